// Value up-projection of a decode result: out_v[b, h, :] = W_UV[h] . o[b, h, :].
//
// With the key up-projection absorbed into the query, attention runs in latent space and each
// head's value rows of kv_b_proj (W_UV[h], d_v x d_latent) are applied afterwards (automated review
// of the TPLA paper, referee report "significance": matrix absorption; feature request on
// latent-cache sharding, "Background / problem": kv_b_proj sharded per head, o_proj rowwise, then
// the all-reduce).  Applied to one device's shard subset it yields that device's operand of the
// all-reduce.
//
// Per head this is a [batch x d_latent] . [d_latent x d_v] product, so it runs on the matrix cores:
// one workgroup per 32 batch rows x 32 value columns of one head, its four waves splitting the
// latent (32x32x16 bf16 MFMAs), all of a wave's operand loads in flight at once.
// The fp32 input o enters as a bf16 value plus the bf16 remainder o - bf16(o) (two products into
// the same fp32 accumulators), so about 16 significant bits of o take part; W_UV is bf16 as stored.
// HBM-bound: each weight row is read once per 32 batch rows.
#include <type_traits>

#include "kernels.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kSplit = 4;           // waves of a workgroup, each taking a quarter of the latent
constexpr int kChunk = 64;          // latent values of a wave's tiles staged at a time (4 k-steps)
constexpr int kOStride = kChunk + 4;  // floats per staged row of o (16-byte pad: rows shift banks)
constexpr int kWStride = kChunk + 8;  // bf16 per staged row of W_UV (16-byte pad)

// Workgroup = one 32 x 32 output tile (32 batch rows, 32 value columns) of one head; wave q sums the
// k-steps [q K / 4, (q + 1) K / 4) and the four partial tiles are added in LDS in wave order.  A
// wave stages its rows of o and W_UV through its own LDS region, 64 latent values at a time, with
// loads that cover whole 256-byte (o) and 128-byte (W_UV) row pieces, two chunks in flight; the
// MFMA operands are then read from LDS.  Operand layout (32x32x16 bf16): lane l holds
// A[l % 32][8 (l / 32) + i] and B[8 (l / 32) + i][l % 32], i < 8; accumulator r of lane l is
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__global__ __launch_bounds__(64 * kSplit) void up_project_mfma_kernel(const float* __restrict__ o,
                                                                      const uint16_t* __restrict__ w, int batch,
                                                                      int heads, int d_c, int d_v,
                                                                      float* __restrict__ out, int xcds) {
  __shared__ __attribute__((aligned(16))) float o_s[kSplit][32 * kOStride];  // also the partial tiles, at the end
  __shared__ __attribute__((aligned(16))) uint16_t w_s[kSplit][32 * kWStride];
  static_assert(sizeof(o_s) >= (kSplit - 1) * 4 * 64 * sizeof(floatx4_t), "partial tiles fit the staging area");
  const int lane = threadIdx.x & 63, wq = threadIdx.x >> 6;
  // Workgroup id -> (head, batch tile) unit and value tile.  Workgroups are dealt to the device's
  // XCDs round-robin by id; the value tiles of one unit all get ids = unit (mod xcds), so they run
  // on one XCD and read the unit's rows of o through that XCD's L2 once.  Ids past the last unit
  // exit.
  const int vtiles = (d_v + 31) / 32;
  const int xcd = blockIdx.x % xcds, k = blockIdx.x / xcds;
  const int unit = (k / vtiles) * xcds + xcd;
  if (unit >= heads * ((batch + 31) / 32)) return;
  const int v0 = (k % vtiles) * 32, h = unit % heads, b0 = (unit / heads) * 32;
  const int half = lane >> 5, l32 = lane & 31;
  const int ksteps = d_c / 16;
  const int kb = wq * ksteps / kSplit, ke = (wq + 1) * ksteps / kSplit;
  const int nchunks = (ke - kb + 3) / 4;

  // Staging: o rows 4 i + lane / 16, floats 4 (lane % 16) ..; W_UV rows 8 i + lane / 8, values
  // 8 (lane % 8) ...  Rows past the end repeat the last valid row, and pieces past the latent
  // (a chunk overhanging the wave's range, or a wave without k-steps) repeat its last piece; none
  // of these is used.
  const int ob = min(b0 + (lane >> 4), batch - 1), wv = min(v0 + (lane >> 3), d_v - 1);
  float* os = o_s[wq];
  uint16_t* ws = w_s[wq];
  // Two register sets of staged pieces, selected at compile time (S = 0 or 1).
  float4 of0[8], of1[8];
  uint4 wf0[4], wf1[4];
  auto load = [&](auto set, int c) {
    constexpr int S = decltype(set)::value;
    const int kc = 16 * kb + kChunk * min(c, max(nchunks - 1, 0));
    const int co = min(kc + 4 * (lane & 15), d_c - 4), cw = min(kc + 8 * (lane & 7), d_c - 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int b = min(ob + 4 * i, batch - 1);
      const float4 x = *reinterpret_cast<const float4*>(o + (static_cast<int64_t>(b) * heads + h) * d_c + co);
      if constexpr (S == 0) of0[i] = x; else of1[i] = x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = min(wv + 8 * i, d_v - 1);
      const uint4 x = *reinterpret_cast<const uint4*>(w + (static_cast<int64_t>(h) * d_v + v) * d_c + cw);
      if constexpr (S == 0) wf0[i] = x; else wf1[i] = x;
    }
  };
  floatx16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // One staged chunk: write it to LDS, then its (up to) four k-steps.
  auto process = [&](auto set, int c) {
    constexpr int S = decltype(set)::value;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the previous chunk's reads are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<float4*>(os + (4 * i + (lane >> 4)) * kOStride + 4 * (lane & 15)) = S == 0 ? of0[i] : of1[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(ws + (8 * i + (lane >> 3)) * kWStride + 8 * (lane & 7)) = S == 0 ? wf0[i] : wf1[i];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // this wave's chunk is in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (kb + 4 * c + s < ke) {
        const float4 a0 = *reinterpret_cast<const float4*>(os + l32 * kOStride + 16 * s + 8 * half);
        const float4 a1 = *reinterpret_cast<const float4*>(os + l32 * kOStride + 16 * s + 8 * half + 4);
        const uint4 bw4 = *reinterpret_cast<const uint4*>(ws + l32 * kWStride + 16 * s + 8 * half);
        const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
          const float r0 = x[2 * i] - bf16_to_f32(static_cast<uint16_t>(hi[i] & 0xffffu));
          const float r1 = x[2 * i + 1] - bf16_to_f32(static_cast<uint16_t>(hi[i] >> 16));
          lo[i] = pack_bf16x2(r0, r1);
        }
        const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, bw4);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3])), bw, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3])), bw, acc, 0, 0, 0);
      }
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  load(Set0{}, 0);
  if (nchunks > 1) load(Set1{}, 1);
  for (int c = 0; c < nchunks; c += 2) {
    process(Set0{}, c);
    if (c + 2 < nchunks) load(Set0{}, c + 2);
    if (c + 1 < nchunks) {
      process(Set1{}, c + 1);
      if (c + 3 < nchunks) load(Set1{}, c + 3);
    }
  }
  __syncthreads();  // every wave is done with its staging area
  floatx4_t* part = reinterpret_cast<floatx4_t*>(&o_s[0][0]);  // [kSplit - 1][4][64]
  if (wq > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      part[((wq - 1) * 4 + j) * 64 + lane] = floatx4_t{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
  }
  __syncthreads();
  if (wq > 0) return;
#pragma unroll
  for (int q = 0; q < kSplit - 1; ++q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4_t t = part[(q * 4 + j) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * j + e] += t[e];
    }
  }
  const int vv = v0 + l32;
  if (vv >= d_v) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bb = b0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (bb < batch) out[(static_cast<int64_t>(bb) * heads + h) * d_v + vv] = acc[r];
  }
}

// fp32 weights, or latent widths the matrix-core tiles do not cover: one thread per output.
template <typename T>
__global__ __launch_bounds__(256) void up_project_generic_kernel(const float* __restrict__ o, const T* __restrict__ w,
                                                                 int batch, int heads, int d_c, int d_v,
                                                                 float* __restrict__ out) {
  const int64_t total = static_cast<int64_t>(batch) * heads * d_v;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int v = static_cast<int>(idx % d_v);
    const int64_t bh = idx / d_v;
    const int h = static_cast<int>(bh % heads);
    const float* a = o + bh * d_c;
    const T* wr = w + (static_cast<int64_t>(h) * d_v + v) * d_c;
    float acc = 0.f;
    for (int c = 0; c < d_c; ++c) acc = fmaf(a[c], load_as_f32(wr + c), acc);
    out[idx] = acc;
  }
}

}  // namespace

hipError_t launch_up_project(const float* o, const void* w_uv, int w_dtype, int batch, int heads, int d_latent,
                             int d_v, float* out_v, int xcds, hipStream_t stream) {
  if (batch == 0 || heads == 0) return hipSuccess;
  if (xcds < 1) return hipErrorInvalidValue;
  if (w_dtype == 1 && d_latent % 16 == 0) {
    const int64_t units = static_cast<int64_t>(heads) * ((batch + 31) / 32), vt = (d_v + 31) / 32;
    const int64_t blocks = (units + xcds - 1) / xcds * xcds * vt;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(blocks));
    hipLaunchKernelGGL(up_project_mfma_kernel, grid, dim3(64 * kSplit), 0, stream, o,
                       static_cast<const uint16_t*>(w_uv), batch, heads, d_latent, d_v, out_v, xcds);
  } else {
    const int64_t total = static_cast<int64_t>(batch) * heads * d_v;
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 256 * 64));
    if (w_dtype == 1)
      hipLaunchKernelGGL(up_project_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, o,
                         static_cast<const uint16_t*>(w_uv), batch, heads, d_latent, d_v, out_v);
    else
      hipLaunchKernelGGL(up_project_generic_kernel<float>, dim3(blocks), dim3(256), 0, stream, o,
                         static_cast<const float*>(w_uv), batch, heads, d_latent, d_v, out_v);
  }
  return hipGetLastError();
}

}  // namespace tpla
