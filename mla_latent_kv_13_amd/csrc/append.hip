// latent_cache_append: store new cache rows [latent | rope key] at their slots.  With the Hadamard
// reparameterisation the latent is rotated first, x <- H x in fp32, then rounded to the cache dtype
// (round to nearest even for bf16); the rope key is copied unchanged (TPLA abstract and the feature
// request's "Directions under investigation": an orthogonal Hadamard transform before slicing).
#include "kernels.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLatent = 1024;

constexpr int kRowsPerBlock = kThreads / 64;  // one wave per appended row

// One wave per row at a time, the grid striding over the rows: lane l holds latent elements
// V*l .. V*l+V-1 (V = d_latent / 64, or 1 with lanes >= d_latent idle), rotated in registers when
// ROT, and rope-key piece l (16 bytes; the first 64 pieces), copied unchanged.  With norm_lanes > 0
// the (rotated) latent is then RMS-normalised with unit gain over slices of norm_lanes * V values:
// each slice's sum of squares is a reduction over the aligned group of lanes holding it, and the
// slice is scaled by 1 / sqrt(mean square + eps).  The next row's loads are issued before this row
// is processed (a wave's last prefetch re-reads row n - 1, unused).
template <typename T, int V, bool ROT>
__global__ __launch_bounds__(kThreads) void append_row_kernel(T* __restrict__ cache, const T* __restrict__ rows,
                                                               const int64_t* __restrict__ slots, int64_t n,
                                                               int d_latent, int d_rope, int norm_lanes, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRowsPerBlock;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t D = d_latent + d_rope;
  const int lanes = d_latent / V;  // lanes holding latent elements (<= 64)
  const bool on = lane < lanes;
  const int pieces = d_rope * static_cast<int>(sizeof(T)) / 16;  // rope key in 16-byte pieces
  const bool rope_on = lane < pieces;
  const float inv_w = norm_lanes > 0 ? 1.0f / static_cast<float>(norm_lanes * V) : 0.f;
  // every lane loads in bounds: idle lanes repeat piece 0 (of the latent when there is no rope)
  auto load = [&](int64_t r, Pack<T, V>& p, uint4& rk) {
    const T* src = rows + r * D;
    p = reinterpret_cast<const Pack<T, V>*>(src)[on ? lane : 0];
    rk = reinterpret_cast<const uint4*>(pieces > 0 ? src + d_latent : src)[rope_on ? lane : 0];
  };
  Pack<T, V> p;
  uint4 rk;
  load(i, p, rk);
  for (; i < n; i += stride) {
    Pack<T, V> pn;
    uint4 rkn;
    load(min(i + stride, n - 1), pn, rkn);
    T* dst = cache + slots[i] * D;
    float x[V];
#pragma unroll
    for (int r = 0; r < V; ++r) x[r] = on ? load_as_f32(&p.v[r]) : 0.f;
    if constexpr (ROT) wave_wht(x, d_latent, lane);
    if (norm_lanes > 0) {
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < V; ++r) ss = fmaf(x[r], x[r], ss);
      ss = group_reduce<false>(ss, norm_lanes);
      const float scale = 1.0f / sqrtf(ss * inv_w + eps);
#pragma unroll
      for (int r = 0; r < V; ++r) x[r] *= scale;
    }
#pragma unroll
    for (int r = 0; r < V; ++r) p.v[r] = store_from_f32<T>(x[r]);
    if (on) reinterpret_cast<Pack<T, V>*>(dst)[lane] = p;
    if (rope_on) reinterpret_cast<uint4*>(dst + d_latent)[lane] = rk;
    for (int k = lane + 64; k < pieces; k += 64)  // rope keys wider than 64 pieces
      reinterpret_cast<uint4*>(dst + d_latent)[k] = reinterpret_cast<const uint4*>(rows + i * D + d_latent)[k];
    p = pn;
    rk = rkn;
  }
}

template <typename T, bool ROT>
hipError_t launch_rows(T* cache, const T* rows, const int64_t* slots, int64_t n, int d_latent, int d_rope,
                       int norm_lanes, float eps, hipStream_t stream) {
  // enough waves to keep every CU busy, each then striding over the rows
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((n + kRowsPerBlock - 1) / kRowsPerBlock, 256 * 16)));
#define TPLA_ROWS(VV) \
  hipLaunchKernelGGL((append_row_kernel<T, VV, ROT>), grid, dim3(kThreads), 0, stream, cache, rows, slots, n, d_latent, \
                     d_rope, norm_lanes, eps)
  switch (d_latent <= 64 ? 1 : d_latent / 64) {
    case 1: TPLA_ROWS(1); break;
    case 2: TPLA_ROWS(2); break;
    case 4: TPLA_ROWS(4); break;
    case 8: TPLA_ROWS(8); break;
    case 16: TPLA_ROWS(16); break;
    default: return hipErrorInvalidValue;
  }
#undef TPLA_ROWS
  return hipGetLastError();
}

// Plain copy of whole rows in 16-byte pieces (row bytes are a multiple of 16).
__global__ __launch_bounds__(kThreads) void append_copy_kernel(unsigned char* __restrict__ cache,
                                                                const unsigned char* __restrict__ rows,
                                                                const int64_t* __restrict__ slots, int64_t n,
                                                                int row_bytes) {
  const int pieces = row_bytes / 16;
  const int64_t total = n * pieces;
  for (int64_t k = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; k < total;
       k += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t i = k / pieces;
    const int p = static_cast<int>(k % pieces);
    const uint4 v = *reinterpret_cast<const uint4*>(rows + i * row_bytes + p * 16);
    *reinterpret_cast<uint4*>(cache + slots[i] * row_bytes + p * 16) = v;
  }
}

}  // namespace

hipError_t launch_append(void* cache, const void* rows, const int64_t* slots, int64_t n, int d_latent, int d_rope,
                         int dtype, int wht, int norm_slices, float eps, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int elem = dtype == 0 ? 4 : 2;
  if (wht || norm_slices > 0) {
    // a power of two up to 1024 (checked with the descriptor); rows in whole 16-byte pieces
    if (d_latent > kMaxLatent || (d_latent & (d_latent - 1)) != 0 || n > 0x7fffffffLL) return hipErrorInvalidValue;
    if ((d_latent * elem) % 16 != 0 || (d_rope * elem) % 16 != 0) return hipErrorInvalidValue;
    int norm_lanes = 0;  // lanes holding one normalised slice
    if (norm_slices > 0) {
      const int v = d_latent <= 64 ? 1 : d_latent / 64;
      const int w = d_latent / norm_slices;
      if (norm_slices > 64 || d_latent % norm_slices != 0 || w % v != 0) return hipErrorInvalidValue;
      norm_lanes = w / v;
    }
    if (dtype == 0) {
      auto* c = static_cast<float*>(cache);
      auto* r = static_cast<const float*>(rows);
      return wht ? launch_rows<float, true>(c, r, slots, n, d_latent, d_rope, norm_lanes, eps, stream)
                 : launch_rows<float, false>(c, r, slots, n, d_latent, d_rope, norm_lanes, eps, stream);
    }
    auto* c = static_cast<uint16_t*>(cache);
    auto* r = static_cast<const uint16_t*>(rows);
    return wht ? launch_rows<uint16_t, true>(c, r, slots, n, d_latent, d_rope, norm_lanes, eps, stream)
               : launch_rows<uint16_t, false>(c, r, slots, n, d_latent, d_rope, norm_lanes, eps, stream);
  }
  const int row_bytes = (d_latent + d_rope) * elem;
  const int64_t total = n * (row_bytes / 16);
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 256 * 32);
  hipLaunchKernelGGL(append_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<unsigned char*>(cache), static_cast<const unsigned char*>(rows), slots, n, row_bytes);
  return hipGetLastError();
}

}  // namespace tpla
