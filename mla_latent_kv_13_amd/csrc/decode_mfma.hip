// bf16 split-K TPLA decode on the gfx950 matrix cores.
//
// Work unit: one workgroup = (token chunk c, sequence b, shard s, group of 32*NW heads).  It
// streams the chunk's cache rows of that shard -- the latent slice [s*W, (s+1)*W) and the whole
// rope key, i.e. the per-device share of the TPLA review page (320 = 256 + 64 values per token
// at two shards) -- from HBM into double-buffered LDS tiles of 32 tokens.  Every wave owns 32
// heads and, per tile:
//   S^T[token, head] = K_tile[token, :] . Q^T[:, head]       32x32x16 bf16 MFMA, K = W + D_R
//   online softmax over tokens per head (per-lane partials, one cross-half max per tile)
//   O^T[col, head]  += V_tile^T[col, token] . P^T[token, head]  32x32x16 bf16 MFMA, K = tokens
// with the value tile read transposed out of LDS by ds_read_b64_tr_b16.  The chunk's normalised
// output and log-sum-exp go to the workspace; the merge kernel combines chunks exactly
// (feature request on latent-cache sharding, "Directions under investigation": sequence split
// plus log-sum-exp merge).  The slice softmax is plain, with the same scale on every shard
// (TPLA abstract; review page, Eq. 6).
//
// Lane layouts (checked on gfx950): for v_mfma_f32_32x32x16_bf16 lane l holds A[l%32][8*(l/32)+i]
// and B[8*(l/32)+i][l%32], i = 0..7, and accumulator j of lane l is D[8*(j/4)+4*(l/32)+j%4][l%32].
// ds_read_b64_tr_b16 lets lane q of each 16-lane group address row q/4, columns 4*(q%4)..+3 of a
// 4 x 16 block and returns column q (rows 0..3).
#include "kernels.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kNT = 32;  // tokens per LDS tile (the M dimension of the QK product)

template <int W, int DR, int NW>
struct Cfg {
  static constexpr int KW = W + DR;                    // key width of one shard
  static constexpr int KSTEPS = KW / 16;               // 16-deep MFMA steps of the QK product
  static constexpr int ROW_BYTES = KW * 2 + 16;        // LDS row pitch: 16 B of padding spreads banks
  static constexpr int TILE_BYTES = kNT * ROW_BYTES;
  static constexpr int CPR = KW / 8;                   // 16-byte chunks per row
  static constexpr int LAT_CPR = W / 8;
  static constexpr int THREADS = NW * 64;
  static constexpr int LOADS = (kNT * CPR + THREADS - 1) / THREADS;
  static constexpr int CB = W / 32;                    // 32-column blocks of the value
  static constexpr int LDS_BYTES = 2 * TILE_BYTES;
  static_assert(W % 32 == 0 && DR % 16 == 0, "tile shape");
};

typedef __attribute__((address_space(3))) short4_t lds_short4_t;

template <int W, int DR, int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(DecodeLaunch a, float scale_log2) {
  using C = Cfg<W, DR, NW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int c = blockIdx.x, b = blockIdx.y;
  const int groups = a.heads / (32 * NW);
  const int s_local = blockIdx.z / groups, hg = blockIdx.z % groups;
  const int s = a.shard_begin + s_local;
  const int T = a.seq_lens[b];
  const int t_begin = c * a.chunk_tokens;
  if (t_begin >= T) return;
  const int t_end = min(T, t_begin + a.chunk_tokens);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int head = (hg * NW + wv) * 32 + l32;
  const int d_c = a.d_latent;
  const int64_t D = d_c + DR;
  const uint16_t* __restrict__ cache = static_cast<const uint16_t*>(a.cache);

  // Q^T operand of the QK product: lane holds features 16*kk + 8*half .. +7 of its head.
  uint4 qf[C::KSTEPS];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + (static_cast<int64_t>(b) * a.heads + head) * d_c + s * W;
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + (static_cast<int64_t>(b) * a.heads + head) * DR;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int f = 16 * kk + 8 * half;
      qf[kk] = (f < W) ? *reinterpret_cast<const uint4*>(ql + f) : *reinterpret_cast<const uint4*>(qr + (f - W));
    }
  }

  uint4 stage[C::LOADS];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int k = 0; k < C::LOADS; ++k) {
      const int idx = tid + k * C::THREADS;
      const int tok = idx / C::CPR, ch = idx % C::CPR;
      const int t = t0 + tok;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (idx < kNT * C::CPR && t < t_end) {
        const int64_t row = cache_row(a.block_table, b, t, a.page_size, a.max_pages_per_seq);
        const int64_t col = (ch < C::LAT_CPR) ? static_cast<int64_t>(s) * W + ch * 8 : d_c + (ch - C::LAT_CPR) * 8;
        v = *reinterpret_cast<const uint4*>(cache + row * D + col);
      }
      stage[k] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int k = 0; k < C::LOADS; ++k) {
      const int idx = tid + k * C::THREADS;
      if (idx < kNT * C::CPR) {
        const int tok = idx / C::CPR, ch = idx % C::CPR;
        *reinterpret_cast<uint4*>(lds + buf * C::TILE_BYTES + tok * C::ROW_BYTES + ch * 16) = stage[k];
      }
    }
  };

  floatx16_t o_acc[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int j = 0; j < 16; ++j) o_acc[cb][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(t_begin);
  store_tile(0);
  __syncthreads();

  int buf = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += kNT) {
    const bool has_next = t0 + kNT < t_end;
    if (has_next) load_tile(t0 + kNT);
    const unsigned char* tile = lds + buf * C::TILE_BYTES;

    // S^T = K_tile . Q^T  (lane: head l32, tokens 8*(j/4) + 4*half + j%4)
    floatx16_t sacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const uint4 kv = *reinterpret_cast<const uint4*>(tile + l32 * C::ROW_BYTES + (16 * kk + 8 * half) * 2);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                     __builtin_bit_cast(bf16x8_t, qf[kk]), sacc, 0, 0, 0);
    }

    // Online softmax in base 2 (log2 e folded into the scale).
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int tok = 8 * (j >> 2) + 4 * half + (j & 3);
      const float v = (t0 + tok < t_end) ? sacc[j] * scale_log2 : -INFINITY;
      x[j] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);  // finite: every tile holds at least one valid token
    const float alpha = exp2f(m_run - m_new);
    uint32_t pk[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = exp2f(x[2 * i] - m_new), p1 = exp2f(x[2 * i + 1] - m_new);
      psum += p0 + p1;
      pk[i] = pack_bf16x2(p0, p1);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int j = 0; j < 16; ++j) o_acc[cb][j] *= alpha;
    }

    // O^T += V_tile^T . P^T.  k-step ks covers tokens 16*ks .. 16*ks+15 in the order the softmax
    // registers hold them: operand slot 8*half + i <-> token 16*ks + 8*(i/4) + 4*half + i%4.
    const int grp = lane >> 4, q = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]));
      const int row0 = 16 * ks + 4 * half + (q >> 2);
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) {
        const int col = 32 * cb + 16 * (grp & 1) + 4 * (q & 3);
        const unsigned char* p0 = tile + row0 * C::ROW_BYTES + col * 2;
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p0));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p0 + 8 * C::ROW_BYTES));
        const short8_t v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o_acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v8), pb, o_acc[cb], 0, 0, 0);
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // Chunk result: o = O / l, lse = ln 2 * (m + log2 l); the two lane halves hold disjoint tokens.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const int64_t part = ((static_cast<int64_t>(b) * a.num_chunks + c) * a.shard_count + s_local) * a.heads + head;
  float* dst = a.part_o + part * W;
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int col = 32 * cb + 8 * j4 + 4 * half;
      const float4 v = make_float4(o_acc[cb][4 * j4] * inv, o_acc[cb][4 * j4 + 1] * inv, o_acc[cb][4 * j4 + 2] * inv,
                                   o_acc[cb][4 * j4 + 3] * inv);
      *reinterpret_cast<float4*>(dst + col) = v;
    }
  if (half == 0) a.part_lse[part] = (m_run + log2f(l_tot)) * kLn2;
}

template <int W, int DR, int NW>
hipError_t launch_one(const DecodeLaunch& a, hipStream_t stream) {
  using C = Cfg<W, DR, NW>;
  auto kern = decode_mfma_kernel<W, DR, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const dim3 grid(a.num_chunks, a.batch, a.shard_count * (a.heads / (32 * NW)));
  const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
  hipLaunchKernelGGL(kern, grid, dim3(C::THREADS), C::LDS_BYTES, stream, a, scale_log2);
  return hipGetLastError();
}

template <int W, int DR>
hipError_t launch_w(const DecodeLaunch& a, hipStream_t stream) {
  if (a.heads % 128 == 0) return launch_one<W, DR, 4>(a, stream);
  if (a.heads % 64 == 0) return launch_one<W, DR, 2>(a, stream);
  return launch_one<W, DR, 1>(a, stream);
}

}  // namespace

bool mfma_supported(int w, int d_rope, int heads) {
  return (w == 128 || w == 256 || w == 512) && d_rope == 64 && heads % 32 == 0;
}

hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t stream) {
  if (!mfma_supported(a.w, a.d_rope, a.heads)) return hipErrorInvalidValue;
  switch (a.w) {
    case 128: return launch_w<128, 64>(a, stream);
    case 256: return launch_w<256, 64>(a, stream);
    default: return launch_w<512, 64>(a, stream);
  }
}

}  // namespace tpla
