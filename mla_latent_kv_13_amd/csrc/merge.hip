// Split-K merge, shard sum and Hadamard rotations.
//
// merge: for each (sequence b, head h) and each computed shard, the chunk partials (o_k, lse_k)
//   are combined exactly by log-sum-exp, in chunk order: M = max lse_k, lse = M + ln sum e^(lse_k-M),
//   o = sum_k e^(lse_k - lse) o_k (feature request on latent-cache sharding, "Directions under
//   investigation": sequence split with a log-sum-exp merge).  Shard outputs are placed in their
//   latent columns and summed -- the in-device stand-in for the all-reduce after the row-parallel
//   output projection (TPLA abstract; feature request, "Directions").  With the Hadamard-rotated
//   cache the summed row is rotated back, out = H y.
// rotate_query: q~ = H q_lat for a Hadamard-rotated cache, so that logits are unchanged at G = 1
//   (TPLA abstract: an orthogonal transform before slicing).
#include "kernels.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLatent = 1024;
constexpr int kMergeWaves = kThreads / 64;  // one (sequence, head) per wave

// In-place orthonormal Walsh-Hadamard transform (Sylvester order) of the n values a wave holds as
// x[r] = v[lane + 64 r] (n a power of two <= 1024; lanes >= n idle when n < 64): radix-2 butterflies
// on pairs (i, i + span), across lanes for span < 64 and across registers above, then 1/sqrt(n).
__device__ __forceinline__ void wave_fwht(float (&x)[kMaxLatent / 64], int n, int lane) {
  const int lanes = n < 64 ? n : 64;
  for (int span = 1; span < lanes; span <<= 1) {
#pragma unroll
    for (int r = 0; r < kMaxLatent / 64; ++r) {
      const float other = __shfl_xor(x[r], span);
      x[r] = (lane & span) ? other - x[r] : x[r] + other;
    }
  }
  const int regs = n / 64;
  for (int sr = 1; sr < regs; sr <<= 1) {
#pragma unroll
    for (int r = 0; r < kMaxLatent / 64; ++r) {
      if ((r & sr) == 0 && r + sr < kMaxLatent / 64) {
        const float u = x[r], v = x[r + sr];
        x[r] = u + v;
        x[r + sr] = u - v;
      }
    }
  }
  const float norm = 1.0f / sqrtf(static_cast<float>(n));
#pragma unroll
  for (int r = 0; r < kMaxLatent / 64; ++r) x[r] *= norm;
}

// Columns a lane accumulates at once: V = 4 (float4; slice width a multiple of 4) or 1.
template <int V>
struct Vec;
template <>
struct Vec<4> {
  typedef float4 T;
  static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ void fma(float w, const T& v, T& acc) {
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
};
template <>
struct Vec<1> {
  typedef float T;
  static __device__ __forceinline__ T zero() { return 0.f; }
  static __device__ __forceinline__ void fma(float w, const T& v, T& acc) { acc = fmaf(w, v, acc); }
};

template <int V>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeLaunch a) {
  typedef typename Vec<V>::T vec_t;
  __shared__ __attribute__((aligned(16))) float ybuf[kMergeWaves][kMaxLatent];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * kMergeWaves + wv, b = blockIdx.y;
  if (h >= a.heads) return;  // the rest of this kernel is wave-local
  float* y = ybuf[wv];
  // Partials of sequence b: nv consecutive slots from slot0 (chunks holding tokens, or the
  // workers whose tile share meets the sequence under the balanced schedule).
  int nv;
  int64_t slot0;
  if (a.sched == 0) {
    const int T = a.seq_lens[b];
    nv = (T + a.chunk_tokens - 1) / a.chunk_tokens;
    slot0 = static_cast<int64_t>(b) * a.num_chunks;
  } else {
    const int64_t total = a.tile_prefix[a.batch];
    const int64_t p0 = a.tile_prefix[b], p1 = a.tile_prefix[b + 1];
    const int64_t nw = min(static_cast<int64_t>(a.workers), total);  // workers that took part
    // worker holding tile t: the largest w with floor(w * total / nw) <= t
    auto worker_of = [&](int64_t t) { return ((t + 1) * nw - 1) / total; };
    nv = p1 > p0 ? static_cast<int>(worker_of(p1 - 1) - worker_of(p0) + 1) : 0;
    slot0 = p1 > p0 ? b + worker_of(p0) : 0;
  }
  const int lo = a.shard_begin * a.w, hi = lo + a.shard_count * a.w;
  for (int j = lane; j < a.d_latent; j += 64)
    if (j < lo || j >= hi) y[j] = 0.f;  // latent columns of shards that were not computed

  const int64_t stride = static_cast<int64_t>(a.shard_count) * a.heads;  // partial rows between chunks
  const int wv_cols = a.w / V;                                              // vectors per slice row
  for (int sl = 0; sl < a.shard_count; ++sl) {
    const int s = a.shard_begin + sl;
    const int64_t base = (slot0 * a.shard_count + sl) * a.heads + h;
    float mx = -INFINITY;
    for (int k = lane; k < nv; k += 64) mx = fmaxf(mx, a.part_lse[base + k * stride]);
    const float M = wave_max(mx);
    float z = 0.f;
    for (int k = lane; k < nv; k += 64) z += expf(a.part_lse[base + k * stride] - M);
    const float Z = wave_sum(z);
    const float invZ = nv > 0 ? 1.0f / Z : 0.f;
    // Lane c accumulates vectors c and c + 64 of the slice row.  Chunk weights are taken 64 at a
    // time (lane k holds chunk g + k's) and broadcast with readlane; four chunks' loads are issued
    // together so that enough of them are in flight.
    for (int c0 = 0; c0 < wv_cols; c0 += 128) {
      const bool on0 = c0 + lane < wv_cols, on1 = c0 + 64 + lane < wv_cols;
      vec_t acc0 = Vec<V>::zero(), acc1 = Vec<V>::zero();
      for (int g = 0; g < nv; g += 64) {
        const float wl = g + lane < nv ? expf(a.part_lse[base + (g + lane) * stride] - M) * invZ : 0.f;
        const int kn = min(64, nv - g);
        for (int kk = 0; kk < kn; kk += 4) {
          vec_t v0[4], v1[4];
          float wt[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool ok = kk + u < kn;
            wt[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), (kk + u) & 63)) : 0.f;
            const vec_t* src = reinterpret_cast<const vec_t*>(a.part_o + (base + (ok ? g + kk + u : g) * stride) * a.w) + c0 + lane;
            v0[u] = on0 && ok ? src[0] : Vec<V>::zero();
            v1[u] = on1 && ok ? src[64] : Vec<V>::zero();
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            Vec<V>::fma(wt[u], v0[u], acc0);
            Vec<V>::fma(wt[u], v1[u], acc1);
          }
        }
      }
      vec_t* yd = reinterpret_cast<vec_t*>(y + s * a.w) + c0 + lane;
      if (on0) yd[0] = acc0;
      if (on1) yd[64] = acc1;
    }
    if (a.lse != nullptr && lane == 0)
      a.lse[(static_cast<int64_t>(b) * a.shard_count + sl) * a.heads + h] = nv > 0 ? M + logf(Z) : -INFINITY;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // this wave's LDS row is complete
  __builtin_amdgcn_wave_barrier();

  float x[kMaxLatent / 64];
#pragma unroll
  for (int r = 0; r < kMaxLatent / 64; ++r) {
    const int j = lane + 64 * r;
    x[r] = j < a.d_latent ? y[j] : 0.f;
  }
  if (a.wht) wave_fwht(x, a.d_latent, lane);
  float* dst = a.out + (static_cast<int64_t>(b) * a.heads + h) * a.d_latent;
#pragma unroll
  for (int r = 0; r < kMaxLatent / 64; ++r) {
    const int j = lane + 64 * r;
    if (j < a.d_latent) dst[j] = x[r];
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void rotate_query_kernel(const T* __restrict__ q, int d_latent, void* dst,
                                                                 int dst_f32) {
  __shared__ float x[kMaxLatent];
  const int64_t r = blockIdx.x;
  for (int j = threadIdx.x; j < d_latent; j += kThreads) x[j] = load_as_f32(q + r * d_latent + j);
  block_fwht(x, d_latent);
  if (dst_f32) {
    float* o = static_cast<float*>(dst) + r * d_latent;
    for (int j = threadIdx.x; j < d_latent; j += kThreads) o[j] = x[j];
  } else {
    uint16_t* o = static_cast<uint16_t*>(dst) + r * d_latent;
    for (int j = threadIdx.x; j < d_latent; j += kThreads) o[j] = f32_to_bf16(x[j]);
  }
}

// tile_prefix[b] = sum_{b' < b} ceil(seq_lens[b'] / 32) for b = 0..batch, one block: each thread
// sums a contiguous run of sequences, then an exclusive scan over the threads' sums.
__global__ __launch_bounds__(kThreads) void tile_prefix_kernel(const int* __restrict__ seq_lens, int batch,
                                                               int* __restrict__ prefix) {
  __shared__ int sums[kThreads];
  const int per = (batch + kThreads - 1) / kThreads;
  const int b0 = threadIdx.x * per, b1 = min(batch, b0 + per);
  int own = 0;
  for (int b = b0; b < b1; ++b) own += (seq_lens[b] + 31) >> 5;
  sums[threadIdx.x] = own;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = threadIdx.x >= off ? sums[threadIdx.x - off] : 0;
    __syncthreads();
    sums[threadIdx.x] += v;
    __syncthreads();
  }
  int run = sums[threadIdx.x] - own;  // exclusive
  for (int b = b0; b < b1; ++b) {
    prefix[b] = run;
    run += (seq_lens[b] + 31) >> 5;
  }
  if (threadIdx.x == kThreads - 1) prefix[batch] = sums[kThreads - 1];
}

}  // namespace

hipError_t launch_tile_prefix(const int* seq_lens, int batch, int* tile_prefix, hipStream_t stream) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(kThreads), 0, stream, seq_lens, batch, tile_prefix);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream) {
  if (a.d_latent > kMaxLatent) return hipErrorInvalidValue;
  if (a.wht && (a.d_latent & (a.d_latent - 1)) != 0) return hipErrorInvalidValue;
  const dim3 grid((a.heads + kMergeWaves - 1) / kMergeWaves, a.batch);
  if (a.w % 4 == 0)
    hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<1>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rotate_query(const void* q_lat, int dtype, int rows, int d_latent, void* dst, int dst_f32,
                               hipStream_t stream) {
  if (d_latent > kMaxLatent) return hipErrorInvalidValue;
  if (dtype == 0)
    hipLaunchKernelGGL(rotate_query_kernel<float>, dim3(rows), dim3(kThreads), 0, stream,
                       static_cast<const float*>(q_lat), d_latent, dst, dst_f32);
  else
    hipLaunchKernelGGL(rotate_query_kernel<uint16_t>, dim3(rows), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q_lat), d_latent, dst, dst_f32);
  return hipGetLastError();
}

}  // namespace tpla
