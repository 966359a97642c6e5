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
constexpr int kMaxChunks = 4096;

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeLaunch a) {
  __shared__ float y[kMaxLatent];
  __shared__ float wts[kMaxChunks];
  __shared__ float scratch[16];
  const int h = blockIdx.x, b = blockIdx.y;
  const int T = a.seq_lens[b];
  const int nv = (T + a.chunk_tokens - 1) / a.chunk_tokens;  // chunks holding tokens
  for (int j = threadIdx.x; j < a.d_latent; j += kThreads) y[j] = 0.f;

  for (int sl = 0; sl < a.shard_count; ++sl) {
    const int s = a.shard_begin + sl;
    const int64_t stride = static_cast<int64_t>(a.shard_count) * a.heads;  // between chunks
    const int64_t base = (static_cast<int64_t>(b) * a.num_chunks * a.shard_count + sl) * a.heads + h;
    float mx = -INFINITY;
    for (int k = threadIdx.x; k < nv; k += kThreads) mx = fmaxf(mx, a.part_lse[base + k * stride]);
    const float M = block_max(mx, scratch);
    float sum = 0.f;
    for (int k = threadIdx.x; k < nv; k += kThreads) {
      const float e = expf(a.part_lse[base + k * stride] - M);
      wts[k] = e;
      sum += e;
    }
    const float Z = block_sum(sum, scratch);  // also publishes wts[]
    const float lse_s = (nv > 0) ? M + logf(Z) : -INFINITY;
    const float invZ = (nv > 0) ? 1.0f / Z : 0.f;
    for (int j = threadIdx.x; j < a.w; j += kThreads) {
      float acc = 0.f;
      for (int k = 0; k < nv; ++k) acc = fmaf(wts[k], a.part_o[(base + k * stride) * a.w + j], acc);
      y[s * a.w + j] = acc * invZ;
    }
    if (a.lse != nullptr && threadIdx.x == 0) a.lse[(static_cast<int64_t>(b) * a.shard_count + sl) * a.heads + h] = lse_s;
    __syncthreads();
  }
  if (a.wht) block_fwht(y, a.d_latent);
  __syncthreads();
  float* dst = a.out + (static_cast<int64_t>(b) * a.heads + h) * a.d_latent;
  for (int j = threadIdx.x; j < a.d_latent; j += kThreads) dst[j] = y[j];
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

}  // namespace

hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream) {
  if (a.d_latent > kMaxLatent || a.num_chunks > kMaxChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3(a.heads, a.batch), dim3(kThreads), 0, stream, a);
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
