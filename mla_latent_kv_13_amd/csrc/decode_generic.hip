// Generic split-K TPLA decode kernel (VALU, fp32 arithmetic) for any supported shape and for
// fp32 caches.  One workgroup computes one (chunk, sequence, shard, head): the logits of the
// chunk's tokens, their softmax, and the normalised chunk output with its log-sum-exp, which
// the merge kernel combines across chunks ("Directions under investigation" of the feature
// request on latent-cache sharding: sequence split with a log-sum-exp merge).  Per shard the
// logit is scale * (latent-slice dot + whole rope dot) and the value is the latent slice
// (TPLA abstract; review page, Eq. 6: a plain softmax per slice).
#include "kernels.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunk = 2048;     // tokens per chunk (logits and row offsets kept in LDS)
constexpr int kMaxKey = 1024 + 256; // w + d_rope

template <typename E>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(DecodeLaunch a) {
  __shared__ float q[kMaxKey];
  __shared__ float prob[kMaxChunk];
  __shared__ int64_t rowoff[kMaxChunk];
  __shared__ float scratch[16];

  const int c = blockIdx.x, b = blockIdx.y;
  const int s_local = blockIdx.z / a.heads, h = blockIdx.z % a.heads;
  const int s = a.shard_begin + s_local;
  const int T = a.seq_lens[b];
  const int t0 = c * a.chunk_tokens;
  if (t0 >= T) return;
  const int n = min(T - t0, a.chunk_tokens);
  const int w = a.w, d_r = a.d_rope, d_c = a.d_latent;
  const int64_t D = d_c + d_r;
  const E* cache = static_cast<const E*>(a.cache);

  const int64_t qrow = static_cast<int64_t>(b) * a.heads + h;
  for (int j = threadIdx.x; j < w; j += kThreads) {
    q[j] = a.q_lat_f32 ? static_cast<const float*>(a.q_lat)[qrow * d_c + s * w + j]
                       : load_as_f32(static_cast<const E*>(a.q_lat) + qrow * d_c + s * w + j);
  }
  for (int j = threadIdx.x; j < d_r; j += kThreads) q[w + j] = load_as_f32(static_cast<const E*>(a.q_rope) + qrow * d_r + j);
  const int bs = a.row_seq ? a.row_seq[b] : b;  // cache sequence of query row b
  for (int i = threadIdx.x; i < n; i += kThreads)
    rowoff[i] = cache_row(a.block_table, bs, t0 + i, a.page_size, a.max_pages_per_seq) * D;
  __syncthreads();

  float local_max = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const E* row = cache + rowoff[i];
    float acc = 0.f;
    for (int j = 0; j < w; ++j) acc = fmaf(q[j], load_as_f32(row + s * w + j), acc);
    for (int j = 0; j < d_r; ++j) acc = fmaf(q[w + j], load_as_f32(row + d_c + j), acc);
    const float logit = acc * a.scale;
    prob[i] = logit;
    local_max = fmaxf(local_max, logit);
  }
  const float m = block_max(local_max, scratch);
  float local_sum = 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const float p = expf(prob[i] - m);
    prob[i] = p;
    local_sum += p;
  }
  const float l = block_sum(local_sum, scratch);  // also orders the prob[] writes before the reads below
  const float inv = 1.0f / l;

  const int64_t part = ((static_cast<int64_t>(b) * a.num_chunks + c) * a.shard_count + s_local) * a.heads + h;
  float* dst = a.part_o + part * w;
  for (int j = threadIdx.x; j < w; j += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < n; ++i) acc = fmaf(prob[i], load_as_f32(cache + rowoff[i] + s * w + j), acc);
    dst[j] = acc * inv;
  }
  if (threadIdx.x == 0) a.part_lse[part] = m + logf(l);
}

}  // namespace

hipError_t launch_decode_generic(const DecodeLaunch& a, int dtype, hipStream_t stream) {
  if (a.chunk_tokens > kMaxChunk || a.w + a.d_rope > kMaxKey) return hipErrorInvalidValue;
  const dim3 grid(a.num_chunks, a.batch, a.shard_count * a.heads);
  if (dtype == 0)
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tpla
