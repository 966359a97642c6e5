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

template <typename T>
__global__ __launch_bounds__(kThreads) void append_wht_kernel(T* __restrict__ cache, const T* __restrict__ rows,
                                                               const int64_t* __restrict__ slots, int d_latent,
                                                               int d_rope) {
  __shared__ float x[kMaxLatent];
  const int64_t i = blockIdx.x;
  const int64_t D = d_latent + d_rope;
  const T* src = rows + i * D;
  T* dst = cache + slots[i] * D;
  for (int j = threadIdx.x; j < d_latent; j += kThreads) x[j] = load_as_f32(src + j);
  block_fwht(x, d_latent);
  for (int j = threadIdx.x; j < d_latent; j += kThreads) dst[j] = store_from_f32<T>(x[j]);
  for (int j = threadIdx.x; j < d_rope; j += kThreads) dst[d_latent + j] = src[d_latent + j];
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
                         int dtype, int wht, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int elem = dtype == 0 ? 4 : 2;
  if (wht) {
    if (d_latent > kMaxLatent || n > 0x7fffffffLL) return hipErrorInvalidValue;
    if (dtype == 0)
      hipLaunchKernelGGL(append_wht_kernel<float>, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream,
                         static_cast<float*>(cache), static_cast<const float*>(rows), slots, d_latent, d_rope);
    else
      hipLaunchKernelGGL(append_wht_kernel<uint16_t>, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream,
                         static_cast<uint16_t*>(cache), static_cast<const uint16_t*>(rows), slots, d_latent, d_rope);
  } else {
    const int row_bytes = (d_latent + d_rope) * elem;
    const int64_t total = n * (row_bytes / 16);
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 256 * 32);
    hipLaunchKernelGGL(append_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       static_cast<unsigned char*>(cache), static_cast<const unsigned char*>(rows), slots, n, row_bytes);
  }
  return hipGetLastError();
}

}  // namespace tpla
