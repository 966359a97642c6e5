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
// V*l .. V*l+V-1 (V = d_latent / 64, or 1 with lanes >= d_latent idle), rotated in registers,
// and rope-key piece l (16 bytes; the first 64 pieces), copied unchanged.  The next row's loads
// are issued before this row is rotated (a wave's last prefetch re-reads row n - 1, unused).
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void append_wht_kernel(T* __restrict__ cache, const T* __restrict__ rows,
                                                               const int64_t* __restrict__ slots, int64_t n,
                                                               int d_latent, int d_rope) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRowsPerBlock;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t D = d_latent + d_rope;
  const int lanes = d_latent / V;  // lanes holding latent elements (<= 64)
  const bool on = lane < lanes;
  const int pieces = d_rope * static_cast<int>(sizeof(T)) / 16;  // rope key in 16-byte pieces
  const bool rope_on = lane < pieces;
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
    wave_wht(x, d_latent, lane);
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

template <typename T>
hipError_t launch_wht(T* cache, const T* rows, const int64_t* slots, int64_t n, int d_latent, int d_rope,
                      hipStream_t stream) {
  // enough waves to keep every CU busy, each then striding over the rows
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((n + kRowsPerBlock - 1) / kRowsPerBlock, 256 * 16)));
  switch (d_latent <= 64 ? 1 : d_latent / 64) {
    case 1: hipLaunchKernelGGL((append_wht_kernel<T, 1>), grid, dim3(kThreads), 0, stream, cache, rows, slots, n, d_latent, d_rope); break;
    case 2: hipLaunchKernelGGL((append_wht_kernel<T, 2>), grid, dim3(kThreads), 0, stream, cache, rows, slots, n, d_latent, d_rope); break;
    case 4: hipLaunchKernelGGL((append_wht_kernel<T, 4>), grid, dim3(kThreads), 0, stream, cache, rows, slots, n, d_latent, d_rope); break;
    case 8: hipLaunchKernelGGL((append_wht_kernel<T, 8>), grid, dim3(kThreads), 0, stream, cache, rows, slots, n, d_latent, d_rope); break;
    case 16: hipLaunchKernelGGL((append_wht_kernel<T, 16>), grid, dim3(kThreads), 0, stream, cache, rows, slots, n, d_latent, d_rope); break;
    default: return hipErrorInvalidValue;
  }
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
                         int dtype, int wht, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int elem = dtype == 0 ? 4 : 2;
  if (wht) {
    // a power of two up to 1024 (checked with the descriptor); rows in whole 16-byte pieces
    if (d_latent > kMaxLatent || (d_latent & (d_latent - 1)) != 0 || n > 0x7fffffffLL) return hipErrorInvalidValue;
    if ((d_latent * elem) % 16 != 0 || (d_rope * elem) % 16 != 0) return hipErrorInvalidValue;
    if (dtype == 0)
      return launch_wht(static_cast<float*>(cache), static_cast<const float*>(rows), slots, n, d_latent, d_rope, stream);
    return launch_wht(static_cast<uint16_t*>(cache), static_cast<const uint16_t*>(rows), slots, n, d_latent, d_rope,
                      stream);
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
