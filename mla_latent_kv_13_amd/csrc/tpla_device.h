// Device-side helpers shared by the HIP kernels of the latent-cache decode library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994530942f;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }

// float -> bf16 bit pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two bf16 (round to nearest even) packed in one word, low half = a.
// Uses the gfx950 packed conversion; the vector is read back whole, never per element.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  floatx2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ T store_from_f32(float v);
template <>
__device__ __forceinline__ float store_from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t store_from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

// Block-wide reductions over blockDim.x threads (a multiple of 64); `scratch` holds >= 16 floats.
__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wv] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, scratch[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wv] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < nw; ++i) r += scratch[i];
  return r;
}

// V elements of T read or written as one aligned access.
template <typename T, int V>
struct alignas(sizeof(T) * V) Pack {
  T v[V];
};

// Lane v's value from another lane of its row of 16 (DPP; every lane reads a valid source).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Maximum (MAX) or sum over aligned groups of gw lanes (gw a power of two <= 64); every lane of a
// group receives its group's result.  Below 16 lanes: DPP swaps of lane pairs (lane ^ 1, lane ^ 2),
// then of the two quads of each 8 and the two halves of each 16 (mirrors).
template <bool MAX>
__device__ __forceinline__ float group_reduce(float v, int gw) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if (gw > 1) v = op(v, dpp_mov<0xb1>(v));   // quad_perm(1, 0, 3, 2)
  if (gw > 2) v = op(v, dpp_mov<0x4e>(v));   // quad_perm(2, 3, 0, 1)
  if (gw > 4) v = op(v, dpp_mov<0x141>(v));  // row_half_mirror
  if (gw > 8) v = op(v, dpp_mov<0x140>(v));  // row_mirror
  if (gw > 16) v = op(v, __shfl_xor(v, 16));
  if (gw > 32) v = op(v, __shfl_xor(v, 32));
  return v;
}

// One butterfly of a Walsh-Hadamard stage across lanes: the pair (lane, lane ^ M) becomes
// (a + c, a - c), a the value of the lane with bit M clear.  The partner's value comes from a
// VALU lane swap: DPP within rows of 16 (M = 4: the half-row mirror, then the quad reversal,
// lands on lane ^ 4), permlane swaps across rows (results: lane with bit M clear, lane with it set).
template <int M>
__device__ __forceinline__ float wht_lane_pair(float x, int lane) {
  if constexpr (M >= 16) {
    const auto sw = M == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                            : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float lo = __uint_as_float(sw[0]), hi = __uint_as_float(sw[1]);
    return __builtin_fmaf(hi, (lane & M) ? -1.0f : 1.0f, lo);  // lo -/+ hi, one rounding
  } else {
    float other;
    if constexpr (M == 1) other = dpp_mov<0xb1>(x);                 // quad_perm(1, 0, 3, 2)
    else if constexpr (M == 2) other = dpp_mov<0x4e>(x);            // quad_perm(2, 3, 0, 1)
    else if constexpr (M == 4) other = dpp_mov<0x1b>(dpp_mov<0x141>(x));  // row_half_mirror, quad_perm(3, 2, 1, 0)
    else other = dpp_mov<0x128>(x);                                  // row_ror:8
    return __builtin_fmaf(x, (lane & M) ? -1.0f : 1.0f, other);  // other -/+ x, one rounding
  }
}

// In-register orthonormal Walsh-Hadamard transform (Sylvester order) of n values held V per
// lane: element e = V * lane + r is x[r], n = V * lanes with lanes = n / V a power of two: 64
// when V > 1, up to 64 when V = 1 (lanes past n hold values that are never used).  Butterflies on pairs (e, e + span), span
// increasing: within a lane's registers while span < V, then across lanes; then 1/sqrt(n).
template <int V>
__device__ __forceinline__ void wave_wht(float (&x)[V], int n, int lane) {
#pragma unroll
  for (int span = 1; span < V; span <<= 1) {
#pragma unroll
    for (int r = 0; r < V; ++r) {
      if ((r & span) == 0) {
        const float u = x[r], w = x[r + span];
        x[r] = u + w;
        x[r + span] = u - w;
      }
    }
  }
  const int lanes = n / V;
#define TPLA_WHT_LANE_STAGE(M)                                            \
  if (V > 1 || lanes > M) {                                               \
    _Pragma("unroll") for (int r = 0; r < V; ++r) x[r] = wht_lane_pair<M>(x[r], lane); \
  }
  TPLA_WHT_LANE_STAGE(1)
  TPLA_WHT_LANE_STAGE(2)
  TPLA_WHT_LANE_STAGE(4)
  TPLA_WHT_LANE_STAGE(8)
  TPLA_WHT_LANE_STAGE(16)
  TPLA_WHT_LANE_STAGE(32)
#undef TPLA_WHT_LANE_STAGE
  const float norm = 1.0f / sqrtf(static_cast<float>(n));
#pragma unroll
  for (int r = 0; r < V; ++r) x[r] *= norm;
}

// Row of the cache pool holding token t of sequence b.
__device__ __forceinline__ int64_t cache_row(const int* __restrict__ block_table, int b, int t, int page_size,
                                             int max_pages_per_seq) {
  const int page = block_table ? block_table[static_cast<int64_t>(b) * max_pages_per_seq + t / page_size] : b;
  return static_cast<int64_t>(page) * page_size + (t % page_size);
}

}  // namespace tpla
