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
#include <algorithm>

#include "kernels.h"
#include "project.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLatent = 1024;
constexpr int kMergeWaves = kThreads / 64;  // one (sequence, head) per wave

// out = H y for the summed latent row y (LDS), V consecutive values per lane.
template <int V>
__device__ __forceinline__ void rotate_out(const float* y, float* dst, int n, int lane) {
  const bool on = lane < n / V;
  Pack<float, V> p = on ? reinterpret_cast<const Pack<float, V>*>(y)[lane] : Pack<float, V>{};
  wave_wht(p.v, n, lane);
  if (on) reinterpret_cast<Pack<float, V>*>(dst)[lane] = p;
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

// Merge of one (sequence, head) for nb computed shards from s0, in a single pass.  Shard s0 + q's
// partials are rows q * n2 + k, k < n2 (n2 = a power of two >= the slots per shard nr and >= P;
// rows k >= nr are padding).  A shard's arithmetic does not depend on s0 or nb.  A
// load step covers P rows (lane group g = lane / (64 / P) takes row step * P + g, P > 1 when a
// slice row is at most 32 float4) and E float4 per lane of each (E = 2 when it is 65..128
// float4); S steps.  Lane j also holds row j's log-sum-exp, so each shard's maximum and sum are
// reductions over an aligned group of n2 lanes, all shards at once.  Every load is issued before
// any value is needed (no branch around a load: rows and vectors past the end are clamped to
// valid ones and never used), so the wave waits on memory once; the number of slots holding
// tokens, nv <= nr, comes from get_nv() after the loads.
template <int E, int P, int S, typename NV>
__device__ __forceinline__ void merge_one_pass(const MergeLaunch& a, int b, int h, int lane, int64_t slot0, int nr,
                                               int lg2, int s0, int nb, NV get_nv, float* y) {
  constexpr int GW = 64 / P;  // lanes per row of a load step
  const int n2 = 1 << lg2, sc = a.shard_count, nvec = a.w / 4;
  const int64_t heads = a.heads;
  const int g = lane / GW, c = lane % GW;
  auto part_row = [&](int j) {  // partial row of row j (padding rows read slot nr - 1)
    const int sl = s0 + (j >> lg2), k = min(j & (n2 - 1), nr - 1);
    return ((slot0 + k) * sc + sl) * heads + h;
  };
  const int R = nb * n2;
  const float lse_raw = a.part_lse[part_row(min(lane, R - 1))];
  float4 v[S][E];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const float4* src = reinterpret_cast<const float4*>(a.part_o + part_row(min(i * P + g, R - 1)) * a.w);
#pragma unroll
    for (int e = 0; e < E; ++e) v[i][e] = src[min(c + 64 * e, nvec - 1)];
  }
  const int nv = get_nv();
  const int kl = lane & (n2 - 1);
  const bool live = lane < R && kl < nv;
  const float lse_l = live ? lse_raw : -INFINITY;
  const float M = group_reduce<true>(lse_l, n2);
  const float Z = group_reduce<false>(live ? expf(lse_l - M) : 0.f, n2);
  const float wl = live ? expf(lse_l - M) * (1.0f / Z) : 0.f;
  if (a.lse != nullptr && kl == 0 && lane < R)
    a.lse[(static_cast<int64_t>(b) * sc + s0 + (lane >> lg2)) * heads + h] = nv > 0 ? M + logf(Z) : -INFINITY;
  float4 acc[E];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int j0 = i * P;  // first row of this step (uniform)
    if (j0 < R) {
      if ((j0 & (n2 - 1)) == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0));
#pragma unroll
      for (int gg = 1; gg < P; ++gg) {
        const float wg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0 + gg));
        wt = g == gg ? wg : wt;
      }
      if (((j0 + g) & (n2 - 1)) < nv) {  // rows without tokens may hold stale values: never multiplied
#pragma unroll
        for (int e = 0; e < E; ++e) Vec<4>::fma(wt, v[i][e], acc[e]);
      }
      if (((j0 + P) & (n2 - 1)) == 0) {  // last step of shard j0 / n2: add the P groups, store
#pragma unroll
        for (int e = 0; e < E; ++e) {
#pragma unroll
          for (int off = GW; off < 64; off <<= 1) {
            acc[e].x += __shfl_xor(acc[e].x, off);
            acc[e].y += __shfl_xor(acc[e].y, off);
            acc[e].z += __shfl_xor(acc[e].z, off);
            acc[e].w += __shfl_xor(acc[e].w, off);
          }
        }
        float4* yd = reinterpret_cast<float4*>(y + (a.shard_begin + s0 + (j0 >> lg2)) * a.w);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (g == 0 && c + 64 * e < nvec) yd[c + 64 * e] = acc[e];
      }
    }
  }
}

// Slots per shard padded to a power of two no less than p: log2.
__device__ __forceinline__ int pad_log2(int nr, int p) {
  const int m = max(nr, p);
  return 32 - __clz(m - 1);
}

// The summed latent row y of (sequence b, head h), d_latent floats at y (16-byte aligned; LDS),
// and the log-sum-exps of the computed shards (when a.lse is set).  Wave-local.  E > 0: the
// one-pass path (E, P, S as above) is compiled in for waves whose partials fit it.
template <int V, int E, int P, int S>
__device__ __forceinline__ void merge_row(const MergeLaunch& a, int b, int h, int lane, float* y) {
  typedef typename Vec<V>::T vec_t;
  const int lo = a.shard_begin * a.w, hi = lo + a.shard_count * a.w;
  for (int j = lane; j < a.d_latent; j += 64)
    if (j < lo || j >= hi) y[j] = 0.f;  // latent columns of shards that were not computed
  if constexpr (E > 0) {
    // chunked schedule: the loads of every chunk slot go out before the context length arrives
    if (a.sched == 0) {
      const int lg2 = pad_log2(a.num_chunks, P);
      if ((1 << lg2) <= min(64, S * P)) {
        const int per = min(64, S * P) >> lg2;  // shards per pass
        for (int s0 = 0; s0 < a.shard_count; s0 += per)
          merge_one_pass<E, P, S>(a, b, h, lane, static_cast<int64_t>(b) * a.num_chunks, a.num_chunks, lg2, s0,
                                  min(per, a.shard_count - s0), [&] {
                                    return (a.seq_lens[b] + a.chunk_tokens - 1) / a.chunk_tokens;
                                  }, y);
        return;
      }
    }
  }
  {
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
  if constexpr (E > 0) {
    const int lg2 = pad_log2(max(nv, 1), P);
    if ((1 << lg2) <= min(64, S * P)) {
      const int per = min(64, S * P) >> lg2;
      for (int s0 = 0; s0 < a.shard_count; s0 += per)
        merge_one_pass<E, P, S>(a, b, h, lane, slot0, max(nv, 1), lg2, s0, min(per, a.shard_count - s0),
                                [&] { return nv; }, y);
      return;
    }
  }

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
  }
}

// dst = H y for a row of n values (n a power of two <= 1024); dst may be y itself.
__device__ __forceinline__ void rotate_row(const float* y, float* dst, int n, int lane) {
  switch (n <= 64 ? 1 : n / 64) {
    case 1: rotate_out<1>(y, dst, n, lane); break;
    case 2: rotate_out<2>(y, dst, n, lane); break;
    case 4: rotate_out<4>(y, dst, n, lane); break;
    case 8: rotate_out<8>(y, dst, n, lane); break;
    default: rotate_out<16>(y, dst, n, lane); break;
  }
}

template <int V, int E, int P, int S>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeLaunch a) {
  __shared__ __attribute__((aligned(64))) float ybuf[kMergeWaves][kMaxLatent];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * kMergeWaves + wv, b = blockIdx.y;
  if (h >= a.heads) return;  // the rest of this kernel is wave-local
  if (a.skip_whole && a.sched == 1) {
    // rows whose tiles all fall in one worker's share were finished by the decode kernel (the
    // same share boundaries as its segments: worker w takes tiles [w*total/nw, (w+1)*total/nw))
    const int64_t total = a.tile_prefix[a.batch];
    const int64_t p0 = a.tile_prefix[b], p1 = a.tile_prefix[b + 1];
    const int64_t nw = min(static_cast<int64_t>(a.workers), total);
    if (p1 > p0 && ((p0 + 1) * nw - 1) / total == (p1 * nw - 1) / total) return;
  }
  float* y = ybuf[wv];
  merge_row<V, E, P, S>(a, b, h, lane, y);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // this wave's LDS row is complete
  __builtin_amdgcn_wave_barrier();

  float* dst = a.out + (static_cast<int64_t>(b) * a.heads + h) * a.d_latent;
  if (!a.wht) {
    for (int j = lane; j < a.d_latent / 4; j += 64)
      reinterpret_cast<float4*>(dst)[j] = reinterpret_cast<const float4*>(y)[j];
    return;
  }
  rotate_row(y, dst, a.d_latent, lane);
}

// Merge with the value up-projection fused in: out_v[b, h, :] = W_UV[h] . o[b, h, :], o being the
// row merge_kernel would write (the projection and its sources: project.h).  The merged rows
// never leave the CU.  Workgroup = one head h and kProjRows consecutive sequences; wave i merges
// sequences b0 + i, b0 + i + kProjWaves, ... into LDS rows i, i + kProjWaves, ... (rotated back in
// place under the Hadamard transform), requesting its weight operands as soon as its last row is
// merged; then the waves apply W_UV[h] to the rows.
template <int V, int E, int P, int S>
__global__ __launch_bounds__(kProjThreads) void merge_project_kernel(MergeLaunch a, ProjectArgs p) {
  extern __shared__ __attribute__((aligned(16))) float rows_s[];  // [kProjRows][d_latent + 4], then the k-part tiles
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int h, b0;
  if (!proj_unit(a.batch, a.heads, p.xcds, h, b0)) return;  // uniform over the workgroup
  const int ys = a.d_latent + 4;
  const ProjWave pw(p, h, a.d_latent, wv, lane);
  uint4 wf[8];
  for (int i = wv; i < kProjRows; i += kProjWaves) {
    float* y = rows_s + i * ys;
    const int b = b0 + i;
    const bool last = i + kProjWaves >= kProjRows;
    if (b < a.batch) {
      merge_row<V, E, P, S>(a, b, h, lane, y);
      if (pw.active && last) pw.load_w(wf, pw.kb);  // in flight during the rotation and the wait for the other rows
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // this wave's LDS row is complete
      __builtin_amdgcn_wave_barrier();
      if (a.wht) rotate_row(y, y, a.d_latent, lane);
    } else {
      if (pw.active && last) pw.load_w(wf, pw.kb);
      for (int j = lane; j < a.d_latent; j += 64) y[j] = 0.f;
    }
  }
  __syncthreads();
  const floatx16_t acc = proj_mfma(pw, rows_s, ys, wf, lane);
  proj_reduce_store(pw, acc, rows_s, p, h, a.heads, b0, a.batch, lane);
}

// Context merge: decode results over P disjoint parts of every sequence's context combined by
// log-sum-exp into the result over the whole context (feature request on latent-cache sharding,
// "Directions under investigation": context parallelism, a sequence split with a log-sum-exp
// merge).  One wave per (sequence, head).  Lane i < shard_count gathers local shard i's
// log-sum-exps over the parts: lse_i = M + ln sum_p e^(lse_p,i - M).  Then, part by part, the
// latent row y_p (= H out_p under the Hadamard transform, H being its own inverse) is added with
// the weight e^(lse_p,i - lse_i) of each column's shard; the sum is rotated back (out = H y).
// Parts with lse = -inf add nothing; a shard with no tokens anywhere gives 0 and -inf.  The rows
// of the first PB parts are requested before the log-sum-exps are combined, and PB parts at a
// time after that (indices clamped to the last part, branches only around the arithmetic).
// V > 0: V consecutive values per lane (d_latent = 64 V, or V = 1 below 64), rotated when WHT;
// V = 0: value lane + 64 r in register r (other widths, no rotation).
template <int V, bool WHT>
__global__ __launch_bounds__(kThreads) void context_merge_kernel(ContextMergeLaunch a) {
  constexpr int R = V > 0 ? V : kMaxLatent / 64;  // values a lane holds
  constexpr int PB = 4;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * kMergeWaves + wv, b = blockIdx.y;
  if (h >= a.heads) return;  // the rest of this kernel is wave-local
  const int n = a.d_latent, sc = a.shard_count, w = n / a.num_shards;
  const int64_t bh = static_cast<int64_t>(b) * a.heads + h;
  const int64_t part_stride = static_cast<int64_t>(a.batch) * a.heads * n;
  const int64_t lse_stride = static_cast<int64_t>(a.batch) * sc * a.heads;
  const bool mine = lane < sc;  // this lane holds local shard `lane`
  const int64_t lse_at = (static_cast<int64_t>(b) * sc + (mine ? lane : 0)) * a.heads + h;
  const bool on = V > 0 ? lane < n / V : true;
  float x[PB][R];
  float lp[PB];
  auto load = [&](int p0) {
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int p = min(p0 + k, a.parts - 1);
      const float* src = a.out_parts + p * part_stride + bh * n;
      if constexpr (V > 0) {
        const Pack<float, V> pk = reinterpret_cast<const Pack<float, V>*>(src)[on ? lane : 0];
#pragma unroll
        for (int r = 0; r < V; ++r) x[k][r] = pk.v[r];
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) x[k][r] = src[min(lane + 64 * r, n - 1)];
      }
      lp[k] = a.lse_parts[p * lse_stride + lse_at];
    }
  };
  load(0);
  float m = -INFINITY;
  float z = 0.f;
  if (a.parts <= PB) {
    // every part's log-sum-exp arrived with the first load: no further round trip to memory
#pragma unroll
    for (int k = 0; k < PB; ++k) m = fmaxf(m, lp[k]);  // a repeated last part does not change the maximum
    if (m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < PB; ++k)
        if (k < a.parts) z += expf(lp[k] - m);
    }
  } else {
    for (int p0 = 0; p0 < a.parts; p0 += PB) {
      float l[PB];
#pragma unroll
      for (int k = 0; k < PB; ++k) l[k] = a.lse_parts[min(p0 + k, a.parts - 1) * lse_stride + lse_at];
#pragma unroll
      for (int k = 0; k < PB; ++k) m = fmaxf(m, l[k]);
    }
    if (m != -INFINITY)
      for (int p = 0; p < a.parts; ++p) z += expf(a.lse_parts[p * lse_stride + lse_at] - m);
  }
  const float lse_i = m != -INFINITY ? m + logf(z) : -INFINITY;
  if (a.lse != nullptr && mine) a.lse[lse_at] = lse_i;

  // local shard of each value this lane holds (-1: a shard that was not computed, or padding)
  int shard_of[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = V > 0 ? V * lane + r : lane + 64 * r;
    const int i = j < n ? j / w - a.shard_begin : -1;
    shard_of[r] = i >= 0 && i < sc ? i : -1;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  for (int p0 = 0; p0 < a.parts; p0 += PB) {
    if (p0 > 0) load(p0);
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      if (p0 + k >= a.parts) break;
      if constexpr (WHT) wave_wht(x[k], n, lane);  // y_p = H out_p
      const float wl = mine && lse_i != -INFINITY ? expf(lp[k] - lse_i) : 0.f;  // weight of part p for shard `lane`
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float wt = __shfl(wl, shard_of[r] >= 0 ? shard_of[r] : 0);
        if (shard_of[r] >= 0) acc[r] = fmaf(wt, x[k][r], acc[r]);
      }
    }
  }
  float* dst = a.out + bh * n;
  if constexpr (V > 0) {
    if constexpr (WHT) wave_wht(acc, n, lane);  // out = H y
    Pack<float, V> pk;
#pragma unroll
    for (int r = 0; r < V; ++r) pk.v[r] = acc[r];
    if (on) reinterpret_cast<Pack<float, V>*>(dst)[lane] = pk;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane + 64 * r < n) dst[lane + 64 * r] = acc[r];
  }
}

// tile_prefix[b] = sum_{b' < b} ceil(seq_lens[b'] / 32) for b = 0..batch, by one whole block: each
// thread sums a contiguous run of sequences, then an exclusive scan over the threads' sums.
__device__ __forceinline__ void tile_prefix_block(const int* __restrict__ seq_lens, int batch, int* __restrict__ prefix) {
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

__global__ __launch_bounds__(kThreads) void tile_prefix_kernel(const int* __restrict__ seq_lens, int batch,
                                                               int* __restrict__ prefix) {
  tile_prefix_block(seq_lens, batch, prefix);
}

// One wave per query row, four rows per block: V consecutive values per lane, rotated in registers.
// With a tile prefix to compute (prefix non-null) one more block, the last, computes it, so that a
// call that needs both launches one kernel.
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void rotate_query_kernel(const T* __restrict__ q, int rows, int d_latent,
                                                                 void* dst, int dst_f32, const int* __restrict__ seq_lens,
                                                                 int batch, int* __restrict__ prefix) {
  // With a prefix to compute, block 0 computes it (dispatched first, so that it runs beside the
  // rotation rather than after it) and the rows start at block 1.
  const int blk = static_cast<int>(blockIdx.x) - (prefix != nullptr ? 1 : 0);
  if (blk < 0) {  // uniform over the block
    tile_prefix_block(seq_lens, batch, prefix);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blk) * kMergeWaves + (threadIdx.x >> 6);
  if (r >= rows) return;
  const bool on = lane < d_latent / V;
  const Pack<T, V> p = on ? reinterpret_cast<const Pack<T, V>*>(q + r * d_latent)[lane] : Pack<T, V>{};
  float x[V];
#pragma unroll
  for (int i = 0; i < V; ++i) x[i] = load_as_f32(&p.v[i]);
  wave_wht(x, d_latent, lane);
  if (!on) return;
  if (dst_f32) {
    Pack<float, V> o;
#pragma unroll
    for (int i = 0; i < V; ++i) o.v[i] = x[i];
    reinterpret_cast<Pack<float, V>*>(static_cast<float*>(dst) + r * d_latent)[lane] = o;
  } else {
    Pack<uint16_t, V> o;
#pragma unroll
    for (int i = 0; i < V; ++i) o.v[i] = f32_to_bf16(x[i]);
    reinterpret_cast<Pack<uint16_t, V>*>(static_cast<uint16_t*>(dst) + r * d_latent)[lane] = o;
  }
}

template <typename T>
hipError_t launch_rotate(const T* q, int rows, int d_latent, void* dst, int dst_f32, const int* seq_lens, int batch,
                         int* prefix, hipStream_t stream) {
  const dim3 grid((rows + kMergeWaves - 1) / kMergeWaves + (prefix != nullptr ? 1 : 0));
#define TPLA_ROT(VV)                                                                                            \
  hipLaunchKernelGGL((rotate_query_kernel<T, VV>), grid, dim3(kThreads), 0, stream, q, rows, d_latent, dst, dst_f32, \
                     seq_lens, batch, prefix)
  switch (d_latent <= 64 ? 1 : d_latent / 64) {
    case 1: TPLA_ROT(1); break;
    case 2: TPLA_ROT(2); break;
    case 4: TPLA_ROT(4); break;
    case 8: TPLA_ROT(8); break;
    case 16: TPLA_ROT(16); break;
    default: return hipErrorInvalidValue;
  }
#undef TPLA_ROT
  return hipGetLastError();
}

// Merge kernel variants <V, E, P, S>, indexed by merge_variant().
#define TPLA_MERGE_VARIANTS(X)                                                                  \
  X(0, 4, 0, 1, 1) X(1, 1, 0, 1, 1) X(2, 4, 2, 1, 4) X(3, 4, 2, 1, 8) X(4, 4, 1, 1, 4)           \
  X(5, 4, 1, 1, 8) X(6, 4, 1, 1, 16) X(7, 4, 1, 2, 4) X(8, 4, 1, 2, 8) X(9, 4, 1, 2, 16)         \
  X(10, 4, 1, 4, 4) X(11, 4, 1, 4, 8) X(12, 4, 1, 4, 16)

// One-pass shape: float4 per lane per row (E) or rows per load step (P) from the slice width;
// steps S: the fewest of 4, 8 and 16 / E that hold every chunk row of all shards under the
// chunked schedule (else 16 / E, shards in several passes), and 16 / E under the balanced
// schedule, where the rows per sequence vary.
int merge_variant(const MergeLaunch& a) {
  const int nvec = a.w / 4;
  const int e = a.w % 4 != 0 || nvec > 128 ? 0 : (nvec > 64 ? 2 : 1);
  const int pr = nvec > 32 ? 1 : (nvec > 16 ? 2 : 4);
  int steps = 16 / max(e, 1);
  if (a.sched == 0) {
    int n2 = pr;
    while (n2 < a.num_chunks) n2 <<= 1;
    const int need = a.shard_count * n2 / pr;
    steps = need <= 4 ? 4 : (need <= 8 ? 8 : steps);
  }
  const int si = steps == 4 ? 0 : (steps == 8 ? 1 : 2);
  if (e == 0) return a.w % 4 == 0 ? 0 : 1;
  if (e == 2) return steps == 4 ? 2 : 3;
  return (pr == 1 ? 4 : (pr == 2 ? 7 : 10)) + si;
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
  using K = void (*)(MergeLaunch);
  K kern = nullptr;
  switch (merge_variant(a)) {
#define TPLA_X(i, V, E, P, S) \
  case i: kern = merge_kernel<V, E, P, S>; break;
    TPLA_MERGE_VARIANTS(TPLA_X)
#undef TPLA_X
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_project(const MergeLaunch& a, const uint16_t* w_uv, int d_v, float* out_v, int xcds,
                                hipStream_t stream) {
  if (a.d_latent > kMaxLatent || a.d_latent % 16 != 0 || d_v < 1 || d_v > kProjMaxDv || xcds < 1)
    return hipErrorInvalidValue;
  if (a.wht && (a.d_latent & (a.d_latent - 1)) != 0) return hipErrorInvalidValue;
  ProjectArgs p;
  p.w = w_uv;
  p.d_v = d_v;
  p.vp = proj_vp(d_v);
  p.out_v = out_v;
  p.xcds = xcds;
  const int btiles = (a.batch + kProjRows - 1) / kProjRows;
  const int64_t blocks = static_cast<int64_t>((a.heads + xcds - 1) / xcds) * xcds * btiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t lds = proj_lds_bytes(a.d_latent, p.vp);
  // Sixteen waves per workgroup leave 128 registers per lane: the one-pass shapes holding 32 or
  // more float4 per lane (S E = 16) would spill, so they run with half the steps (sequences with
  // more partials than that take the general loop).
  using K = void (*)(MergeLaunch, ProjectArgs);
  K kern = nullptr;
  switch (merge_variant(a)) {
    case 0: kern = merge_project_kernel<4, 0, 1, 1>; break;
    case 1: kern = merge_project_kernel<1, 0, 1, 1>; break;
    case 2: case 3: kern = merge_project_kernel<4, 2, 1, 4>; break;
    case 4: kern = merge_project_kernel<4, 1, 1, 4>; break;
    case 5: case 6: kern = merge_project_kernel<4, 1, 1, 8>; break;
    case 7: kern = merge_project_kernel<4, 1, 2, 4>; break;
    case 8: case 9: kern = merge_project_kernel<4, 1, 2, 8>; break;
    case 10: kern = merge_project_kernel<4, 1, 4, 4>; break;
    case 11: case 12: kern = merge_project_kernel<4, 1, 4, 8>; break;
    default: return hipErrorInvalidValue;
  }
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kProjThreads), lds, stream, a, p);
  return hipGetLastError();
}

hipError_t launch_context_merge(const ContextMergeLaunch& a, hipStream_t stream) {
  if (a.d_latent > kMaxLatent || a.shard_count > 64) return hipErrorInvalidValue;
  if (a.wht && (a.d_latent & (a.d_latent - 1)) != 0) return hipErrorInvalidValue;
  if (a.batch == 0 || a.heads == 0) return hipSuccess;
  const dim3 grid((a.heads + kMergeWaves - 1) / kMergeWaves, a.batch);
  // the packed layout needs d_latent = 64 V (V a power of two), or V = 1 below 64 (rotated rows only)
  const int v = a.d_latent <= 64 ? (a.wht ? 1 : (a.d_latent == 64 ? 1 : 0)) : a.d_latent / 64;
  const bool packed = v > 0 && (v & (v - 1)) == 0 && (a.d_latent <= 64 || a.d_latent % 64 == 0);
#define TPLA_CM(VV)                                                                             \
  if (a.wht)                                                                                    \
    hipLaunchKernelGGL((context_merge_kernel<VV, true>), grid, dim3(kThreads), 0, stream, a);   \
  else                                                                                          \
    hipLaunchKernelGGL((context_merge_kernel<VV, false>), grid, dim3(kThreads), 0, stream, a)
  if (!packed) {
    hipLaunchKernelGGL((context_merge_kernel<0, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    switch (v) {
      case 1: TPLA_CM(1); break;
      case 2: TPLA_CM(2); break;
      case 4: TPLA_CM(4); break;
      case 8: TPLA_CM(8); break;
      default: TPLA_CM(16); break;
    }
  }
#undef TPLA_CM
  return hipGetLastError();
}

hipError_t launch_rotate_query(const void* q_lat, int dtype, int rows, int d_latent, void* dst, int dst_f32,
                               hipStream_t stream, const int* seq_lens, int batch, int* tile_prefix) {
  if (d_latent > kMaxLatent || (d_latent & (d_latent - 1)) != 0) return hipErrorInvalidValue;
  if (dtype == 0)
    return launch_rotate(static_cast<const float*>(q_lat), rows, d_latent, dst, dst_f32, seq_lens, batch, tile_prefix,
                         stream);
  return launch_rotate(static_cast<const uint16_t*>(q_lat), rows, d_latent, dst, dst_f32, seq_lens, batch, tile_prefix,
                       stream);
}

}  // namespace tpla
