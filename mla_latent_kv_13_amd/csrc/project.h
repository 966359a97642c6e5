// Value up-projection of latent rows held in LDS, on the matrix cores: out_v[b, h, :] =
// W_UV[h] . o[b, h, :] for kProjRows consecutive rows b of one head h (value rows of kv_b_proj
// applied after latent attention: automated review of the TPLA paper, referee report
// "significance", matrix absorption; feature request on latent-cache sharding, "Background /
// problem": kv_b_proj per head, o_proj rowwise, then the all-reduce), as the merge kernel with the
// projection fused in applies it to the decode results it has just merged into LDS.
//
// A workgroup has kProjWaves waves.  Wave (vt, kq) -- vt = wave % vp, kq = wave / vp -- takes
// value columns [32 vt, 32 vt + 32) over k-part kq of kparts = kProjWaves / vp equal parts of the
// latent's 16-wide k-steps, with 32x32x16 bf16 MFMAs; vp is a power of two >= ceil(d_v / 32) and
// at least 4, so with at most four value tiles (d_v <= 128) there are four k-parts.  A row of o
// enters as bf16(o) plus the bf16 remainder (two products into one fp32 sum), so about 16
// significant bits take part; W_UV is bf16 as stored.  The k-parts' tiles are added in LDS in kq
// order.  MFMA rows past kProjRows are zero and never stored.
//
// Operand layout (32x32x16 bf16): lane l holds A[l % 32][8 (l / 32) + i] and B[8 (l / 32) + i][l % 32],
// i < 8; accumulator r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpla_device.h"

namespace tpla {

constexpr int kProjWaves = 16;
constexpr int kProjRows = 16;                  // a multiple of kProjWaves and of 8, at most 32
constexpr int kProjThreads = 64 * kProjWaves;
constexpr int kProjAcc = kProjRows / 2;        // accumulators of a lane that hold rows < kProjRows
constexpr int kProjMaxDv = 32 * kProjWaves;

struct ProjectArgs {
  const uint16_t* w;  // bf16 [heads, d_v, d_latent]
  int d_v;
  int vp;             // waves per k-part
  float* out_v;       // fp32 [batch, heads, d_v]
  int xcds;
};

// Waves per k-part for d_v value columns (d_v <= kProjMaxDv).
inline int proj_vp(int d_v) {
  int vp = 4;
  while (vp * 32 < d_v) vp <<= 1;
  return vp;
}

// LDS of a workgroup: the rows (16-byte pad between rows, so that they start 4 banks apart), later
// reused for the k-parts' partial tiles.
inline size_t proj_lds_bytes(int d_latent, int vp) {
  const size_t rows = static_cast<size_t>(kProjRows) * (d_latent + 4) * sizeof(float);
  const size_t parts = static_cast<size_t>(vp) * (kProjWaves / vp - 1) * (kProjAcc / 4) * 64 * sizeof(floatx4_t);
  return rows > parts ? rows : parts;
}

// Workgroup id -> (head, first row).  Ids are dealt to the XCDs round-robin; the row tiles of head
// h get ids = h (mod xcds), so they run on one XCD and read W_UV[h] through its L2.  Returns false
// for the padding ids past the last head.
__device__ __forceinline__ bool proj_unit(int batch, int heads, int xcds, int& h, int& b0) {
  const int btiles = (batch + kProjRows - 1) / kProjRows;
  const int xcd = blockIdx.x % xcds, k = blockIdx.x / xcds;
  h = (k / btiles) * xcds + xcd;
  b0 = (k % btiles) * kProjRows;
  return h < heads;
}

struct ProjWave {
  int vt, kq, kparts, ksteps, kb, ke;
  bool active;
  const uint16_t* wrow;  // this lane's weight row, at its 8-value half of a k-step

  __device__ __forceinline__ ProjWave(const ProjectArgs& p, int h, int d_c, int wv, int lane) {
    vt = wv & (p.vp - 1);
    kq = wv / p.vp;
    kparts = kProjWaves / p.vp;
    ksteps = d_c / 16;
    kb = kq * ksteps / kparts;
    ke = (kq + 1) * ksteps / kparts;
    active = vt * 32 < p.d_v;
    // B operand of k-step s: lane l holds W_UV[h][32 vt + l % 32][16 s + 8 (l / 32) + i] (rows
    // past d_v repeat the last one, k-steps past the latent the last one; neither is used)
    wrow = p.w + (static_cast<int64_t>(h) * p.d_v + min(vt * 32 + (lane & 31), p.d_v - 1)) * d_c + 8 * (lane >> 5);
  }
  // Weight operands of k-steps g .. g + 7.
  __device__ __forceinline__ void load_w(uint4 (&wf)[8], int g) const {
#pragma unroll
    for (int s = 0; s < 8; ++s) wf[s] = *reinterpret_cast<const uint4*>(wrow + 16 * min(g + s, ksteps - 1));
  }
};

// This wave's partial tile over its k-part, the rows read from LDS (rows_s, ys floats apart,
// written and published by the caller); wf holds the operands of k-steps kb .. kb + 7 on entry.
__device__ __forceinline__ floatx16_t proj_mfma(const ProjWave& pw, const float* rows_s, int ys, uint4 (&wf)[8],
                                                int lane) {
  floatx16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (!pw.active) return acc;
  const int half = lane >> 5, l32 = lane & 31;
  const float* arow = rows_s + l32 * ys + 8 * half;  // A operand: lane l holds o[b0 + l % 32][16 s + 8 (l / 32) + i]
  for (int g = pw.kb; g < pw.ke; g += 8) {
    uint4 cur[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) cur[s] = wf[s];
    if (g + 8 < pw.ke) pw.load_w(wf, g + 8);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (g + s < pw.ke) {
        float x[8];
        if (l32 < kProjRows) {
          const float4 a0 = *reinterpret_cast<const float4*>(arow + 16 * (g + s));
          const float4 a1 = *reinterpret_cast<const float4*>(arow + 16 * (g + s) + 4);
          x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
          x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
          const float r0 = x[2 * i] - bf16_to_f32(static_cast<uint16_t>(hi[i] & 0xffffu));
          const float r1 = x[2 * i + 1] - bf16_to_f32(static_cast<uint16_t>(hi[i] >> 16));
          lo[i] = pack_bf16x2(r0, r1);
        }
        const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, cur[s]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3])), bw, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3])), bw, acc, 0, 0, 0);
      }
    }
  }
  return acc;
}

// The k-parts' tiles added in LDS in kq order (rows_s reused: every wave must be done reading the
// rows, which the first barrier ensures) and rows b0 .. b0 + kProjRows - 1 (< batch) of head h
// stored.  Every wave of the workgroup calls this.
__device__ __forceinline__ void proj_reduce_store(const ProjWave& pw, floatx16_t acc, float* rows_s,
                                                  const ProjectArgs& p, int h, int heads, int b0, int batch, int lane) {
  constexpr int NG = kProjAcc / 4;
  const int kparts = pw.kparts, vt = pw.vt, kq = pw.kq;
  __syncthreads();  // every wave is done reading the rows
  floatx4_t* part = reinterpret_cast<floatx4_t*>(rows_s);  // [vp][kparts - 1][NG][64]
  if (pw.active && kq > 0) {
#pragma unroll
    for (int j = 0; j < NG; ++j)
      part[((vt * (kparts - 1) + kq - 1) * NG + j) * 64 + lane] = floatx4_t{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
  }
  __syncthreads();
  if (!pw.active || kq > 0) return;
  for (int q = 0; q < kparts - 1; ++q) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const floatx4_t t = part[((vt * (kparts - 1) + q) * NG + j) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * j + e] += t[e];
    }
  }
  const int half = lane >> 5, vv = vt * 32 + (lane & 31);
  if (vv >= p.d_v) return;
#pragma unroll
  for (int r = 0; r < kProjAcc; ++r) {
    const int bb = b0 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (bb < batch) p.out_v[(static_cast<int64_t>(bb) * heads + h) * p.d_v + vv] = acc[r];
  }
}

}  // namespace tpla
