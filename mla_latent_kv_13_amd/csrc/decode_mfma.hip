// bf16 split-K TPLA decode on the gfx950 matrix cores.
//
// Work unit: one workgroup = (token chunk of sequence b -- or, with the balanced schedule, an
// equal share of all the batch's tiles, one segment per sequence it touches --, shard s, group of
// 32*HB heads).  It streams the segment's cache rows of that shard -- the latent slice
// [s*W, (s+1)*W) and the whole rope key,
// the per-device share of the TPLA review page (320 = 256 + 64 values per token at two shards) --
// from HBM straight into a ring of ST LDS tiles of 32 tokens with global_load_lds_dwordx4 (no
// register staging), keeping ST-1 tiles in flight per workgroup so that enough bytes are
// outstanding to cover HBM latency.  Per tile, every wave owns 32 heads and:
//   S^T[token, head] = K_tile[token, :] . Q^T[:, head]        32x32x16 bf16 MFMA over key width
//   online softmax over tokens per head, in base 2
//   O^T[col, head]  += V_tile^T[col, token] . P^T[token, head]  32x32x16 bf16 MFMA over tokens
// with the value tile read transposed out of LDS by ds_read_b64_tr_b16.  With KS = 2 the two waves
// of a pair split the key width for S (exchanging fp32 partial logits through LDS) and the value
// columns for O, which halves the registers each wave needs for the wide single-shard case.
// One wave per SIMD, except at W = 128 with two or more head blocks, where a wave fits in half the
// register file and two share each SIMD (see waves_per_simd).
// The chunk's normalised output and log-sum-exp go to the workspace and the merge kernel combines
// chunks exactly (feature request on latent-cache sharding, "Directions under investigation":
// sequence split plus log-sum-exp merge).  The slice softmax is plain, with the same scale on
// every shard (TPLA abstract; review page, Eq. 6).
//
// Lane layouts (checked on gfx950): for v_mfma_f32_32x32x16_bf16 lane l holds A[l%32][8*(l/32)+i]
// and B[8*(l/32)+i][l%32], i = 0..7, and accumulator j of lane l is D[8*(j/4)+4*(l/32)+j%4][l%32].
// ds_read_b64_tr_b16 lets lane q of each 16-lane group address row q/4, columns 4*(q%4)..+3 of a
// 4 x 16 block and returns column q (rows 0..3).  global_load_lds_dwordx4 writes lane i's 16 bytes
// at LDS base + 16*i, so a tile is laid out in 1 KiB pieces, one per wave instruction.
//
// LDS tile layout: token-major rows of KW bf16 (KW = W + D_R) in 16-byte chunks; chunk c of token t
// sits at position c ^ f(t), f(t) = 4*((t/2)%2) + (t/4)%4 (a permutation within each group of 8
// chunks, period 16 in t).  LDS serves a 16-byte-per-lane read 16 lanes (256 bytes, all 64
// banks) per cycle and an 8-byte read 32 lanes per cycle.  A row is 128 bytes modulo 256 for
// every supported width, so the 16 tokens of a K-operand read group (same chunk) land on 16
// distinct 16-byte bank groups exactly when f is one-to-one on the even and on the odd tokens of
// each 16; the transposed V read (4 tokens x 4 adjacent chunks per 32 lanes) needs bit 2 of f to
// differ between tokens t and t+2.
//
// Cache layouts: LAYOUT 0 = contiguous (sequence b owns rows b*page_size...), 1 = paged with
// page_size a power of two of at least 32 (a tile never straddles a page, and the page of a
// token is a shift away), 2 = any other paging.  In layouts 0 and 1 a full tile is 32
// consecutive rows, so each lane's DMA source is a fixed byte offset from one wave-uniform row
// address, which layout 1 forms in scalar registers from the tile's page number.
#include <type_traits>

#include "kernels.h"
#include "lds_dma.h"
#include "tpla_device.h"

namespace tpla {
namespace {

constexpr int kNT = 32;          // tokens per LDS tile (the M dimension of the QK product)
constexpr int kMaxPages = 1024;  // block-table entries of one chunk kept in LDS


// Waves per SIMD a configuration is built for: two where a wave's registers fit half the file
// (value width 128 with at least two head blocks of 32), else one.  Two waves per SIMD let one
// wave's barrier, LDS and softmax stalls be covered by the other's matrix work.
constexpr int waves_per_simd(int w, int hb, int ks) { return w == 128 && hb >= 2 && ks == 1 ? 2 : 1; }

template <int W, int DR, int HB, int KS, int STQ, int LAYOUT>
struct Cfg {
  static constexpr int KW = W + DR;                // key width of one shard
  static constexpr int ROW_BYTES = KW * 2;
  static constexpr int CPR = KW / 8;               // 16-byte chunks per token row
  static constexpr int LAT_CPR = W / 8;
  static constexpr int TILE_BYTES = kNT * ROW_BYTES;
  static constexpr int NWAVES = HB * KS;
  static constexpr int THREADS = NWAVES * 64;
  static constexpr int INSTR = kNT * CPR / 64;     // 1 KiB DMA pieces per tile
  static constexpr int PER_LO = INSTR / NWAVES;    // pieces per wave; the first REM waves take one more
  static constexpr int REM = INSTR % NWAVES;
  static constexpr int PER_MAX = PER_LO + (REM ? 1 : 0);
  static constexpr int KSTEPS = KW / 16 / KS;      // QK k-steps of one wave
  static constexpr int CB = W / 32 / KS;           // 32-column value blocks of one wave
  // LDS a workgroup may take: all of it, or with two waves per SIMD its share among the
  // workgroups that the CU then holds together.  It holds ST ring stages, the partial-logit
  // exchange buffer (KS > 1), the page list of paged layouts.  Ring stages: as requested, but
  // never more loads in flight per lane than vmcnt can count (63), and only as many as fit.
  static constexpr int OCC = waves_per_simd(W, HB, KS);
  static constexpr int LDS_BUDGET = OCC > 1 ? 160 * 1024 / ((NWAVES >= 4 ? 1 : 4 / NWAVES) * OCC) : 160 * 1024;
  static constexpr int PAGE_BYTES = LAYOUT != 0 ? kMaxPages * 4 : 0;
  static constexpr int SX_BYTES = KS > 1 ? NWAVES * 4096 : 0;
  static constexpr bool fits(int st) { return st * TILE_BYTES + SX_BYTES + PAGE_BYTES <= LDS_BUDGET; }
  static constexpr int ST0 = STQ < 2 + 63 / PER_MAX ? STQ : 2 + 63 / PER_MAX;
  static constexpr int largest_fit(int st) { return st <= 3 || fits(st) ? st : largest_fit(st - 1); }
  static constexpr int ST = largest_fit(ST0);
  static constexpr int SX_OFF = ST * TILE_BYTES;
  static constexpr int PAGES_OFF = SX_OFF + SX_BYTES;
  static constexpr int LDS_BYTES = PAGES_OFF + PAGE_BYTES;
  static_assert(W % 32 == 0 && DR % 16 == 0 && CPR % 8 == 0, "tile shape");
  static_assert(kNT * CPR % 64 == 0, "a tile is a whole number of 1 KiB pieces");
  static_assert((KW / 16) % KS == 0 && (W / 32) % KS == 0, "key/value split");
  static_assert(KS == 1 || KS == 2, "key split");
  static_assert(ST >= 3, "ring of at least three tiles (two resident, one in flight)");
  static_assert(LDS_BYTES <= LDS_BUDGET, "LDS budget");
};

__device__ __forceinline__ int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }

// Order of the MFMAs of one steady-state step of the one-wave-per-32-heads tiles: NQ logit
// k-steps of the next tile (a dependent chain into one accumulator) spread evenly among NP value
// steps of the current tile (independent: consecutive ones go to different column blocks).  A
// dependent 32x32x16 MFMA cannot start until its predecessor's result is written back, which
// takes about three times as long as the matrix core needs to accept an independent one, so the
// value steps fill the gaps of the chain.  Op n is a value step when the running share of value
// steps crosses an integer there; index(n) is its position among the ops of its kind.
template <int NQ, int NP>
struct Stream {
  static constexpr int N = NQ + NP;
  static constexpr bool pv(int n) { return ((n + 1) * NP) / N > (n * NP) / N; }
  static constexpr int index(int n) {
    int c = 0;
    for (int m = 0; m < n; ++m) c += pv(m) == pv(n) ? 1 : 0;
    return c;
  }
};

// Tiles that finish whole rows themselves (DecodeLaunch::direct_out): the full 512-wide latent
// of one shard split between the two waves of a pair, 256 value columns each.
constexpr bool direct_rows(int w, int ks) { return w == 512 && ks == 2; }

// H2 butterfly on one index bit: the lower index takes the sum, the upper the difference.
__device__ __forceinline__ void bfly(float& lo, float& hi) {
  const float u = lo, v = hi;
  lo = u + v;
  hi = u - v;
}

// Butterflies on index bit K of N registers (every index a compile-time constant, so that the
// array stays in registers).
template <int K, int N>
__device__ __forceinline__ void bfly_bit(float (&z)[N]) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const int r = ((i >> K) << (K + 1)) | (i & ((1 << K) - 1));
    bfly(z[r], z[r | (1 << K)]);
  }
}

// Final output of a row that one workgroup computed whole, from one wave of a pair: this wave's
// O^T accumulators (CB = 8 blocks of 32 columns, kh * 256 + 32 * cb + 8 * (j / 4) + 4 * half +
// j % 4 for accumulator j, head = lane % 32) are normalised, rotated back by the orthonormal
// Sylvester Hadamard matrix when the cache is rotated (out = H y, the merge's definition), and
// written with the log-sum-exp.  H is the product of one 2-point butterfly per bit of the column
// index: the accumulator-index bits are butterflied in registers, the lane-half bit across the
// two halves of the wave (permlane32 swaps), and the wave bit through LDS: wave kh = 0 finishes
// columns c and c + 256 for c in [0, 128), wave kh = 1 for c in [128, 256), each sending the other
// the half of its values it does not finish (16 KiB per wave at `mine`, read back at `theirs`).
template <int CB>
__device__ __forceinline__ void finish_row(const floatx16_t (&o_acc)[CB], float l_tot, float m_ref, const DecodeLaunch& a,
                                           int b, int head, int kh, int half, int lane, unsigned char* mine,
                                           const unsigned char* theirs) {
  static_assert(CB == 8, "a pair of 256-column halves");
  float z[CB * 16];  // z[16 * cb + j]
  const float f = (a.direct_wht ? 0.044194173824159216f : 1.0f) / l_tot;  // 1/sqrt(512) with H
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int j = 0; j < 16; ++j) z[16 * cb + j] = o_acc[cb][j] * f;
  float* out = a.direct_out + (static_cast<int64_t>(b) * a.heads + head) * 512;
  if (!a.direct_wht) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        *reinterpret_cast<float4*>(out + kh * 256 + 32 * cb + 8 * j4 + 4 * half) =
            make_float4(z[16 * cb + 4 * j4], z[16 * cb + 4 * j4 + 1], z[16 * cb + 4 * j4 + 2], z[16 * cb + 4 * j4 + 3]);
  } else {
    // register bits: z index bits 0-1 = column bits 0-1, bits 2-3 = column bits 3-4, bits 4-6 =
    // column bits 5-7 (the lower column always has the lower index)
    bfly_bit<0>(z);
    bfly_bit<1>(z);
    bfly_bit<2>(z);
    bfly_bit<3>(z);
    bfly_bit<4>(z);
    bfly_bit<5>(z);
    bfly_bit<6>(z);
    // lane-half bit (column bit 2): swap halves between register pairs, butterfly in the lane,
    // swap back.  After the first swap a lane below 32 holds both halves of z[r], a lane above 32
    // both halves of z[r + 1].
#pragma unroll
    for (int r = 0; r < CB * 16; r += 2) {
      const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[r]), __float_as_uint(z[r + 1]), false, false);
      float lo = __uint_as_float(s1[0]), hi = __uint_as_float(s1[1]);
      bfly(lo, hi);
      const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
      z[r] = __uint_as_float(s2[0]);
      z[r + 1] = __uint_as_float(s2[1]);
    }
    // wave bit (column bit 8): blocks cb = 4 .. 7 (kh = 0) or 0 .. 3 (kh = 1) go to the partner
    // (selected per value, so that every register index stays a constant)
    const bool k0 = kh == 0;
    __syncthreads();  // every wave is done with the ring, which now holds the exchange
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float g[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] = k0 ? z[64 + 4 * i + e] : z[4 * i + e];
      reinterpret_cast<float4*>(mine)[i * 64 + lane] = make_float4(g[0], g[1], g[2], g[3]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 t = reinterpret_cast<const float4*>(theirs)[i * 64 + lane];
      const float o4[4] = {t.x, t.y, t.z, t.w};
      float lo4[4], hi4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // kh = 0 holds column c, the partner c + 256; kh = 1 the reverse
        const float own = k0 ? z[4 * i + e] : z[64 + 4 * i + e];
        lo4[e] = k0 ? own + o4[e] : o4[e] + own;
        hi4[e] = k0 ? own - o4[e] : o4[e] - own;
      }
      const int cb = (k0 ? 0 : 4) + i / 4, j4 = i % 4;
      const int col = 32 * cb + 8 * j4 + 4 * half;
      *reinterpret_cast<float4*>(out + col) = make_float4(lo4[0], lo4[1], lo4[2], lo4[3]);
      *reinterpret_cast<float4*>(out + col + 256) = make_float4(hi4[0], hi4[1], hi4[2], hi4[3]);
    }
  }
  if (a.direct_lse != nullptr && half == 0 && kh == 0)
    a.direct_lse[static_cast<int64_t>(b) * a.heads + head] = (m_ref + log2f(l_tot)) * kLn2;
}

template <int W, int DR, int HB, int KS, int STQ, int LAYOUT, bool DIRECT>
__global__ __launch_bounds__(HB * KS * 64, waves_per_simd(W, HB, KS)) void decode_mfma_kernel(DecodeLaunch a, float scale_log2, int units,
                                                                       int members, int page_shift) {
  using C = Cfg<W, DR, HB, KS, STQ, LAYOUT>;
  constexpr int ST = C::ST;
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];

  // XCD-aware placement: consecutive workgroups go to the device's XCDs in turn, so the members
  // of one unit (its shards and head groups, which read the same tokens) take ids `xcds` apart:
  // same XCD, adjacent in dispatch order, sharing that XCD's L2 for the common rows.
  const int xcds = a.xcds;
  const int L = blockIdx.x, xcd = L % xcds, slot = L / xcds;
  const int member = slot % members;
  // Prefill rows under the balanced schedule: each XCD takes a contiguous block of workers
  // instead, so that the rows of one sequence -- which all read the same prefix tiles -- run on
  // one XCD and share its L2.
  int u = (slot / members) * xcds + xcd;
  if (a.row_seq != nullptr && a.sched == 1) u = xcd * ((units + xcds - 1) / xcds) + slot / members;
  if (u >= units) return;
  const int groups = a.heads / (32 * HB);
  const int s_local = member / groups, hg = member % groups;
  const int s = a.shard_begin + s_local;

  // Work of this workgroup.  Chunked schedule: unit u is chunk c of sequence b (one segment).
  // Balanced schedule: unit u is worker u, which takes the u-th equal share of all 32-token
  // tiles of the batch (tile_prefix[b] = tiles of sequences before b; min(workers, tiles)
  // workers take part) and works through it sequence by sequence; its partial for sequence b
  // goes to slot b + u.
  int64_t g_next = 0, g_end = 0;
  if (a.sched == 1) {
    // min(workers, tiles) workers take part, so that every share holds at least one tile
    const int64_t total = a.tile_prefix[a.batch];
    const int64_t nw = min(static_cast<int64_t>(units), total);
    if (u >= nw) return;
    g_next = static_cast<int64_t>(u) * total / nw;
    g_end = static_cast<int64_t>(u + 1) * total / nw;
  }
  for (;;) {
  int b, t_begin, t_end;
  int64_t part_row0;  // partial row of head 0 of this segment
  bool whole = false;  // the segment is its row's whole context (balanced schedule)
  if (a.sched == 0) {
    const int c = u % a.num_chunks;
    b = u / a.num_chunks;
    t_begin = c * a.chunk_tokens;
    const int T = a.seq_lens[b];
    if (t_begin >= T) return;
    t_end = min(T, t_begin + a.chunk_tokens);
    part_row0 = ((static_cast<int64_t>(b) * a.num_chunks + c) * a.shard_count + s_local) * a.heads;
  } else {
    if (g_next >= g_end) return;
    // sequence holding global tile g_next: the last b with tile_prefix[b] <= g_next
    int lo = 0, hi = a.batch;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_prefix[mid] <= g_next) lo = mid; else hi = mid - 1;
    }
    b = lo;
    const int64_t p0 = a.tile_prefix[b], p1 = a.tile_prefix[b + 1];
    const int64_t seg_end = min(g_end, p1);
    t_begin = static_cast<int>((g_next - p0) * kNT);
    t_end = min(a.seq_lens[b], static_cast<int>((seg_end - p0) * kNT));
    part_row0 = ((static_cast<int64_t>(b) + u) * a.shard_count + s_local) * a.heads;
    whole = g_next == p0 && seg_end == p1;
    g_next = seg_end;
  }
  const int n_tiles = (t_end - t_begin + kNT - 1) / kNT;
  const int bs = a.row_seq ? a.row_seq[b] : b;  // cache sequence of query row b

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = wv / KS, kh = wv % KS;
  const int half = lane >> 5, l32 = lane & 31;
  const int head = (hg * HB + hb) * 32 + l32;
  const int d_c = a.d_latent;
  const int64_t D = d_c + DR;
  const unsigned char* __restrict__ cache = static_cast<const unsigned char*>(a.cache);
  const int page_size = a.page_size;

  int* pages = reinterpret_cast<int*>(lds + C::PAGES_OFF);
  const int first_page = LAYOUT == 1 ? (t_begin >> page_shift)
                         : (LAYOUT ? (page_shift >= 0 ? (t_begin >> page_shift) : t_begin / page_size) : 0);
  if constexpr (LAYOUT != 0) {
    const int last_page = page_shift >= 0 ? ((t_end - 1) >> page_shift) : (t_end - 1) / page_size;
    const int* bt = a.block_table + static_cast<int64_t>(bs) * a.max_pages_per_seq + first_page;
    for (int i = tid; i <= last_page - first_page; i += C::THREADS) pages[i] = bt[i];
  }
  __syncthreads();

  // This wave's DMA pieces are [first_piece, first_piece + n_pieces); piece k covers tile slots
  // k*64 + lane; slot -> (token tt, position p) -> source chunk p ^ f(tt).  dofs[k] is the lane's
  // byte offset from the tile's first row when the tile is 32 consecutive rows.
  const int n_pieces = C::PER_LO + (wv < C::REM ? 1 : 0);
  const int first_piece = wv * C::PER_LO + min(wv, C::REM);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds)) + first_piece * 1024);
  uint32_t dofs[C::PER_MAX];
#pragma unroll
  for (int k = 0; k < C::PER_MAX; ++k) {
    const int sigma = (first_piece + k) * 64 + lane;
    const int tt = sigma / C::CPR, p = sigma % C::CPR;
    const int ch = p ^ swz(tt);
    const int col = (ch < C::LAT_CPR) ? s * W + ch * 8 : d_c + (ch - C::LAT_CPR) * 8;
    dofs[k] = static_cast<uint32_t>(tt * D * 2 + col * 2);
  }
  // Byte address of cache row `row`.
  auto row_addr = [&](int64_t row) { return cache + row * D * 2; };
  // Full tiles of layouts 0 and 1 address their first row in 32 x 32 -> 64-bit scalar products:
  // layout 0 from the sequence's first row (once per segment), layout 1 from its page (the host
  // takes layout 1 only when a page's bytes fit 32 bits).
  const uint32_t row_bytes = static_cast<uint32_t>(D * 2);
  const uint32_t page_bytes = static_cast<uint32_t>(page_size) * row_bytes;
  const unsigned char* seq_rows = LAYOUT == 0 ? cache + static_cast<int64_t>(bs) * page_size * (D * 2) : cache;
  auto row_of = [&](int t) -> int64_t {
    if constexpr (LAYOUT == 0) {
      return static_cast<int64_t>(bs) * page_size + t;
    } else {
      const bool sh = LAYOUT == 1 || page_shift >= 0;
      const int pi = sh ? (t >> page_shift) : t / page_size;
      const int off = sh ? (t & (page_size - 1)) : t - pi * page_size;
      return static_cast<int64_t>(pages[pi - first_page]) * page_size + off;
    }
  };

  auto issue = [&](int j, int stage) {
    // wave-uniform; taken as such so that the tile's address arithmetic stays on the scalar unit
    const int t0 = __builtin_amdgcn_readfirstlane(t_begin + j * kNT);
    const uint32_t dst = lds_base + stage * C::TILE_BYTES;
    if (LAYOUT != 2 && t0 + kNT <= t_end) {
      // 32 consecutive rows: one uniform base, per-lane constant offsets
      const void* base;
      if constexpr (LAYOUT == 1) {
        // power-of-two pages of at least 32 rows: the tile sits in one page; its address is
        // formed in scalar registers from the page number
        const uint32_t pg = __builtin_amdgcn_readfirstlane(pages[(t0 >> page_shift) - first_page]);
        base = uniform_ptr(cache + static_cast<uint64_t>(pg) * page_bytes +
                           static_cast<uint32_t>(t0 & (page_size - 1)) * row_bytes);
      } else {
        base = uniform_ptr(seq_rows + static_cast<uint64_t>(static_cast<uint32_t>(t0)) * row_bytes);
      }
#pragma unroll
      for (int k = 0; k < C::PER_MAX; ++k) {
        if (C::REM != 0 && k >= n_pieces) break;
        dma16_sbase(dofs[k], base, dst + k * 1024);
      }
    } else {
#pragma unroll
      for (int k = 0; k < C::PER_MAX; ++k) {
        if (C::REM != 0 && k >= n_pieces) break;
        const int sigma = (first_piece + k) * 64 + lane;
        const int tt = sigma / C::CPR, p = sigma % C::CPR;
        const int ch = p ^ swz(tt);
        const int col = (ch < C::LAT_CPR) ? s * W + ch * 8 : d_c + (ch - C::LAT_CPR) * 8;
        const int t = min(t0 + tt, t_end - 1);  // rows past the end repeat a valid row; their p is 0
        dma16(row_addr(row_of(t)) + col * 2, dst + k * 1024);
      }
    }
  };

  // The k-step of the key width that this wave's k-th step covers.  KS = 2: the waves of a pair
  // take alternate pairs of k-steps (wave kh the steps 4j + 2kh and 4j + 2kh + 1), so that within
  // a wave the LDS offsets of the K operand differ by compile-time amounts (see koff).
  auto kstep = [&](int k) { return KS == 1 ? k : 4 * (k >> 1) + 2 * kh + (k & 1); };
  static_assert(KS == 1 || (C::KW / 16) % 4 == 0, "whole groups of four k-steps per pair");

  // Q^T operand of this wave's k-steps: lane holds features 16*kk + 8*half .. +7 of its head.
  uint4 qf[C::KSTEPS];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(a.q_lat) + (static_cast<int64_t>(b) * a.heads + head) * d_c + s * W;
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_rope) + (static_cast<int64_t>(b) * a.heads + head) * DR;
#pragma unroll
    for (int k = 0; k < C::KSTEPS; ++k) {
      const int f = 16 * kstep(k) + 8 * half;
      qf[k] = (f < W) ? *reinterpret_cast<const uint4*>(ql + f) : *reinterpret_cast<const uint4*>(qr + (f - W));
    }
  }
  // Wait for the query now, before the ring starts: otherwise the compiler's own wait for these
  // loads would sit inside the tile loop and drain the tile DMA with it.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
#pragma unroll
  for (int k = 0; k < C::KSTEPS; ++k) asm volatile("" : "+v"(qf[k].x), "+v"(qf[k].y), "+v"(qf[k].z), "+v"(qf[k].w));
  // Logits are scale*log2(e)*(q.k).  A negative scale is moved into the query (exact bf16 sign
  // flips), so the factor applied in the softmax, cs, is never negative.
  const float cs = fabsf(scale_log2);
  if (scale_log2 < 0.f) {
#pragma unroll
    for (int k = 0; k < C::KSTEPS; ++k) {
      qf[k].x ^= 0x80008000u; qf[k].y ^= 0x80008000u; qf[k].z ^= 0x80008000u; qf[k].w ^= 0x80008000u;
    }
  }

#pragma unroll
  for (int j = 0; j < ST - 1; ++j)
    if (j < n_tiles) issue(j, j);

  // Per-lane LDS offsets (bytes) of the swizzled operand reads.
  const int swk = swz(l32);  // K operand: token l32
  // koff[m]: k-steps kk with kk % 4 = m (KS = 1), or with kk % 4 = 2 kh + m (KS = 2, m < 2); the
  // rest of a step's offset, 128 bytes per group of four k-steps, is a compile-time constant.
  int koff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int mm = KS == 1 ? m : 2 * kh + (m & 1);
    koff[m] = l32 * C::ROW_BYTES + ((((2 * mm) | half) ^ swk) << 4);
  }
  const int grp = lane >> 4, q = lane & 15;
  const int vt = 4 * half + (q >> 2);  // V operand: token vt (low read) and vt + 8 (high read) of a 16-token step
  int voff[2][2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int m = 0; m < 2; ++m)
      voff[hi][m] = (vt + 8 * hi) * C::ROW_BYTES + (((4 * m + 2 * (grp & 1) + ((q & 3) >> 1)) ^ swz(vt + 8 * hi)) << 4) + 8 * (q & 1);

  floatx16_t o_acc[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int j = 0; j < 16; ++j) o_acc[cb][j] = 0.f;
  // Online softmax state of the lane's head, in base-2 logit units.  m_ref is the reference
  // maximum the exponentials are taken against; it is raised (and O, l rescaled) only when a
  // logit exceeds it by more than 8, so p stays in (0, 2^8] and the rescale almost never runs.
  // l holds the lane's partial sum over its half of the tokens.
  float m_ref = -INFINITY, l_run = 0.f;
#ifndef TPLA_NPF
#define TPLA_NPF 4
#endif
#ifndef TPLA_NPV
#define TPLA_NPV 4
#endif
  constexpr int KST = C::KSTEPS;
  constexpr int NV = 2 * C::CB;                       // value fragments (MFMAs) per tile
  constexpr int NPF = KST < TPLA_NPF ? KST : TPLA_NPF;  // K fragments read ahead of their MFMA
  constexpr int NPV = NV < TPLA_NPV ? NV : TPLA_NPV;    // value fragments read ahead of their MFMA
  static_assert(NPV <= KST, "value prefetch rides on the k-steps of the next tile's logits");

  auto tile_at = [&](int stage) { return lds + stage * C::TILE_BYTES; };
  auto kread = [&](const unsigned char* tile, int k) {
    if constexpr (KS == 1) return *reinterpret_cast<const uint4*>(tile + koff[k & 3] + ((k >> 2) << 7));
    return *reinterpret_cast<const uint4*>(tile + koff[k & 1] + ((k >> 1) << 7));
  };
  // Value fragment v = ks * CB + cbl: tokens 16*ks.., value block kh*CB + cbl.
  auto vread = [&](const unsigned char* tile, int v) {
    const int ks = v / C::CB, cb = kh * C::CB + v % C::CB;
    const unsigned char* p0 = tile + 16 * ks * C::ROW_BYTES + ((cb >> 1) << 7);
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p0 + voff[0][cb & 1]));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p0 + voff[1][cb & 1]));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto mfma = [](const auto& a_op, const auto& b_op, const floatx16_t& c_acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a_op), __builtin_bit_cast(bf16x8_t, b_op),
                                                   c_acc, 0, 0, 0);
  };
  // Partial logits of a wave pair (KS = 2): one buffer, written after a tile's logit product and
  // read by the partner after the barrier that follows the write.
  auto sx_write = [&](const floatx16_t& v) {
    float4* dst = reinterpret_cast<float4*>(lds + C::SX_OFF + wv * 4096);
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) dst[j4 * 64 + lane] = make_float4(v[4 * j4], v[4 * j4 + 1], v[4 * j4 + 2], v[4 * j4 + 3]);
  };
  auto sx_read = [&](float4 (&pv)[4]) {
    const float4* src = reinterpret_cast<const float4*>(lds + C::SX_OFF + (wv ^ 1) * 4096);
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) pv[j4] = src[j4 * 64 + lane];
  };
  // Full logits of a tile from this wave's partial and (KS = 2) the partner's; both waves of a
  // pair add the halves in the same order, so they agree bit for bit.
  auto logits = [&](const floatx16_t& sv, const float4 (&pv)[4], float (&x)[16]) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const float o4[4] = {pv[j4].x, pv[j4].y, pv[j4].z, pv[j4].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float own = sv[4 * j4 + e];
        x[4 * j4 + e] = KS == 1 ? own : (kh == 0 ? own + o4[e] : o4[e] + own);
      }
    }
  };
  // First half of the online softmax of a tile: the new reference maximum (over both lane halves,
  // i.e. all 32 tokens of the lane's head) and the rescale factor alpha of O and l (exactly 1
  // unless the reference was raised).  Tokens past the end of a partial tile may take part: their
  // rows repeat the last valid row, so they do not change the maximum.
  auto max8 = [](const float (&x)[16], int o) {
    return fmaxf(fmaxf(fmaxf(x[o], x[o + 1]), fmaxf(x[o + 2], x[o + 3])), fmaxf(fmaxf(x[o + 4], x[o + 5]), fmaxf(x[o + 6], x[o + 7])));
  };
  auto max_final = [&](float rmax, float& neg_m) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
    rmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float tmax = rmax * cs;
    const float m_new = tmax > m_ref + 8.0f ? tmax : m_ref;      // first tile: m_ref = -inf
    float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);         // exactly 1 when not raised, 0 first
    asm volatile("" : "+v"(alpha));  // computed here, in a value step, not sunk to the loop's end
    m_ref = m_new;
    neg_m = -m_new;
    return alpha;
  };
  auto softmax_max = [&](const float (&x)[16], float& neg_m) { return max_final(fmaxf(max8(x, 0), max8(x, 8)), neg_m); };
  // A tile's maximum logit of the lane's head, scaled: over both lane halves (all 32 tokens).
  auto tile_max = [&](const float (&x)[16]) {
    const float rmax = fmaxf(max8(x, 0), max8(x, 8));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * cs;
  };
  // Second half of the online softmax, one logit e (0..15) at a time: p = 2^(cs*x - m_ref), packed
  // to bf16 by pairs for the value product and added to the running sum ps by pairs (started by
  // pair 0); the first of a pair waits in p_lo.  One exponential per logit step, so that each
  // hides under its step's MFMA.  The empty asm holds each addition in the step that computes
  // its pair: otherwise the compiler sinks the whole dependent chain of additions to the end of
  // the iteration, after the last value MFMA and before the next barrier.
  // KS = 1: a pair is summed and packed one step after its second exponential, so that the
  // exponential's latency passes under that step's MFMA (the last pair after the loop); at KS = 2
  // finishing a pair in its own step measured faster.
  constexpr bool DEFER = KS == 1;
  auto finish_pair = [&](int j, float p0, float p1, uint32_t (&pk)[8], float& ps) {
    ps = j == 0 ? p0 + p1 : ps + (p0 + p1);
    asm volatile("" : "+v"(ps));
    pk[j] = pack_bf16x2(p0, p1);
  };
  auto softmax_one = [&](const float (&x)[16], int e, float neg_m, uint32_t (&pk)[8], float& p_lo, float& p_hi,
                         float& ps) {
    if (DEFER && (e & 1) == 0 && e > 0) finish_pair((e >> 1) - 1, p_lo, p_hi, pk, ps);
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], cs, neg_m));
    if ((e & 1) == 0) p_lo = p; else p_hi = p;
    if (!DEFER && (e & 1) == 1) finish_pair(e >> 1, p_lo, p_hi, pk, ps);
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int j = 0; j < 16; ++j) o_acc[cb][j] *= alpha;
  };
  // O^T += V_tile^T . P^T.  k-step ks covers tokens 16*ks .. 16*ks+15 in the order the softmax
  // registers hold them: operand slot 8*half + i <-> token 16*ks + 8*(i/4) + 4*half + i%4.
  // The first NPV value fragments are already in vf.
  auto pv = [&](const unsigned char* tile, const uint32_t (&pk)[8], short8_t (&vf)[NPV]) {
    const uint4 pb[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      o_acc[v % C::CB] = mfma(vf[v % NPV], pb[v / C::CB], o_acc[v % C::CB]);
      if (v + NPV < NV) vf[v % NPV] = vread(tile, v + NPV);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The value product of one tile with the softmax maximum of the next tile riding on its steps:
  // (KS = 2) the barrier that publishes the pair's partial logits and the read of the partner's,
  // then the logit sum, the maximum and the new reference.  sn = this wave's logits of the next
  // tile; writes its full logits to x and its -m to neg_m, returns its alpha.
  auto pv_next = [&](const unsigned char* tile, const uint32_t (&pk)[8], short8_t (&vf)[NPV], const floatx16_t& sn,
                     float (&x)[16], float& neg_m) {
    constexpr int VB = 1;                  // exchange barrier and partner read
    constexpr int VL = NV >= 12 ? 5 : 3;   // logit sum, the partner's logits having arrived
    constexpr int VF = VL + 3;             // last reduction step, new reference and alpha
    static_assert(VF < NV, "value steps to carry the maximum");
    const uint4 pb[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
    float4 pvx[4];
    float rmax = 0.f, alpha = 1.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (KS > 1) {
        if (v == VB) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own partial logits written
          raw_barrier();
          sx_read(pvx);
        }
      }
      o_acc[v % C::CB] = mfma(vf[v % NPV], pb[v / C::CB], o_acc[v % C::CB]);
      if (v + NPV < NV) vf[v % NPV] = vread(tile, v + NPV);
      if (v == VL) logits(sn, pvx, x);
      if (v == VL + 1) rmax = max8(x, 0);
      if (v == VL + 2) rmax = fmaxf(rmax, max8(x, 8));
      if (v == VF) alpha = max_final(rmax, neg_m);
      __builtin_amdgcn_sched_barrier(0);
    }
    return alpha;
  };

  // Tile j sits in ring stage j % ST.  Waiting for tile j when `newer` tiles were issued after
  // it: the loads of those may stay in flight, which the wait can express only for the steady
  // state count; otherwise it drains everything.
  auto wait_tile = [&](int newer, auto steady) {
    constexpr int NS = decltype(steady)::value;
    if (newer == NS) {
      if (C::REM != 0 && wv < C::REM)
        wait_vm_lgkm0<NS * (C::PER_LO + 1)>();
      else
        wait_vm_lgkm0<NS * C::PER_LO>();
    } else {
      wait_vm_lgkm0<0>();
    }
  };

  // Prologue: tiles 0..ST-2 are in flight.  Wait for tile 0, compute its logits and maximum.
  wait_tile(min(n_tiles - 1, ST - 2), std::integral_constant<int, ST - 2>{});
  raw_barrier();
  // Softmax state of the tile about to be weighted: its full logits x (unscaled), -m_ref and
  // alpha, the factor O and l take before its weights are added.
  float x[16], neg_m, alpha;
  {
    const unsigned char* t0 = tile_at(0);
    uint4 kf[NPF];
#pragma unroll
    for (int k = 0; k < NPF; ++k) kf[k] = kread(t0, k);
    floatx16_t s0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s0[j] = 0.f;
#pragma unroll
    for (int k = 0; k < KST; ++k) {
      s0 = mfma(kf[k % NPF], qf[k], s0);
      if (k + NPF < KST) kf[k % NPF] = kread(t0, k + NPF);
    }
    float4 pvx[4];
    if constexpr (KS > 1) {
      sx_write(s0);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      raw_barrier();
      sx_read(pvx);
    }
    logits(s0, pvx, x);
    alpha = softmax_max(x, neg_m);  // the first tile: O and l are still zero
  }
  __builtin_amdgcn_sched_barrier(0);

  // Two steady-state loops.  w = 128 (two waves per SIMD): one stream of MFMAs, the next tile's
  // logits interleaved with this tile's value product, no per-tile maximum (weights are taken against
  // the reference and their sum checked instead).  Other widths: the fenced loop below, which keeps
  // the exponentials between the logit MFMAs and the next maximum between the value MFMAs.
  constexpr bool STREAM = W == 128 && KS == 1;
  if constexpr (STREAM) {
    // Steady state, iteration i: tile i with tile i+1 resident.  Tile i's weights are taken first,
    // against the reference m_ref, and their sum checked: every weight is at most the sum, so a
    // sum above kOverflow (or not finite) means a logit more than log2(kOverflow) above m_ref,
    // rare since m_ref starts at the segment's first tile's maximum; such a tile is refitted
    // (m_ref raised to the tile's maximum, O and l rescaled, the weights taken again) before its
    // value product.  Then one stream of MFMAs interleaves the logits of tile i+1 with tile i's
    // value product (Stream above), each operand read out of LDS DQ steps ahead.
    constexpr float kOverflow = 4096.0f;
    constexpr int DQ = 4;
    using S = Stream<KST, NV>;
    int st_cur = 0, st_next = 1 % ST, st_issue = ST - 1;
    float ps = 0.f;
    uint32_t pk[8];
    auto weights_of = [&](int valid) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool k0 = 8 * ((2 * j) >> 2) + 4 * half + ((2 * j) & 3) < valid;
        const bool k1 = 8 * ((2 * j + 1) >> 2) + 4 * half + ((2 * j + 1) & 3) < valid;
        const float p0 = k0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j], cs, neg_m)) : 0.f;
        const float p1 = k1 ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j + 1], cs, neg_m)) : 0.f;
        ps = j == 0 ? p0 + p1 : ps + (p0 + p1);  // weights are >= +0: the same sum as from 0
        pk[j] = pack_bf16x2(p0, p1);
      }
    };
    auto refit = [&](int valid) {
      const float m_new = fmaxf(m_ref, tile_max(x));
      const float f = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      neg_m = -m_new;
      l_run *= f;
      rescale(f);
      weights_of(valid);
    };
    for (int i = 0; i + 1 < n_tiles; ++i) {
      wait_tile(min(n_tiles - 1, ST + i - 2) - (i + 1), std::integral_constant<int, ST - 3>{});
      raw_barrier();  // tile i+1 visible; tile i-1's stage free
      if (i + ST - 1 < n_tiles) issue(i + ST - 1, st_issue);
      st_issue = st_issue + 1 == ST ? 0 : st_issue + 1;
      const unsigned char* tn = tile_at(st_next);
      const unsigned char* tc = tile_at(st_cur);
      auto frag = [&](int n) -> uint4 {
        if (S::pv(n)) return __builtin_bit_cast(uint4, vread(tc, S::index(n)));
        return kread(tn, S::index(n));
      };
      uint4 fr[DQ];
#pragma unroll
      for (int n = 0; n < DQ; ++n)
        if (n < S::N) fr[n] = frag(n);
      weights_of(kNT);
      if (__builtin_expect(__any(!(ps <= kOverflow)), 0)) refit(kNT);  // wave-uniform, rare
      l_run += ps;
      const uint4 pb[2] = {make_uint4(pk[0], pk[1], pk[2], pk[3]), make_uint4(pk[4], pk[5], pk[6], pk[7])};
      __builtin_amdgcn_sched_barrier(0);
      floatx16_t s_nxt;
#pragma unroll
      for (int j = 0; j < 16; ++j) s_nxt[j] = 0.f;
#pragma unroll
      for (int n = 0; n < S::N; ++n) {
        if (S::pv(n)) {
          const int v = S::index(n);
          o_acc[v % C::CB] = mfma(fr[n % DQ], pb[v / C::CB], o_acc[v % C::CB]);
        } else {
          s_nxt = mfma(fr[n % DQ], qf[S::index(n)], s_nxt);
        }
        if (n + DQ < S::N) fr[n % DQ] = frag(n + DQ);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = s_nxt[j];
      st_cur = st_next;
      st_next = st_next + 1 == ST ? 0 : st_next + 1;
    }
    // Last tile (possibly partial): weights of the tokens past the end are exactly 0, also when
    // the scale is zero; the same overflow check.
    {
      const int valid = t_end - (t_begin + (n_tiles - 1) * kNT);
      weights_of(valid);
      if (__any(!(ps <= kOverflow))) refit(valid);
      l_run += ps;
      const unsigned char* tile = tile_at(st_cur);
      short8_t vf[NPV];
#pragma unroll
      for (int v = 0; v < NPV; ++v) vf[v] = vread(tile, v);
      pv(tile, pk, vf);
    }
  } else {
  // Steady state, iteration i: tile i with tile i+1 resident.  Each k-step of the logits of tile
  // i+1 (one MFMA) also carries one read-ahead K fragment, up to one of tile i's softmax weights
  // and, in the last NPV steps, one value fragment of tile i; then comes tile i's value
  // product, whose steps carry the maximum of tile i+1 (with the pair's exchange at KS = 2).  The
  // steps are fenced so that the compiler keeps this order, which hides the LDS latency behind
  // the matrix cores and the softmax arithmetic in the gaps between MFMA issues.
  // When tile i+1 raises the reference maximum (rare), the iteration leaves the inner loop after
  // its value product, so that the rescale of O -- which needs O out of the accumulation
  // registers -- stays outside the steady-state loop.
  int st_cur = 0, st_next = 1 % ST, st_issue = ST - 1;
  int i = 0;
  uint32_t pk[8];
  while (i + 1 < n_tiles) {
    bool raised = false;
    for (; i + 1 < n_tiles; ++i) {
      wait_tile(min(n_tiles - 1, ST + i - 2) - (i + 1), std::integral_constant<int, ST - 3>{});
      raw_barrier();  // tile i+1 visible; tile i-1's stage and the exchange buffer free
      if (i + ST - 1 < n_tiles) issue(i + ST - 1, st_issue);
      st_issue = st_issue + 1 == ST ? 0 : st_issue + 1;
      const unsigned char* tn = tile_at(st_next);
      const unsigned char* tc = tile_at(st_cur);
      uint4 kf[NPF];
#pragma unroll
      for (int k = 0; k < NPF; ++k) kf[k] = kread(tn, k);
      __builtin_amdgcn_sched_barrier(0);

      floatx16_t s_nxt;
#pragma unroll
      for (int j = 0; j < 16; ++j) s_nxt[j] = 0.f;
      float ps = 0.f, p_lo = 0.f, p_hi = 0.f;
      short8_t vf[NPV];
#pragma unroll
      for (int k = 0; k < KST; ++k) {
        s_nxt = mfma(kf[k % NPF], qf[k], s_nxt);
        if (k + NPF < KST) kf[k % NPF] = kread(tn, k + NPF);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if ((e * KST) / 16 == k) softmax_one(x, e, neg_m, pk, p_lo, p_hi, ps);
        if (k >= KST - NPV) vf[k - (KST - NPV)] = vread(tc, k - (KST - NPV));
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (DEFER) finish_pair(7, p_lo, p_hi, pk, ps);
      l_run = __builtin_fmaf(l_run, alpha, ps);
      if constexpr (KS > 1) sx_write(s_nxt);
      const float m_old = m_ref;
      __builtin_amdgcn_sched_barrier(0);
      alpha = pv_next(tc, pk, vf, s_nxt, x, neg_m);
      st_cur = st_next;
      st_next = st_next + 1 == ST ? 0 : st_next + 1;
      if (__any(alpha != 1.0f && m_old != -INFINITY)) {  // wave-uniform, rare
        raised = true;
        ++i;
        break;
      }
    }
    if (!raised) break;
    rescale(alpha);  // before tile i's weights are added
  }

  // Last tile (possibly partial): weights of the tokens past the end are exactly 0, also when
  // the scale is zero.  Its maximum is known and O already rescaled.
  {
    const int i = n_tiles - 1;
    const int valid = t_end - (t_begin + i * kNT);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool k0 = 8 * ((2 * j) >> 2) + 4 * half + ((2 * j) & 3) < valid;
      const bool k1 = 8 * ((2 * j + 1) >> 2) + 4 * half + ((2 * j + 1) & 3) < valid;
      const float p0 = k0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j], cs, neg_m)) : 0.f;
      const float p1 = k1 ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j + 1], cs, neg_m)) : 0.f;
      ps = j == 0 ? p0 + p1 : ps + (p0 + p1);
      pk[j] = pack_bf16x2(p0, p1);
    }
    l_run = __builtin_fmaf(l_run, alpha, ps);
    const unsigned char* tile = tile_at(st_cur);
    short8_t vf[NPV];
#pragma unroll
    for (int v = 0; v < NPV; ++v) vf[v] = vread(tile, v);
    pv(tile, pk, vf);
  }

  }

  // Chunk result: o = O / l, lse = ln 2 * (m + log2 l); the two lane halves hold disjoint tokens.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  // A separate instantiation (DIRECT) carries this, so that the decode kernels' registers are
  // allocated without it.
  if constexpr (DIRECT) {
    static_assert(direct_rows(W, KS), "tiles that finish rows");
    static_assert(C::NWAVES * 16384 <= C::ST * C::TILE_BYTES, "the row exchange fits in the ring");
    if (whole && a.direct_out != nullptr) {  // workgroup-uniform
      finish_row<C::CB>(o_acc, l_tot, m_ref, a, b, head, kh, half, lane, lds + static_cast<size_t>(wv) * 16384,
                        lds + static_cast<size_t>(wv ^ 1) * 16384);
      __syncthreads();  // the next segment reuses the ring, which held the exchange
      continue;
    }
  }
  const float inv = 1.0f / l_tot;
  const int64_t part = part_row0 + head;
  float* dst = a.part_o + part * W;
#pragma unroll
  for (int cbl = 0; cbl < C::CB; ++cbl) {
    const int cb = kh * C::CB + cbl;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int col = 32 * cb + 8 * j4 + 4 * half;
      const float4 v = make_float4(o_acc[cbl][4 * j4] * inv, o_acc[cbl][4 * j4 + 1] * inv, o_acc[cbl][4 * j4 + 2] * inv,
                                   o_acc[cbl][4 * j4 + 3] * inv);
      *reinterpret_cast<float4*>(dst + col) = v;
    }
  }
  if (half == 0 && kh == 0) a.part_lse[part] = (m_ref + log2f(l_tot)) * kLn2;
  if (a.sched == 0) return;  // a chunk is a single segment
  __syncthreads();           // the next segment reuses the ring and the page list
  }
}

template <int W, int DR, int HB, int KS, int STQ, int LAYOUT>
hipError_t launch_one(const DecodeLaunch& a, hipStream_t stream) {
  using C = Cfg<W, DR, HB, KS, STQ, LAYOUT>;
  auto kern = decode_mfma_kernel<W, DR, HB, KS, STQ, LAYOUT, false>;
  if constexpr (direct_rows(W, KS))
    if (a.direct_out != nullptr) kern = decode_mfma_kernel<W, DR, HB, KS, STQ, LAYOUT, true>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t units = a.sched == 1 ? a.workers : static_cast<int64_t>(a.num_chunks) * a.batch;
  const int members = a.shard_count * (a.heads / (32 * HB));
  const int64_t blocks = (units + a.xcds - 1) / a.xcds * a.xcds * members;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  int page_shift = -1;
  if (LAYOUT != 0 && (a.page_size & (a.page_size - 1)) == 0) page_shift = __builtin_ctz(a.page_size);
  const float scale_log2 = static_cast<float>(static_cast<double>(a.scale) * 1.4426950408889634);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(C::THREADS), C::LDS_BYTES, stream, a, scale_log2,
                     static_cast<int>(units), members, page_shift);
  return hipGetLastError();
}

template <int W, int DR, int HB, int KS, int STQ>
hipError_t launch_layout(const DecodeLaunch& a, hipStream_t stream) {
  if (a.block_table == nullptr) return launch_one<W, DR, HB, KS, STQ, 0>(a, stream);
  // layout 1: power-of-two pages of whole tiles whose bytes fit 32 bits (the kernel's page address)
  const bool page_fits = static_cast<int64_t>(a.page_size) * (a.d_latent + DR) * 2 < (int64_t{1} << 32);
  if (a.page_size % kNT == 0 && (a.page_size & (a.page_size - 1)) == 0 && page_fits)
    return launch_one<W, DR, HB, KS, STQ, 1>(a, stream);
  return launch_one<W, DR, HB, KS, STQ, 2>(a, stream);
}

// Tile configuration per value width: (largest head-block count per workgroup, key split, ring
// stages).  Overridable at build time for tuning sweeps.
#ifndef TPLA_W128_CFG
#define TPLA_W128_CFG 4, 1, 6
#endif
#ifndef TPLA_W256_CFG
#define TPLA_W256_CFG 4, 1, 5
#endif
#ifndef TPLA_W512_CFG
#define TPLA_W512_CFG 2, 2, 3
#endif
struct TileCfg {
  int hb_max, ks, st;
};
constexpr TileCfg kW128{TPLA_W128_CFG}, kW256{TPLA_W256_CFG}, kW512{TPLA_W512_CFG};

constexpr TileCfg tile_cfg(int w) { return w == 128 ? kW128 : (w == 256 ? kW256 : kW512); }

// Head blocks of 32 per workgroup: the largest of (hb_max, 2, 1) that divides the heads.
int pick_hb(int w, int heads) {
  const int cap = tile_cfg(w).hb_max;
  if (cap >= 4 && heads % 128 == 0) return 4;
  if (cap >= 2 && heads % 64 == 0) return 2;
  return 1;
}

template <int W, int HBMAX, int KS, int ST>
hipError_t launch_w(const DecodeLaunch& a, hipStream_t stream) {
  const int hb = pick_hb(W, a.heads);
  if constexpr (HBMAX >= 4)
    if (hb == 4) return launch_layout<W, 64, 4, KS, ST>(a, stream);
  if constexpr (HBMAX >= 2)
    if (hb == 2) return launch_layout<W, 64, 2, KS, ST>(a, stream);
  return launch_layout<W, 64, 1, KS, ST>(a, stream);
}

}  // namespace

bool mfma_supported(int w, int d_rope, int heads) {
  return (w == 128 || w == 256 || w == 512) && d_rope == 64 && heads % 32 == 0;
}

void mfma_plan_info(int w, int heads, int* head_groups, int* wgs_per_cu) {
  const int hb = pick_hb(w, heads);
  *head_groups = heads / (32 * hb);
  // one wave per SIMD (or two, see waves_per_simd), so a CU holds 4 / (waves per workgroup)
  // workgroups, times the waves per SIMD
  const int waves = hb * tile_cfg(w).ks;
  *wgs_per_cu = (waves >= 4 ? 1 : 4 / waves) * waves_per_simd(w, hb, tile_cfg(w).ks);
}

int mfma_max_chunk_pages() { return kMaxPages - 2; }

bool mfma_direct_rows(int w) { return direct_rows(w, tile_cfg(w).ks); }

int mfma_max_segment_pages() { return kMaxPages - 2; }

hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t stream) {
  if (!mfma_supported(a.w, a.d_rope, a.heads)) return hipErrorInvalidValue;
  // the chunk's block-table entries must fit the LDS page list
  if (a.block_table != nullptr && a.sched == 0 && a.chunk_tokens / a.page_size + 2 > kMaxPages) return hipErrorInvalidValue;
  switch (a.w) {
    case 128: return launch_w<128, kW128.hb_max, kW128.ks, kW128.st>(a, stream);
    case 256: return launch_w<256, kW256.hb_max, kW256.ks, kW256.st>(a, stream);
    default: return launch_w<512, kW512.hb_max, kW512.ks, kW512.st>(a, stream);
  }
}

}  // namespace tpla
