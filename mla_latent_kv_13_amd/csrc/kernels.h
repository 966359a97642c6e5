// Host-side launchers of the HIP kernels (internal to the library; the C ABI is include/tpla.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpla {

// Everything a split-K decode launch needs.  Partial results of chunk c of
// sequence b, computed shard s_local and head h live at
//   part_o  [((b * num_chunks + c) * shard_count + s_local) * heads + h] * w   (w floats)
//   part_lse [((b * num_chunks + c) * shard_count + s_local) * heads + h]
// and exist only for chunks with c * chunk_tokens < seq_lens[b].
struct DecodeLaunch {
  const void* cache;
  const int* block_table;
  const int* seq_lens;
  const void* q_lat;     // [B, H, d_c]: the caller's query, or the rotated copy in the workspace
  const void* q_rope;    // [B, H, d_r]
  int q_lat_f32;         // 1 when q_lat holds fp32 values (the generic kernel's rotated query)
  float scale;
  int batch, heads, d_latent, d_rope, w;
  int page_size, max_pages_per_seq;
  int shard_begin, shard_count;
  int chunk_tokens, num_chunks;
  float* part_o;
  float* part_lse;
  // Balanced schedule (sched = 1, MFMA kernel): min(workers, tiles) workgroups per (shard, head
  // group) take equal shares of all 32-token tiles of the batch; tile_prefix[b] (b = 0..batch)
  // counts the tiles of the sequences before b.  The partial of sequence b from worker w is
  // slot b + w:
  //   part_o [((b + w) * shard_count + s_local) * heads + h] * w_cols   (w_cols = w floats)
  // Chunked schedule (sched = 0): chunk c of sequence b is slot b * num_chunks + c.
  int sched;
  int workers;
  const int* tile_prefix;
  // Cache sequence of query row b (prefill: several query rows of one sequence, each over its
  // own causal prefix, seq_lens[b] being the prefix length); null: row b is sequence b.
  const int* row_seq;
  // XCDs of the device: consecutive workgroup ids are dispatched to the XCDs in turn.
  int xcds;
  // Rows finished in the kernel (balanced schedule, one shard of the whole latent, MFMA kernels
  // for which mfma_direct_rows() holds; null otherwise): a row whose tiles all fall in one
  // worker's share gets its final output written here, [batch, heads, d_latent] (rotated back by
  // H when direct_wht), and its log-sum-exp to direct_lse [batch, heads] (may be null), instead
  // of a partial; the merge then leaves that row alone (MergeLaunch::skip_whole).
  float* direct_out;
  float* direct_lse;
  int direct_wht;
};

struct MergeLaunch {
  const float* part_o;
  const float* part_lse;
  const int* seq_lens;
  int batch, heads, d_latent, w;
  int shard_begin, shard_count;
  int chunk_tokens, num_chunks;
  int sched, workers;
  const int* tile_prefix;
  int wht;
  float* out;
  float* lse;   // may be null
  // 1: rows whose tiles all fall in one worker's share were finished by the decode kernel
  // (DecodeLaunch::direct_out) and are skipped (balanced schedule only)
  int skip_whole;
};

// dtype: 0 = fp32, 1 = bf16 storage.
hipError_t launch_decode_generic(const DecodeLaunch& a, int dtype, hipStream_t stream);
// Decode results over P disjoint parts of each context, merged by log-sum-exp.
struct ContextMergeLaunch {
  const float* out_parts;  // [parts, batch, heads, d_latent]
  const float* lse_parts;  // [parts, batch, shard_count, heads]
  int parts, batch, heads, d_latent;
  int num_shards, shard_begin, shard_count;
  int wht;
  float* out;  // [batch, heads, d_latent]
  float* lse;  // [batch, shard_count, heads] or null
};
hipError_t launch_context_merge(const ContextMergeLaunch& a, hipStream_t stream);

// Returns hipErrorInvalidValue when no MFMA tile covers the shape (checked by mfma_supported first).
bool mfma_supported(int w, int d_rope, int heads);
hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t stream);
// Workgroups the MFMA kernel runs per (sequence, chunk, shard), and how many fit on one CU.
void mfma_plan_info(int w, int heads, int* head_groups, int* wgs_per_cu);
// Largest number of cache pages one chunk of the MFMA kernel may span.
int mfma_max_chunk_pages();
// Whether the MFMA kernel of value width w finishes whole rows itself (DecodeLaunch::direct_out).
bool mfma_direct_rows(int w);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream);
// The merge with the value up-projection fused in: out_v[b,h,:] = W_UV[h] . (the row launch_merge
// would write to a.out, which is not written); bf16 weights [heads, d_v, d_latent], d_latent a
// multiple of 16, 1 <= d_v <= 512.
hipError_t launch_merge_project(const MergeLaunch& a, const uint16_t* w_uv, int d_v, float* out_v, int xcds,
                                hipStream_t stream);
// tile_prefix[b] = sum over b' < b of ceil(seq_lens[b'] / 32), b = 0..batch.
hipError_t launch_tile_prefix(const int* seq_lens, int batch, int* tile_prefix, hipStream_t stream);
// Query rows of a prefill call: row r in [query_start[b], query_start[b+1]) belongs to sequence
// b, sits at position seq_lens[b] - n_b + (r - query_start[b]) of its n_b new tokens and sees the
// cache prefix up to itself: row_len[r] = that position + 1 (clamped to [0, max_seq_len]),
// row_seq[r] = b.  Rows past query_start[batch] get length 0.
hipError_t launch_prefill_rows(const int* query_start, const int* seq_lens, int batch, int num_queries,
                               int max_seq_len, int* row_len, int* row_seq, hipStream_t stream);
// Largest number of cache pages one segment of the MFMA kernel may span (its LDS page list).
int mfma_max_segment_pages();
// Rotate q_lat [B*H, d_c] by the Hadamard matrix into dst (fp32 if dst_f32, else bf16).  With
// tile_prefix non-null the same launch also computes the tile prefix of seq_lens [batch] (as
// launch_tile_prefix).
hipError_t launch_rotate_query(const void* q_lat, int dtype, int rows, int d_latent, void* dst, int dst_f32,
                               hipStream_t stream, const int* seq_lens = nullptr, int batch = 0,
                               int* tile_prefix = nullptr);
// norm_slices > 0: RMS-normalise the (rotated) latent over that many equal slices, unit gain.
hipError_t launch_append(void* cache, const void* rows, const int64_t* slots, int64_t n, int d_latent, int d_rope,
                         int dtype, int wht, int norm_slices, float eps, hipStream_t stream);
// out_v[b,h,:] = W_UV[h] . o[b,h,:]; w_dtype 0 = fp32, 1 = bf16 weights [heads, d_v, d_latent].
hipError_t launch_up_project(const float* o, const void* w_uv, int w_dtype, int batch, int heads, int d_latent,
                             int d_v, float* out_v, int xcds, hipStream_t stream);

}  // namespace tpla
