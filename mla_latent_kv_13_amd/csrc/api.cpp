// C ABI of the latent-cache decode library: argument checks, split-K planning, workspace layout
// and kernel launches.  Declarations and the contract of every entry point: include/tpla.h.
#include "../../include/tpla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int32_t ok() {
  g_last_error[0] = '\0';
  return TPLA_OK;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(TPLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxChunksMerge = 4096;

// Compute units and XCDs (accelerator complex dies, each with its own L2) of the current device.
// The split-K plan sizes its grid to fill every CU once, and the kernels place workgroups that
// share rows on one XCD.  Read once per device from the runtime, so that a partitioned device (one
// XCD per partition) or a part with fewer CUs gets a plan of its own shape.  Without a device
// (e.g. a workspace-size query on a host with no GPU) a whole MI355X is assumed: 256 CUs in 8
// XCDs.
constexpr int kMaxDevices = 64;
struct DeviceShape {
  int cus, xcds;
};
DeviceShape device_shape() {
  static std::atomic<int> cached[kMaxDevices];  // cus << 8 | xcds, 0 while unknown
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return {256, 8};
  }
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1 || xcds > 255)
      xcds = 1;
    (void)hipGetLastError();
    v = (std::min(cus, 1 << 22) << 8) | xcds;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return {v >> 8, v & 255};
}

// Scratch of the allocation-free decode entry point (tpla_decode_sharded_noalloc): one
// file-scope device array, which every GPU the library runs on holds from the module's load until
// the process ends.  Host code never passes `scratch` itself (in host code the name is a host-side
// stand-in, not a device address): the device address is read once per device with
// hipGetSymbolAddress, with that device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int32_t scratch_address(void** ptr) {
  static std::atomic<void*> per_device[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TPLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TPLA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
  void* p = per_device[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TPLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    per_device[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return TPLA_OK;
}

struct Plan {
  int kernel;        // 1 generic, 2 MFMA
  int chunk_tokens;
  int num_chunks;
  int sched;         // 0 chunked, 1 balanced
  int workers;       // balanced: workgroups per (shard, head group)
  int64_t slots;     // partial slots per (shard, head)
  size_t off_rows, off_qrot, off_prefix, off_part_o, off_part_lse, total;
};

int32_t check_desc(const tpla_cache_desc_t* d) {
  if (d == nullptr) return fail(TPLA_ERR_INVALID_ARGUMENT, "cache descriptor is NULL");
  if (d->dtype != TPLA_F32 && d->dtype != TPLA_BF16) return fail(TPLA_ERR_UNSUPPORTED, "dtype %d is not fp32 or bf16", d->dtype);
  if (d->d_latent < 1 || d->d_rope < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "d_latent must be >= 1 and d_rope >= 0");
  if (d->page_size < 1 || d->num_pages < 1) return fail(TPLA_ERR_INVALID_ARGUMENT, "page_size and num_pages must be >= 1");
  if (d->max_pages_per_seq < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq must be >= 0");
  if (d->transform != TPLA_LATENT_IDENTITY && d->transform != TPLA_LATENT_WHT)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "unknown latent transform %d", d->transform);
  const int vec = d->dtype == TPLA_BF16 ? 8 : 4;
  if (d->d_latent % vec != 0 || d->d_rope % vec != 0)
    return fail(TPLA_ERR_UNSUPPORTED, "d_latent and d_rope must be multiples of %d for this dtype", vec);
  if (d->transform == TPLA_LATENT_WHT && (d->d_latent > 1024 || (d->d_latent & (d->d_latent - 1)) != 0))
    return fail(TPLA_ERR_UNSUPPORTED, "the Hadamard transform needs d_latent a power of two <= 1024");
  const int64_t pool_rows = static_cast<int64_t>(d->num_pages) * d->page_size;
  if (pool_rows * (d->d_latent + d->d_rope) > (int64_t(1) << 40))
    return fail(TPLA_ERR_UNSUPPORTED, "cache pool larger than 2^40 elements");
  return TPLA_OK;
}

// `batch` counts query rows: sequences for a decode call, new tokens for a prefill call
// (prefill = true), whose row map (prefix length and sequence per row) the workspace also holds.
int32_t make_plan(const tpla_cache_desc_t* d, int32_t batch, int32_t heads, int32_t num_shards, int32_t shard_count,
                  int32_t max_seq_len, const tpla_decode_opts_t* opts, Plan* plan, bool prefill = false) {
  int32_t st = check_desc(d);
  if (st != TPLA_OK) return st;
  if (batch < 1 || heads < 1) return fail(TPLA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
  if (batch > 65535 || static_cast<int64_t>(heads) * shard_count > 65535)
    return fail(TPLA_ERR_UNSUPPORTED, prefill ? "num_queries and heads must be <= 65535"
                                              : "batch and heads * shard_count must be <= 65535");
  if (max_seq_len < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0");
  if (num_shards < 1 || d->d_latent % num_shards != 0)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "num_shards=%d must be >= 1 and divide d_latent=%d", num_shards, d->d_latent);
  if (shard_count < 1 || shard_count > num_shards)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "shard_count=%d outside [1, num_shards]", shard_count);
  const int w = d->d_latent / num_shards;
  const int req_kernel = opts ? opts->kernel : 0;
  if (req_kernel < 0 || req_kernel > 2) return fail(TPLA_ERR_INVALID_ARGUMENT, "opts->kernel must be 0, 1 or 2");
  const bool mfma_ok = d->dtype == TPLA_BF16 && tpla::mfma_supported(w, d->d_rope, heads);
  if (req_kernel == 2 && !mfma_ok)
    return fail(TPLA_ERR_UNSUPPORTED, "no MFMA tile for bf16 w=%d d_rope=%d heads=%d (needs w in {128,256,512}, d_rope 64, heads %% 32 == 0)",
                w, d->d_rope, heads);
  plan->kernel = req_kernel != 0 ? req_kernel : (mfma_ok ? 2 : 1);
  if (plan->kernel == 1 && (w > 1024 || w + d->d_rope > 1024 + 256))
    return fail(TPLA_ERR_UNSUPPORTED, "generic kernel supports w <= 1024 and w + d_rope <= 1280");

  const int span = std::max(max_seq_len, 1);
  int ct = opts ? opts->chunk_tokens : 0;
  if (ct < 0 || ct % 64 != 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "chunk_tokens=%d must be 0 or a multiple of 64", ct);
  if (ct == 0) {
    if (plan->kernel == 2) {
      // One round of workgroups fills the chip: chunks per sequence so that
      // sequences x chunks x shards x head groups = CUs x workgroups per CU.  Fewer, longer chunks
      // keep the split-K partials (heads x d_latent fp32 per chunk) small next to the cache bytes.
      int head_groups = 1, per_cu = 1;
      tpla::mfma_plan_info(w, heads, &head_groups, &per_cu);
      const int64_t per_index = static_cast<int64_t>(batch) * shard_count * head_groups;
      const int64_t slots = static_cast<int64_t>(device_shape().cus) * per_cu;
      int64_t per_seq = std::max<int64_t>(1, (slots + per_index - 1) / per_index);
      if (d->max_pages_per_seq > 0) per_seq = std::max<int64_t>(per_seq, 32);  // ragged lengths: finer chunks balance better
      ct = static_cast<int>(round_up((span + per_seq - 1) / per_seq, 64));
      ct = std::max(ct, 256);
    } else {
      ct = static_cast<int>(std::min<int64_t>(round_up(span, 64), 1024));
    }
  }
  // Longest chunk each kernel takes: the generic kernel keeps a chunk's logits in LDS; the MFMA
  // kernel on a paged cache stages a chunk's block-table entries there.
  int max_ct = 1 << 30;
  if (plan->kernel == 1) max_ct = 2048;
  if (plan->kernel == 2 && d->max_pages_per_seq > 0)
    max_ct = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(tpla::mfma_max_chunk_pages() - 1) * d->page_size, 1 << 30));
  max_ct = std::max(64, max_ct / 64 * 64);
  if (ct > max_ct) {
    if (opts && opts->chunk_tokens)
      return fail(TPLA_ERR_UNSUPPORTED, plan->kernel == 1 ? "generic kernel chunk_tokens must be <= 2048"
                                                           : "chunk_tokens spans more cache pages than the kernel stages");
    ct = max_ct;
  }
  int nc = (span + ct - 1) / ct;
  if (nc > kMaxChunksMerge) {
    // Past this many chunks, chunks grow (up to the kernel's limit) rather than the partials.
    if (opts && opts->chunk_tokens) return fail(TPLA_ERR_UNSUPPORTED, "more than %d chunks per sequence", kMaxChunksMerge);
    ct = static_cast<int>(std::min<int64_t>(round_up((span + kMaxChunksMerge - 1) / kMaxChunksMerge, 64), max_ct));
    nc = (span + ct - 1) / ct;
  }
  plan->chunk_tokens = ct;
  plan->num_chunks = nc;
  plan->sched = 0;
  plan->workers = 0;
  plan->slots = static_cast<int64_t>(batch) * nc;
  const int req_sched = opts ? opts->schedule : 0;
  if (req_sched < 0 || req_sched > 2) return fail(TPLA_ERR_INVALID_ARGUMENT, "opts->schedule must be 0, 1 or 2");
  const int64_t max_tiles = static_cast<int64_t>(batch) * ((static_cast<int64_t>(span) + 31) / 32);
  const bool balanced_ok = plan->kernel == 2 && max_tiles < (int64_t(1) << 30);
  if (req_sched == 2 && !balanced_ok)
    return fail(TPLA_ERR_UNSUPPORTED, "the balanced schedule needs the MFMA kernel and fewer than 2^30 tiles");
  if (balanced_ok && (req_sched == 2 || (req_sched == 0 && d->max_pages_per_seq > 0))) {
    // One workgroup per slot of the chip.  A segment (a share's tiles of one sequence) must not
    // span more cache pages than a workgroup stages; a segment never outgrows its sequence, so
    // only contexts longer than that bound call for more, shorter shares.
    int head_groups = 1, per_cu = 1;
    tpla::mfma_plan_info(w, heads, &head_groups, &per_cu);
    const int64_t members = static_cast<int64_t>(shard_count) * head_groups;
    int64_t workers = std::max<int64_t>(1, static_cast<int64_t>(device_shape().cus) * per_cu / members);
    if (d->max_pages_per_seq > 0) {
      const int64_t cap_tiles = std::max<int64_t>(1, static_cast<int64_t>(tpla::mfma_max_segment_pages() - 1) * d->page_size / 32 - 1);
      const int64_t span_tiles = (static_cast<int64_t>(span) + 31) / 32;
      if (span_tiles > cap_tiles) workers = std::max(workers, (max_tiles + cap_tiles - 1) / cap_tiles);
    }
    workers = std::min<int64_t>(workers, std::max<int64_t>(1, max_tiles));
    plan->sched = 1;
    plan->workers = static_cast<int>(workers);
    plan->slots = batch + workers;
  }

  size_t off = 0;
  plan->off_rows = off;
  if (prefill) off += 2 * round_up(static_cast<size_t>(batch) * 4, 256);
  plan->off_qrot = off;
  if (d->transform == TPLA_LATENT_WHT) {
    const size_t elem = plan->kernel == 1 ? 4 : 2;
    off += round_up(static_cast<size_t>(batch) * heads * d->d_latent * elem, 256);
  }
  plan->off_prefix = off;
  if (plan->sched == 1) off += round_up(static_cast<size_t>(batch + 1) * 4, 256);
  plan->off_part_o = off;
  off += round_up(static_cast<size_t>(plan->slots) * shard_count * heads * static_cast<size_t>(w) * 4, 256);
  plan->off_part_lse = off;
  off += round_up(static_cast<size_t>(plan->slots) * shard_count * heads * 4, 256);
  plan->total = off;
  return TPLA_OK;
}

// Query rows of a prefill call (see mla_prefill_absorbed): query_start [sequences + 1].
struct PrefillRows {
  const int32_t* query_start;
  int32_t sequences;
};

// The value up-projection fused into the merge (tpla_decode_sharded_projected).
struct Projection {
  int32_t w_dtype;
  const void* w_uv;
  int32_t d_v;
  float* out_v;
};

// One decode call over `batch` query rows.  Decode: row b is sequence b over seq_lens[b] tokens.
// Prefill (pf non-null): `batch` new-token rows of pf->sequences sequences, each over its causal
// prefix of the cache (the row map is built on the device first).
int32_t decode_impl(const tpla_cache_desc_t* d, const void* cache, const int32_t* block_table,
                    const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t max_seq_len, const void* q_latent,
                    const void* q_rope, float scale, int32_t num_shards, int32_t shard_begin, int32_t shard_count,
                    float* out, float* lse, void* workspace, size_t workspace_bytes, const tpla_decode_opts_t* opts,
                    void* stream_ptr, const PrefillRows* pf = nullptr, const Projection* proj = nullptr) {
  Plan plan;
  int32_t st = make_plan(d, batch, heads, num_shards, shard_count, max_seq_len, opts, &plan, pf != nullptr);
  if (st != TPLA_OK) return st;
  const int32_t sequences = pf ? pf->sequences : batch;
  if (shard_begin < 0 || shard_begin + shard_count > num_shards)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "shard range [%d, %d) outside [0, %d)", shard_begin, shard_begin + shard_count, num_shards);
  if (!cache || !seq_lens || !q_latent || (!proj && !out) || (d->d_rope > 0 && !q_rope))
    return fail(TPLA_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  if (!aligned(cache, 16) || !aligned(q_latent, 16) || (q_rope && !aligned(q_rope, 16)) || (out && !aligned(out, 16)))
    return fail(TPLA_ERR_INVALID_ARGUMENT, "cache, q_latent, q_rope and out must be 16-byte aligned");
  if (proj) {
    if (proj->w_dtype != TPLA_BF16)
      return fail(TPLA_ERR_UNSUPPORTED, "the fused up-projection takes bf16 weights (w_dtype %d); fp32 weights: "
                  "tpla_decode_sharded then tpla_value_up_projection", proj->w_dtype);
    if (proj->d_v < 1) return fail(TPLA_ERR_INVALID_ARGUMENT, "d_v must be >= 1");
    if (proj->d_v > 512 || d->d_latent % 16 != 0)
      return fail(TPLA_ERR_UNSUPPORTED, "the fused up-projection needs d_v <= 512 and d_latent a multiple of 16 (d_v=%d, d_latent=%d)",
                  proj->d_v, d->d_latent);
    if (!proj->w_uv || !proj->out_v) return fail(TPLA_ERR_INVALID_ARGUMENT, "w_uv and out_v must not be NULL");
    if (!aligned(proj->w_uv, 16) || !aligned(proj->out_v, 16))
      return fail(TPLA_ERR_INVALID_ARGUMENT, "w_uv and out_v must be 16-byte aligned");
  }
  if (!(scale == scale)) return fail(TPLA_ERR_INVALID_ARGUMENT, "scale is NaN");
  if (block_table == nullptr) {
    if (d->num_pages < sequences || d->page_size < max_seq_len)
      return fail(TPLA_ERR_INVALID_ARGUMENT, "without a block table sequence b uses page b: need num_pages >= batch and page_size >= max_seq_len");
  } else {
    if (static_cast<int64_t>(d->max_pages_per_seq) * d->page_size < max_seq_len)
      return fail(TPLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq * page_size < max_seq_len");
  }
  if (plan.total > 0 && (workspace == nullptr || !aligned(workspace, 256)))
    return fail(TPLA_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < plan.total)
    return fail(TPLA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, plan.total);

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const int w = d->d_latent / num_shards;
  const bool wht = d->transform == TPLA_LATENT_WHT;

  tpla::DecodeLaunch L;
  L.cache = cache;
  L.block_table = block_table;
  L.seq_lens = seq_lens;
  L.q_lat = q_latent;
  L.q_rope = q_rope;
  L.q_lat_f32 = d->dtype == TPLA_F32 ? 1 : 0;
  L.scale = scale;
  L.batch = batch;
  L.heads = heads;
  L.d_latent = d->d_latent;
  L.d_rope = d->d_rope;
  L.w = w;
  L.page_size = d->page_size;
  L.max_pages_per_seq = d->max_pages_per_seq;
  L.shard_begin = shard_begin;
  L.shard_count = shard_count;
  L.chunk_tokens = plan.chunk_tokens;
  L.num_chunks = plan.num_chunks;
  L.part_o = reinterpret_cast<float*>(ws + plan.off_part_o);
  L.part_lse = reinterpret_cast<float*>(ws + plan.off_part_lse);
  L.sched = plan.sched;
  L.workers = plan.workers;
  L.tile_prefix = reinterpret_cast<const int*>(ws + plan.off_prefix);
  L.row_seq = nullptr;
  L.xcds = device_shape().xcds;
  L.direct_out = nullptr;
  L.direct_lse = nullptr;
  L.direct_wht = wht ? 1 : 0;

  hipError_t e;
  if (pf) {
    int* row_len = reinterpret_cast<int*>(ws + plan.off_rows);
    int* row_seq = reinterpret_cast<int*>(ws + plan.off_rows + round_up(static_cast<size_t>(batch) * 4, 256));
    e = tpla::launch_prefill_rows(pf->query_start, seq_lens, pf->sequences, batch, max_seq_len, row_len, row_seq, stream);
    if (e != hipSuccess) return hip_fail(e, "prefill row map launch");
    seq_lens = row_len;  // from here on every row is a decode row over its own prefix
    L.seq_lens = row_len;
    L.row_seq = row_seq;
    // exact MLA over the whole latent under the balanced schedule: a row that one worker
    // computes whole (most prefill rows) is finished in the decode kernel, not merged
    if (plan.kernel == 2 && plan.sched == 1 && num_shards == 1 && shard_count == 1 && tpla::mfma_direct_rows(w)) {
      L.direct_out = out;
      L.direct_lse = lse;
    }
  }
  int* prefix = reinterpret_cast<int*>(ws + plan.off_prefix);
  if (plan.sched == 1 && !wht) {
    e = tpla::launch_tile_prefix(seq_lens, batch, prefix, stream);
    if (e != hipSuccess) return hip_fail(e, "tile prefix launch");
  }
  if (wht) {
    // the query rotation's launch also computes the tile prefix when the schedule needs one
    void* qrot = ws + plan.off_qrot;
    const int dst_f32 = plan.kernel == 1 ? 1 : 0;
    e = tpla::launch_rotate_query(q_latent, d->dtype == TPLA_BF16 ? 1 : 0, batch * heads, d->d_latent, qrot, dst_f32, stream,
                                  seq_lens, batch, plan.sched == 1 ? prefix : nullptr);
    if (e != hipSuccess) return hip_fail(e, "query rotation launch");
    L.q_lat = qrot;
    L.q_lat_f32 = dst_f32;
  }
  if (opts && opts->decode_begin) {
    e = hipEventRecord(static_cast<hipEvent_t>(opts->decode_begin), stream);
    if (e != hipSuccess) return hip_fail(e, "recording decode_begin");
  }
  if (plan.kernel == 2) {
    e = tpla::launch_decode_mfma(L, stream);
    if (e != hipSuccess) return hip_fail(e, "MFMA decode launch");
  } else {
    e = tpla::launch_decode_generic(L, d->dtype == TPLA_BF16 ? 1 : 0, stream);
    if (e != hipSuccess) return hip_fail(e, "generic decode launch");
  }
  if (opts && opts->decode_end) {
    e = hipEventRecord(static_cast<hipEvent_t>(opts->decode_end), stream);
    if (e != hipSuccess) return hip_fail(e, "recording decode_end");
  }
  tpla::MergeLaunch M;
  M.part_o = L.part_o;
  M.part_lse = L.part_lse;
  M.seq_lens = seq_lens;
  M.batch = batch;
  M.heads = heads;
  M.d_latent = d->d_latent;
  M.w = w;
  M.shard_begin = shard_begin;
  M.shard_count = shard_count;
  M.chunk_tokens = plan.chunk_tokens;
  M.num_chunks = plan.num_chunks;
  M.sched = plan.sched;
  M.workers = plan.workers;
  M.tile_prefix = L.tile_prefix;
  M.wht = wht ? 1 : 0;
  M.out = out;
  M.lse = lse;
  M.skip_whole = L.direct_out != nullptr ? 1 : 0;
  if (proj) {
    e = tpla::launch_merge_project(M, static_cast<const uint16_t*>(proj->w_uv), proj->d_v, proj->out_v,
                                   device_shape().xcds, stream);
    if (e != hipSuccess) return hip_fail(e, "merge with up-projection launch");
    return ok();
  }
  e = tpla::launch_merge(M, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

}  // namespace

extern "C" {

int32_t tpla_abi_version(void) { return TPLA_ABI_VERSION; }

const char* tpla_status_string(int32_t status) {
  switch (status) {
    case TPLA_OK: return "TPLA_OK";
    case TPLA_ERR_INVALID_ARGUMENT: return "TPLA_ERR_INVALID_ARGUMENT";
    case TPLA_ERR_UNSUPPORTED: return "TPLA_ERR_UNSUPPORTED";
    case TPLA_ERR_WORKSPACE_TOO_SMALL: return "TPLA_ERR_WORKSPACE_TOO_SMALL";
    case TPLA_ERR_HIP: return "TPLA_ERR_HIP";
    default: return "TPLA_ERR_UNKNOWN";
  }
}

const char* tpla_last_error(void) { return g_last_error; }

int32_t tpla_workspace_size(const tpla_cache_desc_t* desc, int32_t batch, int32_t heads, int32_t num_shards,
                            int32_t shard_count, int32_t max_seq_len, const tpla_decode_opts_t* opts, size_t* bytes) {
  if (bytes == nullptr) return fail(TPLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan plan;
  const int32_t st = make_plan(desc, batch, heads, num_shards, shard_count, max_seq_len, opts, &plan);
  if (st != TPLA_OK) return st;
  *bytes = plan.total;
  return ok();
}

namespace {

int32_t append_impl(const tpla_cache_desc_t* desc, void* cache, const void* rows, const int64_t* slots, int64_t n,
                    int32_t norm_slices, float eps, void* stream) {
  int32_t st = check_desc(desc);
  if (st != TPLA_OK) return st;
  if (n < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "n must be >= 0");
  if (norm_slices < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "norm_slices must be >= 0");
  if (norm_slices > 0) {
    if (desc->d_latent % norm_slices != 0)
      return fail(TPLA_ERR_INVALID_ARGUMENT, "norm_slices=%d must divide d_latent=%d", norm_slices, desc->d_latent);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(TPLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (desc->d_latent > 1024 || (desc->d_latent & (desc->d_latent - 1)) != 0 || norm_slices > 64)
      return fail(TPLA_ERR_UNSUPPORTED, "normalisation needs d_latent a power of two <= 1024 and norm_slices <= 64");
  }
  if (n == 0) return ok();
  if (!cache || !rows || !slots) return fail(TPLA_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  if (!aligned(cache, 16) || !aligned(rows, 16) || !aligned(slots, 8))
    return fail(TPLA_ERR_INVALID_ARGUMENT, "cache and rows must be 16-byte aligned, slots 8-byte aligned");
  if ((desc->transform == TPLA_LATENT_WHT || norm_slices > 0) && n > 0x7fffffffLL)
    return fail(TPLA_ERR_UNSUPPORTED, "at most 2^31-1 rows per rotated or normalised append");
  const hipError_t e = tpla::launch_append(cache, rows, slots, n, desc->d_latent, desc->d_rope,
                                           desc->dtype == TPLA_BF16 ? 1 : 0, desc->transform == TPLA_LATENT_WHT ? 1 : 0,
                                           norm_slices, eps, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

}  // namespace

int32_t latent_cache_append(const tpla_cache_desc_t* desc, void* cache, const void* rows, const int64_t* slots,
                            int64_t n, void* stream) {
  return append_impl(desc, cache, rows, slots, n, 0, 0.f, stream);
}

int32_t latent_cache_append_normed(const tpla_cache_desc_t* desc, void* cache, const void* rows, const int64_t* slots,
                                   int64_t n, int32_t norm_slices, float eps, void* stream) {
  if (norm_slices < 1) return fail(TPLA_ERR_INVALID_ARGUMENT, "norm_slices must be >= 1");
  return append_impl(desc, cache, rows, slots, n, norm_slices, eps, stream);
}

int32_t tpla_merge_context_parts(int32_t transform, int32_t num_shards, int32_t shard_begin, int32_t shard_count,
                                 int32_t parts, int32_t batch, int32_t heads, int32_t d_latent,
                                 const float* out_parts, const float* lse_parts, float* out, float* lse,
                                 void* stream) {
  if (transform != TPLA_LATENT_IDENTITY && transform != TPLA_LATENT_WHT)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "unknown latent transform %d", transform);
  if (parts < 1 || batch < 0 || heads < 0 || d_latent < 1)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "parts >= 1, batch and heads >= 0, d_latent >= 1 required");
  if (num_shards < 1 || d_latent % num_shards != 0)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "num_shards=%d must be >= 1 and divide d_latent=%d", num_shards, d_latent);
  if (shard_begin < 0 || shard_count < 1 || shard_begin + shard_count > num_shards)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "shard range [%d, %d) outside [0, %d)", shard_begin, shard_begin + shard_count,
                num_shards);
  if (d_latent > 1024 || shard_count > 64) return fail(TPLA_ERR_UNSUPPORTED, "d_latent <= 1024 and shard_count <= 64");
  if (transform == TPLA_LATENT_WHT && (d_latent & (d_latent - 1)) != 0)
    return fail(TPLA_ERR_UNSUPPORTED, "the Hadamard transform needs d_latent a power of two <= 1024");
  if (batch > 65535) return fail(TPLA_ERR_UNSUPPORTED, "batch <= 65535");
  if (batch == 0 || heads == 0) return ok();
  if (!out_parts || !lse_parts || !out) return fail(TPLA_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  if (!aligned(out_parts, 16) || !aligned(out, 16) || !aligned(lse_parts, 4) || (lse && !aligned(lse, 4)))
    return fail(TPLA_ERR_INVALID_ARGUMENT, "out_parts and out must be 16-byte aligned, lse_parts and lse 4-byte");
  tpla::ContextMergeLaunch L{};
  L.out_parts = out_parts;
  L.lse_parts = lse_parts;
  L.parts = parts;
  L.batch = batch;
  L.heads = heads;
  L.d_latent = d_latent;
  L.num_shards = num_shards;
  L.shard_begin = shard_begin;
  L.shard_count = shard_count;
  L.wht = transform == TPLA_LATENT_WHT ? 1 : 0;
  L.out = out;
  L.lse = lse;
  const hipError_t e = tpla::launch_context_merge(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "context merge launch");
  return ok();
}

int32_t tpla_value_up_projection(int32_t w_dtype, const float* o, const void* w_uv, int32_t batch, int32_t heads,
                                 int32_t d_latent, int32_t d_v, float* out_v, void* stream) {
  if (w_dtype != TPLA_F32 && w_dtype != TPLA_BF16) return fail(TPLA_ERR_UNSUPPORTED, "w_dtype %d is not fp32 or bf16", w_dtype);
  if (batch < 0 || heads < 0 || d_latent < 1 || d_v < 1)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 0, d_latent and d_v >= 1");
  if (batch == 0 || heads == 0) return ok();
  if (!o || !w_uv || !out_v) return fail(TPLA_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  if (!aligned(o, 16) || !aligned(w_uv, 16) || !aligned(out_v, 16))
    return fail(TPLA_ERR_INVALID_ARGUMENT, "o, w_uv and out_v must be 16-byte aligned");
  if (heads > 65535 || batch > 65535 * 32) return fail(TPLA_ERR_UNSUPPORTED, "heads <= 65535 and batch <= 2097120");
  const hipError_t e = tpla::launch_up_project(o, w_uv, w_dtype, batch, heads, d_latent, d_v, out_v,
                                               device_shape().xcds, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "up-projection launch");
  return ok();
}

int32_t tpla_decode_sharded(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t max_seq_len,
                            const void* q_latent, const void* q_rope, float scale, int32_t num_shards,
                            int32_t shard_begin, int32_t shard_count, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_impl(desc, cache, block_table, seq_lens, batch, heads, max_seq_len, q_latent, q_rope, scale, num_shards,
                     shard_begin, shard_count, out, lse, workspace, workspace_bytes, nullptr, stream);
}

int32_t tpla_decode_sharded_ex(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t max_seq_len,
                               const void* q_latent, const void* q_rope, float scale, int32_t num_shards,
                               int32_t shard_begin, int32_t shard_count, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, const tpla_decode_opts_t* opts, void* stream) {
  return decode_impl(desc, cache, block_table, seq_lens, batch, heads, max_seq_len, q_latent, q_rope, scale, num_shards,
                     shard_begin, shard_count, out, lse, workspace, workspace_bytes, opts, stream);
}

int32_t tpla_decode_sharded_noalloc(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                                    const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t max_seq_len,
                                    const void* q_latent, const void* q_rope, float scale, int32_t num_shards,
                                    int32_t shard_begin, int32_t shard_count, float* out, float* lse, void* stream) {
  // The plan (and with it the scratch this call needs) is the one tpla_decode_sharded makes; the
  // kernels write every scratch byte they later read, so nothing is cleared between calls.
  Plan plan;
  const int32_t st = make_plan(desc, batch, heads, num_shards, shard_count, max_seq_len, nullptr, &plan);
  if (st != TPLA_OK) return st;
  if (plan.total > kScratchBytes)
    return fail(TPLA_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use tpla_decode_sharded with a caller workspace)", plan.total, kScratchBytes);
  void* ws = nullptr;
  const int32_t sst = scratch_address(&ws);
  if (sst != TPLA_OK) return sst;
  return decode_impl(desc, cache, block_table, seq_lens, batch, heads, max_seq_len, q_latent, q_rope, scale, num_shards,
                     shard_begin, shard_count, out, lse, ws, kScratchBytes, nullptr, stream);
}

int32_t tpla_decode_sharded_projected(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t max_seq_len,
                                      const void* q_latent, const void* q_rope, float scale, int32_t num_shards,
                                      int32_t shard_begin, int32_t shard_count, int32_t w_dtype, const void* w_uv,
                                      int32_t d_v, float* out_v, float* lse, void* workspace, size_t workspace_bytes,
                                      const tpla_decode_opts_t* opts, void* stream) {
  const Projection proj{w_dtype, w_uv, d_v, out_v};
  return decode_impl(desc, cache, block_table, seq_lens, batch, heads, max_seq_len, q_latent, q_rope, scale, num_shards,
                     shard_begin, shard_count, nullptr, lse, workspace, workspace_bytes, opts, stream, nullptr, &proj);
}

int32_t mla_decode_absorbed(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t batch, int32_t heads, int32_t max_seq_len,
                            const void* q_latent, const void* q_rope, float scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(desc, cache, block_table, seq_lens, batch, heads, max_seq_len, q_latent, q_rope, scale, 1, 0, 1,
                     out, lse, workspace, workspace_bytes, nullptr, stream);
}

int32_t mla_prefill_workspace_size(const tpla_cache_desc_t* desc, int32_t num_queries, int32_t heads,
                                   int32_t max_seq_len, const tpla_decode_opts_t* opts, size_t* bytes) {
  if (bytes == nullptr) return fail(TPLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (num_queries < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "num_queries must be >= 0");
  if (num_queries == 0) {
    const int32_t st = check_desc(desc);
    if (st != TPLA_OK) return st;
    *bytes = 0;
    return ok();
  }
  Plan plan;
  const int32_t st = make_plan(desc, num_queries, heads, 1, 1, max_seq_len, opts, &plan, true);
  if (st != TPLA_OK) return st;
  *bytes = plan.total;
  return ok();
}

int32_t mla_prefill_absorbed_ex(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* query_start, int32_t batch,
                                int32_t num_queries, int32_t heads, int32_t max_seq_len, const void* q_latent,
                                const void* q_rope, float scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, const tpla_decode_opts_t* opts, void* stream) {
  const int32_t st = check_desc(desc);
  if (st != TPLA_OK) return st;
  if (batch < 1 || heads < 1) return fail(TPLA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
  if (num_queries < 0) return fail(TPLA_ERR_INVALID_ARGUMENT, "num_queries must be >= 0");
  if (query_start == nullptr || seq_lens == nullptr)
    return fail(TPLA_ERR_INVALID_ARGUMENT, "query_start and seq_lens must not be NULL");
  if (num_queries == 0) return ok();  // no new tokens: nothing to compute
  const PrefillRows pf{query_start, batch};
  return decode_impl(desc, cache, block_table, seq_lens, num_queries, heads, max_seq_len, q_latent, q_rope, scale, 1,
                     0, 1, out, lse, workspace, workspace_bytes, opts, stream, &pf);
}

int32_t mla_prefill_absorbed(const tpla_cache_desc_t* desc, const void* cache, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* query_start, int32_t batch, int32_t num_queries,
                             int32_t heads, int32_t max_seq_len, const void* q_latent, const void* q_rope,
                             float scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return mla_prefill_absorbed_ex(desc, cache, block_table, seq_lens, query_start, batch, num_queries, heads,
                                 max_seq_len, q_latent, q_rope, scale, out, lse, workspace, workspace_bytes, nullptr,
                                 stream);
}

}  // extern "C"
