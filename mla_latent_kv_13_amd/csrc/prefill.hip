// Query-row map of an absorbed MLA prefill call.  Prefill keeps exact MLA (the prefill/decode
// separation of the TPLA review page: referee report, summary; forward implications): every new
// token of a sequence attends to the cached tokens up to and including its own.  One query row
// over its causal prefix is a decode row over a cache of that length, so a prefill call runs the
// decode kernels over its query rows once this map gives each row its sequence (for the cache
// rows) and its prefix length (for the token range).
#include "kernels.h"

namespace tpla {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void prefill_rows_kernel(const int* __restrict__ query_start,
                                                                const int* __restrict__ seq_lens, int batch,
                                                                int num_queries, int max_seq_len,
                                                                int* __restrict__ row_len, int* __restrict__ row_seq) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= num_queries) return;
  // sequence of row r: the last b in [0, batch) with query_start[b] <= r
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (query_start[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int q0 = query_start[lo], q1 = query_start[lo + 1];
  int64_t len = 0;
  if (r >= q0 && r < q1) {
    // the n_b = q1 - q0 new tokens are the last n_b of the sequence's seq_lens[b] cached tokens
    len = static_cast<int64_t>(seq_lens[lo]) - (q1 - q0) + (r - q0) + 1;
    len = len < 0 ? 0 : (len > max_seq_len ? max_seq_len : len);
  }
  row_len[r] = static_cast<int>(len);
  row_seq[r] = lo;
}

}  // namespace

hipError_t launch_prefill_rows(const int* query_start, const int* seq_lens, int batch, int num_queries,
                               int max_seq_len, int* row_len, int* row_seq, hipStream_t stream) {
  if (batch < 1 || num_queries < 1) return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>((num_queries + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(prefill_rows_kernel, dim3(blocks), dim3(kThreads), 0, stream, query_start, seq_lens, batch,
                     num_queries, max_seq_len, row_len, row_seq);
  return hipGetLastError();
}

}  // namespace tpla
