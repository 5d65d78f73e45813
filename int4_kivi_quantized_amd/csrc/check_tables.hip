// On-demand device check of the block table and context lengths that the
// append and decode kernels trust (their device preconditions, include/s4kv.h).
//
// One work-group walks every (sequence, page) entry of the table: a length
// outside [0, 16 * max_pages] (or above max_ctx, when given) counts once per
// sequence; a block id outside [0, num_pages) counts when its page holds one
// of the sequence's tokens. The first fault is the smallest (sequence, page)
// key, with page -1 standing for a length fault. Counts and the first fault
// are reduced in LDS in a fixed order and written by one thread, so the
// report needs no clearing beforehand and is the same on every run.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace s4kv {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int32_t B,
    int32_t max_pages, int32_t num_pages, int32_t max_ctx, int32_t* __restrict__ report) {
  __shared__ int32_t red_len[kCheckThreads], red_ids[kCheckThreads];
  __shared__ int64_t red_key[kCheckThreads];
  const int t = threadIdx.x;
  const int64_t row = (int64_t)max_pages + 1;  // key = b * row + (page + 1)
  const int64_t none = (int64_t)B * row;       // larger than every key
  const int64_t limit = (int64_t)max_pages * kPage;
  int32_t bad_len = 0, bad_ids = 0;
  int64_t first = none;
  // lengths, one sequence per thread and step
  for (int b = t; b < B; b += kCheckThreads) {
    const int32_t c = ctx_lens[b];
    if (c < 0 || c > limit || (max_ctx > 0 && c > max_ctx)) {
      ++bad_len;
      first = min(first, (int64_t)b * row);
    }
  }
  // block ids of the pages in use, one table entry per thread and step
  const int64_t entries = (int64_t)B * max_pages;
  for (int64_t i = t; i < entries; i += kCheckThreads) {
    const int b = static_cast<int>(i / max_pages);
    const int p = static_cast<int>(i - (int64_t)b * max_pages);
    const int64_t c = min(max((int64_t)ctx_lens[b], (int64_t)0), limit);
    if (p >= (c + kPage - 1) / kPage) continue;
    const int32_t id = block_table[i];
    if (id < 0 || id >= num_pages) {
      ++bad_ids;
      first = min(first, (int64_t)b * row + p + 1);
    }
  }
  red_len[t] = bad_len;
  red_ids[t] = bad_ids;
  red_key[t] = first;
  __syncthreads();
  for (int stride = kCheckThreads / 2; stride > 0; stride /= 2) {
    if (t < stride) {
      red_len[t] += red_len[t + stride];
      red_ids[t] += red_ids[t + stride];
      red_key[t] = min(red_key[t], red_key[t + stride]);
    }
    __syncthreads();
  }
  if (t == 0) {
    const int64_t k = red_key[0];
    report[0] = red_len[0];
    report[1] = red_ids[0];
    report[2] = k == none ? -1 : static_cast<int32_t>(k / row);
    report[3] = k == none ? -1 : static_cast<int32_t>(k % row) - 1;
  }
}

}  // namespace

hipError_t launch_check_tables(const s4kv_shape& s, const int32_t* block_table,
                               const int32_t* ctx_lens, int32_t max_ctx, int32_t* report,
                               hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, block_table,
                     ctx_lens, s.num_seqs, s.max_pages_per_seq, s.num_pages, max_ctx, report);
  return hipGetLastError();
}

}  // namespace s4kv
