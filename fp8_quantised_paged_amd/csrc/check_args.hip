// Device-side check of the attention calls' caller contract: the block table,
// context lengths and query offsets live in device memory, so the host checks
// of every entry point cannot see them. This pass reads them once and reports,
// per rule, whether it is broken and the first sequence that breaks it.
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

constexpr int kCheckThreads = 256;

// result[0]: rule bits (kCheckBadSeqLen, kCheckBadQueries, kCheckBadPage); result[1..3]: the
// lowest offending sequence of each rule (INT32_MAX when none).
__global__ void check_init_kernel(int32_t* result) {
  if (threadIdx.x == 0) {
    result[0] = 0;
    result[1] = INT32_MAX;
    result[2] = INT32_MAX;
    result[3] = INT32_MAX;
  }
}

// One thread per (sequence, logical page) entry, grid-stride. The per-sequence
// rules are checked by the thread of page 0 of each sequence.
__global__ __launch_bounds__(kCheckThreads) void check_paged_args_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q_lens, int32_t batch, int32_t max_pages, int32_t page_size,
    int64_t num_pages, int32_t total_q, int32_t max_q_len, int32_t* __restrict__ result) {
  __shared__ int32_t s_bits;
  __shared__ int32_t s_first[3];
  if (threadIdx.x == 0) {
    s_bits = 0;
    s_first[0] = s_first[1] = s_first[2] = INT32_MAX;
  }
  __syncthreads();
  const int64_t cap = (int64_t)max_pages * page_size;
  const int64_t n = (int64_t)batch * max_pages;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int32_t b = (int32_t)(idx / max_pages);
    const int32_t j = (int32_t)(idx % max_pages);
    const int32_t L = seq_lens[b];
    if (j == 0) {
      int32_t ql = 1;
      bool bad_q = false;
      if (cu_q_lens != nullptr) {
        const int32_t c0 = cu_q_lens[b];
        const int32_t c1 = cu_q_lens[b + 1];
        ql = c1 - c0;
        bad_q = ql < 0 || ql > max_q_len || (b == 0 && c0 != 0) || (b == batch - 1 && c1 != total_q);
      }
      const bool bad_len = L < 0 || (int64_t)L > cap;
      // a verify row would sit before key 0 (a decode row over no keys is allowed:
      // its output is zero, its partials empty)
      if (cu_q_lens != nullptr && !bad_len && !bad_q && ql > L) bad_q = true;
      if (bad_len) {
        atomicOr(&s_bits, kCheckBadSeqLen);
        atomicMin(&s_first[0], b);
      }
      if (bad_q) {
        atomicOr(&s_bits, kCheckBadQueries);
        atomicMin(&s_first[1], b);
      }
    }
    // only the pages that hold keys are read by the kernels
    const int64_t used = (L <= 0) ? 0 : ((int64_t)min((int64_t)L, cap) + page_size - 1) / page_size;
    if (j < used) {
      const int32_t pg = block_table[idx];
      if (pg < 0 || (int64_t)pg >= num_pages) {
        atomicOr(&s_bits, kCheckBadPage);
        atomicMin(&s_first[2], b);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && s_bits != 0) {
    atomicOr(&result[0], s_bits);
    atomicMin(&result[1], s_first[0]);
    atomicMin(&result[2], s_first[1]);
    atomicMin(&result[3], s_first[2]);
  }
}

}  // namespace

hipError_t launch_check_paged_args(const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q_lens,
                                   int32_t batch, int32_t max_pages, int32_t page_size, int64_t num_pages,
                                   int32_t total_q, int32_t max_q_len, int32_t* result, hipStream_t stream) {
  check_init_kernel<<<1, 64, 0, stream>>>(result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)batch * max_pages;
  const int64_t want = (n + kCheckThreads - 1) / kCheckThreads;
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 1024 ? 1024 : want));
  check_paged_args_kernel<<<grid, kCheckThreads, 0, stream>>>(block_table, seq_lens, cu_q_lens, batch, max_pages,
                                                              page_size, num_pages, total_q, max_q_len, result);
  return hipGetLastError();
}

}  // namespace kvfp8
