// Host side of the kvfp8 C ABI: argument validation (fail closed, before any
// HIP call), workspace sizing, kernel selection and launch. The library keeps
// no state besides a thread-local error string and allocates nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <vector>

#include "../../include/kvfp8.h"
#include "kvfp8_internal.h"

#define KVFP8_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int32_t ok() {
  g_err[0] = '\0';
  return KVFP8_OK;
}

}  // namespace

namespace kvfp8 {
void set_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }
void clear_error() { g_err[0] = '\0'; }
}  // namespace kvfp8

namespace {

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVFP8_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// finite, positive and normal (a subnormal scale is rejected: no calibrated
// amax / 448 of a non-zero fp16 tensor is subnormal)
bool good_scale(float s) { return std::isfinite(s) && s >= 1.17549435e-38f; }

bool supported_page(int32_t p) { return p == 4 || p == 8 || p == 16 || p == 32 || p == 64; }

constexpr int32_t kMaxSplits = 256;
constexpr int32_t kSplitRows = 32;  // query rows per kv-head handled by the split kernel

struct AttnCommon {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t batch, n_q_heads, n_kv_heads, head_dim, page_size, max_pages;
  float k_scale, v_scale, sm_scale;
  int32_t num_splits;
  float* workspace;
  size_t workspace_bytes;
  uint16_t* out;
};

int32_t check_common(const AttnCommon& c, int64_t n_rows) {
  if (!c.q || !c.k_cache || !c.v_cache || !c.block_table || !c.seq_lens)
    return fail(KVFP8_INVALID_ARG, "null input pointer");
  if (c.batch < 0 || n_rows < 0) return fail(KVFP8_INVALID_ARG, "negative batch or row count");
  if (c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.max_pages <= 0)
    return fail(KVFP8_INVALID_ARG, "heads and max_pages_per_seq must be positive");
  if (c.batch > 65535 || c.n_kv_heads > 65535)
    return fail(KVFP8_UNSUPPORTED, "batch and n_kv_heads must be at most 65535 (launch grid)");
  if (c.n_q_heads % c.n_kv_heads != 0)
    return fail(KVFP8_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                c.n_q_heads, c.n_kv_heads);
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(KVFP8_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c.head_dim);
  if (!supported_page(c.page_size))
    return fail(KVFP8_UNSUPPORTED, "page_size %d (supported: 4, 8, 16, 32, 64)", c.page_size);
  if (c.num_splits < 1 || c.num_splits > kMaxSplits)
    return fail(KVFP8_UNSUPPORTED, "num_splits %d (supported: 1..%d)", c.num_splits, kMaxSplits);
  if (!good_scale(c.k_scale) || !good_scale(c.v_scale) || !good_scale(c.sm_scale))
    return fail(KVFP8_BAD_SCALE, "k_scale, v_scale and sm_scale must be finite, positive and normal "
                "(got %g, %g, %g)", (double)c.k_scale, (double)c.v_scale, (double)c.sm_scale);
  if (!good_scale(c.k_scale * c.sm_scale * kvfp8::kLog2e))
    return fail(KVFP8_BAD_SCALE, "k_scale * sm_scale * log2(e) = %g leaves the normal fp32 range",
                (double)(c.k_scale * c.sm_scale * kvfp8::kLog2e));
  if (!aligned16(c.q) || !aligned16(c.k_cache) || !aligned16(c.v_cache))
    return fail(KVFP8_INVALID_ARG, "q, k_cache and v_cache must be 16-byte aligned");
  if (c.out && !aligned16(c.out)) return fail(KVFP8_INVALID_ARG, "out must be 16-byte aligned");
  if (c.num_splits == 1 && !c.out)
    return fail(KVFP8_INVALID_ARG, "out may be NULL only with num_splits > 1");
  if (c.num_splits > 1) {
    size_t need = kvfp8_attn_workspace_bytes(n_rows, c.n_q_heads, c.head_dim, c.num_splits);
    if (!c.workspace) return fail(KVFP8_WORKSPACE, "num_splits > 1 needs an FP32 workspace");
    if (c.workspace_bytes < need)
      return fail(KVFP8_WORKSPACE, "workspace holds %zu bytes, %zu needed", c.workspace_bytes, need);
    if (!aligned16(c.workspace)) return fail(KVFP8_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  return KVFP8_OK;
}

kvfp8::AttnArgs make_args(const AttnCommon& c, const int32_t* cu_q, int64_t n_rows, int32_t max_q) {
  kvfp8::AttnArgs a{};
  a.q = c.q;
  a.k_cache = c.k_cache;
  a.v_cache = c.v_cache;
  a.block_table = c.block_table;
  a.seq_lens = c.seq_lens;
  a.cu_q_lens = cu_q;
  a.batch = c.batch;
  a.n_q_heads = c.n_q_heads;
  a.n_kv_heads = c.n_kv_heads;
  a.group = c.n_q_heads / c.n_kv_heads;
  a.head_dim = c.head_dim;
  a.page_size = c.page_size;
  a.max_pages = c.max_pages;
  a.num_splits = c.num_splits;
  a.max_q_len = max_q;
  a.score_scale = c.k_scale * c.sm_scale * kvfp8::kLog2e;
  a.v_scale = c.v_scale;
  a.k_scale = c.k_scale;
  if (c.num_splits > 1) {
    float* ws = c.workspace;
    int64_t units = n_rows * c.n_q_heads * (int64_t)c.num_splits;
    a.ws_o = ws;
    a.ws_m = ws + units * c.head_dim;
    a.ws_l = a.ws_m + units;
    a.out = nullptr;
  } else {
    a.out = c.out;
  }
  return a;
}

struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_cache;
  uint8_t* v_cache;
};

int32_t run_attention(const AttnCommon& c, const int32_t* cu_q, int64_t n_rows, int32_t max_q,
                      hipStream_t stream, const AppendArgs* app = nullptr, bool f16_kv = false) {
  if (c.batch == 0 || n_rows == 0) return ok();
  const int32_t group = c.n_q_heads / c.n_kv_heads;
  const int64_t rows = (int64_t)max_q * group;
  kvfp8::AttnArgs a = make_args(c, cu_q, n_rows, max_q);
  if (app) {
    a.k_new = app->k_new;
    a.v_new = app->v_new;
    a.k_cache_w = app->k_cache;
    a.v_cache_w = app->v_cache;
  }
  hipError_t e;
  if (f16_kv) {
    if (rows > kSplitRows)
      return fail(KVFP8_UNSUPPORTED, "the fp16-cache kernel takes at most %d query rows per kv-head", kSplitRows);
    e = kvfp8::launch_attn_split_f16(a, (int)rows, stream);
  } else if (rows <= kSplitRows) {
    e = kvfp8::launch_attn_split(a, (int)rows, stream);
  } else {
    if (c.num_splits != 1)
      return fail(KVFP8_UNSUPPORTED, "chunks longer than %d rows per kv-head need num_splits == 1",
                  kSplitRows);
    e = kvfp8::launch_attn_chunk(a, stream);
  }
  if (e == hipErrorNotSupported) return fail(KVFP8_UNSUPPORTED, "no kernel for this shape");
  if (e != hipSuccess) return hip_status(e, "attention launch");
  if (c.num_splits > 1 && c.out) {
    e = kvfp8::launch_split_reduce(a.ws_o, a.ws_m, a.ws_l, (int32_t)n_rows, c.n_q_heads, c.head_dim,
                                   c.num_splits, c.out, nullptr, stream);
    if (e != hipSuccess) return hip_status(e, "split reduce launch");
  }
  return ok();
}

}  // namespace

// ------------------------------------------------------------ static scratch
// The FP32 split workspace of paged_attn_e4m3_decode_append_noalloc, for
// callers that cannot allocate: a file-scope device array of
// KVFP8_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns for the current device may reach a
// kernel.
static __device__ __align__(256) float scratch[KVFP8_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current GPU's copy of `scratch`, looked up once per
// device with that device current and kept.
int32_t device_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(KVFP8_UNSUPPORTED, "device %d: the scratch table holds devices 0..%d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(KVFP8_HIP_ERROR, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return KVFP8_OK;
}

// Host checks of a decode step with appended tokens (the arguments of
// paged_attn_e4m3_decode_append).
int32_t check_decode_append(const AttnCommon& c, const uint16_t* k_new, const uint16_t* v_new) {
  int32_t st = check_common(c, c.batch);
  if (st != KVFP8_OK) return st;
  if (c.n_q_heads / c.n_kv_heads > kSplitRows)
    return fail(KVFP8_UNSUPPORTED, "GQA group of %d heads (at most %d)", c.n_q_heads / c.n_kv_heads, kSplitRows);
  if (c.batch > 0 && (!k_new || !v_new)) return fail(KVFP8_INVALID_ARG, "null new-token pointer");
  if (c.batch > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(KVFP8_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  return KVFP8_OK;
}

}  // namespace

KVFP8_API const char* kvfp8_status_str(int32_t status) {
  switch (status) {
    case KVFP8_OK: return "KVFP8_OK";
    case KVFP8_INVALID_ARG: return "KVFP8_INVALID_ARG";
    case KVFP8_BAD_SCALE: return "KVFP8_BAD_SCALE";
    case KVFP8_NONFINITE_INPUT: return "KVFP8_NONFINITE_INPUT";
    case KVFP8_WORKSPACE: return "KVFP8_WORKSPACE";
    case KVFP8_UNSUPPORTED: return "KVFP8_UNSUPPORTED";
    case KVFP8_HIP_ERROR: return "KVFP8_HIP_ERROR";
    default: return "KVFP8_UNKNOWN_STATUS";
  }
}

KVFP8_API const char* kvfp8_last_error(void) { return g_err; }

KVFP8_API size_t kvfp8_attn_workspace_bytes(int64_t n_rows, int32_t n_q_heads, int32_t head_dim,
                                            int32_t num_splits) {
  if (n_rows <= 0 || n_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  return (size_t)n_rows * (size_t)n_q_heads * (size_t)num_splits * ((size_t)head_dim + 2) *
         sizeof(float);
}

KVFP8_API const char* kvfp8_attn_kernel_name(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t page_size, int32_t max_pages_per_seq,
                                             int32_t max_q_len, int32_t num_splits, int32_t f16_kv) {
  thread_local char name[96];
  name[0] = '\0';
  if (batch <= 0 || batch > 65535 || n_q_heads <= 0 || n_kv_heads <= 0 || n_kv_heads > 65535 ||
      n_q_heads % n_kv_heads != 0 || (head_dim != 64 && head_dim != 128) || !supported_page(page_size) ||
      max_pages_per_seq <= 0 || max_q_len < 1 || num_splits < 1 || num_splits > kMaxSplits)
    return name;
  kvfp8::AttnArgs a{};
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.max_pages = max_pages_per_seq;
  a.num_splits = num_splits;
  a.max_q_len = max_q_len;
  const int64_t rows = (int64_t)max_q_len * a.group;
  if (f16_kv) {
    if (rows <= kSplitRows) kvfp8::attn_split_f16_kernel_name(a, (int)rows, name, sizeof(name));
  } else if (rows <= kSplitRows) {
    kvfp8::attn_split_kernel_name(a, (int)rows, name, sizeof(name));
  } else if (num_splits == 1) {
    kvfp8::attn_chunk_kernel_name(a, name, sizeof(name));
  }
  return name;
}

KVFP8_API int32_t kv_calibrate_amax(const uint16_t* x_f16, int64_t n_tensors, int64_t n_elems,
                                    float* amax_out, float* scale_out, hipStream_t stream) {
  if (n_tensors < 0 || n_elems < 0) return fail(KVFP8_INVALID_ARG, "negative size");
  if (n_tensors == 0) return ok();
  if (!amax_out || !scale_out) return fail(KVFP8_INVALID_ARG, "null output pointer");
  if (n_elems > 0 && !x_f16) return fail(KVFP8_INVALID_ARG, "null input pointer");
  if (n_elems > 0 && !aligned16(x_f16)) return fail(KVFP8_INVALID_ARG, "x_f16 must be 16-byte aligned");
  hipError_t e = kvfp8::launch_calibrate(x_f16, n_tensors, n_elems, amax_out, scale_out, stream);
  if (e != hipSuccess) return hip_status(e, "calibration launch");
  std::vector<float> amax((size_t)n_tensors);
  e = hipMemcpyAsync(amax.data(), amax_out, (size_t)n_tensors * sizeof(float), hipMemcpyDeviceToHost,
                     stream);
  if (e != hipSuccess) return hip_status(e, "calibration readback");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "calibration synchronise");
  int64_t nonfinite = -1, zero = -1;
  for (int64_t t = 0; t < n_tensors; ++t) {
    if (std::isnan(amax[(size_t)t]) && nonfinite < 0) nonfinite = t;
    if (amax[(size_t)t] == 0.0f && zero < 0) zero = t;
  }
  if (nonfinite >= 0)
    return fail(KVFP8_NONFINITE_INPUT, "tensor %lld holds Inf or NaN", (long long)nonfinite);
  if (zero >= 0)
    return fail(KVFP8_BAD_SCALE, "tensor %lld has amax 0: no finite positive scale", (long long)zero);
  return ok();
}

KVFP8_API int32_t kv_quant_write(const uint16_t* k_f16, const uint16_t* v_f16,
                                 const int64_t* slot_mapping, int64_t n_tokens, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t page_size, int64_t num_pages,
                                 float k_scale, float v_scale, uint8_t* k_cache, uint8_t* v_cache,
                                 hipStream_t stream) {
  if (n_tokens < 0 || num_pages < 0) return fail(KVFP8_INVALID_ARG, "negative size");
  if (n_kv_heads <= 0) return fail(KVFP8_INVALID_ARG, "n_kv_heads must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(KVFP8_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (!supported_page(page_size))
    return fail(KVFP8_UNSUPPORTED, "page_size %d (supported: 4, 8, 16, 32, 64)", page_size);
  if (!good_scale(k_scale) || !good_scale(v_scale))
    return fail(KVFP8_BAD_SCALE, "k_scale and v_scale must be finite, positive and normal (got %g, %g)",
                (double)k_scale, (double)v_scale);
  if (n_tokens == 0) return ok();
  if (!k_f16 || !v_f16 || !slot_mapping || !k_cache || !v_cache)
    return fail(KVFP8_INVALID_ARG, "null pointer");
  if (!aligned16(k_f16) || !aligned16(v_f16))
    return fail(KVFP8_INVALID_ARG, "k_f16 and v_f16 must be 16-byte aligned");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(KVFP8_INVALID_ARG, "caches must be 16-byte aligned");
  hipError_t e = kvfp8::launch_quant_write(k_f16, v_f16, slot_mapping, n_tokens, n_kv_heads, head_dim,
                                           page_size, num_pages, k_scale, v_scale, k_cache, v_cache,
                                           stream);
  return hip_status(e, "quant write launch");
}

KVFP8_API int32_t paged_attn_e4m3_decode(const uint16_t* q_f16, const uint8_t* k_cache,
                                         const uint8_t* v_cache, const int32_t* block_table,
                                         const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                         int32_t max_pages_per_seq, float k_scale, float v_scale,
                                         float sm_scale, int32_t num_splits, float* workspace,
                                         size_t workspace_bytes, uint16_t* out_f16,
                                         hipStream_t stream) {
  AttnCommon c{q_f16, k_cache, v_cache, block_table, seq_lens, batch, n_q_heads, n_kv_heads,
               head_dim, page_size, max_pages_per_seq, k_scale, v_scale, sm_scale, num_splits,
               workspace, workspace_bytes, out_f16};
  int32_t st = check_common(c, batch);
  if (st != KVFP8_OK) return st;
  if (n_q_heads / n_kv_heads > kSplitRows)
    return fail(KVFP8_UNSUPPORTED, "GQA group of %d heads (at most %d)", n_q_heads / n_kv_heads,
                kSplitRows);
  return run_attention(c, nullptr, batch, 1, stream);
}

KVFP8_API int32_t paged_attn_e4m3_decode_append(const uint16_t* q_f16, const uint16_t* k_new,
                                                const uint16_t* v_new, uint8_t* k_cache, uint8_t* v_cache,
                                                const int32_t* block_table, const int32_t* seq_lens,
                                                int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                                int32_t head_dim, int32_t page_size,
                                                int32_t max_pages_per_seq, float k_scale, float v_scale,
                                                float sm_scale, int32_t num_splits, float* workspace,
                                                size_t workspace_bytes, uint16_t* out_f16,
                                                hipStream_t stream) {
  AttnCommon c{q_f16, k_cache, v_cache, block_table, seq_lens, batch, n_q_heads, n_kv_heads,
               head_dim, page_size, max_pages_per_seq, k_scale, v_scale, sm_scale, num_splits,
               workspace, workspace_bytes, out_f16};
  int32_t st = check_decode_append(c, k_new, v_new);
  if (st != KVFP8_OK) return st;
  const AppendArgs app{k_new, v_new, k_cache, v_cache};
  return run_attention(c, nullptr, batch, 1, stream, &app);
}

KVFP8_API int32_t paged_attn_e4m3_decode_append_noalloc(const uint16_t* q_f16, const uint16_t* k_new,
                                                        const uint16_t* v_new, uint8_t* k_cache, uint8_t* v_cache,
                                                        const int32_t* block_table, const int32_t* seq_lens,
                                                        int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                                        int32_t head_dim, int32_t page_size,
                                                        int32_t max_pages_per_seq, float k_scale, float v_scale,
                                                        float sm_scale, int32_t num_splits, uint16_t* out_f16,
                                                        hipStream_t stream) {
  if (!out_f16) return fail(KVFP8_INVALID_ARG, "out must not be NULL (the partials stay in the library's scratch)");
  const bool split = num_splits > 1;
  if (split && batch > 0 && n_q_heads > 0 && head_dim > 0) {
    const size_t need = kvfp8_attn_workspace_bytes(batch, n_q_heads, head_dim, num_splits);
    if (need > (size_t)KVFP8_NOALLOC_SCRATCH_BYTES)
      return fail(KVFP8_WORKSPACE, "the split partials need %zu bytes; the static scratch holds %zu "
                  "(fewer splits, a smaller batch, or paged_attn_e4m3_decode_append with a workspace)",
                  need, (size_t)KVFP8_NOALLOC_SCRATCH_BYTES);
  }
  // every argument is checked on the host, with the scratch standing in for
  // the workspace, before the first HIP call
  float* const kStandIn = reinterpret_cast<float*>(uintptr_t{256});
  AttnCommon c{q_f16, k_cache, v_cache, block_table, seq_lens, batch, n_q_heads, n_kv_heads,
               head_dim, page_size, max_pages_per_seq, k_scale, v_scale, sm_scale, num_splits,
               split ? kStandIn : nullptr, split ? (size_t)KVFP8_NOALLOC_SCRATCH_BYTES : 0, out_f16};
  int32_t st = check_decode_append(c, k_new, v_new);
  if (st != KVFP8_OK) return st;
  if (batch == 0) return ok();
  if (split) {
    st = device_scratch(&c.workspace);
    if (st != KVFP8_OK) return st;
  }
  const AppendArgs app{k_new, v_new, k_cache, v_cache};
  return run_attention(c, nullptr, batch, 1, stream, &app);
}

KVFP8_API int32_t paged_attn_e4m3_verify(const uint16_t* q_f16, const int32_t* cu_q_lens,
                                         int32_t total_q, int32_t max_q_len, const uint8_t* k_cache,
                                         const uint8_t* v_cache, const int32_t* block_table,
                                         const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                         int32_t max_pages_per_seq, float k_scale, float v_scale,
                                         float sm_scale, int32_t num_splits, float* workspace,
                                         size_t workspace_bytes, uint16_t* out_f16,
                                         hipStream_t stream) {
  AttnCommon c{q_f16, k_cache, v_cache, block_table, seq_lens, batch, n_q_heads, n_kv_heads,
               head_dim, page_size, max_pages_per_seq, k_scale, v_scale, sm_scale, num_splits,
               workspace, workspace_bytes, out_f16};
  if (!cu_q_lens) return fail(KVFP8_INVALID_ARG, "null cu_q_lens");
  if (total_q < 0) return fail(KVFP8_INVALID_ARG, "negative total_q");
  if (max_q_len < 1 && total_q > 0) return fail(KVFP8_INVALID_ARG, "max_q_len must be >= 1");
  int32_t st = check_common(c, total_q);
  if (st != KVFP8_OK) return st;
  return run_attention(c, cu_q_lens, total_q, max_q_len, stream);
}

KVFP8_API int32_t paged_attn_e4m3_verify_append(const uint16_t* q_f16, const uint16_t* k_new, const uint16_t* v_new,
                                                const int32_t* cu_q_lens, int32_t total_q, int32_t max_q_len,
                                                uint8_t* k_cache, uint8_t* v_cache, const int32_t* block_table,
                                                const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                                int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                                int32_t max_pages_per_seq, float k_scale, float v_scale, float sm_scale,
                                                int32_t num_splits, float* workspace, size_t workspace_bytes,
                                                uint16_t* out_f16, hipStream_t stream) {
  AttnCommon c{q_f16, k_cache, v_cache, block_table, seq_lens, batch, n_q_heads, n_kv_heads,
               head_dim, page_size, max_pages_per_seq, k_scale, v_scale, sm_scale, num_splits,
               workspace, workspace_bytes, out_f16};
  if (!cu_q_lens) return fail(KVFP8_INVALID_ARG, "null cu_q_lens");
  if (total_q < 0) return fail(KVFP8_INVALID_ARG, "negative total_q");
  if (max_q_len < 1 && total_q > 0) return fail(KVFP8_INVALID_ARG, "max_q_len must be >= 1");
  int32_t st = check_common(c, total_q);
  if (st != KVFP8_OK) return st;
  if ((int64_t)max_q_len * (n_q_heads / n_kv_heads) > kSplitRows)
    return fail(KVFP8_UNSUPPORTED, "appending takes at most %d query rows per kv-head (max_q_len * group)",
                kSplitRows);
  if (total_q > 0 && (!k_new || !v_new)) return fail(KVFP8_INVALID_ARG, "null new-token pointer");
  if (total_q > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(KVFP8_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  const AppendArgs app{k_new, v_new, k_cache, v_cache};
  return run_attention(c, cu_q_lens, total_q, max_q_len, stream, &app);
}

KVFP8_API int32_t paged_attn_f16_decode(const uint16_t* q_f16, const uint16_t* k_cache_f16,
                                        const uint16_t* v_cache_f16, const int32_t* block_table,
                                        const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                        int32_t max_pages_per_seq, float sm_scale, int32_t num_splits,
                                        float* workspace, size_t workspace_bytes, uint16_t* out_f16,
                                        hipStream_t stream) {
  AttnCommon c{q_f16, reinterpret_cast<const uint8_t*>(k_cache_f16), reinterpret_cast<const uint8_t*>(v_cache_f16),
               block_table, seq_lens, batch, n_q_heads, n_kv_heads, head_dim, page_size, max_pages_per_seq,
               1.0f, 1.0f, sm_scale, num_splits, workspace, workspace_bytes, out_f16};
  int32_t st = check_common(c, batch);
  if (st != KVFP8_OK) return st;
  if (n_q_heads / n_kv_heads > kSplitRows)
    return fail(KVFP8_UNSUPPORTED, "GQA group of %d heads (at most %d)", n_q_heads / n_kv_heads,
                kSplitRows);
  return run_attention(c, nullptr, batch, 1, stream, nullptr, true);
}

KVFP8_API int32_t paged_attn_f16_verify(const uint16_t* q_f16, const int32_t* cu_q_lens, int32_t total_q,
                                        int32_t max_q_len, const uint16_t* k_cache_f16,
                                        const uint16_t* v_cache_f16, const int32_t* block_table,
                                        const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                        int32_t max_pages_per_seq, float sm_scale, int32_t num_splits,
                                        float* workspace, size_t workspace_bytes, uint16_t* out_f16,
                                        hipStream_t stream) {
  AttnCommon c{q_f16, reinterpret_cast<const uint8_t*>(k_cache_f16), reinterpret_cast<const uint8_t*>(v_cache_f16),
               block_table, seq_lens, batch, n_q_heads, n_kv_heads, head_dim, page_size, max_pages_per_seq,
               1.0f, 1.0f, sm_scale, num_splits, workspace, workspace_bytes, out_f16};
  if (!cu_q_lens) return fail(KVFP8_INVALID_ARG, "null cu_q_lens");
  if (total_q < 0) return fail(KVFP8_INVALID_ARG, "negative total_q");
  if (max_q_len < 1 && total_q > 0) return fail(KVFP8_INVALID_ARG, "max_q_len must be >= 1");
  int32_t st = check_common(c, total_q);
  if (st != KVFP8_OK) return st;
  return run_attention(c, cu_q_lens, total_q, max_q_len, stream, nullptr, true);
}

KVFP8_API int32_t split_reduce_fp32(const float* ws_o, const float* ws_m, const float* ws_l,
                                    int32_t n_rows, int32_t n_q_heads, int32_t head_dim,
                                    int32_t num_splits, uint16_t* out_f16, float* lse_out,
                                    hipStream_t stream) {
  if (n_rows < 0 || n_q_heads <= 0) return fail(KVFP8_INVALID_ARG, "bad row or head count");
  if (head_dim != 64 && head_dim != 128)
    return fail(KVFP8_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(KVFP8_UNSUPPORTED, "num_splits %d (supported: 1..%d)", num_splits, kMaxSplits);
  if (n_rows == 0) return ok();
  if (!ws_o || !ws_m || !ws_l || !out_f16) return fail(KVFP8_INVALID_ARG, "null pointer");
  if ((reinterpret_cast<uintptr_t>(ws_o) & 7u) != 0)
    return fail(KVFP8_INVALID_ARG, "ws_o must be 8-byte aligned");
  hipError_t e = kvfp8::launch_split_reduce(ws_o, ws_m, ws_l, n_rows, n_q_heads, head_dim, num_splits,
                                            out_f16, lse_out, stream);
  return hip_status(e, "split reduce launch");
}

KVFP8_API int32_t kvfp8_e4m3_encode_f32(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
  if (n < 0) return fail(KVFP8_INVALID_ARG, "negative size");
  if (n == 0) return ok();
  if (!x || !codes) return fail(KVFP8_INVALID_ARG, "null pointer");
  return hip_status(kvfp8::launch_encode(x, codes, n, stream), "encode launch");
}

KVFP8_API int32_t kvfp8_e4m3_decode_f32(const uint8_t* codes, float* x, int64_t n, hipStream_t stream) {
  if (n < 0) return fail(KVFP8_INVALID_ARG, "negative size");
  if (n == 0) return ok();
  if (!x || !codes) return fail(KVFP8_INVALID_ARG, "null pointer");
  return hip_status(kvfp8::launch_decode(codes, x, n, stream), "decode launch");
}

KVFP8_API int32_t kvfp8_check_paged_args(const int32_t* block_table, const int32_t* seq_lens,
                                         const int32_t* cu_q_lens, int32_t batch, int32_t max_pages_per_seq,
                                         int32_t page_size, int64_t num_pages, int32_t total_q, int32_t max_q_len,
                                         int32_t* result, hipStream_t stream) {
  if (batch < 0) return fail(KVFP8_INVALID_ARG, "negative batch");
  if (max_pages_per_seq <= 0 || page_size <= 0 || num_pages < 0)
    return fail(KVFP8_INVALID_ARG, "max_pages_per_seq and page_size must be positive, num_pages non-negative");
  if (cu_q_lens && (total_q < 0 || max_q_len < 0)) return fail(KVFP8_INVALID_ARG, "negative total_q or max_q_len");
  if (batch == 0) return ok();
  if (!block_table || !seq_lens || !result) return fail(KVFP8_INVALID_ARG, "null pointer");
  if ((reinterpret_cast<uintptr_t>(result) & 3u) != 0) return fail(KVFP8_INVALID_ARG, "result must be 4-byte aligned");
  hipError_t e = kvfp8::launch_check_paged_args(block_table, seq_lens, cu_q_lens, batch, max_pages_per_seq,
                                                page_size, num_pages, total_q, max_q_len, result, stream);
  if (e != hipSuccess) return hip_status(e, "argument check launch");
  int32_t r[4] = {0, 0, 0, 0};
  e = hipMemcpyAsync(r, result, sizeof(r), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_status(e, "argument check readback");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "argument check synchronise");
  if (r[0] == 0) return ok();
  char detail[320];
  int len = 0;
  detail[0] = '\0';
  if (r[0] & kvfp8::kCheckBadSeqLen)
    len += snprintf(detail + len, sizeof(detail) - (size_t)len,
                    "seq_lens outside [0, max_pages_per_seq * page_size] (first at sequence %d); ", r[1]);
  if ((r[0] & kvfp8::kCheckBadQueries) && len < (int)sizeof(detail))
    len += snprintf(detail + len, sizeof(detail) - (size_t)len,
                    "query rows outside [0, max_q_len], above seq_lens, or cu_q_lens not starting at 0 / "
                    "ending at total_q (first at sequence %d); ", r[2]);
  if ((r[0] & kvfp8::kCheckBadPage) && len < (int)sizeof(detail))
    snprintf(detail + len, sizeof(detail) - (size_t)len,
             "block-table entry outside [0, num_pages) (first at sequence %d); ", r[3]);
  return fail(KVFP8_INVALID_ARG, "%s", detail);
}
