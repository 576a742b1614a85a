// Internal declarations shared by the kvfp8 translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace kvfp8 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ E4M3 codec
// gfx950's v_cvt_scalef32_pk_f16_fp8 turns two OCP E4M3 codes into two fp16
// values in one instruction (the word select picks bytes 0-1 or 2-3). With a
// scale of 1 it is exact on all 256 codes, NaN and signed zero included: every
// E4M3 value is representable in fp16. This is half the instructions of
// decoding to fp32 and packing.
__device__ __forceinline__ f16x4 e4m3x4_to_f16(uint32_t w) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);  // bytes 0, 1
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);   // bytes 2, 3
  return __builtin_shufflevector(a, b, 0, 1, 2, 3);
}

__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  f16x4 a = e4m3x4_to_f16(w0);
  f16x4 b = e4m3x4_to_f16(w1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E4M3 code of an fp32 value: round to nearest even, saturate to +-448, NaN
// keeps its sign as 0x7F | sign. v_cvt_pk_fp8_f32 rounds to nearest even but
// does not saturate (it returns NaN from 464 up) and gives 0xFF for every NaN,
// hence the explicit NaN select and the clamp.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  if (q != q) return ((__float_as_uint(q) >> 24) & 0x80u) | 0x7Fu;
  float c = fminf(fmaxf(q, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xFFu;
}

// ------------------------------------------------------------------ launchers
struct AttnArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* cu_q_lens;  // nullptr: one query row per sequence (row == b)
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages;
  int32_t num_splits;
  int32_t max_q_len;
  float score_scale;  // k_scale * sm_scale * log2(e): scores in log2 units
  float v_scale;
  float* ws_o;  // partial mode
  float* ws_m;
  float* ws_l;
  uint16_t* out;  // direct mode (num_splits == 1)
  // with append: the new tokens of sequence b (keys seq_lens[b] - q_len ..
  // seq_lens[b] - 1, its query rows) are quantised into the cache before they
  // are read; nullptr otherwise
  const uint16_t* k_new;  // [query rows][n_kv_heads][head_dim] fp16
  const uint16_t* v_new;
  uint8_t* k_cache_w;  // the same caches, writable
  uint8_t* v_cache_w;
  float k_scale;
};

// Compute units of the current device (queried once per device).
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                   ? n
                   : 256;
  }
  return cus[dev];
}

// the library's thread-local error text (kvfp8_last_error)
void set_error(const char* msg);
void clear_error();

hipError_t launch_calibrate(const uint16_t* x, int64_t n_tensors, int64_t n_elems, float* amax,
                            float* scale, hipStream_t stream);
hipError_t launch_quant_write(const uint16_t* k, const uint16_t* v, const int64_t* slots,
                              int64_t n_tokens, int32_t n_kv_heads, int32_t head_dim,
                              int32_t page_size, int64_t num_pages, float k_scale, float v_scale,
                              uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream);
// Split-context kernel for up to 32 query rows per (sequence, kv-head).
hipError_t launch_attn_split(const AttnArgs& a, int rows_per_kvh, hipStream_t stream);
// FP16-KV twin of the split-context kernel (k_cache / v_cache hold fp16).
hipError_t launch_attn_split_f16(const AttnArgs& a, int rows_per_kvh, hipStream_t stream);
// Query-tiled causal chunk kernel (long q_len).
hipError_t launch_attn_chunk(const AttnArgs& a, hipStream_t stream);
// Name of the kernel instantiation each attention launcher chooses for these
// arguments (rows_per_kvh: query rows per kv-head), written to buf.
void attn_split_kernel_name(const AttnArgs& a, int rows_per_kvh, char* buf, size_t n);
void attn_split_f16_kernel_name(const AttnArgs& a, int rows_per_kvh, char* buf, size_t n);
void attn_chunk_kernel_name(const AttnArgs& a, char* buf, size_t n);
hipError_t launch_split_reduce(const float* ws_o, const float* ws_m, const float* ws_l,
                               int32_t n_rows, int32_t n_q_heads, int32_t head_dim,
                               int32_t num_splits, uint16_t* out, float* lse,
                               hipStream_t stream);
// Device-side check of the attention calls' caller contract; result: int32[4]
// (rule bits, then the first offending sequence per rule).
constexpr int32_t kCheckBadSeqLen = 1;   // seq_lens[b] < 0 or > max_pages * page_size
constexpr int32_t kCheckBadQueries = 2;  // q_len out of [0, max_q_len], above seq_lens[b], or bad cu_q_lens ends
constexpr int32_t kCheckBadPage = 4;     // a block-table entry of a page holding keys outside [0, num_pages)
hipError_t launch_check_paged_args(const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q_lens,
                                   int32_t batch, int32_t max_pages, int32_t page_size, int64_t num_pages,
                                   int32_t total_q, int32_t max_q_len, int32_t* result, hipStream_t stream);
hipError_t launch_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);
hipError_t launch_decode(const uint8_t* codes, float* x, int64_t n, hipStream_t stream);

}  // namespace kvfp8
