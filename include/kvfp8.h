/*
 * kvfp8 -- paged KV-cache attention over calibrated FP8 E4M3 on MI355X (gfx950).
 *
 * C ABI of libkvfp8.so. Every entry point takes plain pointers and sizes; all
 * pointers are DEVICE pointers unless marked "host". The library allocates no
 * memory and keeps no state besides a thread-local error string: the caller
 * owns every buffer. Work is enqueued on the caller's HIP stream and the calls
 * do not synchronise, except kv_calibrate_amax, which is an offline call and
 * waits for its own result, and kvfp8_check_paged_args, a debug-time check
 * that does the same. Every call validates its arguments on the host
 * before touching the GPU and returns a kvfp8_status; on any non-zero status
 * nothing has been launched (except for kv_calibrate_amax and
 * kvfp8_check_paged_args, whose statuses report what their kernels found).
 *
 * The method is described by three pull-request pages:
 *   [P1] "[Model][SM70] Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP"
 *   [P2] "[Model][SM70][FP8] Integrate calibrated E4M3 QSA KV capacity path"
 *   [P3] "[Experiment][SM70] Qualify E4M3 KV with MTP3"
 * Each declaration names the passage that defines its operation.
 *
 * Cache layout (the pages leave it open): two caches, K and V, each
 * uint8 E4M3 codes (OCP OFP8 E4M3: bias 7, no infinities, max 448).
 *   k_cache: [num_pages][n_kv_heads][page_size][head_dim]  (token-major)
 *   v_cache: [num_pages][n_kv_heads][head_dim][page_size]  (dimension-major)
 * A slot is page * page_size + offset. The block table maps logical page i of
 * sequence b to block_table[b * max_pages_per_seq + i].
 *
 * Attention semantics shared by the attention calls: seq_lens[b] counts every
 * key of sequence b including this step's query tokens (written to the cache
 * beforehand); query row i of a sequence with q_len query tokens sits at
 * position seq_lens[b] - q_len + i and sees keys 0 .. that position; query head
 * h reads kv-head h / (n_q_heads / n_kv_heads); the score of key j is
 * sm_scale * k_scale * (q . decode(k_code_j)) and the output is
 * v_scale * sum_j softmax_j * decode(v_code_j). The K/V scales are applied once
 * per tile and per split accumulator, never per element ([P2] Changes: the K/V
 * scaling is hoisted out of the per-element loads).
 *
 * Caller contract that the host cannot check without a synchronisation (device
 * data): block-table entries of pages that hold keys are valid page ids below
 * num_pages; seq_lens[b] <= max_pages_per_seq * page_size, and for verify
 * q_len <= seq_lens[b] (a decode sequence may have no keys: its output is zero
 * and its partials empty, as for a context shard holding none of its pages); the
 * slots passed to kv_quant_write are distinct. Entries of the block table past
 * a sequence's last page are never read. kvfp8_check_paged_args checks the
 * block-table and length parts on the device.
 */
#ifndef KVFP8_H
#define KVFP8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvfp8_status {
  KVFP8_OK = 0,
  KVFP8_INVALID_ARG = 1,      /* null pointer, bad size, misaligned pointer            */
  KVFP8_BAD_SCALE = 2,        /* scale not finite, not positive, or subnormal; amax 0  */
  KVFP8_NONFINITE_INPUT = 3,  /* calibration input holds Inf or NaN                    */
  KVFP8_WORKSPACE = 4,        /* split workspace missing or too small                  */
  KVFP8_UNSUPPORTED = 5,      /* shape outside the compiled kernels' range             */
  KVFP8_HIP_ERROR = 6         /* a HIP call or kernel launch failed                    */
} kvfp8_status;

/* Human-readable name of a status code (static string). */
const char* kvfp8_status_str(int32_t status);

/* Detail of the last non-OK status returned on the calling thread (static
 * thread-local buffer, valid until the next call on that thread). */
const char* kvfp8_last_error(void);

/* Bytes of the FP32 split workspace needed by the attention calls for n_rows
 * query rows (batch for decode, total_q for verify) and num_splits splits:
 * n_rows * n_q_heads * num_splits * (head_dim + 2) * 4. Layout, all fp32,
 * contiguous in this order:
 *   ws_o [n_rows][n_q_heads][num_splits][head_dim]  unnormalised, v_scale applied
 *   ws_m [n_rows][n_q_heads][num_splits]            running max, natural-log units
 *   ws_l [n_rows][n_q_heads][num_splits]            sum of exp(score - m)
 * An empty split holds m = -inf and l = 0; its o slot is not written (the
 * reduce gives it weight zero and never multiplies it). The workspace is FP32 by
 * contract ([P1] Status and history and [P3] Problem and resulting behavior:
 * a half-precision split temporary broke the E4M3 route). Calls sharing one
 * workspace must not overlap. Returns 0 for non-positive arguments. */
size_t kvfp8_attn_workspace_bytes(int64_t n_rows, int32_t n_q_heads, int32_t head_dim,
                                  int32_t num_splits);

/* Name of the kernel instantiation an attention call with these arguments
 * launches on the current device, e.g. "attn_split_kernel<128,16,1,8,false>"
 * (template arguments: head_dim, page_size, 16-row query blocks, wavefronts
 * per workgroup, short start-up), "attn_split_f16_kernel<...>" (f16_kv != 0:
 * the FP16-cache twins) or "attn_chunk_kernel<head_dim,page_size>". Decode
 * calls pass max_q_len = 1. Returns "" for arguments no call accepts. A static
 * thread-local string, valid until the next call on that thread; launches
 * nothing. For tests and benchmarks that must name the kernel they exercise. */
const char* kvfp8_attn_kernel_name(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                   int32_t page_size, int32_t max_pages_per_seq, int32_t max_q_len,
                                   int32_t num_splits, int32_t f16_kv);

/* Per-tensor calibration ([P2] Changes: offline calibration of the per-layer
 * K/V scales; [P2] Validation boundary: no unit-scale fallback). For each of
 * n_tensors contiguous fp16 rows of n_elems elements:
 *   amax_out[t]  = max |x| (exact; an fp16 value),
 *   scale_out[t] = amax / 448 rounded once to fp32 (IEEE division).
 * x_f16: [n_tensors][n_elems] fp16 bits, 16-byte aligned; amax_out, scale_out:
 * [n_tensors] fp32 (device). Offline and synchronous: waits on `stream` for its
 * result. A tensor holding any Inf/NaN gets NaN in both outputs and the call
 * returns KVFP8_NONFINITE_INPUT; otherwise a tensor with amax 0 gets 0 in both
 * outputs and the call returns KVFP8_BAD_SCALE. The outputs are written in
 * both error cases. Not capturable in a graph. */
int32_t kv_calibrate_amax(const uint16_t* x_f16, int64_t n_tensors, int64_t n_elems,
                          float* amax_out, float* scale_out, hipStream_t stream);

/* Quantising cache write ([P2] Changes: the main K/V cache is stored as
 * calibrated E4M3). For token t, kv-head h, dimension d:
 *   code = E4M3(fl32(x) / scale), round to nearest even, |q| >= 448 saturates
 *   to +-448, NaN gives 0x7F with its sign bit, the sign of zero is kept;
 * K codes go to k_cache[page][h][off][d] and V codes to v_cache[page][h][d][off]
 * with page = slot / page_size, off = slot % page_size, slot = slot_mapping[t].
 * Slots < 0 or >= num_pages * page_size are skipped.
 * k_f16, v_f16: [n_tokens][n_kv_heads][head_dim] fp16 bits, contiguous, 16-byte
 * aligned; slot_mapping: [n_tokens] int64. n_tokens == 0 is a no-op.
 * k_scale, v_scale: finite, positive, normal fp32 ([P2] Changes and Validation
 * boundary: scales are finite and positive, startup refuses anything else). */
int32_t kv_quant_write(const uint16_t* k_f16, const uint16_t* v_f16, const int64_t* slot_mapping,
                       int64_t n_tokens, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                       int64_t num_pages, float k_scale, float v_scale, uint8_t* k_cache,
                       uint8_t* v_cache, hipStream_t stream);

/* Decode attention, one query token per sequence ([P2] Changes: grouped-page
 * decode and split routes over the E4M3 cache). q_f16: [batch][n_q_heads]
 * [head_dim] fp16; block_table: [batch][max_pages_per_seq] int32; seq_lens:
 * [batch] int32 (>= 0; a sequence with no keys gets out = 0 and empty
 * partials). out_f16: [batch][n_q_heads][head_dim] fp16.
 * num_splits >= 1 splits the keys of every sequence into ranges of one size
 * for the whole call, C = ceil(L_max / (64 * num_splits)) * 64 keys with L_max
 * the longest context of the batch: split s covers keys [s*C, min((s+1)*C, L)),
 * so the longest sequence uses all num_splits splits and a shorter one
 * ceil(L / C) of them (the others are empty). In a ragged batch every
 * non-empty split then carries the same work.
 * num_splits == 1 writes out_f16 directly (workspace may be NULL). With
 * num_splits > 1 the FP32 partials go to `workspace` (see
 * kvfp8_attn_workspace_bytes) and, when out_f16 is not NULL, split_reduce_fp32
 * runs on the same stream to produce out_f16; with out_f16 == NULL only the
 * partials are produced (for callers that combine partials themselves, e.g.
 * from several context shards). Supported: head_dim 64 or 128, page_size 4, 8,
 * 16, 32 or 64, n_q_heads a multiple of n_kv_heads with a group of at most 32
 * heads, 1 <= num_splits <= 256. q, caches, workspace and out must be 16-byte
 * aligned. k_scale, v_scale, sm_scale: finite, positive, normal fp32, and so
 * must be k_scale * sm_scale * log2(e) (else KVFP8_BAD_SCALE). */
int32_t paged_attn_e4m3_decode(const uint16_t* q_f16, const uint8_t* k_cache, const uint8_t* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t max_pages_per_seq, float k_scale,
                               float v_scale, float sm_scale, int32_t num_splits, float* workspace,
                               size_t workspace_bytes, uint16_t* out_f16, hipStream_t stream);

/* Decode step with the new token appended ([P2] Changes: the quantising cache
 * write and the decode route over the E4M3 cache, one step). For every
 * sequence b with L = seq_lens[b] >= 1, the new token's K and V (k_new, v_new:
 * [batch][n_kv_heads][head_dim] fp16, 16-byte aligned) are quantised exactly
 * as kv_quant_write does (same scales, same rounding and saturation) into key
 * position L - 1, i.e. slot block_table[b][(L-1)/page_size] * page_size +
 * (L-1) % page_size; then attention runs as paged_attn_e4m3_decode over keys
 * 0 .. L-1, the new one included. seq_lens counts the new token. The result
 * (cache bytes and output) equals kv_quant_write with those slots followed by
 * paged_attn_e4m3_decode. k_cache and v_cache are written (the new tokens'
 * bytes only). Other arguments, errors and the workspace as for
 * paged_attn_e4m3_decode. */
int32_t paged_attn_e4m3_decode_append(const uint16_t* q_f16, const uint16_t* k_new, const uint16_t* v_new,
                                      uint8_t* k_cache, uint8_t* v_cache, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                      int32_t max_pages_per_seq, float k_scale, float v_scale, float sm_scale,
                                      int32_t num_splits, float* workspace, size_t workspace_bytes,
                                      uint16_t* out_f16, hipStream_t stream);

/* Bytes of the library's static FP32 scratch used by
 * paged_attn_e4m3_decode_append_noalloc: one copy per GPU the library runs on,
 * held until the process ends. */
#define KVFP8_NOALLOC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the decode step of
 * paged_attn_e4m3_decode_append with the FP32 split partials kept in the
 * library's static per-GPU scratch (KVFP8_NOALLOC_SCRATCH_BYTES) instead of a
 * caller workspace. Same arguments, kernels, results and errors as
 * paged_attn_e4m3_decode_append without workspace and workspace_bytes; out_f16
 * must not be NULL. The call allocates nothing (no hipMalloc, no library
 * allocation); its first call on a device looks up that device's scratch
 * address. Returns KVFP8_WORKSPACE, before any HIP call, when num_splits > 1
 * needs more than KVFP8_NOALLOC_SCRATCH_BYTES, i.e. when
 * kvfp8_attn_workspace_bytes(batch, n_q_heads, head_dim, num_splits) exceeds it.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * partials (each call writes every partial it reads, so nothing needs
 * clearing): calls on one GPU must not overlap (issue them on one stream, or
 * order them), or they race. */
int32_t paged_attn_e4m3_decode_append_noalloc(const uint16_t* q_f16, const uint16_t* k_new, const uint16_t* v_new,
                                              uint8_t* k_cache, uint8_t* v_cache, const int32_t* block_table,
                                              const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                              int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                              int32_t max_pages_per_seq, float k_scale, float v_scale,
                                              float sm_scale, int32_t num_splits, uint16_t* out_f16,
                                              hipStream_t stream);

/* Multi-query attention with a causal mask among each sequence's query tokens:
 * MTP verify of 1 + drafted tokens ([P1] Purpose and Validation on 4xV100 TP4:
 * MTP3 verifies up to four tokens per step) and prefill/catch-up chunks in mixed
 * batches ([P2] Changes). q_f16: [total_q][n_q_heads][head_dim] fp16, rows of
 * sequence b at cu_q_lens[b] .. cu_q_lens[b+1]-1; cu_q_lens: [batch+1] int32
 * (device) with cu_q_lens[batch] == total_q; max_q_len (host) bounds every
 * q_len and selects the kernel: max_q_len * group <= 32 runs the split kernel
 * (num_splits as for decode), larger chunks run the query-tiled chunk kernel,
 * which requires num_splits == 1. out_f16: [total_q][n_q_heads][head_dim].
 * Workspace rows are query rows (n_rows = total_q). Other arguments as for
 * paged_attn_e4m3_decode. */
int32_t paged_attn_e4m3_verify(const uint16_t* q_f16, const int32_t* cu_q_lens, int32_t total_q,
                               int32_t max_q_len, const uint8_t* k_cache, const uint8_t* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t max_pages_per_seq, float k_scale,
                               float v_scale, float sm_scale, int32_t num_splits, float* workspace,
                               size_t workspace_bytes, uint16_t* out_f16, hipStream_t stream);

/* MTP verify step with its new tokens appended ([P1] Purpose and Validation on
 * 4xV100 TP4: MTP3 verifies the drafted tokens of a step; [P2] Changes: the
 * quantising cache write). The query tokens of sequence b are its new tokens:
 * row cu_q_lens[b] + i is key position seq_lens[b] - q_len + i. Their K and V
 * (k_new, v_new: [total_q][n_kv_heads][head_dim] fp16, 16-byte aligned, rows in
 * the order of q) are quantised exactly as kv_quant_write does into those
 * positions (slots found through the block table), then attention runs as
 * paged_attn_e4m3_verify. The result (cache bytes and output) equals
 * kv_quant_write of those slots followed by paged_attn_e4m3_verify. Takes at
 * most 32 query rows per kv-head (max_q_len * group <= 32); larger chunks
 * return KVFP8_UNSUPPORTED. Other arguments, errors and the workspace as for
 * paged_attn_e4m3_verify. */
int32_t paged_attn_e4m3_verify_append(const uint16_t* q_f16, const uint16_t* k_new, const uint16_t* v_new,
                                      const int32_t* cu_q_lens, int32_t total_q, int32_t max_q_len,
                                      uint8_t* k_cache, uint8_t* v_cache, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                      int32_t max_pages_per_seq, float k_scale, float v_scale, float sm_scale,
                                      int32_t num_splits, float* workspace, size_t workspace_bytes,
                                      uint16_t* out_f16, hipStream_t stream);

/* FP16-cache twins of paged_attn_e4m3_decode and paged_attn_e4m3_verify, for
 * the single-variable comparison of cache formats that the pages make (only
 * kv_cache_dtype differs between the arms: [P1] Validation on 4xV100 TP4).
 * k_cache_f16: [num_pages][n_kv_heads][page_size][head_dim] fp16 and
 * v_cache_f16: [num_pages][n_kv_heads][head_dim][page_size] fp16 (the E4M3
 * layout with two-byte elements); there are no K/V scales. The work plan, split
 * boundaries, workspace, reduce, arguments, errors and limits are those of the
 * E4M3 calls; the verify twin takes at most 32 query rows per kv-head
 * (max_q_len * group <= 32), larger chunks return KVFP8_UNSUPPORTED. */
int32_t paged_attn_f16_decode(const uint16_t* q_f16, const uint16_t* k_cache_f16, const uint16_t* v_cache_f16,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t max_pages_per_seq, float sm_scale, int32_t num_splits, float* workspace,
                              size_t workspace_bytes, uint16_t* out_f16, hipStream_t stream);
int32_t paged_attn_f16_verify(const uint16_t* q_f16, const int32_t* cu_q_lens, int32_t total_q,
                              int32_t max_q_len, const uint16_t* k_cache_f16, const uint16_t* v_cache_f16,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t max_pages_per_seq, float sm_scale, int32_t num_splits, float* workspace,
                              size_t workspace_bytes, uint16_t* out_f16, hipStream_t stream);

/* Reduction of FP32 split partials ([P1] Status and history, [P3] Problem and
 * resulting behavior: the split temporary output is FP32). For each row r and
 * head h, with M = max_s m_s and w_s = exp(m_s - M) (0 for an empty split):
 *   out = sum_s w_s o_s / sum_s w_s l_s,   lse = M + log(sum_s w_s l_s).
 * ws_o: [n_rows][n_q_heads][num_splits][head_dim], ws_m, ws_l:
 * [n_rows][n_q_heads][num_splits], all fp32 (the layout of the attention
 * workspace, whose three parts may also come from elsewhere, e.g. partials
 * gathered from context shards). out_f16: [n_rows][n_q_heads][head_dim] fp16;
 * lse_out: [n_rows][n_q_heads] fp32 or NULL. A row whose splits are all empty
 * gets out = 0 and lse = -inf. Only splits up to the last one with a finite m
 * are read in full: o of the splits after it need not have been written.
 * head_dim 64 or 128; 1 <= num_splits <= 256. */
int32_t split_reduce_fp32(const float* ws_o, const float* ws_m, const float* ws_l, int32_t n_rows,
                          int32_t n_q_heads, int32_t head_dim, int32_t num_splits, uint16_t* out_f16,
                          float* lse_out, hipStream_t stream);

/* Check of the device-side caller contract above ([P2] Purpose: unsupported
 * combinations fail closed). The attention calls cannot see their block table,
 * context lengths and query offsets from the host; a caller that cannot vouch
 * for them (a debug build, a fuzzer, a new scheduler) runs this check first with
 * the same arguments. block_table: [batch][max_pages_per_seq] int32;
 * seq_lens: [batch] int32; cu_q_lens: [batch+1] int32 for verify, or NULL for
 * decode (one query row per sequence); num_pages: pages in the caches;
 * total_q, max_q_len: as for paged_attn_e4m3_verify (ignored without
 * cu_q_lens); result: int32[4] device scratch owned by the caller, overwritten.
 * Returns KVFP8_OK when for every sequence b, with q_len =
 * cu_q_lens[b+1] - cu_q_lens[b] (verify):
 *   0 <= seq_lens[b] <= max_pages_per_seq * page_size,
 *   0 <= q_len <= max_q_len and q_len <= seq_lens[b] (verify),
 *   cu_q_lens[0] == 0 and cu_q_lens[batch] == total_q (verify),
 *   0 <= block_table[b][i] < num_pages for i < ceil(seq_lens[b] / page_size);
 * otherwise KVFP8_INVALID_ARG, and kvfp8_last_error() names each broken rule
 * with the first sequence that breaks it. Synchronous (waits on `stream` for
 * its result); not capturable in a graph. batch == 0 is a no-op. */
int32_t kvfp8_check_paged_args(const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_q_lens,
                               int32_t batch, int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                               int32_t total_q, int32_t max_q_len, int32_t* result, hipStream_t stream);

/* Device E4M3 codec exposed for testing the conversions the kernels use.
 * kvfp8_e4m3_encode_f32: codes[i] = E4M3(x[i]) with the rounding and
 * saturation of kv_quant_write (no scale). kvfp8_e4m3_decode_f32: x[i] = value
 * of codes[i] (NaN for 0x7F/0xFF). n >= 0; no alignment requirement. */
int32_t kvfp8_e4m3_encode_f32(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);
int32_t kvfp8_e4m3_decode_f32(const uint8_t* codes, float* x, int64_t n, hipStream_t stream);

/* Revision-bound per-layer scale file ([P2] Changes: the E4M3 mode requires
 * every per-layer K/V scale, finite and positive, and refuses to start when the
 * calibrated overlay is missing or incomplete; [P2] Validation boundary: the
 * overlay must have been generated for the exact checkpoint revision, with no
 * generic or unit-scale fallback). Host-only; all pointers are host pointers.
 * kvfp8_scale_overlay_write stores n_layers (k_scale, v_scale) pairs for
 * `revision` (1..255 printable characters, no whitespace) at `path` (written to
 * path.tmp, then renamed); the scales are written as hexadecimal floats, so
 * reading returns them bit for bit. It refuses a scale that is not finite,
 * positive and normal (KVFP8_BAD_SCALE).
 * kvfp8_scale_overlay_read fails closed: a missing or malformed file, another
 * revision, another layer count, a layer missing or given twice
 * (KVFP8_INVALID_ARG) or an invalid scale (KVFP8_BAD_SCALE) returns an error and
 * leaves k_scales and v_scales untouched; on success both are filled
 * ([n_layers] fp32, layer order). */
int32_t kvfp8_scale_overlay_write(const char* path, const char* revision, int32_t n_layers, const float* k_scales,
                                  const float* v_scales);
int32_t kvfp8_scale_overlay_read(const char* path, const char* revision, int32_t n_layers, float* k_scales,
                                 float* v_scales);

#ifdef __cplusplus
}
#endif

#endif /* KVFP8_H */
