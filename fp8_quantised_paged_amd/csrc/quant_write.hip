// Quantising paged cache write: code = E4M3(fl32(x) / scale), scattered to the
// K page ([P][D] per kv-head) and the V page ([D][P] per kv-head).
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

// One thread per (token, kv-head, group of 8 dims). Reads 16 bytes of K and of
// V, writes 8 contiguous K codes and 8 V codes at a stride of page_size.
__global__ __launch_bounds__(256) void quant_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t n_tokens, int n_kv_heads, int head_dim,
    int page_size, int64_t num_pages, float k_scale, float v_scale, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache) {
  const int groups = head_dim >> 3;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = n_tokens * n_kv_heads * groups;
  if (idx >= total) return;
  const int g = (int)(idx % groups);
  const int h = (int)((idx / groups) % n_kv_heads);
  const int64_t t = idx / ((int64_t)groups * n_kv_heads);
  // the slot and the K/V values are independent loads: issue them together
  const int64_t src = (t * n_kv_heads + h) * head_dim + (int64_t)g * 8;
  const int64_t slot = slots[t];
  const u32x4 kw = *reinterpret_cast<const u32x4*>(k + src);
  const u32x4 vw = *reinterpret_cast<const u32x4*>(v + src);
  if (slot < 0 || slot >= num_pages * page_size) return;
  const int64_t page = slot / page_size;
  const int off = (int)(slot - page * page_size);

  uint32_t kc[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t bits = (kw[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
    float x = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    kc[j >> 2] |= e4m3_encode(x / k_scale) << ((j & 3) * 8);
  }
  uint8_t* kdst = k_cache + ((page * n_kv_heads + h) * page_size + off) * head_dim + g * 8;
  *reinterpret_cast<u32x2*>(kdst) = u32x2{kc[0], kc[1]};

  uint8_t* vdst = v_cache + ((page * n_kv_heads + h) * head_dim + (int64_t)g * 8) * page_size + off;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t bits = (vw[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
    float x = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    vdst[(int64_t)j * page_size] = (uint8_t)e4m3_encode(x / v_scale);
  }
}

__global__ void encode_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) codes[i] = (uint8_t)e4m3_encode(x[i]);
}

__global__ void decode_kernel(const uint8_t* __restrict__ codes, float* __restrict__ x, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    f16x4 h = e4m3x4_to_f16((uint32_t)codes[i]);
    x[i] = (float)h[0];
  }
}

}  // namespace

hipError_t launch_quant_write(const uint16_t* k, const uint16_t* v, const int64_t* slots,
                              int64_t n_tokens, int32_t n_kv_heads, int32_t head_dim,
                              int32_t page_size, int64_t num_pages, float k_scale, float v_scale,
                              uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream) {
  int64_t total = n_tokens * n_kv_heads * (head_dim / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  quant_write_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      k, v, slots, n_tokens, n_kv_heads, head_dim, page_size, num_pages, k_scale, v_scale, k_cache,
      v_cache);
  return hipGetLastError();
}

hipError_t launch_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  encode_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(x, codes, n);
  return hipGetLastError();
}

hipError_t launch_decode(const uint8_t* codes, float* x, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  decode_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(codes, x, n);
  return hipGetLastError();
}

}  // namespace kvfp8
