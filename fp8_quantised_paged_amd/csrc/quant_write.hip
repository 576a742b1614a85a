// Quantising paged cache write: code = E4M3(fl32(x) / scale), scattered to the
// K page ([P][D] per kv-head) and the V page ([D][P] per kv-head).
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// E4M3 codes of two fp32 values that are not NaN, written into the low
// (HI = false) or high half of `old` (the other half is kept): the same codes
// as e4m3_encode, with the clamp to +-448 as one median instruction and one
// convert for the pair.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                                  __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), (int)old, HI);
}

// The fp32 quotient x / scale, correctly rounded, for an fp32 x and a normal
// fp32 scale, as one fp64 multiply by rcp = 1 / scale rounded to fp64
// (computed once on the host) and one rounding to fp32, instead of an fp32
// division (about ten instructions, one of them a reciprocal). Why the result
// is the same: write x = X 2^a with |X| < 2^24 and scale = S 2^c with
// 2^23 <= S < 2^24. An fp32 rounding midpoint next to x / scale (in the fp32
// normal range) is m = M 2^k with M odd and 2^24 <= M < 2^25; x = m scale
// would need M to divide X, so x - m scale is a non-zero multiple of 2^(k+c),
// and |x / scale - m| >= |m| / (M S) > 2^-49 |m|. The fp64 product is within
// about 2^-52 of x / scale (two roundings to 53 bits), so no midpoint lies
// between the two and both round to the same fp32 value. Zero, Inf and NaN
// pass through; quotients below the fp32 normal range encode to a signed zero
// either way.
__device__ __forceinline__ float div_by_scale(float x, double rcp) {
  return (float)((double)x * rcp);
}

// Calls with at most this many tokens use the one-thread-per-8-dims kernel.
constexpr int64_t kDirectMaxTokens = 256;

// Small calls (a decode step's new tokens): one thread per (token, kv-head,
// group of 8 dims), which reads 16 bytes of K and of V and writes 8 contiguous
// K codes and 8 V codes at a stride of page_size. With few tokens this spreads
// the work over the most threads; the V bytes go out one by one.
__global__ __launch_bounds__(256) void quant_write_direct_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t n_tokens, int n_kv_heads, int head_dim,
    int page_size, int64_t num_pages, double k_rcp, double v_rcp, uint8_t* __restrict__ k_cache,
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
    kc[j >> 2] |= e4m3_encode(div_by_scale(x, k_rcp)) << ((j & 3) * 8);
  }
  uint8_t* kdst = k_cache + ((page * n_kv_heads + h) * page_size + off) * head_dim + g * 8;
  *reinterpret_cast<u32x2*>(kdst) = u32x2{kc[0], kc[1]};

  uint8_t* vdst = v_cache + ((page * n_kv_heads + h) * head_dim + (int64_t)g * 8) * page_size + off;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t bits = (vw[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
    float x = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    vdst[(int64_t)j * page_size] = (uint8_t)e4m3_encode(div_by_scale(x, v_rcp));
  }
}

// One workgroup takes a block of TB = 8192 / D consecutive tokens of the call
// and one kv-head; each thread encodes TPT tokens x 8 dims, so the workgroup
// has TB * D / (8 * TPT) threads (TPT = 2: 512 threads for large calls;
// TPT = 1: 1024 threads, for calls too small to fill the chip otherwise).
//
// K: a token's codes are one contiguous row of its page, so every thread
// stores its 8 codes per token directly (16 lanes cover a 128-byte row).
//
// V: a page row holds one dimension of up to P consecutive slots, so a direct
// store is one byte per (token, dim) at a stride of P. Instead the codes go to
// LDS as [D][TB] and are stored from there in the widest aligned pieces the
// slots allow, each piece a part of one page row:
//   run:  a token whose slot is a multiple of R = min(16, P) and whose next
//         R - 1 tokens in the block hold the next R - 1 slots: R bytes per dim;
//   quad: the same with 4 in place of R, for tokens no run covers (the ends of
//         runs cut by the block's edges): 4 bytes per dim;
//   byte: any other token with a valid slot.
// The lanes of a wavefront take consecutive dimensions of one piece, so at
// P <= 16 a wavefront's run stores are one contiguous KiB. Prefill and chunk
// writes are runs almost everywhere; scattered tokens are single bytes, which
// is why calls of a decode step's size take the kernel above. The fp16 inputs
// are read once, with non-temporal loads.
template <int D, int TPT>
__global__ __launch_bounds__(8192 / (8 * TPT)) void quant_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t n_tokens, int n_kv_heads, int page_shift,
    int64_t num_pages, double k_rcp, double v_rcp, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache) {
  constexpr int TB = 8192 / D;              // tokens per block: 64 or 128
  constexpr int NT = 8192 / (8 * TPT);      // threads per block
  constexpr int G = D / 8;                  // 8-dim groups per token
  constexpr int RS = TB + 4;                // LDS row stride in bytes; the 4 spare bytes
                                            // keep a piece's last aligned word in the row
  enum : int { kByte = 0, kQuad = 1, kRun = 2 };
  __shared__ uint32_t vbuf[D * RS / 4];
  __shared__ int64_t sslot[TB];
  __shared__ uint8_t skind[TB];             // piece a token leads: kRun, kQuad or kByte
  __shared__ uint8_t scov[TB];              // 1: inside a run
  __shared__ uint16_t sent[TB];
  __shared__ int64_t sbase[TB];
  __shared__ uint64_t smask[TB / 64];

  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int page_size = 1 << page_shift;
  const int64_t cap = num_pages << page_shift;

  // slots of the block; -1 for tokens past the end and for skipped slots
  if (tid < TB) {
    int64_t s = -1;
    if (t0 + tid < n_tokens) {
      s = slots[t0 + tid];
      if (s < 0 || s >= cap) s = -1;
    }
    sslot[tid] = s;
  }

  // encode: thread (q, g) takes tokens TPT*q .. TPT*q + TPT-1 of the block, dims 8g .. 8g+7
  const int g = tid % G;
  const int q = tid / G;
  u32x4 kw[TPT], vw[TPT];
  int64_t sl[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t t = t0 + TPT * q + i;
    sl[i] = -1;
    kw[i] = u32x4{0u, 0u, 0u, 0u};
    vw[i] = u32x4{0u, 0u, 0u, 0u};
    if (t < n_tokens) {
      const int64_t src = (t * n_kv_heads + h) * D + 8 * g;
      sl[i] = slots[t];
      kw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + src));
      vw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + src));
    }
  }
  // Encode. Without NaN inputs (the rule) two codes come from each convert,
  // written into the chosen half of their word, after a one-instruction clamp
  // to +-448; a NaN must keep its sign as 0x7F | sign, which the convert does
  // not do, so a thread with any NaN input takes the per-value encoder. A NaN
  // fp16 input is one whose magnitude bits exceed 0x7C00.
  u16x2 mag = {0, 0};
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2, kw[i][w] & 0x7FFF7FFFu));
      mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2, vw[i][w] & 0x7FFF7FFFu));
    }
  const bool nan_in = (mag[0] > 0x7C00u) || (mag[1] > 0x7C00u);
  auto kq = [&](int i, int j) {  // fp32 quotient of K value (token i, dim 8g + j)
    return div_by_scale((float)__builtin_bit_cast(_Float16, (uint16_t)(kw[i][j >> 1] >> ((j & 1) * 16))), k_rcp);
  };
  auto vq = [&](int i, int j) {
    return div_by_scale((float)__builtin_bit_cast(_Float16, (uint16_t)(vw[i][j >> 1] >> ((j & 1) * 16))), v_rcp);
  };
  uint32_t kc[TPT][2];
  uint32_t vword[8];
  if (!nan_in) {
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t lo = e4m3_pack2<false>(kq(i, 4 * h2), kq(i, 4 * h2 + 1), 0u);
        kc[i][h2] = e4m3_pack2<true>(kq(i, 4 * h2 + 2), kq(i, 4 * h2 + 3), lo);
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (TPT == 1) {
        vword[j] = e4m3_pack2<false>(vq(0, j), 0.0f, 0u);
      } else {
        vword[j] = e4m3_pack2<false>(vq(0, j), vq(1, j), 0u);
        if constexpr (TPT == 4) vword[j] = e4m3_pack2<true>(vq(2, j), vq(3, j), vword[j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) vword[j] = 0u;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      kc[i][0] = kc[i][1] = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kc[i][j >> 2] |= e4m3_encode(kq(i, j)) << ((j & 3) * 8);
        vword[j] |= e4m3_encode(vq(i, j)) << (i * 8);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t s = sl[i];
    if (s >= 0 && s < cap) {
      const int64_t page = s >> page_shift;
      const int off = (int)(s & (page_size - 1));
      uint8_t* kdst = k_cache + ((page * n_kv_heads + h) * page_size + off) * D + 8 * g;
      *reinterpret_cast<u32x2*>(kdst) = u32x2{kc[i][0], kc[i][1]};
    }
  }
  uint8_t* vrow = reinterpret_cast<uint8_t*>(vbuf) + TPT * q;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint8_t* p = vrow + (8 * g + j) * RS;
    if constexpr (TPT == 4) *reinterpret_cast<uint32_t*>(p) = vword[j];
    else if constexpr (TPT == 2) *reinterpret_cast<uint16_t*>(p) = (uint16_t)vword[j];
    else *p = (uint8_t)vword[j];
  }
  __syncthreads();

  // pieces: runs first, then quads among the tokens no run covers
  const int R = page_size < 16 ? page_size : 16;
  bool lead_run = false;
  if (tid < TB) {
    const int64_t s = sslot[tid];
    lead_run = s >= 0 && (s & (R - 1)) == 0 && tid + R <= TB;
    for (int i = 1; lead_run && i < R; ++i) lead_run = sslot[tid + i] == s + i;
    skind[tid] = lead_run ? kRun : kByte;
  }
  __syncthreads();
  if (tid < TB) {
    const int64_t s = sslot[tid];
    const int first = tid - (int)(s & (R - 1));
    scov[tid] = (s >= 0 && first >= 0 && skind[first] == kRun) ? 1 : 0;
  }
  __syncthreads();
  if (tid < TB && R > 4) {
    // a quad lead: not in a run, slot a multiple of 4, the next 3 tokens hold the next 3 slots
    // (those three are then outside every run as well)
    const int64_t s = sslot[tid];
    bool lead_quad = s >= 0 && scov[tid] == 0 && (s & 3) == 0 && tid + 4 <= TB;
    for (int i = 1; lead_quad && i < 4; ++i) lead_quad = sslot[tid + i] == s + i;
    if (lead_quad) skind[tid] = kQuad;
  }
  __syncthreads();
  // entries: every piece lead, and every valid token that no piece covers
  if (tid < TB) {
    const int64_t s = sslot[tid];
    const int kind = skind[tid];
    bool entry = kind != kByte;
    if (s >= 0 && kind == kByte && scov[tid] == 0) {
      const int firstq = tid - (int)(s & 3);
      entry = !(R > 4 && firstq >= 0 && skind[firstq] == kQuad);
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(entry);
    if ((tid & 63) == 0) smask[tid >> 6] = m;
  }
  __syncthreads();
  int n_ent = 0;
#pragma unroll
  for (int w = 0; w < TB / 64; ++w) n_ent += __builtin_popcountll(smask[w]);
  if (tid < TB) {
    const uint64_t m = smask[tid >> 6];
    if ((m >> (tid & 63)) & 1) {
      int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (tid >= 64) pos += __builtin_popcountll(smask[0]);
      sent[pos] = (uint16_t)(tid | (skind[tid] << 8));
      const int64_t s = sslot[tid];
      sbase[pos] = (((s >> page_shift) * n_kv_heads + h) * D << page_shift) + (s & (page_size - 1));
    }
  }
  __syncthreads();

  // V stores: item = entry * D + dim, dims fastest across the lanes
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(vbuf);
  for (int item = tid; item < n_ent * D; item += NT) {
    const int e = item / D;
    const int d = item % D;
    const int ti = sent[e] & 0xFF;
    const int kind = sent[e] >> 8;
    uint8_t* dst = v_cache + sbase[e] + ((int64_t)d << page_shift);
    if (kind == kByte) {
      *dst = vb8[d * RS + ti];
      continue;
    }
    // the piece's bytes from row d at byte ti: aligned words, then a byte funnel shift
    const uint32_t* row = vbuf + d * (RS / 4) + (ti >> 2);
    const uint32_t sh = (uint32_t)(ti & 3);
    if (kind == kQuad) {
      *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_alignbyte(row[1], row[0], sh);
      continue;
    }
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = (i <= R / 4) ? row[i] : 0u;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
    if (R == 16) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{o[0], o[1], o[2], o[3]};
    } else if (R == 8) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{o[0], o[1]};
    } else {
      *reinterpret_cast<uint32_t*>(dst) = o[0];
    }
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
  if (n_tokens == 0) return hipSuccess;
  // reciprocals of the scales rounded to fp64, for div_by_scale
  const double k_rcp = 1.0 / (double)k_scale;
  const double v_rcp = 1.0 / (double)v_scale;
  if (n_tokens <= kDirectMaxTokens) {
    const int64_t total = n_tokens * n_kv_heads * (head_dim / 8);
    quant_write_direct_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
        k, v, slots, n_tokens, n_kv_heads, head_dim, page_size, num_pages, k_rcp, v_rcp, k_cache,
        v_cache);
    return hipGetLastError();
  }
  const int tb = 8192 / head_dim;
  const int64_t blocks = (n_tokens + tb - 1) / tb;
  if (blocks > 0x7FFFFFFF || n_kv_heads > 65535) return hipErrorInvalidValue;
  const int shift = __builtin_ctz((unsigned)page_size);
  const dim3 grid((unsigned)blocks, (unsigned)n_kv_heads);
  // 1,024-thread workgroups (one token per thread) until the grid holds about
  // four workgroups per CU, then 512-thread ones (two tokens per thread)
  const bool wide = blocks * n_kv_heads < 4 * (int64_t)device_cus();
#define QW_LAUNCH(DD, TT) quant_write_kernel<DD, TT><<<grid, dim3(8192 / (8 * TT)), 0, stream>>>( \
      k, v, slots, n_tokens, n_kv_heads, shift, num_pages, k_rcp, v_rcp, k_cache, v_cache)
  if (head_dim == 128) {
    if (wide) QW_LAUNCH(128, 1); else QW_LAUNCH(128, 2);
  } else {
    if (wide) QW_LAUNCH(64, 1); else QW_LAUNCH(64, 2);
  }
#undef QW_LAUNCH
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
