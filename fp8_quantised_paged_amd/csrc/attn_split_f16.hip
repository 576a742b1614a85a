// FP16-KV twin of the split-context attention kernel, for the single-variable
// comparison of cache formats: the same work plan, MFMA mapping, online
// softmax, wavefront merge and FP32 partials as the E4M3 kernel, over K/V pages
// that hold fp16 values (no decode and no K/V scale).
//
// Cache layout as for E4M3 with two-byte elements: K [pages][Hkv][P][D],
// V [pages][Hkv][D][P] (dimension-major).
//
// A tile is 32 keys, so a wavefront's K+V bytes per tile (16 KB at D = 128)
// and the registers holding them (64) equal those of the E4M3 kernel's 64-key
// tile, and the same two-tile register pipeline fits. Key permutation over the
// tile's two 16-key M-tiles: MFMA row m of M-tile t is key 8(m/4) + 4t + m%4,
// so lane group g's accumulators hold keys 8g .. 8g+7 of every query row, in
// order: the B operand of the PV product as it stands. Dimensions: QK chunk c
// of lane group g covers dims 32c + 8g .. 32c + 8g + 7, so each 16-byte load
// instruction reads 64 contiguous bytes of every key row; the Q operand
// matches.
#include <cstdio>

#include "kvfp8_internal.h"
#include "split_plan.h"

namespace kvfp8 {
namespace {

constexpr int kTileF = 32;
constexpr float kLazyF = 8.0f;  // lazy rescale threshold (log2 units), as in the E4M3 kernel

__device__ __forceinline__ float group_max(float x) {
  // lanes l and l ^ 16 meet by a swap of neighbouring 16-lane rows, then lanes
  // l and l ^ 32 by a swap of the two halves (gfx950 cross-row moves on the
  // vector ALU: no LDS round trip, no wait)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum(float x) {
  // the same two swaps as the maximum; every lane of a group adds the same
  // two values in the same order, so the group agrees bit for bit
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
struct TileF16 {
  u32x4 k[2][D / 32];  // M-tile t, chunk c: dims 32c + 8g .. +7 of key row 8(n/4) + 4t + n%4
  u32x4 v[D / 16];     // dim block blk: keys 8g .. 8g+7 of dim 16*blk + n
};

// Page ids of one lane's K rows (one per M-tile) and V keys (two halves of
// four keys; they differ only with pages of 4 tokens), clamped to the last page.
struct PagesF16 {
  int32_t k[2];
  int32_t v[2];
};

template <int P>
__device__ __forceinline__ void pages_f16(PagesF16& pg, const int32_t* __restrict__ btrow, int t0, int last, int n,
                                          int g) {
#pragma unroll
  for (int t = 0; t < 2; ++t) pg.k[t] = btrow[min((int)((uint32_t)(t0 + 8 * (n >> 2) + 4 * t + (n & 3)) / P), last)];
  pg.v[0] = btrow[min((int)((uint32_t)(t0 + 8 * g) / P), last)];
  pg.v[1] = P == 4 ? btrow[min((int)((uint32_t)(t0 + 8 * g + 4) / P), last)] : pg.v[0];
}

// Loads are unconditional: keys past the end of the sequence read the clamped
// last page and are masked (scores) and cleared (V) in compute_f16.
template <int D, int P>
__device__ __forceinline__ void load_f16(TileF16<D>& r, const PagesF16& pg, int t0, int n, int g,
                                         const uint8_t* __restrict__ kbase, const uint8_t* __restrict__ vbase,
                                         uint32_t page_bytes) {
  // The contraction order over dims is free: chunk c of lane group g holds
  // dims 32c + 8g .. +7, so each load instruction reads 64 contiguous bytes of
  // every key row (the four lane groups side by side), not four 16-byte pieces
  // 64 bytes apart. Q uses the same order.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int off = (t0 + 8 * (n >> 2) + 4 * t + (n & 3)) % P;
    const u32x4* p = reinterpret_cast<const u32x4*>(kbase + (uint64_t)(uint32_t)pg.k[t] * page_bytes +
                                                    (uint32_t)(2 * (off * D + 8 * g)));
#pragma unroll
    for (int j = 0; j < D / 32; ++j) r.k[t][j] = __builtin_nontemporal_load(p + 4 * j);
  }
#pragma unroll
  for (int blk = 0; blk < D / 16; ++blk) {
    const int d = 16 * blk + n;
    if constexpr (P >= 8) {
      const int off = (t0 + 8 * g) % P;
      r.v[blk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          vbase + (uint64_t)(uint32_t)pg.v[0] * page_bytes + (uint32_t)(2 * (d * P + off))));
    } else {
      // pages of 4: keys 8g .. 8g+3 start page v[0], keys 8g+4 .. 8g+7 page v[1]
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vbase + (uint64_t)(uint32_t)pg.v[0] * page_bytes +
                                                       (uint32_t)(2 * d * P));
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vbase + (uint64_t)(uint32_t)pg.v[1] * page_bytes +
                                                       (uint32_t)(2 * d * P));
      r.v[blk] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }
}

template <int D, int NB>
__device__ __forceinline__ void compute_f16(TileF16<D>& r, int t0, int L, int g, const f16x8 (*sq)[D / 32][64],
                                            const int (&lim)[NB], bool masked, float score_scale, float (&m_ref)[NB],
                                            float (&m_max)[NB], float (&l_run)[NB], f32x4 (&o)[NB][D / 16]) {
  constexpr int NBLK = D / 16;
  // keys at or past the end of the sequence may hold anything, NaN included:
  // clear their V values so a zero probability never meets one
  if (t0 + kTileF > L) {
    const int c = L - (t0 + 8 * g);  // valid keys among this lane group's 8
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t mask = c >= 2 * w + 2 ? 0xFFFFFFFFu : (c == 2 * w + 1 ? 0x0000FFFFu : 0u);
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) r.v[blk][w] &= mask;
    }
  }
  // ---- S^T = K Q^T, with Q re-read from LDS every tile (the empty asm keeps
  // the compiler from hoisting it into registers the K/V double buffer needs)
  __asm__ volatile("" ::: "memory");
  const int lane = threadIdx.x & 63;
  f32x4 sc[2][NB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    f16x8 qop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) qop[nb] = sq[nb][c][lane];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f16x8 ka = __builtin_bit_cast(f16x8, r.k[t][c]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        sc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[nb], sc[t][nb], 0, 0, 0);
    }
  }
  // ---- online softmax in log2 units, as in the E4M3 kernel
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  f16x8 pk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // tiles below every row's limit skip the mask (masked is wave-uniform)
    if (masked) {
      const int rem = lim[nb] - t0 - 8 * g;  // keys 8g + j of the tile with j < rem are visible
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * t + i >= rem) sc[t][nb][i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[t][nb][i]);
    m_max[nb] = fmaxf(m_max[nb], group_max(tmax) * score_scale);
    if (__builtin_amdgcn_ballot_w64(m_max[nb] > m_ref[nb] + kLazyF) != 0) {
      const float m_new = m_max[nb];
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
      m_ref[nb] = m_new;
      l_run[nb] *= alpha;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) o[nb][blk] *= alpha;
    }
    const float nref = (m_ref[nb] == -INFINITY) ? 0.0f : -m_ref[nb];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pk[nb][j] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[j >> 2][nb][j & 3], score_scale, nref));
    float lsum = l_run[nb];
    lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb], pk[nb], 0, 1), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb], pk[nb], 2, 3), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb], pk[nb], 4, 5), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb], pk[nb], 6, 7), ones, lsum, false);
    l_run[nb] = lsum;
  }
  // ---- O^T += V^T P^T
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
    const f16x8 va = __builtin_bit_cast(f16x8, r.v[blk]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pk[nb], o[nb][blk], 0, 0, 0);
  }
}

template <int D, int P, int NB, int W>
__global__ __launch_bounds__(64 * W, 2) void attn_split_f16_kernel(const AttnArgs a) {
  constexpr int NC = D / 32;
  constexpr int NBLK = D / 16;
  constexpr int ROWS = NB * 16;
  constexpr int OPAD = D + 4;
  __shared__ float sm_m[W][ROWS];
  __shared__ float sm_l[W][ROWS];
  __shared__ __attribute__((aligned(16))) float sm_o[W][ROWS][OPAD];
  __shared__ f16x8 sm_q[NB][NC][64];  // Q rows, the B operand of each lane

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  const int S = a.num_splits;
  const SplitItem itm = plan_item(a.seq_lens, a.batch, a.n_kv_heads, S,
                                  blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), lane);
  if (!itm.valid) return;  // past the last item (uniform over the workgroup)
  const int s = itm.s;
  const int kvh = itm.kvh;
  const int b = itm.b;
  const int L = itm.L;
  int q0, T;
  if (a.cu_q_lens != nullptr) {
    q0 = a.cu_q_lens[b];
    T = a.cu_q_lens[b + 1] - q0;
  } else {
    q0 = b;
    T = 1;
  }
  T = min(T, a.max_q_len);
  const int G = a.group;
  const int nrows = T * G;
  const int start = s * itm.chunk;
  const int end = min(start + itm.chunk, L);
  const int ntiles = end > start ? (end - start + kTileF - 1) / kTileF : 0;
  const int s_fill_end = (s == itm.n_used - 1) ? S : s + 1;

  // An item with no keys (a sequence of length 0) returns before any K/V load:
  // its page ids would not name a page. It writes m = -inf and l = 0 for its
  // split slots, or zero output rows when there is no workspace.
  if (ntiles == 0) {
    for (int rr = threadIdx.x; rr < nrows; rr += 64 * W) {
      const int64_t row = (int64_t)(q0 + rr / G) * a.n_q_heads + kvh * G + rr % G;
      if (a.out != nullptr) {
        for (int d = 0; d < D; d += 8) *reinterpret_cast<u32x4*>(a.out + row * D + d) = u32x4{0u, 0u, 0u, 0u};
      } else {
        for (int s2 = s; s2 < s_fill_end; ++s2) {
          a.ws_m[row * S + s2] = -INFINITY;
          a.ws_l[row * S + s2] = 0.0f;
        }
      }
    }
    return;
  }

  // ---- Q operand (dims 32c + 8g + i of row n of each 16-row block) and
  // each row's visible-key limit; tiles that end at or below the smallest
  // limit over the query rows, min(end, L - T + 1), need no mask
  const int mask_from = min(end, L - T + 1);
  f16x8 qb[NB][NC];
  int lim[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int rr = nb * 16 + n;
    const int i = rr / G;
    lim[nb] = rr < nrows ? min(end, L - T + i + 1) : 0;
    if (rr < nrows) {
      const uint16_t* qp = a.q + ((int64_t)(q0 + i) * a.n_q_heads + kvh * G + rr % G) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NC; ++c) qb[nb][c] = *reinterpret_cast<const f16x8*>(qp + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) qb[nb][c] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  const uint32_t page_bytes = 2u * (uint32_t)a.n_kv_heads * P * D;  // < 2^32: n_kv_heads <= 65535
  const uint8_t* kbase = a.k_cache + (int64_t)kvh * P * D * 2;
  const uint8_t* vbase = a.v_cache + (int64_t)kvh * P * D * 2;
  const int32_t* btrow = a.block_table + (int64_t)b * a.max_pages;
  const int last = L > 0 ? (L - 1) / P : 0;

  float m_ref[NB], m_max[NB], l_run[NB];
  f32x4 o[NB][NBLK];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_ref[nb] = -INFINITY;
    m_max[nb] = -INFINITY;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) o[nb][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- start-up: Q and the first page ids load together (every wavefront
  // loads Q, so no load sits on one side of a branch); wavefront 0 stores Q to
  // LDS before any tile byte is issued, and the barrier waits for LDS only, so
  // the first tile stays in flight across it
  int it = wave;
  PagesF16 pa, pb;
  pages_f16<P>(pa, btrow, start + it * kTileF, last, n, g);
  pages_f16<P>(pb, btrow, start + (it + W) * kTileF, last, n, g);
  if (wave == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < NC; ++c) sm_q[nb][c][lane] = qb[nb][c];
  }
  __asm__ volatile("" ::: "memory");
  TileF16<D> ra;
  load_f16<D, P>(ra, pa, start + it * kTileF, n, g, kbase, vbase, page_bytes);
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  if constexpr (NB == 1) {
    // two register buffers keep the next tile in flight while the current one
    // is computed; page ids run two tiles ahead of the bytes (the vector
    // memory counter is in-order)
    TileF16<D> rb;
    if (it < ntiles) {
      while (true) {
        pages_f16<P>(pa, btrow, start + (it + 2 * W) * kTileF, last, n, g);
        if (it + W < ntiles) load_f16<D, P>(rb, pb, start + (it + W) * kTileF, n, g, kbase, vbase, page_bytes);
        compute_f16<D, NB>(ra, start + it * kTileF, L, g, sm_q, lim,
                           start + (it + 1) * kTileF > mask_from, a.score_scale, m_ref, m_max, l_run, o);
        it += W;
        if (it >= ntiles) break;
        pages_f16<P>(pb, btrow, start + (it + 2 * W) * kTileF, last, n, g);
        if (it + W < ntiles) load_f16<D, P>(ra, pa, start + (it + W) * kTileF, n, g, kbase, vbase, page_bytes);
        compute_f16<D, NB>(rb, start + it * kTileF, L, g, sm_q, lim,
                           start + (it + 1) * kTileF > mask_from, a.score_scale, m_ref, m_max, l_run, o);
        it += W;
        if (it >= ntiles) break;
      }
    }
  } else {
    // with two 16-row blocks the accumulators leave room for one register
    // tile: the next tile is issued once the current one is computed, with
    // its page ids already loaded
    if (it < ntiles) {
      while (true) {
        compute_f16<D, NB>(ra, start + it * kTileF, L, g, sm_q, lim,
                           start + (it + 1) * kTileF > mask_from, a.score_scale, m_ref, m_max, l_run, o);
        it += W;
        if (it >= ntiles) break;
        load_f16<D, P>(ra, pb, start + it * kTileF, n, g, kbase, vbase, page_bytes);
        pages_f16<P>(pb, btrow, start + (it + W) * kTileF, last, n, g);
      }
    }
  }

  // ---- bring each wavefront's state to its true maximum and merge the
  // wavefronts' states through LDS
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float fac = (m_max[nb] == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_max[nb]);
    const float lrow = group_sum(l_run[nb]) * fac;
    const int rr = nb * 16 + n;
    if (g == 0) {
      sm_m[wave][rr] = m_max[nb];
      sm_l[wave][rr] = lrow;
    }
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
      *reinterpret_cast<f32x4*>(&sm_o[wave][rr][16 * blk + 4 * g]) = o[nb][blk] * fac;
  }
  __syncthreads();

  constexpr int DG8 = D / 8;
  const bool direct = (a.out != nullptr);
  for (int item = threadIdx.x; item < ROWS * DG8; item += 64 * W) {
    const int rr = item / DG8;
    const int dg = item % DG8;
    if (rr >= nrows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][rr]);
    const float ref = (M == -INFINITY) ? 0.0f : M;
    float lsum = 0.0f;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm_m[w][rr];
      const float wt = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - ref);
      lsum += wt * sm_l[w][rr];
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sm_o[w][rr][8 * dg]);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sm_o[w][rr][8 * dg + 4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += wt * x0[j];
        acc[4 + j] += wt * x1[j];
      }
    }
    const int64_t qrow = q0 + rr / G;
    const int h = kvh * G + rr % G;
    if (direct) {
      const float f = lsum > 0.0f ? 1.0f / lsum : 0.0f;
      uint32_t pk4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 lo = (_Float16)(acc[2 * j] * f);
        const _Float16 hi = (_Float16)(acc[2 * j + 1] * f);
        pk4[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x4*>(a.out + (qrow * a.n_q_heads + h) * D + 8 * dg) = u32x4{pk4[0], pk4[1], pk4[2], pk4[3]};
    } else {
      const int64_t unit = (qrow * a.n_q_heads + h) * S + s;
      float* dst = a.ws_o + unit * D + 8 * dg;
      *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
      if (dg == 0) {
        a.ws_m[unit] = (M == -INFINITY) ? -INFINITY : M * kLn2;
        a.ws_l[unit] = lsum;
        for (int s2 = s + 1; s2 < s_fill_end; ++s2) {
          a.ws_m[unit - s + s2] = -INFINITY;
          a.ws_l[unit - s + s2] = 0.0f;
        }
      }
    }
  }
}

template <int D, int P, int NB>
hipError_t launch3_f16(const AttnArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.num_splits, (unsigned)a.n_kv_heads, (unsigned)a.batch);
  // wavefronts per workgroup chosen as for the E4M3 kernel
  if constexpr (NB == 1) {
    if ((int64_t)a.num_splits * a.n_kv_heads * a.batch <= device_cus()) {
      attn_split_f16_kernel<D, P, 1, 8><<<grid, dim3(64 * 8), 0, stream>>>(a);
      return hipGetLastError();
    }
  }
  attn_split_f16_kernel<D, P, NB, 4><<<grid, dim3(64 * 4), 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int P>
hipError_t launch2_f16(const AttnArgs& a, int rows, hipStream_t stream) {
  if (rows <= 16) return launch3_f16<D, P, 1>(a, stream);
  return launch3_f16<D, P, 2>(a, stream);
}

template <int D>
hipError_t launch1_f16(const AttnArgs& a, int rows, hipStream_t stream) {
  switch (a.page_size) {
    case 4: return launch2_f16<D, 4>(a, rows, stream);
    case 8: return launch2_f16<D, 8>(a, rows, stream);
    case 16: return launch2_f16<D, 16>(a, rows, stream);
    case 32: return launch2_f16<D, 32>(a, rows, stream);
    case 64: return launch2_f16<D, 64>(a, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

void attn_split_f16_kernel_name(const AttnArgs& a, int rows_per_kvh, char* buf, size_t n) {
  const int nb = rows_per_kvh <= 16 ? 1 : 2;
  const int w = (nb == 1 && (int64_t)a.num_splits * a.n_kv_heads * a.batch <= device_cus()) ? 8 : 4;
  snprintf(buf, n, "attn_split_f16_kernel<%d,%d,%d,%d>", a.head_dim, a.page_size, nb, w);
}

hipError_t launch_attn_split_f16(const AttnArgs& a, int rows_per_kvh, hipStream_t stream) {
  if (rows_per_kvh < 1 || rows_per_kvh > 32) return hipErrorNotSupported;
  if (a.head_dim == 128) return launch1_f16<128>(a, rows_per_kvh, stream);
  if (a.head_dim == 64) return launch1_f16<64>(a, rows_per_kvh, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvfp8
