// Split-context paged attention over an E4M3 cache for up to 32 query rows per
// (sequence, kv-head): decode (1 query token, the GQA group as rows) and MTP
// verify (a few query tokens with a causal mask among them).
//
// Work decomposition: one workgroup per (sequence, kv-head, split) item of the
// work plan (split_plan.h: one split size for the whole batch, the items with
// keys numbered first); its W wavefronts (8 for a decode grid that fits one
// round of the compute units, else 4) take interleaved 64-key tiles of the
// split and merge their online-softmax states through LDS at the end. With
// new tokens to append (decode or MTP verify), each is quantised into the cache
// by the wavefront that will load the tile holding it, before its first load.
//
// Per 64-key tile a wavefront computes S^T = K Q^T and O^T += V^T P^T with
// v_mfma_f32_16x16x32_f16:
//  * QK: A = 16 keys x 32 dims of K (decoded from E4M3 in registers), B = the
//    same 32 dims x 16 query rows of Q (fp16; decode re-reads it from LDS every
//    tile, verify keeps it in registers).
//    The contraction order over dims is free, so MFMA c takes, in lane group
//    g (lanes 16g..16g+15), dims 16g + 64*(c/2) + 8*(c%2) + i: each load
//    instruction then reads 64 contiguous bytes of 16 key rows. The key of
//    MFMA row m in M-tile t is 16*(m/4) + 4t + m%4, which puts keys
//    16g + 4t + i of every query row in lane group g's accumulators.
//  * PV: A = 16 dims x 32 keys of V^T, B = the 32 keys x 16 rows of P taken
//    straight from the QK accumulators (no cross-lane movement). Lane group g
//    needs keys 16g .. 16g+15 of one dimension: 16 contiguous bytes of the
//    dimension-major V page.
// Scores are scaled once per tile by k_scale * sm_scale * log2(e) (folded into
// the exp2 argument); v_scale is applied once to the merged accumulator.
#include <cstdio>

#include "kvfp8_internal.h"
#include "split_plan.h"

namespace kvfp8 {
namespace {

constexpr int kTile = 64;

template <int D, int P>
struct TileRegs {
  uint32_t k[4][D / 16];   // 4 M-tiles x D/4 bytes of one key row
  uint32_t v[D / 16][4];   // D/16 dim blocks x 16 key bytes of one dimension
};

__device__ __forceinline__ float wave_max_groups(float x) {
  // lanes l and l ^ 16 meet by a swap of neighbouring 16-lane rows, then lanes
  // l and l ^ 32 by a swap of the two halves (gfx950 cross-row moves on the
  // vector ALU: no LDS round trip, no wait)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  // the same two swaps as the maximum; every lane of a group adds the same
  // two values in the same order, so the group agrees bit for bit
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


// Per-lane page ids of one 64-key tile: the page of this lane's K rows (one per
// M-tile when pages are shorter than 16 keys) and of its 16 V keys (one per
// piece of P keys when P < 16). Indices are clamped to the sequence's last
// page, so no entry past it is ever read.
template <int P>
struct PageRegs {
  static constexpr int NK = (P >= 16) ? 1 : 4;
  static constexpr int NV = (P >= 16) ? 1 : 16 / P;
  int32_t k[NK];
  int32_t v[NV];
};

// Vector loads, issued two tiles ahead of use: the in-order vector memory
// counter then never makes a wait on these ids wait on K/V bytes that are
// still in flight for the tile being computed. Key positions are never
// negative, so the page index is an unsigned (shift) division.
template <int P>
__device__ __forceinline__ void load_pages(PageRegs<P>& pr, const int32_t* __restrict__ btrow, int t0,
                                           int last, int n, int g) {
  const int krel = 16 * (n >> 2) + (n & 3);
#pragma unroll
  for (int t = 0; t < PageRegs<P>::NK; ++t)
    pr.k[t] = btrow[min((int)((uint32_t)(t0 + krel + 4 * t) / P), last)];
#pragma unroll
  for (int pc = 0; pc < PageRegs<P>::NV; ++pc)
    pr.v[pc] = btrow[min((int)((uint32_t)(t0 + 16 * g + pc * P) / P), last)];
}

// Page ids of one 64-key tile (pages of >= 16 keys) taken from a block-table
// row held across the wavefront: lane l holds row entries l, l + 64, l + 128
// and l + 192 (rows of at most 256 pages). Same indices as load_pages, no
// memory access.
__device__ __forceinline__ int32_t row_entry(const int32_t (&rowv)[4], int idx) {
  const int addr = (idx & 63) << 2;
  const int32_t v0 = __builtin_amdgcn_ds_bpermute(addr, rowv[0]);
  const int32_t v1 = __builtin_amdgcn_ds_bpermute(addr, rowv[1]);
  const int32_t v2 = __builtin_amdgcn_ds_bpermute(addr, rowv[2]);
  const int32_t v3 = __builtin_amdgcn_ds_bpermute(addr, rowv[3]);
  const int k = idx >> 6;
  return k == 0 ? v0 : (k == 1 ? v1 : (k == 2 ? v2 : v3));
}

template <int P>
__device__ __forceinline__ void pages_from_row(PageRegs<P>& pr, const int32_t (&rowv)[4], int t0, int last, int n,
                                               int g) {
  static_assert(P >= 16, "one page id per lane for K and for V");
  const int krel = 16 * (n >> 2) + (n & 3);
  pr.k[0] = row_entry(rowv, min((int)((uint32_t)(t0 + krel) / P), last));
  pr.v[0] = row_entry(rowv, min((int)((uint32_t)(t0 + 16 * g) / P), last));
}

// K/V bytes are read exactly once per call, so they are loaded non-temporally
// (streamed past the caches instead of evicting the block table, Q and the
// partials). The loads are unconditional: a tile never extends past the split
// unless the split ends the sequence, and page ids are clamped to the last
// page, so keys past the end read rows of an allocated page. Their scores are
// masked and their V bytes cleared in compute_tile, which is cheaper than
// branching and zero-filling the registers on every tile.
// In-page byte offsets of this lane's K rows and V bytes. Tiles start at
// multiples of 64 keys, so the offsets are the same for every tile.
template <int D, int P>
struct LaneOffsets {
  uint32_t k[4];  // K row of M-tile t, dims from 16g
  uint32_t v;     // V bytes of dimension n, keys from 16g (piece 0)
  __device__ __forceinline__ LaneOffsets(int n, int g) {
    const int krel = 16 * (n >> 2) + (n & 3);
#pragma unroll
    for (int t = 0; t < 4; ++t) k[t] = (uint32_t)(((krel + 4 * t) % P) * D + 16 * g);
    v = (uint32_t)(n * P + (16 * g) % P);
  }
};

template <int D, int P>
__device__ __forceinline__ void load_tile(TileRegs<D, P>& r, const PageRegs<P>& pr, const LaneOffsets<D, P>& lo,
                                          const uint8_t* __restrict__ kbase,
                                          const uint8_t* __restrict__ vbase, uint32_t page_stride) {
  constexpr int KD = D / 16;  // dwords of K per lane and M-tile
  // ---- K: the key row of this lane in M-tile t is t0 + 16*(n/4) + 4t + n%4.
  // Lane group g reads dims [16g, 16g+16) (and [64+16g, 80+16g) for D = 128),
  // so each load instruction covers 64 contiguous bytes of every key row.
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t pg = (uint32_t)pr.k[PageRegs<P>::NK == 1 ? 0 : t];
    const uint8_t* p = kbase + (uint64_t)pg * page_stride + lo.k[t];
#pragma unroll
    for (int j = 0; j < KD / 4; ++j) {
      u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 64 * j));
      r.k[t][4 * j + 0] = w[0];
      r.k[t][4 * j + 1] = w[1];
      r.k[t][4 * j + 2] = w[2];
      r.k[t][4 * j + 3] = w[3];
    }
  }
  // ---- V: keys t0 + 16g .. +15 of dimensions 16*blk + n
  if constexpr (P >= 16) {
    const uint8_t* p = vbase + (uint64_t)(uint32_t)pr.v[0] * page_stride + lo.v;
#pragma unroll
    for (int blk = 0; blk < D / 16; ++blk) {
      u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + blk * 16 * P));
      r.v[blk][0] = w[0];
      r.v[blk][1] = w[1];
      r.v[blk][2] = w[2];
      r.v[blk][3] = w[3];
    }
  } else {
    constexpr int PIECES = 16 / P;  // pages covered by 16 keys
    constexpr int PD = P / 4;       // dwords per piece
#pragma unroll
    for (int pc = 0; pc < PIECES; ++pc) {
      const uint8_t* p = vbase + (uint64_t)(uint32_t)pr.v[pc] * page_stride + lo.v;
#pragma unroll
      for (int blk = 0; blk < D / 16; ++blk) {
        const uint8_t* q = p + blk * 16 * P;
        if constexpr (PD == 2) {
          u32x2 w = *reinterpret_cast<const u32x2*>(q);
          r.v[blk][pc * 2 + 0] = w[0];
          r.v[blk][pc * 2 + 1] = w[1];
        } else {
          r.v[blk][pc] = *reinterpret_cast<const uint32_t*>(q);
        }
      }
    }
  }
}

// Bytes of one tile per wavefront (K and V codes): the LDS staging area of the
// verify pipeline.
template <int D>
constexpr int kTileBytes = 2 * kTile * D;

// The same 16-byte loads as load_tile (P >= 16), issued as direct-to-LDS
// loads: load i writes each lane's 16 bytes at lds + 1024 i + 16 lane, so the
// tile occupies no registers while in flight. The caller waits for the
// vector memory counter before read_tile_lds.
template <int D, int P>
__device__ __forceinline__ void load_tile_lds(uint8_t* lds, const PageRegs<P>& pr, const LaneOffsets<D, P>& lo,
                                              const uint8_t* __restrict__ kbase,
                                              const uint8_t* __restrict__ vbase, uint32_t page_stride) {
  static_assert(P >= 16, "V bytes of one dimension must be 16 contiguous bytes");
  constexpr int KD = D / 16;
  // both page addresses first: no page-id register is read once loads of this
  // tile are in flight
  const uint8_t* kp = kbase + (uint64_t)(uint32_t)pr.k[0] * page_stride;
  const uint8_t* vp = vbase + (uint64_t)(uint32_t)pr.v[0] * page_stride + lo.v;
  __asm__ volatile("" ::"v"(kp), "v"(vp));
  int i = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < KD / 4; ++j, ++i)
      __builtin_amdgcn_global_load_lds(kp + lo.k[t] + 64 * j, (__attribute__((address_space(3))) void*)(lds + 1024 * i),
                                       16, 0, 0);
#pragma unroll
  for (int blk = 0; blk < D / 16; ++blk, ++i)
    __builtin_amdgcn_global_load_lds(vp + blk * 16 * P, (__attribute__((address_space(3))) void*)(lds + 1024 * i), 16,
                                     0, 0);
}

// Each lane reads back its own 16-byte pieces (conflict-free: consecutive
// lanes, consecutive 16 bytes) into the register tile.
template <int D, int P>
__device__ __forceinline__ void read_tile_lds(TileRegs<D, P>& r, const uint8_t* lds, int lane) {
  constexpr int KD = D / 16;
  int i = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < KD / 4; ++j, ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(lds + 1024 * i + 16 * lane);
      r.k[t][4 * j + 0] = w[0];
      r.k[t][4 * j + 1] = w[1];
      r.k[t][4 * j + 2] = w[2];
      r.k[t][4 * j + 3] = w[3];
    }
#pragma unroll
  for (int blk = 0; blk < D / 16; ++blk, ++i) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(lds + 1024 * i + 16 * lane);
    r.v[blk][0] = w[0];
    r.v[blk][1] = w[1];
    r.v[blk][2] = w[2];
    r.v[blk][3] = w[3];
  }
}

// Rows keep a reference maximum m_ref for their probabilities and rescale
// their accumulators only when some row's maximum moves more than kLazy (log2
// units) above it: probabilities are then at most 2^kLazy, which fp16 and the
// fp32 accumulators hold exactly as well as values below 1. The true running
// maximum m_max is tracked beside it; the state is brought to m_max once, at
// the end.
constexpr float kLazy = 8.0f;

template <int D, int P, int NB, bool QREG>
__device__ __forceinline__ void compute_tile(TileRegs<D, P>& r, int t0, int L, int g,
                                             const f16x8 (*sq)[D / 32][64], const f16x8 (&qreg)[NB][D / 32],
                                             const int (&lim)[NB], bool masked,
                                             float score_scale, float (&m_ref)[NB], float (&m_max)[NB],
                                             float (&l_run)[NB], f32x4 (&o)[NB][D / 16]) {
  constexpr int NBLK = D / 16;
  // keys at or past the end of the sequence may hold poison codes: zero their
  // V bytes so that a zero probability cannot meet a NaN in the PV product
  if (t0 + kTile > L) {
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const int c = L - (t0 + 16 * g + 4 * w4);
      const uint32_t mask = c >= 4 ? 0xFFFFFFFFu : (c <= 0 ? 0u : ((1u << (8 * c)) - 1u));
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) r.v[blk][w4] &= mask;
    }
  }
  // ---- S^T = K Q^T. Q is in registers (QREG) or re-read from LDS every tile
  // (the empty asm keeps the compiler from hoisting it into registers, which
  // the K/V double buffer needs).
  __asm__ volatile("" ::: "memory");
  const int lane = threadIdx.x & 63;
  f32x4 sc[4][NB];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    f16x8 qop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (QREG)
        qop[nb] = qreg[nb][c];
      else
        qop[nb] = sq[nb][c][lane];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 ka = e4m3x8_to_f16(r.k[t][2 * c], r.k[t][2 * c + 1]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        sc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[nb], sc[t][nb], 0, 0, 0);
    }
  }

  // ---- online softmax (log2 units); rows are lane columns. The maximum is
  // taken on raw scores (score_scale > 0) and the scale folded into exp2's FMA.
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  f16x8 pk[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // mask keys at or past each row's limit (the end of the split, or the
    // row's causal position); the compare constants are the lane's key offsets.
    // Tiles below every row's limit skip it (masked is wave-uniform).
    if (masked) {
      const int rem = lim[nb] - t0 - 16 * g;  // keys 16g + k of the tile with k < rem are visible
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * t + i >= rem) sc[t][nb][i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[t][nb][i]);
    tmax = wave_max_groups(tmax) * score_scale;
    m_max[nb] = fmaxf(m_max[nb], tmax);
    if (__builtin_amdgcn_ballot_w64(m_max[nb] > m_ref[nb] + kLazy) != 0) {
      const float m_new = m_max[nb];
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
      m_ref[nb] = m_new;
      l_run[nb] *= alpha;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) o[nb][blk] *= alpha;
    }
    const float nref = (m_ref[nb] == -INFINITY) ? 0.0f : -m_ref[nb];
    float lsum = l_run[nb];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 2 * u + (j >> 2);
        pk[nb][u][j] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][nb][j & 3], score_scale, nref));
      }
      lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb][u], pk[nb][u], 0, 1), ones, lsum, false);
      lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb][u], pk[nb][u], 2, 3), ones, lsum, false);
      lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb][u], pk[nb][u], 4, 5), ones, lsum, false);
      lsum = __builtin_amdgcn_fdot2(__builtin_shufflevector(pk[nb][u], pk[nb][u], 6, 7), ones, lsum, false);
    }
    l_run[nb] = lsum;
  }
  // ---- O^T += V^T P^T
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f16x8 va = e4m3x8_to_f16(r.v[blk][2 * u], r.v[blk][2 * u + 1]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        o[nb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pk[nb][u], o[nb][blk], 0, 0, 0);
    }
  }
}

template <int D, int P, int NB, int W, bool SHORT = false>
__global__ __launch_bounds__(64 * W, 2) void attn_split_kernel(const AttnArgs a) {
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
  // SHORT (decode over pages of >= 16 keys, one round of 8-wavefront
  // workgroups, at most one tile per wavefront): the start-up is most of the
  // kernel, so it is cut short. The block-table row of sequence blockIdx.z
  // (the plan's sequence whenever the plan is the plain grid, e.g. equal
  // lengths) loads beside the work plan's context lengths; when the plan
  // confirms it and the row has at most 256 pages, the first tiles' page ids
  // come from it, one round trip earlier. Indices stay inside the row.
  constexpr bool kRowPrefetch = SHORT;
  static_assert(!SHORT || (NB == 1 && P >= 16 && W == 8), "short start-up: decode, pages of >= 16 keys, 8 waves");
  int32_t rowv[4] = {0, 0, 0, 0};
  if constexpr (kRowPrefetch) {
    const int32_t* grow = a.block_table + (int64_t)blockIdx.z * a.max_pages;
#pragma unroll
    for (int k = 0; k < 4; ++k) rowv[k] = grow[min(lane + 64 * k, a.max_pages - 1)];
  }
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
  // no query rows (a verify sequence without tokens): nothing to write; the
  // short start-up relies on it (it clamps row indices to nrows - 1)
  if (SHORT && nrows <= 0) return;
  const int start = s * itm.chunk;
  const int end = min(start + itm.chunk, L);
  const int ntiles = end > start ? (end - start + kTile - 1) / kTile : 0;
  // the smallest limit over the query rows (row i of the sequence sees keys
  // below min(end, L - T + i + 1)): tiles that end at or below it need no mask
  const int mask_from = min(end, L - T + 1);
  // the sequence's last item also marks its unused split slots as empty
  // (m = -inf, l = 0: weight zero in the reduce, which never multiplies their o)
  const int s_fill_end = (s == itm.n_used - 1) ? S : s + 1;

  // An item with no keys (a sequence of length 0) writes only m and l.
  if (ntiles == 0 && a.out == nullptr) {
    for (int rr = threadIdx.x; rr < nrows; rr += 64 * W) {
      const int i = rr / G;
      const int64_t unit = ((int64_t)(q0 + i) * a.n_q_heads + kvh * G + rr % G) * S;
      for (int s2 = s; s2 < s_fill_end; ++s2) {
        a.ws_m[unit + s2] = -INFINITY;
        a.ws_l[unit + s2] = 0.0f;
      }
    }
    return;
  }

  // ---- append: each of the sequence's new tokens (key positions L - T ..
  // L - 1, this step's query tokens) is quantised into its slot, exactly as
  // the cache write does, by the wavefront that will load the tile holding it;
  // no other wavefront or workgroup reads that tile (tiles and splits start on
  // multiples of 64 keys, and pages hold at most 64), and the wavefront's other
  // tiles lie on other pages. Its stores must be complete before it issues the
  // load of that tile (see below for where each pipeline waits).
  constexpr bool kStaged = NB == 2 && P >= 16;
  constexpr int PER = D / 64;  // dims per lane
  constexpr int kBatch = 4;
  bool first_wait = false;
  // Staged verify: a wavefront whose new tokens are one batch in one tile that
  // is not its first issues their loads here and encodes and stores them once
  // its first tile has landed (deferred), so the loads' round trip overlaps
  // that tile's instead of delaying it.
  bool deferred = false;
  int d_p0 = 0, d_tile = -1;
  bool d_mine[kBatch];
  uint64_t d_page[kBatch];
  uint16_t d_kx[kBatch][PER], d_vx[kBatch][PER];
  auto store_batch = [&](int p0, const bool (&mine)[kBatch], const uint64_t (&page)[kBatch],
                         const uint16_t (&kx)[kBatch][PER], const uint16_t (&vx)[kBatch][PER]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!mine[u]) continue;
      const int off = (p0 + u) % P;
      uint8_t* kd = a.k_cache_w + ((page[u] * a.n_kv_heads + kvh) * P + off) * D + PER * lane;
      uint8_t* vd = a.v_cache_w + ((page[u] * a.n_kv_heads + kvh) * D + PER * lane) * P + off;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        kd[j] = (uint8_t)e4m3_encode((float)__builtin_bit_cast(_Float16, kx[u][j]) / a.k_scale);
        vd[(int64_t)j * P] = (uint8_t)e4m3_encode((float)__builtin_bit_cast(_Float16, vx[u][j]) / a.v_scale);
      }
    }
  };
  if (a.k_new != nullptr && ntiles > 0) {
    const int first_new = max(start, L - T);
    if (first_new < end) {
      bool wrote = false;
      int wrote_tile = -1;
      bool one_tile = true;
      if constexpr (kStaged) {
        // Staged verify (several new tokens): up to four tokens at a time, every
        // load first (block-table entries and new values), then the encodes and
        // stores; the wait counter retires loads and stores in issue order, so a
        // token's loads placed after the previous token's stores would cost a
        // memory round trip per token.
        for (int p0 = first_new; p0 < end; p0 += kBatch) {
          bool mine[kBatch];
          bool any = false;
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            mine[u] = p0 + u < end && wave == ((p0 + u - start) / kTile) % W;
            any = any || mine[u];
          }
          if (!any) continue;
          // unconditional loads (positions clamped to the split's new tokens):
          // loads on one side of a branch would make the compiler wait for each
          uint64_t page[kBatch];
          uint16_t kx[kBatch][PER], vx[kBatch][PER];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int pos = min(p0 + u, end - 1);
            page[u] = (uint32_t)a.block_table[(int64_t)b * a.max_pages + pos / P];
            const int64_t src = ((int64_t)(q0 + pos - (L - T)) * a.n_kv_heads + kvh) * D + PER * lane;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
              kx[u][j] = a.k_new[src + j];
              vx[u][j] = a.v_new[src + j];
            }
          }
          int btile = -1;
          bool bone = true;
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            if (!mine[u]) continue;
            const int tile = (p0 + u - start) / kTile;
            bone = bone && (btile < 0 || btile == tile);
            btile = tile;
          }
          if (end - first_new <= kBatch && bone && btile != wave) {
            deferred = true;
            d_p0 = p0;
            d_tile = btile;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
              d_mine[u] = mine[u];
              d_page[u] = page[u];
#pragma unroll
              for (int j = 0; j < PER; ++j) {
                d_kx[u][j] = kx[u][j];
                d_vx[u][j] = vx[u][j];
              }
            }
            continue;
          }
          store_batch(p0, mine, page, kx, vx);
          one_tile = one_tile && bone && (wrote_tile < 0 || wrote_tile == btile);
          wrote_tile = btile;
          wrote = true;
        }
      } else {
        for (int pos = first_new; pos < end; ++pos) {
          if (wave != ((pos - start) / kTile) % W) continue;
          const uint64_t page = (uint32_t)a.block_table[(int64_t)b * a.max_pages + pos / P];
          const int off = pos % P;
          const int64_t src = ((int64_t)(q0 + pos - (L - T)) * a.n_kv_heads + kvh) * D + PER * lane;
          uint8_t* kd = a.k_cache_w + ((page * a.n_kv_heads + kvh) * P + off) * D + PER * lane;
          uint8_t* vd = a.v_cache_w + ((page * a.n_kv_heads + kvh) * D + PER * lane) * P + off;
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const float kx = (float)__builtin_bit_cast(_Float16, a.k_new[src + j]);
            const float vx = (float)__builtin_bit_cast(_Float16, a.v_new[src + j]);
            kd[j] = (uint8_t)e4m3_encode(kx / a.k_scale);
            vd[(int64_t)j * P] = (uint8_t)e4m3_encode(vx / a.v_scale);
          }
          wrote = true;
        }
      }
      if (wrote) {
        // The staged pipeline issues every tile load but its first behind a
        // full wait, so it waits only when the tile is its first one; the
        // register pipelines wait here (deferring it measured slower there).
        if (kStaged && one_tile)
          first_wait = wrote_tile == wave;
        else
          __builtin_amdgcn_s_waitcnt(0);
      }
    }
  }

  const uint32_t page_stride = (uint32_t)a.n_kv_heads * P * D;  // < 2^32: n_kv_heads <= 65535
  const LaneOffsets<D, P> lo(n, g);
  const uint8_t* kbase = a.k_cache + (int64_t)kvh * P * D;
  const uint8_t* vbase = a.v_cache + (int64_t)kvh * P * D;
  const int32_t* btrow = a.block_table + (int64_t)b * a.max_pages;
  const int last = L > 0 ? (L - 1) / P : 0;

  // ---- start-up: the Q rows and the first page ids load together; Q goes to
  // LDS before the first tile's K/V are issued, so the latencies overlap
  // instead of adding up. Every wavefront loads Q (a few KB, cache hits) and
  // wavefront 0 stores it: with the loads in a wave-uniform branch the
  // compiler could no longer count them exactly, and its wait before reusing
  // their registers would also wait for the tile in flight.
  // (The short start-up differs: see kRowPrefetch and kOwnQ.)
  // Page ids of the wavefront's first two tiles. The short start-up takes
  // them before Q is loaded: the fallback's loads then precede Q's, and the
  // first tile waits for no Q load.
  int it = wave;
  PageRegs<P> pa, pb;
  TileRegs<D, P> ra;
  auto first_pages = [&]() {
    // Page ids are loaded unconditionally (they are clamped to the sequence's
    // last page, and every block-table row has an entry): a load on only one
    // side of a branch would make the compiler's wait counts inexact.
    if constexpr (kRowPrefetch) {
      if (a.max_pages <= 256 && b == (int)blockIdx.z) {
        pages_from_row<P>(pa, rowv, start + it * kTile, last, n, g);
        pages_from_row<P>(pb, rowv, start + (it + W) * kTile, last, n, g);
      } else {
        load_pages<P>(pa, btrow, start + it * kTile, last, n, g);
        load_pages<P>(pb, btrow, start + (it + W) * kTile, last, n, g);
      }
    } else {
      load_pages<P>(pa, btrow, start + it * kTile, last, n, g);
      load_pages<P>(pb, btrow, start + (it + W) * kTile, last, n, g);
    }
  };
  if constexpr (kRowPrefetch) first_pages();
  // Q operand: dims g*D/4 + 8c + i of row n of each 16-row block.
  f16x8 qraw[NB][NC];
  int lim[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // the short start-up loads a real row for the padding rows too (masked,
    // never written): no lane skips the loads, so no path through the
    // start-up has a different number of loads in flight
    const int rr = kRowPrefetch ? min(n, nrows - 1) : nb * 16 + n;
    const int i = rr / G;
    lim[nb] = nb * 16 + n < nrows ? min(end, L - T + i + 1) : 0;
    if (kRowPrefetch || rr < nrows) {
      const int h = kvh * G + rr % G;
      const uint16_t* qp = a.q + ((int64_t)(q0 + i) * a.n_q_heads + h) * D + 16 * g;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        qraw[nb][c] = *reinterpret_cast<const f16x8*>(qp + 64 * (c >> 1) + 8 * (c & 1));
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) qraw[nb][c] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if constexpr (!kRowPrefetch) first_pages();
  // Short start-up: the first tile is issued before Q is stored, and every
  // wavefront stores its own copy of Q (the same bytes in the same place) and
  // reads only after its own store, so no barrier.
  constexpr bool kOwnQ = kRowPrefetch;
  if (!kOwnQ && wave == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < NC; ++c) sm_q[nb][c][lane] = qraw[nb][c];
  }
  // The tile bytes are issued only after Q is in LDS (the vector memory
  // counter is in-order: a wait for Q issued behind them would wait for
  // them), and the barrier waits for LDS only, so they stay in flight
  // across it (a full __syncthreads would also wait for every vector load).
  // the verify pipeline stages every tile, the first included, through LDS
  __asm__ volatile("" ::: "memory");
  if (!kStaged && it < ntiles) {
    load_tile<D, P>(ra, pa, lo, kbase, vbase, page_stride);
    // a wavefront without tiles never reads Q
    if constexpr (kOwnQ) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sm_q[0][c][lane] = qraw[0][c];
    }
  }
  if constexpr (!kOwnQ) __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

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

  // ---- tiles. With one 16-row block (decode) two register buffers keep the
  // next tile's K/V in flight while the current one is computed, and page ids
  // are fetched two tiles ahead.
  if constexpr (NB == 1) {
    if (it < ntiles) {
      TileRegs<D, P> rb;
      while (true) {
        load_pages<P>(pa, btrow, start + (it + 2 * W) * kTile, last, n, g);
        if (it + W < ntiles) load_tile<D, P>(rb, pb, lo, kbase, vbase, page_stride);
        compute_tile<D, P, NB, false>(ra, start + it * kTile, L, g, sm_q, qraw, lim,
                               start + (it + 1) * kTile > mask_from, a.score_scale, m_ref, m_max, l_run, o);
        it += W;
        if (it >= ntiles) break;
        load_pages<P>(pb, btrow, start + (it + 2 * W) * kTile, last, n, g);
        if (it + W < ntiles) load_tile<D, P>(ra, pa, lo, kbase, vbase, page_stride);
        compute_tile<D, P, NB, false>(rb, start + it * kTile, L, g, sm_q, qraw, lim,
                               start + (it + 1) * kTile > mask_from, a.score_scale, m_ref, m_max, l_run, o);
        it += W;
        if (it >= ntiles) break;
      }
    }
  } else if constexpr (kStaged) {
    // With two blocks (verify) the accumulators leave room for one register
    // tile; the next tile streams into this wavefront's part of the merge
    // area (unused until the merge) with direct-to-LDS loads, and Q stays in
    // registers (reading it from LDS would make the compiler wait for the
    // staged loads, which it cannot tell apart from Q).
    static_assert(W * kTileBytes<D> <= (int)sizeof(sm_o), "tile staging must fit in the merge area");
    uint8_t* tb = reinterpret_cast<uint8_t*>(&sm_o[0][0][0]) + __builtin_amdgcn_readfirstlane(wave) * kTileBytes<D>;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < NC; ++c) __asm__ volatile("" ::"v"(qraw[nb][c]));  // Q complete before the loop
    if (it < ntiles) {
      if (first_wait) __builtin_amdgcn_s_waitcnt(0);  // this step's new tokens are in this tile
      load_tile_lds<D, P>(tb, pa, lo, kbase, vbase, page_stride);
      __builtin_amdgcn_s_waitcnt(0);
      if (deferred) {
        store_batch(d_p0, d_mine, d_page, d_kx, d_vx);
        if (d_tile == it + W) __builtin_amdgcn_s_waitcnt(0);  // the next load reads them
      }
      read_tile_lds<D, P>(ra, tb, lane);
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (it + W < ntiles) load_tile_lds<D, P>(tb, pb, lo, kbase, vbase, page_stride);
      while (true) {
        load_pages<P>(pb, btrow, start + (it + 2 * W) * kTile, last, n, g);
        compute_tile<D, P, NB, true>(ra, start + it * kTile, L, g, nullptr, qraw, lim,
                               start + (it + 1) * kTile > mask_from, a.score_scale, m_ref, m_max, l_run,
                               o);
        it += W;
        if (it >= ntiles) break;
        __builtin_amdgcn_s_waitcnt(0);  // the staged tile (and the page ids) have landed
        read_tile_lds<D, P>(ra, tb, lane);
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before it is overwritten
        if (it + W < ntiles) load_tile_lds<D, P>(tb, pb, lo, kbase, vbase, page_stride);
      }
    }
    __syncthreads();  // every wavefront is done with its staging area before the merge
  } else {
    if (it < ntiles) {
      while (true) {
        load_pages<P>(pb, btrow, start + (it + W) * kTile, last, n, g);
        compute_tile<D, P, NB, false>(ra, start + it * kTile, L, g, sm_q, qraw, lim,
                               start + (it + 1) * kTile > mask_from, a.score_scale, m_ref, m_max, l_run, o);
        it += W;
        if (it >= ntiles) break;
        load_tile<D, P>(ra, pb, lo, kbase, vbase, page_stride);
      }
    }
  }

  // ---- bring each wavefront's state to its true maximum and merge the
  // wavefronts' states through LDS
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float fac = (m_max[nb] == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_max[nb]);
    const float lrow = wave_sum_groups(l_run[nb]) * fac;
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
    const int i = rr / G;
    const int h = kvh * G + rr % G;
    const int64_t qrow = q0 + i;
    if (direct) {
      const float f = lsum > 0.0f ? a.v_scale / lsum : 0.0f;
      uint32_t pk4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 lo = (_Float16)(acc[2 * j] * f);
        const _Float16 hi = (_Float16)(acc[2 * j + 1] * f);
        pk4[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x4*>(a.out + (qrow * a.n_q_heads + h) * D + 8 * dg) =
          u32x4{pk4[0], pk4[1], pk4[2], pk4[3]};
    } else {
      const int64_t unit = (qrow * a.n_q_heads + h) * S + s;
      float* dst = a.ws_o + unit * D + 8 * dg;
      *reinterpret_cast<f32x4*>(dst) =
          f32x4{acc[0] * a.v_scale, acc[1] * a.v_scale, acc[2] * a.v_scale, acc[3] * a.v_scale};
      *reinterpret_cast<f32x4*>(dst + 4) =
          f32x4{acc[4] * a.v_scale, acc[5] * a.v_scale, acc[6] * a.v_scale, acc[7] * a.v_scale};
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

// The launch shape for a call. One 16-row block (decode) whose whole grid fits
// in one round of the compute units runs 8 wavefronts per workgroup, one
// workgroup per CU, so a CU's wavefronts are of one age and finish together
// (two 4-wavefront workgroups on one CU finish apart under the hardware's
// oldest-first issue). Larger grids, and two blocks (verify, LDS-bound), run 4
// wavefronts, two workgroups per CU, which halves the number of rounds. An
// 8-wavefront decode launch over pages of >= 16 keys whose splits hold at most
// one 64-key tile per wavefront takes the short start-up.
struct SplitLaunch {
  int nb;
  int w;
  bool short_start;
};

SplitLaunch choose_split_launch(const AttnArgs& a, int rows) {
  SplitLaunch c{rows <= 16 ? 1 : 2, 4, false};
  if (c.nb == 1 && (int64_t)a.num_splits * a.n_kv_heads * a.batch <= device_cus()) {
    c.w = 8;
    c.short_start = a.page_size >= 16 && a.max_pages <= 256 &&
                    (int64_t)a.max_pages * a.page_size <= (int64_t)kTile * 8 * a.num_splits;
  }
  return c;
}

template <int D, int P, int NB>
hipError_t launch3(const AttnArgs& a, const SplitLaunch& c, hipStream_t stream) {
  dim3 grid((unsigned)a.num_splits, (unsigned)a.n_kv_heads, (unsigned)a.batch);
  if constexpr (NB == 1) {
    if (c.w == 8) {
      if constexpr (P >= 16) {
        if (c.short_start) {
          attn_split_kernel<D, P, 1, 8, true><<<grid, dim3(64 * 8), 0, stream>>>(a);
          return hipGetLastError();
        }
      }
      attn_split_kernel<D, P, 1, 8><<<grid, dim3(64 * 8), 0, stream>>>(a);
      return hipGetLastError();
    }
  }
  attn_split_kernel<D, P, NB, 4><<<grid, dim3(64 * 4), 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int P>
hipError_t launch2(const AttnArgs& a, int rows, hipStream_t stream) {
  const SplitLaunch c = choose_split_launch(a, rows);
  if (c.nb == 1) return launch3<D, P, 1>(a, c, stream);
  return launch3<D, P, 2>(a, c, stream);
}

template <int D>
hipError_t launch1(const AttnArgs& a, int rows, hipStream_t stream) {
  switch (a.page_size) {
    case 4: return launch2<D, 4>(a, rows, stream);
    case 8: return launch2<D, 8>(a, rows, stream);
    case 16: return launch2<D, 16>(a, rows, stream);
    case 32: return launch2<D, 32>(a, rows, stream);
    case 64: return launch2<D, 64>(a, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

void attn_split_kernel_name(const AttnArgs& a, int rows_per_kvh, char* buf, size_t n) {
  const SplitLaunch c = choose_split_launch(a, rows_per_kvh);
  snprintf(buf, n, "attn_split_kernel<%d,%d,%d,%d,%s>", a.head_dim, a.page_size, c.nb, c.w,
           c.short_start ? "true" : "false");
}

hipError_t launch_attn_split(const AttnArgs& a, int rows_per_kvh, hipStream_t stream) {
  if (a.head_dim == 128) return launch1<128>(a, rows_per_kvh, stream);
  if (a.head_dim == 64) return launch1<64>(a, rows_per_kvh, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvfp8
