// Query-tiled causal chunk attention over an E4M3 paged cache: the prefill /
// catch-up chunk of a mixed batch (many query tokens per sequence).
//
// One workgroup of W = 8 wavefronts owns R = 256 query rows (row = token * G +
// head-in-group) of one (sequence, kv-head) and walks the keys visible to them
// in 64-key tiles. Every tile is loaded from HBM once per workgroup, decoded
// from E4M3 to fp16 once, and staged in LDS (K token-major, V dimension-major,
// three buffers: the tile being finished, the next tile whose QK products are
// already running, and the one after that being stored).
// Each wavefront then computes S^T = K Q^T and O^T += V^T P^T for its 32 rows
// with v_mfma_f32_16x16x32_f16, exactly as the split kernel does per lane (the
// same key permutation makes the QK accumulators the PV B operand).
//
// XCD-aware placement: workgroups are dispatched round-robin over the 8 XCDs;
// when the (query tile, kv-head) plane divides evenly, the linear index is
// remapped so that each XCD serves a contiguous run of query tiles of as few
// kv-heads as possible, and its L2 holds one head's K/V stream.
#include <cstdio>

#include "kvfp8_internal.h"

#include <type_traits>


namespace kvfp8 {
namespace {

constexpr int kTile = 64;
constexpr int kWaves = 8;
constexpr int kNB = 2;                       // 16-row blocks per wavefront
constexpr int kRows = kWaves * kNB * 16;     // rows per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;

// LDS rows are 256 bytes: 16 chunks of 8 fp16 values, chunk c of row r stored
// at position c ^ (r % 16). An MFMA operand read (16 rows, lane group g taking
// chunk 4c + g of row n) then falls on all 64 banks at once with no conflict,
// where padded rows (272 or 144 bytes) conflict two-way on gfx950.
// K rows (keys) hold the D dims in order; V^T rows (dims) hold the tile's 64
// keys with keys 16g + 8u .. +7 in chunk 4u + g.
constexpr int kRowHalfs = 128;

__device__ __forceinline__ int swz(int chunk, int row) { return 8 * ((chunk ^ row) & 15); }

template <int D>
struct ChunkLds {
  _Float16 k[3][kTile][kRowHalfs];
  _Float16 v[3][D][kRowHalfs];
};

__device__ __forceinline__ float wave_max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}


// Raw bytes of one tile held by one thread: 16 K bytes (16 dims of one key) and
// 16 V bytes (16 keys of one dim).
template <int D>
struct ChunkRegs {
  static constexpr int KPT = (kTile * D / 16 + kThreads - 1) / kThreads;  // K segments per thread
  static constexpr int VPT = (D * 4 + kThreads - 1) / kThreads;           // V segments per thread
  u32x4 k[KPT];
  u32x4 v[VPT];
};

// Page ids of one thread's K row and V keys in one tile, clamped to the
// sequence's last page (so no block-table entry past it is read). They are
// fetched one tile ahead of the K/V bytes: the vector memory counter is
// in-order, and a wait on an id issued just before the bytes of another tile
// would also wait for those bytes.
template <int D, int P>
struct ChunkPages {
  static constexpr int NV = P >= 16 ? 1 : 16 / P;
  int32_t k[ChunkRegs<D>::KPT];
  int32_t v[ChunkRegs<D>::VPT][NV];
};

template <int D, int P>
__device__ __forceinline__ void chunk_pages(ChunkPages<D, P>& pg, int tid, int t0, int last,
                                            const int32_t* __restrict__ btrow) {
  constexpr int KSEG = D / 16;  // 16-byte segments per key row
#pragma unroll
  for (int j = 0; j < ChunkRegs<D>::KPT; ++j) {
    const int e = tid + j * kThreads;
    if (e < kTile * KSEG) pg.k[j] = btrow[min((t0 + e / KSEG) / P, last)];
  }
#pragma unroll
  for (int j = 0; j < ChunkRegs<D>::VPT; ++j) {
    const int e = tid + j * kThreads;
    if (e < D * 4) {
      const int tv = t0 + 16 * (e & 3);
#pragma unroll
      for (int pc = 0; pc < ChunkPages<D, P>::NV; ++pc) pg.v[j][pc] = btrow[min((tv + pc * P) / P, last)];
    }
  }
}

// Unconditional loads: keys past the end of the sequence read rows of the
// (clamped) last page; their scores are masked and their V bytes cleared in
// chunk_store.
template <int D, int P>
__device__ __forceinline__ void chunk_load(ChunkRegs<D>& r, const ChunkPages<D, P>& pg, int tid, int t0,
                                           const uint8_t* __restrict__ kbase,
                                           const uint8_t* __restrict__ vbase, uint32_t page_stride) {
  constexpr int KSEG = D / 16;
#pragma unroll
  for (int j = 0; j < ChunkRegs<D>::KPT; ++j) {
    const int e = tid + j * kThreads;
    if (e < kTile * KSEG) {
      const int kk = e / KSEG;
      const int seg = e % KSEG;
      const uint32_t off = (uint32_t)(((t0 + kk) % P) * D + 16 * seg);
      r.k[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + (uint64_t)(uint32_t)pg.k[j] * page_stride + off));
    }
  }
#pragma unroll
  for (int j = 0; j < ChunkRegs<D>::VPT; ++j) {
    const int e = tid + j * kThreads;
    if (e < D * 4) {
      const int d = e >> 2;
      const int tv = t0 + 16 * (e & 3);
      if constexpr (P >= 16) {
        r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            vbase + (uint64_t)(uint32_t)pg.v[j][0] * page_stride + (uint32_t)(d * P + tv % P)));
      } else {
#pragma unroll
        for (int pc = 0; pc < ChunkPages<D, P>::NV; ++pc) {
          const uint8_t* q = vbase + (uint64_t)(uint32_t)pg.v[j][pc] * page_stride + (uint32_t)(d * P);
          if constexpr (P == 8) {
            u32x2 w = *reinterpret_cast<const u32x2*>(q);
            r.v[j][2 * pc] = w[0];
            r.v[j][2 * pc + 1] = w[1];
          } else {
            r.v[j][pc] = *reinterpret_cast<const uint32_t*>(q);
          }
        }
      }
    }
  }
}

// Decode the thread's bytes to fp16 and store them in LDS buffer `buf`. Keys at
// or past the sequence end are stored as zeros (their slots may hold poison).
template <int D>
__device__ __forceinline__ void chunk_store(ChunkLds<D>& s, int buf, const ChunkRegs<D>& r, int tid, int t0,
                                            int L) {
  constexpr int KSEG = D / 16;
#pragma unroll
  for (int j = 0; j < ChunkRegs<D>::KPT; ++j) {
    const int e = tid + j * kThreads;
    if (e < kTile * KSEG) {
      const int kk = e / KSEG;
      const int seg = e % KSEG;
      f16x8 a = e4m3x8_to_f16(r.k[j][0], r.k[j][1]);
      f16x8 b = e4m3x8_to_f16(r.k[j][2], r.k[j][3]);
      // key kk is MFMA row m = 4*(kk/16) + kk%4 of M-tile t = (kk/4)%4; storing it
      // at LDS row 16t + m makes each QK operand read 16 consecutive rows
      const int row = 16 * ((kk >> 2) & 3) + 4 * (kk >> 4) + (kk & 3);
      *reinterpret_cast<f16x8*>(&s.k[buf][row][swz(2 * seg, row)]) = a;
      *reinterpret_cast<f16x8*>(&s.k[buf][row][swz(2 * seg + 1, row)]) = b;
    }
  }
#pragma unroll
  for (int j = 0; j < ChunkRegs<D>::VPT; ++j) {
    const int e = tid + j * kThreads;
    if (e < D * 4) {
      const int d = e >> 2;
      const int kseg = e & 3;
      u32x4 w = r.v[j];
      // only the tiles reaching past the sequence end need the per-key mask; the
      // test is uniform over the workgroup, so other tiles skip it entirely
      if (t0 + kTile > L) {
        const int c = L - (t0 + 16 * kseg);  // valid keys among the 16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ci = c - 4 * i;
          w[i] &= ci >= 4 ? 0xFFFFFFFFu : (ci <= 0 ? 0u : ((1u << (8 * ci)) - 1u));
        }
      }
      f16x8 a = e4m3x8_to_f16(w[0], w[1]);
      f16x8 b = e4m3x8_to_f16(w[2], w[3]);
      *reinterpret_cast<f16x8*>(&s.v[buf][d][swz(kseg, d)]) = a;      // keys 16 kseg + 0..7: chunk kseg
      *reinterpret_cast<f16x8*>(&s.v[buf][d][swz(4 + kseg, d)]) = b;  // keys 16 kseg + 8..15: chunk 4 + kseg
    }
  }
}

// S^T = K Q^T of one tile for this wavefront's rows (raw dot products).
template <int D>
__device__ __forceinline__ void chunk_qk(const ChunkLds<D>& sm, int buf, int n, int g,
                                         const f16x8 (&qb)[kNB][D / 32], f32x4 (&sc)[4][kNB]) {
  constexpr int NC = D / 32;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const _Float16* krow = &sm.k[buf][16 * t + n][0];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // dims 32c + 8g .. +7 (the Q operand holds the same dims)
      const f16x8 ka = *reinterpret_cast<const f16x8*>(krow + swz(4 * c + g, n));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        sc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            ka, qb[nb][c], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[t][nb], 0, 0, 0);
    }
  }
}

// Online softmax of one tile (log2 units; the positive scale is applied to
// the raw max and folded into the exponent's FMA). A row keeps a reference
// maximum m_ref for its probabilities and moves it (rescaling o and l) only
// when some row's maximum grows more than kLazy above its reference: the
// probabilities are then at most 2^kLazy, which fp16 and the fp32 sums hold as
// well as values below 1, and after the first tiles the rescale almost never
// runs. The new reference is chosen without a branch, so the maxima and the
// probabilities are straight-line code the scheduler can interleave with the
// next tile's QK products; only the rescale multiplies sit behind a
// (wave-uniform, rare) branch. m_max tracks the true maximum; the state is
// brought to it at the end. MASKED selects out keys at or past a row's limit.
constexpr float kLazy = 8.0f;

template <int D, bool MASKED>
__device__ __forceinline__ void chunk_softmax(f32x4 (&sc)[4][kNB], int t0, int g, const int (&lim)[kNB],
                                              float score_scale, float (&m_ref)[kNB], float (&m_max)[kNB],
                                              f32x4 (&lacc)[kNB], f32x4 (&o)[kNB][D / 16],
                                              u32x4 (&pk)[kNB][2]) {
  constexpr int NBLK = D / 16;
  float alpha[kNB];
  bool moved[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if constexpr (MASKED) {
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
    m_max[nb] = fmaxf(m_max[nb], wave_max_groups(tmax) * score_scale);
    moved[nb] = __builtin_amdgcn_ballot_w64(m_max[nb] > m_ref[nb] + kLazy) != 0;
    const float m_new = moved[nb] ? m_max[nb] : m_ref[nb];
    alpha[nb] = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
    m_ref[nb] = m_new;
    const float nref = (m_new == -INFINITY) ? 0.0f : -m_new;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 2 * u + (j >> 1);
        const int i = 2 * (j & 1);
        f32x2 pp;
        pp[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][nb][i], score_scale, nref));
        pp[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][nb][i + 1], score_scale, nref));
        pk[nb][u][j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, f16x2));
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (moved[nb]) {
      lacc[nb] *= alpha[nb];
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) o[nb][blk] *= alpha[nb];
    }
  }
}

// O^T += V^T P^T and l += 1^T P^T of one tile.
template <int D>
__device__ __forceinline__ void chunk_pv(const ChunkLds<D>& sm, int buf, int n, int g,
                                         const u32x4 (&pk)[kNB][2], f32x4 (&lacc)[kNB],
                                         f32x4 (&o)[kNB][D / 16]) {
  constexpr int NBLK = D / 16;
  const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f16x8 va = *reinterpret_cast<const f16x8*>(&sm.v[buf][16 * blk + n][swz(4 * u + g, n)]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        o[nb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, __builtin_bit_cast(f16x8, pk[nb][u]),
                                                           o[nb][blk], 0, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      lacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, __builtin_bit_cast(f16x8, pk[nb][u]),
                                                       lacc[nb], 0, 0, 0);
}

template <int D, int P>
__global__ __launch_bounds__(kThreads, 1) void attn_chunk_kernel(const AttnArgs a) {
  constexpr int NC = D / 32;
  constexpr int NBLK = D / 16;
  __shared__ __attribute__((aligned(16))) ChunkLds<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.z;

  // ---- XCD-aware (query tile, kv-head) assignment
  const int nx = gridDim.x;
  const int total = nx * a.n_kv_heads;
  int lin = blockIdx.x + nx * blockIdx.y;
  if (total % kXcds == 0) {
    const int per = total / kXcds;
    lin = (lin % kXcds) * per + lin / kXcds;
  }
  const int qt = lin % nx;
  const int kvh = lin / nx;

  const int L = a.seq_lens[b];
  const int q0 = a.cu_q_lens[b];
  const int T = min(a.cu_q_lens[b + 1] - q0, a.max_q_len);
  const int G = a.group;
  const int nrows = T * G;
  const int row0 = qt * kRows;
  if (row0 >= nrows) return;  // whole workgroup exits together
  const int row_end = min(row0 + kRows, nrows);
  // keys visible to the workgroup's last row
  const int n_keys = min(L, L - T + (row_end - 1) / G + 1);
  const int ntiles = n_keys > 0 ? (n_keys + kTile - 1) / kTile : 0;

  // ---- this wavefront's 32 rows: Q operand and causal limits
  f16x8 qb[kNB][NC];
  int lim[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int rr = row0 + wave * (kNB * 16) + nb * 16 + n;
    if (rr < nrows) {
      const int i = rr / G;
      const int h = kvh * G + rr % G;
      const uint16_t* qp = a.q + ((int64_t)(q0 + i) * a.n_q_heads + h) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NC; ++c) qb[nb][c] = *reinterpret_cast<const f16x8*>(qp + 32 * c);
      lim[nb] = L - T + i + 1;
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) qb[nb][c] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      lim[nb] = 0;
    }
  }
  // smallest limit among the wavefront's rows: tiles below it need no mask
  int wave_lim;
  {
    const int first = row0 + wave * (kNB * 16);
    wave_lim = first < nrows ? L - T + first / G + 1 : 0;
  }

  float m_ref[kNB], m_max[kNB];
  f32x4 lacc[kNB];  // row sums of P, accumulated on the matrix core (A = ones)
  f32x4 o[kNB][NBLK];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m_ref[nb] = -INFINITY;
    m_max[nb] = -INFINITY;
    lacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) o[nb][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint32_t page_stride = (uint32_t)a.n_kv_heads * P * D;  // < 2^32: n_kv_heads <= 65535
  const uint8_t* kbase = a.k_cache + (int64_t)kvh * P * D;
  const uint8_t* vbase = a.v_cache + (int64_t)kvh * P * D;
  const int32_t* btrow = a.block_table + (int64_t)b * a.max_pages;
  const int last = L > 0 ? (L - 1) / P : 0;

  // ---- software pipeline over tiles: the QK products of tile it+1 are
  // issued next to the softmax of tile it, so the matrix cores have work
  // while the vector units run the softmax; the bytes of tile it+2 are in
  // flight meanwhile and the page ids of tile it+3 behind them
  ChunkRegs<D> regs;
  ChunkPages<D, P> pg;
  if (ntiles > 0) {
    chunk_pages<D, P>(pg, tid, 0, last, btrow);
    chunk_load<D, P>(regs, pg, tid, 0, kbase, vbase, page_stride);
    if (ntiles > 1) chunk_pages<D, P>(pg, tid, kTile, last, btrow);
    chunk_store<D>(sm, 0, regs, tid, 0, L);
  }
  if (ntiles > 1) {
    chunk_load<D, P>(regs, pg, tid, kTile, kbase, vbase, page_stride);
    if (ntiles > 2) chunk_pages<D, P>(pg, tid, 2 * kTile, last, btrow);
    chunk_store<D>(sm, 1, regs, tid, kTile, L);
  }
  // Q must have arrived before the loop: otherwise the waits for it that the
  // compiler places at its first use inside the loop would, on every later
  // iteration, also wait for the tile loads in flight
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int c = 0; c < NC; ++c) __asm__ volatile("" ::"v"(qb[nb][c]));
  __syncthreads();
  f32x4 sa[4][kNB], sb[4][kNB];
  u32x4 pk[kNB][2];
  if (ntiles > 0) chunk_qk<D>(sm, 0, n, g, qb, sa);
  int buf = 0;  // buffer of tile it
  // Loop body without data-dependent branches in the common case: the loads
  // of tiles t+2 / page ids of t+3, the next tile's QK and the stores run even
  // past the last tile (clamped pages, buffers no one reads afterwards), so the
  // QK products and the softmax form one block the scheduler can interleave.
  auto body = [&](auto masked_tag, int t, f32x4 (&cur)[4][kNB], f32x4 (&nxt)[4][kNB]) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf1 = buf == 2 ? 0 : buf + 1;
    const int buf2 = buf1 == 2 ? 0 : buf1 + 1;
    chunk_load<D, P>(regs, pg, tid, (t + 2) * kTile, kbase, vbase, page_stride);
    chunk_pages<D, P>(pg, tid, (t + 3) * kTile, last, btrow);
    // The per-tile barrier keeps every wavefront on the same tile. The two
    // wavefronts that share a SIMD (w and w + 4) take that tile's steps in
    // opposite orders, matrix core first against vector ALU first, so the
    // SIMD has one wavefront in each kind of work more of the time. Each
    // wavefront's own arithmetic is the same in both orders.
    if (wave < kWaves / 2) {
      chunk_qk<D>(sm, buf1, n, g, qb, nxt);
      chunk_softmax<D, MASKED>(cur, t * kTile, g, lim, a.score_scale, m_ref, m_max, lacc, o, pk);
      chunk_pv<D>(sm, buf, n, g, pk, lacc, o);
      chunk_store<D>(sm, buf2, regs, tid, (t + 2) * kTile, L);
    } else {
      chunk_softmax<D, MASKED>(cur, t * kTile, g, lim, a.score_scale, m_ref, m_max, lacc, o, pk);
      chunk_qk<D>(sm, buf1, n, g, qb, nxt);
      chunk_store<D>(sm, buf2, regs, tid, (t + 2) * kTile, L);
      chunk_pv<D>(sm, buf, n, g, pk, lacc, o);
    }
    __syncthreads();
    buf = buf1;
  };
  for (int it = 0; it < ntiles; it += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t = it + half;
      if (t < ntiles) {
        f32x4 (&cur)[4][kNB] = half == 0 ? sa : sb;
        f32x4 (&nxt)[4][kNB] = half == 0 ? sb : sa;
        if (t * kTile + kTile > wave_lim)
          body(std::true_type{}, t, cur, nxt);
        else
          body(std::false_type{}, t, cur, nxt);
      }
    }
  }
  // bring the state to the true row maxima
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const float fac = (m_max[nb] == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[nb] - m_max[nb]);
    lacc[nb] *= fac;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) o[nb][blk] *= fac;
  }

  // ---- normalise and write fp16 rows (lane holds dims 16*blk + 4g + i of row n)
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const float lrow = lacc[nb][0];
    const int rr = row0 + wave * (kNB * 16) + nb * 16 + n;
    if (rr >= nrows) continue;
    const int i = rr / G;
    const int h = kvh * G + rr % G;
    const float f = lrow > 0.0f ? a.v_scale / lrow : 0.0f;
    uint16_t* dst = a.out + ((int64_t)(q0 + i) * a.n_q_heads + h) * D + 4 * g;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const _Float16 h0 = (_Float16)(o[nb][blk][0] * f);
      const _Float16 h1 = (_Float16)(o[nb][blk][1] * f);
      const _Float16 h2 = (_Float16)(o[nb][blk][2] * f);
      const _Float16 h3 = (_Float16)(o[nb][blk][3] * f);
      const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
      *reinterpret_cast<u32x2*>(dst + 16 * blk) = u32x2{w0, w1};
    }
  }
}

template <int D, int P>
hipError_t launch_p(const AttnArgs& a, hipStream_t stream) {
  const int rows = a.max_q_len * a.group;
  dim3 grid((unsigned)((rows + kRows - 1) / kRows), (unsigned)a.n_kv_heads, (unsigned)a.batch);
  attn_chunk_kernel<D, P><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  switch (a.page_size) {
    case 4: return launch_p<D, 4>(a, stream);
    case 8: return launch_p<D, 8>(a, stream);
    case 16: return launch_p<D, 16>(a, stream);
    case 32: return launch_p<D, 32>(a, stream);
    case 64: return launch_p<D, 64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

void attn_chunk_kernel_name(const AttnArgs& a, char* buf, size_t n) {
  snprintf(buf, n, "attn_chunk_kernel<%d,%d>", a.head_dim, a.page_size);
}

hipError_t launch_attn_chunk(const AttnArgs& a, hipStream_t stream) {
  if (a.out == nullptr || a.cu_q_lens == nullptr) return hipErrorInvalidValue;
  if (a.head_dim == 128) return launch_d<128>(a, stream);
  if (a.head_dim == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvfp8
