"""Seeded synthetic paged-KV workloads.

Every array here is drawn from numpy's PCG64 generator with sub-streams
spawned from one seed, so the oracle and the HIP path consume identical
inputs. K, V and Q are fp16 draws of N(0, 1) (optionally with Student-t
outlier channels); physical pages are a seeded permutation so that the
block table is never the identity.

Layout conventions (shared vocabulary, no arithmetic of the method):

* positions of sequence b are 0 .. seq_lens[b]-1; the last q_lens[b] of them
  are the query tokens of this step;
* ``k``/``v`` hold the fp16 key/value of *every* position, sequence-major,
  shape [sum(seq_lens), n_kv_heads, head_dim];
* ``slot_mapping[t]`` is the cache slot (page * page_size + offset) of the
  t-th row of ``k``/``v``;
* ``block_table[b, i]`` is the physical page of logical page i of sequence b,
  and -1 past the sequence's last page.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

SEED_BASE = 20260000

CONFIG_NAMES = {
    1: "tiny_e4m3_paged_decode_b2_ctx100_257_h8kv2_d64_p4",
    2: "decode_b32_ctx4096_h32kv4_d128_p16",
    3: "mtp3_verify_b16_ctx1k_4k_8k_32k_q4_h32kv4_d128_p16",
    4: "long_b4_ctx262144_h32kv4_d128_p64_splits64_outliers",
    5: "mixed_24layers_8x8192_decode_plus_2048_chunk_over_30000",
}


@dataclass
class PagedBatch:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    seq_lens: np.ndarray  # int32 [B]
    q_lens: np.ndarray  # int32 [B]
    cu_q_lens: np.ndarray  # int32 [B+1]
    cu_seq_lens: np.ndarray  # int64 [B+1] row offsets of each sequence in k/v
    block_table: np.ndarray  # int32 [B, max_pages]
    num_pages: int
    slot_mapping: np.ndarray  # int64 [sum(seq_lens)]
    k: np.ndarray  # fp16 [sum(seq_lens), Hkv, D]
    v: np.ndarray  # fp16 [sum(seq_lens), Hkv, D]
    q: np.ndarray  # fp16 [sum(q_lens), Hq, D]
    calib_k: Optional[np.ndarray] = None  # fp16 [n_calib, Hkv, D]
    calib_v: Optional[np.ndarray] = None
    seed: int = 0
    outlier_channels_k: List[int] = field(default_factory=list)
    outlier_channels_v: List[int] = field(default_factory=list)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    def new_token_rows(self) -> np.ndarray:
        """Rows of k/v that are the query tokens of this step (the last
        q_lens[b] positions of every sequence)."""
        rows = []
        for b in range(self.batch):
            end = int(self.cu_seq_lens[b + 1])
            rows.append(np.arange(end - int(self.q_lens[b]), end))
        return np.concatenate(rows) if rows else np.zeros(0, np.int64)

    def prior_rows(self) -> np.ndarray:
        """Rows of k/v that precede this step's query tokens."""
        rows = []
        for b in range(self.batch):
            beg = int(self.cu_seq_lens[b])
            end = int(self.cu_seq_lens[b + 1])
            rows.append(np.arange(beg, end - int(self.q_lens[b])))
        return np.concatenate(rows) if rows else np.zeros(0, np.int64)


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def _with_outliers(x: np.ndarray, channels: Sequence[int], rng, df: float, scale: float) -> np.ndarray:
    """Replace the listed flattened (kv-head, dim) channels of x [n, Hkv, D]
    by scale * Student-t(df) draws, clamped to the finite fp16 range."""
    if len(channels) == 0:
        return x
    n, hkv, d = x.shape
    flat = x.reshape(n, hkv * d)
    t = rng.standard_t(df, size=(n, len(channels))) * scale
    t = np.clip(t, -65504.0, 65504.0)
    flat[:, np.asarray(channels)] = t.astype(np.float16)
    return flat.reshape(n, hkv, d)


def make_batch(
    seq_lens: Sequence[int],
    q_lens: Sequence[int],
    n_q_heads: int,
    n_kv_heads: int,
    head_dim: int,
    page_size: int,
    seed: int,
    name: str = "custom",
    calib_tokens: Optional[int] = None,
    outlier_frac: float = 0.0,
    outlier_df: float = 3.0,
    outlier_scale: float = 8.0,
    spare_pages: int = 3,
    values: bool = True,
) -> PagedBatch:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    assert seq_lens.shape == q_lens.shape
    assert np.all(q_lens >= 0) and np.all(q_lens <= seq_lens)
    B = seq_lens.shape[0]
    P = page_size
    ss = np.random.SeedSequence(seed)
    s_perm, s_k, s_v, s_q, s_cal, s_out = ss.spawn(6)

    pages_per_seq = (seq_lens.astype(np.int64) + P - 1) // P
    used = int(pages_per_seq.sum())
    num_pages = used + spare_pages
    perm = np.random.Generator(np.random.PCG64(s_perm)).permutation(num_pages).astype(np.int32)
    max_pages = int(max(1, pages_per_seq.max() if B else 1))
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    cu_seq = np.zeros(B + 1, dtype=np.int64)
    cu_seq[1:] = np.cumsum(seq_lens.astype(np.int64))
    slot_mapping = np.empty(int(cu_seq[-1]), dtype=np.int64)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        block_table[b, :n] = perm[off:off + n]
        off += n
        j = np.arange(int(seq_lens[b]), dtype=np.int64)
        slot_mapping[cu_seq[b]:cu_seq[b + 1]] = block_table[b, j // P].astype(np.int64) * P + j % P

    n_ch = n_kv_heads * head_dim
    n_out = int(round(outlier_frac * n_ch))
    rng_out = np.random.Generator(np.random.PCG64(s_out))
    out_k = sorted(rng_out.choice(n_ch, size=n_out, replace=False).tolist()) if n_out else []
    out_v = sorted(rng_out.choice(n_ch, size=n_out, replace=False).tolist()) if n_out else []

    total = int(cu_seq[-1])
    shape = (total, n_kv_heads, head_dim) if values else (0, n_kv_heads, head_dim)
    k = np.empty(shape, dtype=np.float16)
    v = np.empty(shape, dtype=np.float16)
    k_seq = s_k.spawn(B)
    v_seq = s_v.spawn(B)
    for b in (range(B) if values else ()):
        rk = np.random.Generator(np.random.PCG64(k_seq[b]))
        rv = np.random.Generator(np.random.PCG64(v_seq[b]))
        L = int(seq_lens[b])
        k[cu_seq[b]:cu_seq[b + 1]] = _with_outliers(
            _normal_f16(rk, (L, n_kv_heads, head_dim)), out_k, rk, outlier_df, outlier_scale)
        v[cu_seq[b]:cu_seq[b + 1]] = _with_outliers(
            _normal_f16(rv, (L, n_kv_heads, head_dim)), out_v, rv, outlier_df, outlier_scale)

    cu_q = np.zeros(B + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    rq = np.random.Generator(np.random.PCG64(s_q))
    q = _normal_f16(rq, (int(cu_q[-1]), n_q_heads, head_dim))

    calib_k = calib_v = None
    if calib_tokens and values:
        rc = np.random.Generator(np.random.PCG64(s_cal))
        calib_k = _with_outliers(_normal_f16(rc, (calib_tokens, n_kv_heads, head_dim)),
                                 out_k, rc, outlier_df, outlier_scale)
        calib_v = _with_outliers(_normal_f16(rc, (calib_tokens, n_kv_heads, head_dim)),
                                 out_v, rc, outlier_df, outlier_scale)

    return PagedBatch(
        name=name, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
        page_size=page_size, seq_lens=seq_lens, q_lens=q_lens, cu_q_lens=cu_q,
        cu_seq_lens=cu_seq, block_table=block_table, num_pages=num_pages,
        slot_mapping=slot_mapping, k=k, v=v, q=q, calib_k=calib_k, calib_v=calib_v,
        seed=seed, outlier_channels_k=out_k, outlier_channels_v=out_v,
    )


def mtp3_context_lengths(seed: int, batch: int = 16) -> np.ndarray:
    """Context lengths drawn uniformly from {1,024, 4,096, 8,192, 32,768}."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return rng.choice(np.array([1024, 4096, 8192, 32768]), size=batch).astype(np.int32)


def make_config(idx: int, layer: int = 0, seq_len_override: Optional[int] = None,
                values: bool = True, page_size_override: Optional[int] = None) -> PagedBatch:
    """The five named workloads. For the mixed workload (5) one layer's batch is
    returned: 8 decode sequences at 8,192 followed by one sequence holding a
    2,048-token chunk over a 30,000-token prior context."""
    seed = SEED_BASE + idx
    if idx == 1:
        return make_batch([100, 257], [1, 1], 8, 2, 64, 4, seed, name=CONFIG_NAMES[1], values=values)
    if idx == 2:
        L = seq_len_override or 4096
        return make_batch([L] * 32, [1] * 32, 32, 4, 128, page_size_override or 16, seed, name=CONFIG_NAMES[2],
                          calib_tokens=2048, values=values)
    if idx == 3:
        lens = mtp3_context_lengths(seed)
        return make_batch(lens, [4] * 16, 32, 4, 128, 16, seed, name=CONFIG_NAMES[3],
                          calib_tokens=2048, values=values)
    if idx == 4:
        L = seq_len_override or 262144
        return make_batch([L] * 4, [1] * 4, 32, 4, 128, 64, seed, name=CONFIG_NAMES[4],
                          calib_tokens=2048, outlier_frac=0.02, values=values)
    if idx == 5:
        return make_batch([8192] * 8 + [32048], [1] * 8 + [2048], 32, 4, 128, 16,
                          seed * 100 + layer, name=f"{CONFIG_NAMES[5]}_layer{layer}", values=values)
    raise ValueError(f"unknown config {idx}")


def make_mixed_calibration(n_layers: int = 24, tokens: int = 4096, n_kv_heads: int = 4,
                           head_dim: int = 128, seed: int = SEED_BASE + 5) -> np.ndarray:
    """Per-layer K and V calibration draws of the mixed workload, as fp16
    [2 * n_layers, tokens * n_kv_heads * head_dim]; row 2l is layer l's K, row
    2l+1 its V."""
    ss = np.random.SeedSequence([seed, 11]).spawn(2 * n_layers)
    out = np.empty((2 * n_layers, tokens * n_kv_heads * head_dim), dtype=np.float16)
    for i in range(2 * n_layers):
        out[i] = _normal_f16(np.random.Generator(np.random.PCG64(ss[i])), out.shape[1])
    return out


def f16_caches(bt: PagedBatch, poison=np.float16(np.nan)):
    """fp16 K and V caches of a batch in the paged layout (K [pages][Hkv][P][D],
    V [pages][Hkv][D][P]) with every token stored at its slot; unused slots hold
    `poison` (NaN by default). A plain layout scatter: it computes nothing."""
    P, D, H = bt.page_size, bt.head_dim, bt.n_kv_heads
    kc = np.full((bt.num_pages, H, P, D), poison, dtype=np.float16)
    vc = np.full((bt.num_pages, H, D, P), poison, dtype=np.float16)
    pages = bt.slot_mapping // P
    offs = bt.slot_mapping % P
    kc[pages, :, offs, :] = bt.k
    vc[pages, :, :, offs] = bt.v
    return kc, vc
