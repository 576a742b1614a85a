"""Context-parallel decode emulated on one GPU: each sequence's pages are cut
into disjoint shares (the pages a rank would hold), the decode kernel produces
FP32 partials over each share alone (out = NULL), the partials are gathered
along the split axis as an all-gather would, and split_reduce_fp32 combines
them. The result must match the fp64 oracle over the whole context. A rank
may hold none of a sequence's pages (an empty share). Only the exchange itself
is left out (one GPU)."""
import numpy as np
import pytest
import torch

from oracle import paged_attention
from synth import make_batch, make_config
from tests.gpu_common import DeviceBatch, assert_close_attn, dev, oracle_caches, oracle_scales

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def shares(bt, ranks, rng):
    """Per rank: (block_table [B, max_pages], seq_lens [B]) holding a disjoint,
    page-aligned run of every sequence's logical pages (possibly empty)."""
    P = bt.page_size
    out = []
    cuts = []
    for b in range(bt.batch):
        npg = -(-int(bt.seq_lens[b]) // P)
        c = np.sort(rng.integers(0, npg + 1, ranks - 1))
        if b == 0 and ranks >= 3:
            c[1] = c[0]  # rank 1 holds none of sequence 0's pages
        cuts.append(np.concatenate([[0], c, [npg]]))
    for r in range(ranks):
        tab = np.zeros_like(bt.block_table)
        lens = np.zeros(bt.batch, np.int32)
        for b in range(bt.batch):
            p0, p1 = int(cuts[b][r]), int(cuts[b][r + 1])
            tab[b, :p1 - p0] = bt.block_table[b, p0:p1]
            lens[b] = max(0, min(int(bt.seq_lens[b]), p1 * P) - p0 * P)
        out.append((tab, lens))
    return out


def run_dcp(K, bt, db, ks, vs, sm, ranks, s_local, seed):
    rng = np.random.default_rng(seed)
    parts = []
    cut = shares(bt, ranks, rng)
    empty = sum(int((lens == 0).sum()) for _, lens in cut)
    for tab, lens in cut:
        ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, s_local)
        K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, s_local)
        K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, dev(tab), dev(lens), ks, vs, sm,
                                 num_splits=s_local, workspace=ws, partials_only=True)
        parts.append(K.workspace_views(ws, bt.batch, bt.n_q_heads, bt.head_dim, s_local))
    # the all-gather: partials of every rank side by side along the split axis
    o = torch.cat([p[0] for p in parts], dim=2).contiguous()
    m = torch.cat([p[1] for p in parts], dim=2).contiguous()
    l = torch.cat([p[2] for p in parts], dim=2).contiguous()
    return K.split_reduce_fp32(o, m, l), empty


@pytest.mark.parametrize("ranks,s_local", [(2, 2), (2, 3), (4, 2), (8, 2)])  # partials need num_splits > 1
def test_dcp_combine_tiny(K, ranks, s_local):
    bt = make_config(1)  # batch 2, contexts 100 and 257, page 4
    sm = float(np.float32(1.0 / 8.0))
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    out, empty = run_dcp(K, bt, db, float(sc[0]), float(sc[1]), sm, ranks, s_local, seed=61 + ranks * 7 + s_local)
    assert_close_attn(out.cpu().numpy(), ref, f"dcp ranks {ranks} S_local {s_local}")
    if ranks >= 3:
        assert empty > 0, "some rank must hold none of a sequence's pages"


@pytest.mark.parametrize("seed", range(3))
def test_dcp_combine_ragged(K, seed):
    rng = np.random.default_rng(8100 + seed)
    lens = [int(x) for x in rng.integers(1, 5000, 6)]
    bt = make_batch(lens, [1] * 6, 32, 4, 128, 16, seed=8200 + seed)
    sm = float(np.float32(1.0 / np.sqrt(128)))
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    out, _ = run_dcp(K, bt, db, float(sc[0]), float(sc[1]), sm, 2, 4, seed=8300 + seed)
    assert_close_attn(out.cpu().numpy(), ref, f"dcp ragged seed {seed}")


def verify_shares(bt, ranks, rng):
    """Page-aligned shares with every query token in the last one: cuts at or
    before page (L - q_len) // page_size."""
    P = bt.page_size
    cuts = []
    for b in range(bt.batch):
        L, T = int(bt.seq_lens[b]), int(bt.q_lens[b])
        npg = -(-L // P)
        c = np.sort(rng.integers(0, (L - T) // P + 1, ranks - 1))
        cuts.append(np.concatenate([[0], c, [npg]]))
    out = []
    for r in range(ranks):
        tab = np.zeros_like(bt.block_table)
        lens = np.zeros(bt.batch, np.int32)
        for b in range(bt.batch):
            p0, p1 = int(cuts[b][r]), int(cuts[b][r + 1])
            tab[b, :p1 - p0] = bt.block_table[b, p0:p1]
            lens[b] = max(0, min(int(bt.seq_lens[b]), p1 * P) - p0 * P)
        out.append((tab, lens))
    return out


@pytest.mark.parametrize("ranks,seed", [(2, 0), (3, 1), (4, 2)])
def test_dcp_combine_mtp_verify(K, ranks, seed):
    """MTP verify (4 query tokens, causal among them) over context shards: on a
    shard before the query tokens every row sees every key, so each query row
    runs as a decode row of its own over that shard's pages; the last shard
    holds the query tokens and runs the verify call with its local length (the
    causal positions are local positions). The gathered partials reduce to the
    oracle's verify output over the whole context."""
    rng = np.random.default_rng(8400 + seed)
    lens = [int(x) for x in rng.integers(300, 6000, 5)]
    bt = make_batch(lens, [4] * 5, 32, 4, 128, 16, seed=8500 + seed)
    sm = float(np.float32(1.0 / np.sqrt(128)))
    _, sc = oracle_scales(bt)
    ks, vs = float(sc[0]), float(sc[1])
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, ks, vs, db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    S = 2
    rows = bt.total_q
    row_seq = np.repeat(np.arange(bt.batch), bt.q_lens)  # the sequence of every query row
    parts = []
    cut = verify_shares(bt, ranks, rng)
    for r, (tab, lens_r) in enumerate(cut):
        ws = K.workspace(rows, bt.n_q_heads, bt.head_dim, S)
        K.poison_partials(ws, rows, bt.n_q_heads, bt.head_dim, S)
        if r < ranks - 1:  # every key of this shard precedes every query token
            K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, dev(tab[row_seq]), dev(lens_r[row_seq]), ks, vs,
                                     sm, num_splits=S, workspace=ws, partials_only=True)
        else:
            K.paged_attn_e4m3_verify(db.q, db.cu_q, int(bt.q_lens.max()), db.k_cache, db.v_cache, dev(tab),
                                     dev(lens_r), ks, vs, sm, num_splits=S, workspace=ws, partials_only=True)
        parts.append(K.workspace_views(ws, rows, bt.n_q_heads, bt.head_dim, S))
    o = torch.cat([p[0] for p in parts], dim=2).contiguous()
    m = torch.cat([p[1] for p in parts], dim=2).contiguous()
    l = torch.cat([p[2] for p in parts], dim=2).contiguous()
    out = K.split_reduce_fp32(o, m, l)
    assert_close_attn(out.cpu().numpy(), ref, f"dcp verify ranks {ranks}")
