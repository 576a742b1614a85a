"""Decode launches in which every wavefront has at most one 64-key tile (one
round of 8-wavefront workgroups, pages of >= 16 keys, rows of at most 256
pages, splits of at most 512 keys): the split kernel then takes its short
start-up (first page ids from a block-table row loaded beside the work plan,
each wavefront storing its own copy of Q, no start-up barrier). Compared with
the fp64 oracle with equal lengths (the plan is the plain grid, so the
prefetched row is the one used), ragged lengths (the plan packs items
differently, so the page ids are loaded after the plan), a sequence without
keys, a group smaller than the 16-row block (padding rows), an MTP verify
small enough for one 16-row block, with a sequence that has no query tokens,
and the fused step that appends the new token in the same launch."""
import numpy as np
import pytest
import torch

from oracle import paged_attention
from synth import make_batch
from tests.gpu_common import DeviceBatch, assert_close_attn, dev, oracle_caches, oracle_scales

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def short_launch(bt, S, max_q=1):
    """The launch rule of the short start-up, written out for the test's shapes."""
    G = bt.n_q_heads // bt.n_kv_heads
    maxp = bt.block_table.shape[1]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (max_q * G <= 16 and bt.page_size >= 16 and S * bt.n_kv_heads * bt.batch <= cus and maxp <= 256
            and maxp * bt.page_size <= 512 * S)


def run(K, bt, S, lens=None, verify=False):
    _, sc = oracle_scales(bt)
    ks, vs = float(sc[0]), float(sc[1])
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, ks, vs, db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    lens = bt.seq_lens if lens is None else lens
    sm = float(np.float32(1.0 / np.sqrt(bt.head_dim)))
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, lens, bt.cu_q_lens, sc[0], sc[1], sm)
    ws = K.workspace(bt.total_q, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:
        K.poison_partials(ws, bt.total_q, bt.n_q_heads, bt.head_dim, S)
    if verify:
        out = K.paged_attn_e4m3_verify(db.q, db.cu_q, int(bt.q_lens.max()), db.k_cache, db.v_cache, db.block_table,
                                       dev(lens), ks, vs, sm, num_splits=S, workspace=ws)
    else:
        out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, dev(lens), ks, vs, sm,
                                       num_splits=S, workspace=ws)
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("P,S", [(16, 8), (32, 8), (64, 8)])
def test_equal_lengths_prefetched_row(K, P, S):
    """32 sequences of 4096 keys, one kv-head of 8 query heads (a tensor-parallel
    share): 256 workgroups, one tile per wavefront."""
    bt = make_batch([4096] * 32, [1] * 32, 8, 1, 128, P, seed=9800 + P, values=True)
    assert short_launch(bt, S)
    out, ref = run(K, bt, S)
    assert_close_attn(out, ref, f"equal lengths P={P} S={S}")


def test_equal_lengths_head_dim_64(K):
    """head_dim 64, 8 query heads per kv-head, 2 kv-heads: 16 sequences of
    2,048 keys at 4 splits (one tile per wavefront)."""
    bt = make_batch([2048] * 16, [1] * 16, 16, 2, 64, 16, seed=9805)
    S = 4
    assert short_launch(bt, S)
    out, ref = run(K, bt, S)
    assert_close_attn(out, ref, "equal lengths head_dim 64")


@pytest.mark.parametrize("seed,P", [(0, 16), (1, 16), (2, 16), (3, 32), (4, 64)])
def test_ragged_lengths_plan_packs_items(K, seed, P):
    rng = np.random.default_rng(9810 + seed)
    B = 24
    lens = [int(x) for x in rng.integers(1, 2049, B)]
    lens[0] = 2048  # the longest row sets the split size
    bt = make_batch(lens, [1] * B, 16, 2, 128, P, seed=9820 + seed)
    S = 4
    assert short_launch(bt, S)
    out, ref = run(K, bt, S)
    assert_close_attn(out, ref, f"ragged seed {seed}")


def test_sequence_without_keys_and_padding_rows(K):
    """head_dim 64, 4 query heads per kv-head (rows 4..15 of the block are
    padding), one sequence with no keys: its rows are zero."""
    bt = make_batch([900, 1, 1024, 333, 64, 700], [1] * 6, 16, 4, 64, 32, seed=9830)
    lens = bt.seq_lens.copy()
    lens[2] = 0
    for S in (2, 4):
        assert short_launch(bt, S)
        out, ref = run(K, bt, S, lens=lens)
        assert not out[2].astype(np.float64).any()
        assert_close_attn(out, ref, f"no keys S={S}")


def test_small_verify_one_block(K):
    """MTP verify with 2 query tokens per sequence and 8 query heads per
    kv-head (16 rows, one block) and a sequence with no query tokens."""
    bt = make_batch([700, 300, 1500, 64], [2, 0, 2, 1], 16, 2, 128, 16, seed=9840)
    S = 4
    assert short_launch(bt, S, max_q=2)
    out, ref = run(K, bt, S, verify=True)
    assert_close_attn(out, ref, "small verify")


def test_append_with_prefetched_row(K):
    """The fused step (the new token quantised into its slot in the same launch)
    on the tensor-parallel share: cache bytes bit-exact against the oracle and
    the output against the oracle over the whole context."""
    bt = make_batch([4096] * 32, [1] * 32, 8, 1, 128, 16, seed=9850)
    S = 8
    assert short_launch(bt, S)
    _, sc = oracle_scales(bt)
    ks, vs = float(sc[0]), float(sc[1])
    sm = float(np.float32(1.0 / np.sqrt(bt.head_dim)))
    db = DeviceBatch(bt)
    prior, new = dev(bt.prior_rows()), dev(bt.new_token_rows())
    K.kv_quant_write(db.k[prior].contiguous(), db.v[prior].contiguous(), db.slots[prior].contiguous(), ks, vs,
                     db.k_cache, db.v_cache)
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    out = K.paged_attn_e4m3_decode_append(db.q, db.k[new].contiguous(), db.v[new].contiguous(), db.k_cache,
                                          db.v_cache, db.block_table, db.seq_lens, ks, vs, sm, num_splits=S,
                                          workspace=ws).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out, ref, "append, prefetched row")
