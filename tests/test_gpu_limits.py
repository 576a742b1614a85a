"""GPU parity at the largest supported arguments: 256 splits (decode, verify
and the standalone reduce), 32 verify rows per kv-head reached with a group of
one (32 query tokens) and with a group of 32 (one token), page size 64 with
head_dim 64. Same bars as the other parity tests: cache bytes bit-exact,
attention within |gpu - ref| <= 2e-3 + 1e-2 |ref|, workspaces NaN-filled."""
import numpy as np
import pytest
import torch

from oracle import paged_attention, split_partials, split_reduce
from synth import make_batch
from tests.gpu_common import DeviceBatch, assert_close_attn, dev, oracle_caches, oracle_scales

pytestmark = pytest.mark.gpu

MAX_SPLITS = 256


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def _ws(K, rows, bt, S):
    if S == 1:
        return None
    ws = K.workspace(rows, bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, rows, bt.n_q_heads, bt.head_dim, S)
    return ws


def _setup(bt):
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    db.k_cache.copy_(torch.from_numpy(kc))
    db.v_cache.copy_(torch.from_numpy(vc))
    return db, sc, kc, vc, np.float32(1.0 / np.sqrt(bt.head_dim))


def test_decode_at_256_splits(K):
    """The longest sequence fills all 256 splits (64 keys each, the last one
    short); the others use a handful and leave the rest empty."""
    bt = make_batch([MAX_SPLITS * 64 - 23, 700, 1], [1, 1, 1], 8, 2, 128, 16, seed=301)
    db, sc, kc, vc, sm = _setup(bt)
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                   float(sc[1]), float(sm), num_splits=MAX_SPLITS,
                                   workspace=_ws(K, bt.batch, bt, MAX_SPLITS))
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out.cpu().numpy(), ref, "decode S=256")


def test_verify_at_256_splits(K):
    bt = make_batch([MAX_SPLITS * 64 + 5, 40, 4], [4, 2, 4], 16, 4, 128, 16, seed=302)
    db, sc, kc, vc, sm = _setup(bt)
    out = K.paged_attn_e4m3_verify(db.q, db.cu_q, 4, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                   float(sc[0]), float(sc[1]), float(sm), num_splits=MAX_SPLITS,
                                   workspace=_ws(K, bt.total_q, bt, MAX_SPLITS))
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out.cpu().numpy(), ref, "verify S=256")


def test_reduce_of_oracle_partials_at_256_splits(K):
    bt = make_batch([20000, 3000], [1, 1], 8, 2, 64, 16, seed=303)
    _, sc = oracle_scales(bt)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    sm = np.float32(0.125)
    ro, rm, rl = split_partials(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm,
                                MAX_SPLITS, granule=64)
    o32, m32, l32 = ro.astype(np.float32), rm.astype(np.float32), rl.astype(np.float32)
    assert np.isneginf(m32[1]).any()  # the short sequence leaves splits empty
    ref, ref_lse = split_reduce(o32, m32, l32)
    out, lse = K.split_reduce_fp32(dev(o32), dev(m32), dev(l32), with_lse=True)
    assert_close_attn(out.cpu().numpy(), ref, "reduce S=256")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("S", [1, 4])
def test_verify_32_query_tokens_group_1(K, S):
    """32 rows per kv-head from 32 query tokens of one head each (no GQA)."""
    bt = make_batch([300, 33, 32], [32, 17, 32], 4, 4, 128, 16, seed=304)
    db, sc, kc, vc, sm = _setup(bt)
    out = K.paged_attn_e4m3_verify(db.q, db.cu_q, 32, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                   float(sc[0]), float(sc[1]), float(sm), num_splits=S,
                                   workspace=_ws(K, bt.total_q, bt, S))
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out.cpu().numpy(), ref, f"verify q32 g1 S={S}")


@pytest.mark.parametrize("S", [1, 3])
def test_group_32_head_dim_64_page_64(K, S):
    """The widest group (32 query heads on one kv-head) at head_dim 64 and the
    largest page, decode and one-token verify."""
    bt = make_batch([1000, 65, 64, 1], [1, 1, 1, 1], 32, 1, 64, 64, seed=305)
    db, sc, kc, vc, sm = _setup(bt)
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                   float(sc[1]), float(sm), num_splits=S, workspace=_ws(K, bt.batch, bt, S))
    assert_close_attn(out.cpu().numpy(), ref, f"decode g32 S={S}")
    out = K.paged_attn_e4m3_verify(db.q, db.cu_q, 1, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                   float(sc[0]), float(sc[1]), float(sm), num_splits=S,
                                   workspace=_ws(K, bt.total_q, bt, S))
    assert_close_attn(out.cpu().numpy(), ref, f"verify g32 S={S}")
