"""Randomised split plans on the GPU against the fp64 oracle: ragged batches
(1 to 129 sequences, a few long ones, zero-length sequences in verify), split
counts 1 to 40, head_dim 64/128, page sizes 4 to 64, GQA groups 1 to 16, for
the E4M3 kernel and its fp16-cache twin, each within the attention tolerance.
The workspace is NaN-filled, so any partial the reduce uses without it having
been written shows up. Seeded: every case is reproducible. The suite runs 12
seeds; KVFP8_RANDOM_PLAN_SEEDS=N runs seeds 0 .. N-1 for a wider sample."""
import os

import numpy as np
import pytest
import torch

from oracle import paged_attention, paged_attention_f16
from synth import make_batch
from synth.workloads import f16_caches
from tests.gpu_common import DeviceBatch, assert_close_attn, dev, oracle_caches, oracle_scales

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def _draw(seed):
    rng = np.random.default_rng(9000 + seed)
    verify = seed % 2 == 1
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([4, 8, 16, 32, 64]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 4, 8, 16]))
    B = int(rng.integers(1, 130))
    lens = rng.integers(1, 400, B)
    long = rng.random(B) < 0.08
    lens[long] = rng.integers(1000, 3000, int(long.sum()))
    if verify:
        q = rng.integers(1, 5, B).clip(1, max(1, 32 // G))
        q = np.minimum(q, lens)
        empty = rng.random(B) < 0.05
        lens[empty], q[empty] = 0, 0
    else:
        q = np.ones(B, dtype=np.int64)
    S = int(rng.integers(1, 41))
    bt = make_batch(lens.tolist(), q.tolist(), Hkv * G, Hkv, D, P, seed=9500 + seed)
    return bt, S, verify


def _ws(K, rows, bt, S):
    if S == 1:
        return None
    ws = K.workspace(max(rows, 1), bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, max(rows, 1), bt.n_q_heads, bt.head_dim, S)
    return ws


N_SEEDS = int(os.environ.get("KVFP8_RANDOM_PLAN_SEEDS", "12"))


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_random_plan_e4m3_and_f16(K, seed):
    bt, S, verify = _draw(seed)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    rows = bt.total_q
    print(f"seed {seed}: batch {bt.batch} verify {verify} D {bt.head_dim} P {bt.page_size} Hkv {bt.n_kv_heads} "
          f"G {bt.n_q_heads // bt.n_kv_heads} S {S} keys {int(bt.seq_lens.sum())}", flush=True)
    # E4M3: cache written by the library, oracle over its own quantised cache
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    # the generated tables meet the attention calls' device-side contract
    K.kvfp8_check_paged_args(db.block_table, db.seq_lens, bt.page_size, bt.num_pages,
                             db.cu_q if verify else None, bt.total_q, int(bt.q_lens.max()))
    K.kv_quant_write(db.k, db.v, db.slots, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    assert np.array_equal(db.k_cache.cpu().numpy(), kc) and np.array_equal(db.v_cache.cpu().numpy(), vc)
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    if verify:
        out = K.paged_attn_e4m3_verify(db.q, db.cu_q, int(bt.q_lens.max()), db.k_cache, db.v_cache, db.block_table,
                                       db.seq_lens, float(sc[0]), float(sc[1]), float(sm), num_splits=S,
                                       workspace=_ws(K, rows, bt, S))
    else:
        out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                       float(sc[1]), float(sm), num_splits=S, workspace=_ws(K, rows, bt, S))
    assert_close_attn(out.cpu().numpy(), ref, f"e4m3 seed {seed}")
    # fp16 twin
    kf, vf = f16_caches(bt)
    ref16, _ = paged_attention_f16(bt.q, kf, vf, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    if verify:
        out16 = K.paged_attn_f16_verify(db.q, db.cu_q, int(bt.q_lens.max()), dev(kf), dev(vf), db.block_table,
                                        db.seq_lens, float(sm), num_splits=S, workspace=_ws(K, rows, bt, S))
    else:
        out16 = K.paged_attn_f16_decode(db.q, dev(kf), dev(vf), db.block_table, db.seq_lens, float(sm),
                                        num_splits=S, workspace=_ws(K, rows, bt, S))
    assert_close_attn(out16.cpu().numpy(), ref16, f"f16 seed {seed}")


@pytest.mark.parametrize("S", [1, 3])
def test_zero_length_sequences_in_verify(K, S):
    """Sequences with no keys (and no query rows) beside ordinary ones, with
    and without a workspace: no load of theirs may touch the cache, and the
    other rows are unaffected."""
    bt = make_batch([0, 5, 0, 70, 0], [0, 2, 0, 3, 0], 16, 4, 128, 16, seed=9600 + S)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    out = K.paged_attn_e4m3_verify(db.q, db.cu_q, 3, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                   float(sc[0]), float(sc[1]), float(sm), num_splits=S,
                                   workspace=_ws(K, bt.total_q, bt, S))
    assert_close_attn(out.cpu().numpy(), ref, f"e4m3 S={S}")
    kf, vf = f16_caches(bt)
    ref16, _ = paged_attention_f16(bt.q, kf, vf, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    out16 = K.paged_attn_f16_verify(db.q, db.cu_q, 3, dev(kf), dev(vf), db.block_table, db.seq_lens, float(sm),
                                    num_splits=S, workspace=_ws(K, bt.total_q, bt, S))
    assert_close_attn(out16.cpu().numpy(), ref16, f"f16 S={S}")
