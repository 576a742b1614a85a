"""Score patterns that drive the online softmax's rarely taken paths, on the
GPU against the fp64 oracle. With N(0,1) data the running maximum settles in
the first tile and the lazy rescale (taken when a row's maximum grows more
than 2^8 above its reference) almost never runs. Here the keys are built so
that one query head of every group scores key j as alpha * j (the maximum
climbs through every tile and split), as alpha * (L - j) (maximum in the first
tile), or flat with one spike in the middle; the other heads of the group see
the same keys at other angles. Decode (unsplit and split), MTP verify, a
prefill chunk and the fp16-cache twin are each compared with the oracle."""
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


def shaped_batch(lens, q_lens, pattern, seed, alpha=0.05):
    bt = make_batch(lens, q_lens, 32, 4, 128, 16, seed=seed)
    G = bt.n_q_heads // bt.n_kv_heads
    sm = 1.0 / np.sqrt(bt.head_dim)
    for b, L in enumerate(bt.seq_lens):
        L = int(L)
        row = int(bt.cu_q_lens[b])
        j = np.arange(L, dtype=np.float64)
        if pattern == "rising":
            s = alpha * j
        elif pattern == "falling":
            s = alpha * (L - j)
        else:  # flat with a spike in the middle
            s = np.full(L, 0.5)
            s[L // 2] = 40.0
        for h in range(bt.n_kv_heads):
            qr = bt.q[row, h * G].astype(np.float64)
            kk = (s / (sm * qr.dot(qr)))[:, None] * qr[None, :]
            noise = 0.05 * np.random.default_rng(seed + 31 * b + h).standard_normal(kk.shape)
            tok = int(bt.cu_seq_lens[b]) + np.arange(L)
            bt.k[tok, h, :] = (kk + noise).astype(np.float16)
    return bt, float(np.float32(sm))


def run_e4m3(K, bt, sm, S, max_q):
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    ws = K.workspace(bt.total_q, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if max_q == 1:
        out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                       float(sc[1]), sm, num_splits=S, workspace=ws)
    else:
        out = K.paged_attn_e4m3_verify(db.q, db.cu_q, max_q, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                       float(sc[0]), float(sc[1]), sm, num_splits=S, workspace=ws)
    return out.cpu().numpy(), ref, db


@pytest.mark.parametrize("pattern", ["rising", "falling", "spike"])
@pytest.mark.parametrize("S", [1, 3])
def test_decode_extremes(K, pattern, S):
    bt, sm = shaped_batch([4096, 1500, 700], [1, 1, 1], pattern, seed=9700)
    out, ref, _ = run_e4m3(K, bt, sm, S, 1)
    assert_close_attn(out, ref, f"decode {pattern} S={S}")


@pytest.mark.parametrize("pattern", ["rising", "falling", "spike"])
def test_verify_and_chunk_extremes(K, pattern):
    bt, sm = shaped_batch([3000, 900], [4, 4], pattern, seed=9710)
    out, ref, _ = run_e4m3(K, bt, sm, 4, 4)
    assert_close_attn(out, ref, f"verify {pattern}")
    bt, sm = shaped_batch([2600], [40], pattern, seed=9720)
    out, ref, _ = run_e4m3(K, bt, sm, 1, 40)
    assert_close_attn(out, ref, f"chunk {pattern}")


@pytest.mark.parametrize("pattern", ["rising", "spike"])
def test_f16_twin_extremes(K, pattern):
    bt, sm = shaped_batch([4096, 1500], [1, 1], pattern, seed=9730)
    kf, vf = f16_caches(bt)
    ref, _ = paged_attention_f16(bt.q, kf, vf, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    db = DeviceBatch(bt)
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, 3)
    out = K.paged_attn_f16_decode(db.q, dev(kf), dev(vf), db.block_table, db.seq_lens, sm, num_splits=3, workspace=ws)
    assert_close_attn(out.cpu().numpy(), ref, f"f16 decode {pattern}")
