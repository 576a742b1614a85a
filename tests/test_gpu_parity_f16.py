"""GPU parity of the FP16-cache twin (paged_attn_f16_decode / _verify, through
the C ABI) against the fp64 oracle over fp16 caches, within the attention
tolerance |gpu - ref| <= 2e-3 + 1e-2 |ref|. Unused cache slots hold NaN and
the split workspace is NaN-filled, so a read of either shows up."""
import numpy as np
import pytest
import torch

from oracle import e4m3_decode, paged_attention_f16
from synth import make_batch, make_config
from synth.workloads import f16_caches
from tests.gpu_common import DeviceBatch, assert_close_attn, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def _sm(bt):
    return np.float32(1.0 / np.sqrt(bt.head_dim))


def _ws(K, rows, bt, S):
    if S == 1:
        return None
    ws = K.workspace(rows, bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, rows, bt.n_q_heads, bt.head_dim, S)
    return ws


DECODE_CASES = {
    "tiny_p4": lambda: make_config(1),
    "d128_p16_ragged": lambda: make_batch([1, 31, 32, 33, 63, 64, 65, 1000, 333], [1] * 9, 32, 4, 128, 16, seed=151),
    "d64_p8": lambda: make_batch([5, 130, 77], [1] * 3, 16, 4, 64, 8, seed=152),
    "d128_p64_g4": lambda: make_batch([700, 64, 129], [1] * 3, 16, 4, 128, 64, seed=153),
    "d128_p32_g16": lambda: make_batch([300, 41], [1] * 2, 32, 2, 128, 32, seed=154),
    "d64_p4_g32": lambda: make_batch([90, 17], [1] * 2, 32, 1, 64, 4, seed=155),
    "d128_b150_ragged": lambda: make_batch([1 + (37 * i) % 300 for i in range(150)], [1] * 150, 32, 4, 128, 16,
                                           seed=156),
}


@pytest.mark.parametrize("S", [1, 3, 8])
@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_f16_decode_matches_oracle(K, case, S):
    bt = DECODE_CASES[case]()
    kc, vc = f16_caches(bt)
    sm = _sm(bt)
    out = K.paged_attn_f16_decode(dev(bt.q), dev(kc), dev(vc), dev(bt.block_table), dev(bt.seq_lens), float(sm),
                                  num_splits=S, workspace=_ws(K, bt.batch, bt, S)).cpu().numpy()
    ref, _ = paged_attention_f16(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    assert_close_attn(out, ref, f"{case} S={S}")


VERIFY_CASES = {
    "mtp3_small": lambda: make_batch([1024, 70, 4, 300], [4] * 4, 32, 4, 128, 16, seed=161),
    "ragged_q": lambda: make_batch([50, 9, 200, 3], [1, 2, 4, 3], 32, 4, 128, 16, seed=162),
    "d64_p4": lambda: make_batch([100, 257], [4, 2], 8, 2, 64, 4, seed=163),
    "g4_q8": lambda: make_batch([129, 64], [8, 5], 16, 4, 64, 16, seed=164),
    "p64_q4": lambda: make_batch([700, 64, 129], [4, 2, 3], 32, 4, 128, 64, seed=165),
    "p32_g16_q2": lambda: make_batch([300, 41, 5], [2, 2, 1], 32, 2, 128, 32, seed=166),
}


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("case", list(VERIFY_CASES))
def test_f16_verify_matches_oracle(K, case, S):
    bt = VERIFY_CASES[case]()
    kc, vc = f16_caches(bt)
    sm = _sm(bt)
    out = K.paged_attn_f16_verify(dev(bt.q), dev(bt.cu_q_lens), int(bt.q_lens.max()), dev(kc), dev(vc),
                                  dev(bt.block_table), dev(bt.seq_lens), float(sm), num_splits=S,
                                  workspace=_ws(K, bt.total_q, bt, S)).cpu().numpy()
    ref, _ = paged_attention_f16(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    assert_close_attn(out, ref, f"{case} S={S}")


def test_f16_verify_rejects_long_chunks(K):
    bt = make_batch([100], [40], 8, 2, 64, 16, seed=167)  # 40 tokens x 4 heads = 160 rows per kv-head
    kc, vc = f16_caches(bt)
    with pytest.raises(K.KVFP8Error) as e:
        K.paged_attn_f16_verify(dev(bt.q), dev(bt.cu_q_lens), 40, dev(kc), dev(vc), dev(bt.block_table),
                                dev(bt.seq_lens), 0.125)
    assert e.value.status == K.UNSUPPORTED


@pytest.mark.parametrize("S", [1, 4])
def test_f16_arm_on_dequantised_values_agrees_with_e4m3_arm(K, S):
    """The two arms on the same values: the E4M3 kernel over calibrated codes,
    the FP16 kernel over those codes dequantised into fp16 with power-of-two
    scales (exact). Both against the one oracle result, within tolerance."""
    bt = make_batch([4096, 1000, 3000, 64], [1] * 4, 32, 4, 128, 16, seed=168)
    ks, vs = np.float32(2.0 ** -6), np.float32(2.0 ** -7)
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, float(ks), float(vs), db.k_cache, db.v_cache)
    kc, vc = db.k_cache.cpu().numpy(), db.v_cache.cpu().numpy()
    kf = (e4m3_decode(kc) * float(ks)).astype(np.float16)
    vf = (e4m3_decode(vc) * float(vs)).astype(np.float16)
    sm = _sm(bt)
    ref, _ = paged_attention_f16(bt.q, kf, vf, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    ws = _ws(K, bt.batch, bt, S)
    o8 = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(ks), float(vs),
                                  float(sm), num_splits=S, workspace=ws).cpu().numpy()
    o16 = K.paged_attn_f16_decode(db.q, dev(kf), dev(vf), db.block_table, db.seq_lens, float(sm), num_splits=S,
                                  workspace=_ws(K, bt.batch, bt, S)).cpu().numpy()
    assert_close_attn(o8, ref, f"e4m3 S={S}")
    assert_close_attn(o16, ref, f"f16 S={S}")


def test_f16_fullsize_4k_decode_sampled(K):
    """The 4k decode shape (32 x 4,096 keys, 32/4 heads, D 128, page 16) in the
    launch configuration the bench times, checked on sampled sequences."""
    bt = make_config(2)
    kc, vc = f16_caches(bt)
    sm = _sm(bt)
    S = K.default_splits(bt.batch, bt.n_kv_heads, 4096)
    out = K.paged_attn_f16_decode(dev(bt.q), dev(kc), dev(vc), dev(bt.block_table), dev(bt.seq_lens), float(sm),
                                  num_splits=S, workspace=_ws(K, bt.batch, bt, S)).cpu().numpy()
    rows = [0, 13, 31]
    ref, _ = paged_attention_f16(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm, rows=rows)
    assert_close_attn(out[rows], ref[rows], "4k f16 sampled")
