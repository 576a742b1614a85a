"""Pins of the oracle's attention over fp16 K/V caches (CPU only): the other
arm of the pages' comparison of cache formats."""

import numpy as np
import pytest

from oracle import e4m3_decode, new_caches, paged_attention, paged_attention_f16, quant_write
from synth import make_batch
from synth.workloads import f16_caches
from tests import pins


def _tokens(bt, kc, vc):
    P = bt.page_size
    pages, offs = bt.slot_mapping // P, bt.slot_mapping % P
    return kc[pages, :, offs, :], vc[pages, :, :, offs]


def test_brute_force_tiny():
    bt = make_batch([5, 11, 8], [1, 3, 8], 4, 2, 8, 4, seed=121)
    kc, vc = f16_caches(bt)
    sm = np.float32(0.3)
    out, _ = paged_attention_f16(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    for b in range(bt.batch):
        s0, s1 = bt.cu_seq_lens[b], bt.cu_seq_lens[b + 1]
        q0, q1 = bt.cu_q_lens[b], bt.cu_q_lens[b + 1]
        ref = pins.brute_force_attention(bt.q[q0:q1].astype(np.float64).tolist(),
                                         bt.k[s0:s1].astype(np.float64).tolist(),
                                         bt.v[s0:s1].astype(np.float64).tolist(), 1.0, 1.0, float(sm),
                                         int(q1 - q0), float)
        np.testing.assert_allclose(out[q0:q1], np.array(ref), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.25, 2.0 ** -7)])
def test_equals_e4m3_arm_on_the_same_values(scales):
    """An fp16 cache holding exactly the dequantised E4M3 values (power-of-two
    scales keep them exact in fp16) attends exactly as the E4M3 cache does."""
    ks, vs = np.float32(scales[0]), np.float32(scales[1])
    bt = make_batch([1, 63, 64, 65, 200], [1, 1, 4, 1, 3], 16, 4, 64, 16, seed=122)
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, ks, vs, kc, vc)
    kf = (e4m3_decode(kc) * float(ks)).astype(np.float16)
    vf = (e4m3_decode(vc) * float(vs)).astype(np.float16)
    assert np.array_equal(kf.astype(np.float64), e4m3_decode(kc) * float(ks), equal_nan=True)
    sm = np.float32(0.125)
    ref, ref_lse = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, ks, vs, sm)
    out, lse = paged_attention_f16(bt.q, kf, vf, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-15)


def test_single_key_returns_v():
    bt = make_batch([1, 1], [1, 1], 8, 2, 32, 4, seed=123)
    kc, vc = f16_caches(bt)
    out, _ = paged_attention_f16(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, np.float32(0.5))
    for b in range(2):
        for h in range(8):
            np.testing.assert_array_equal(out[b, h], bt.v[b, h // 4].astype(np.float64))


def test_unused_slots_are_invisible():
    """NaN poison in unused slots, or different data there, never reaches an output."""
    bt = make_batch([7, 30, 17], [1, 2, 1], 8, 2, 16, 8, seed=124)
    kc, vc = f16_caches(bt)
    kz, vz = f16_caches(bt, poison=np.float16(1000.0))
    sm = np.float32(0.25)
    a, _ = paged_attention_f16(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    b, _ = paged_attention_f16(bt.q, kz, vz, bt.block_table, bt.seq_lens, bt.cu_q_lens, sm)
    assert np.isfinite(a).all()
    np.testing.assert_array_equal(a, b)
    assert np.isnan(kc).any()  # the poison is really there
    kt, vt = _tokens(bt, kc, vc)
    np.testing.assert_array_equal(kt, bt.k)
    np.testing.assert_array_equal(vt, bt.v)
