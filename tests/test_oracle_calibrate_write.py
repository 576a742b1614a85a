"""Pins of the oracle's calibration and quantising write (CPU only)."""

import numpy as np
import pytest

from oracle import calibrate_amax, e4m3_decode, new_caches, quant_write, quantise, quotient_f32
from oracle.kv_write import POISON
from synth import make_batch, make_config
from tests import pins


def test_quotient_is_correctly_rounded():
    rng = np.random.default_rng(7)
    num = rng.standard_normal(1500).astype(np.float32) * np.float32(100)
    den = np.abs(rng.standard_normal(1500)).astype(np.float32) + np.float32(1e-3)
    got = quotient_f32(num, den)
    for n, d, g in zip(num, den, got):
        assert float(g) == pins.exact_round_f32(n, d)
    # amax / 448 for every positive finite fp16 value
    x = np.arange(1, 0x7C00, 37, dtype=np.uint16).view(np.float16).astype(np.float32)
    got = quotient_f32(x, np.float32(448.0))
    for n, g in zip(x[::7], got[::7]):
        assert float(g) == pins.exact_round_f32(n, 448.0)


def test_calibrate_brute_force_small():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 333)) * rng.uniform(0.1, 50, (5, 1))).astype(np.float16)
    amax, scale, status = calibrate_amax(x)
    assert status == 0
    for r in range(5):
        best = 0.0
        for val in x[r].tolist():
            if abs(val) > best:
                best = abs(val)
        assert float(amax[r]) == best
        assert float(scale[r]) == pins.exact_round_f32(best, 448.0)


def test_calibrate_scale_maps_amax_onto_e4m3_max():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((16, 4096)) * np.exp2(rng.integers(-8, 8, (16, 1)))).astype(np.float16)
    amax, scale, status = calibrate_amax(x)
    assert status == 0
    # the largest element quantises to +-448 and nothing exceeds it
    for r in range(16):
        codes = quantise(x[r], scale[r])
        assert (codes & 0x7F).max() == 0x7E
        assert np.isfinite(e4m3_decode(codes)).all()


def test_calibrate_errors():
    x = np.zeros((3, 8), dtype=np.float16)
    x[0] = 1.0
    x[2, 3] = np.inf
    amax, scale, status = calibrate_amax(x)
    assert status == 3  # non-finite wins over the zero tensor
    assert amax[0] == 1.0 and scale[0] == np.float32(1.0 / 448)
    assert amax[1] == 0.0 and scale[1] == 0.0
    assert np.isnan(amax[2]) and np.isnan(scale[2])
    x[2, 3] = 0.0
    _, _, status = calibrate_amax(x)
    assert status == 2
    x[2, 3] = np.nan
    amax, _, status = calibrate_amax(x)
    assert status == 3 and np.isnan(amax[2])


def _tiny_batch():
    return make_batch([9, 13, 4], [1, 2, 4], 4, 2, 16, 4, seed=11)


def test_quant_write_brute_force_slots():
    bt = _tiny_batch()
    ks, vs = np.float32(0.011), np.float32(0.0093)
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, ks, vs, kc, vc)
    P = bt.page_size
    rng = np.random.default_rng(0)
    for t in range(bt.k.shape[0]):
        page, off = divmod(int(bt.slot_mapping[t]), P)
        for h in range(bt.n_kv_heads):
            d = int(rng.integers(bt.head_dim))
            qk = np.float32(pins.exact_round_f32(float(bt.k[t, h, d]), float(ks)))
            qv = np.float32(pins.exact_round_f32(float(bt.v[t, h, d]), float(vs)))
            assert kc[page, h, off, d] == pins.brute_force_encode(np.array([qk]))[0]
            assert vc[page, h, d, off] == pins.brute_force_encode(np.array([qv]))[0]


def test_quant_write_layout_and_poison():
    bt = make_config(1)
    amax, scale, st = calibrate_amax(np.stack([bt.k.reshape(-1), bt.v.reshape(-1)]))
    assert st == 0
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, scale[0], scale[1], kc, vc)
    P = bt.page_size
    written = np.zeros((bt.num_pages, P), dtype=bool)
    written.reshape(-1)[bt.slot_mapping] = True
    # unwritten slots (spare pages, tail of last pages) keep the poison code
    assert (kc.transpose(0, 2, 1, 3)[~written] == POISON).all()
    assert (vc.transpose(0, 3, 1, 2)[~written] == POISON).all()
    # written slots decode to within half an E4M3 step of the input
    pages, offs = bt.slot_mapping // P, bt.slot_mapping % P
    kd = e4m3_decode(kc[pages, :, offs, :]) * float(scale[0])
    vd = e4m3_decode(vc[pages, :, :, offs]) * float(scale[1])
    for dec, src, sc in ((kd, bt.k, scale[0]), (vd, bt.v, scale[1])):
        err = np.abs(dec - src.astype(np.float64))
        bound = np.maximum(np.abs(src.astype(np.float64)) * 2.0 ** -4, 2.0 ** -10 * float(sc)) * 1.0001
        assert (err <= bound).all()


def test_quant_write_skips_padding_slots():
    bt = _tiny_batch()
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    slots = bt.slot_mapping.copy()
    slots[::2] = -1
    slots[1] = bt.num_pages * bt.page_size  # one past the end: skipped too
    quant_write(bt.k, bt.v, slots, 0.01, 0.01, kc, vc)
    n_written = ((kc != POISON).any(axis=3)).sum()
    expect = sum(1 for s in slots if 0 <= s < bt.num_pages * bt.page_size) * bt.n_kv_heads
    # a written token can legitimately encode to the poison code only for NaN input, which never happens here
    assert n_written == expect
