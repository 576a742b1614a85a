"""The oracle still reproduces the stored values under tests/golden/ (written
by tests/golden/make_golden.py from the oracle alone). A change here means the
oracle's arithmetic changed and must be justified by the passage it follows."""

import os

import numpy as np

from oracle import calibrate_amax, e4m3_decode, new_caches, paged_attention, quant_write
from synth import make_config

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e4m3_code_table():
    vals = e4m3_decode(np.arange(256, dtype=np.uint8))
    for code, v in _rows("e4m3_codes.txt"):
        got = vals[int(code, 16)]
        if v == "nan":
            assert np.isnan(got)
        else:
            assert float.fromhex(v) == got


def test_tiny_attention():
    rows = _rows("tiny_attention.txt")
    bt = make_config(1)
    amax, scale, st = calibrate_amax(np.stack([bt.k.reshape(-1), bt.v.reshape(-1)]))
    assert [float.fromhex(x) for x in rows[0]] == [float(amax[0]), float(amax[1]),
                                                    float(scale[0]), float(scale[1])]
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, scale[0], scale[1], kc, vc)
    out, lse = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens,
                               scale[0], scale[1], np.float32(1.0 / np.sqrt(bt.head_dim)))
    for r, h, l, o0, o1, o2, o63 in rows[1:]:
        r, h = int(r), int(h)
        np.testing.assert_allclose([lse[r, h], out[r, h, 0], out[r, h, 1], out[r, h, 2], out[r, h, 63]],
                                   [float.fromhex(x) for x in (l, o0, o1, o2, o63)], rtol=1e-13, atol=1e-15)
