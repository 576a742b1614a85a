"""The revision-bound scale file (host-only, CPU tests).

Both halves of the gate: what calibration produces is stored and read back bit
for bit, and the reader refuses every missing, foreign, incomplete or invalid
file with an error and no fallback (outputs untouched).
"""

import os

import numpy as np
import pytest

from fp8_quantised_paged_amd import kvfp8
from oracle import calibrate_amax

REV = "ckpt-0123abcd"


def _scales(n, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.uniform(1e-3, 2.0, n).astype(np.float32), rng.uniform(1e-3, 2.0, n).astype(np.float32))


def _status(fn, *args):
    try:
        fn(*args)
    except kvfp8.KVFP8Error as e:
        return e.status
    return kvfp8.OK


def test_round_trip_is_bit_exact(tmp_path):
    k, v = _scales(24)
    # the extremes of the accepted range and values with every mantissa bit set
    k[0], v[0] = np.float32(np.finfo(np.float32).tiny), np.float32(np.finfo(np.float32).max)
    k[1] = np.nextafter(np.float32(1.0), np.float32(2.0))
    path = str(tmp_path / "scales.txt")
    kvfp8.scale_overlay_write(path, REV, k, v)
    rk, rv = kvfp8.scale_overlay_read(path, REV, 24)
    assert np.array_equal(rk.view(np.uint32), k.view(np.uint32))
    assert np.array_equal(rv.view(np.uint32), v.view(np.uint32))
    assert not os.path.exists(path + ".tmp")


def test_calibrated_scales_survive_the_file(tmp_path):
    """The oracle's per-layer calibration (amax/448 over each layer's K and V
    draws) goes through the file unchanged."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((2 * 6, 4096)) * rng.uniform(0.1, 20.0, (12, 1))).astype(np.float16)
    _, scale, st = calibrate_amax(x)
    assert st == 0
    path = str(tmp_path / "scales.txt")
    kvfp8.scale_overlay_write(path, REV, scale[0::2], scale[1::2])
    rk, rv = kvfp8.scale_overlay_read(path, REV, 6)
    assert np.array_equal(rk.view(np.uint32), scale[0::2].view(np.uint32))
    assert np.array_equal(rv.view(np.uint32), scale[1::2].view(np.uint32))


@pytest.mark.parametrize("bad", [0.0, -1.0, float("inf"), float("nan"), 1e-40])
def test_writer_refuses_invalid_scales(tmp_path, bad):
    k, v = _scales(4)
    v[2] = bad
    path = str(tmp_path / "scales.txt")
    assert _status(kvfp8.scale_overlay_write, path, REV, k, v) == kvfp8.BAD_SCALE
    assert not os.path.exists(path)


def test_writer_refuses_bad_revision(tmp_path):
    k, v = _scales(2)
    for rev in ("", "has space", "tab\there", "x" * 300):
        assert _status(kvfp8.scale_overlay_write, str(tmp_path / "s.txt"), rev, k, v) == kvfp8.INVALID_ARG


def _good_text(n=3):
    k, v = _scales(n, seed=1)
    lines = ["kvfp8-scale-overlay 1", f"revision {REV}", f"layers {n}"]
    lines += [f"{i} {float(k[i]).hex()} {float(v[i]).hex()}" for i in range(n)]
    return lines


def _write(tmp_path, lines, name="s.txt"):
    p = tmp_path / name
    p.write_text("\n".join(lines) + "\n")
    return str(p)


def test_hand_written_file_reads(tmp_path):
    lines = _good_text(3)
    lines[3], lines[5] = lines[5], lines[3]  # records in any order
    k, v = kvfp8.scale_overlay_read(_write(tmp_path, lines), REV, 3)
    ek, ev = _scales(3, seed=1)
    assert np.array_equal(k, ek) and np.array_equal(v, ev)


def _mutations():
    g = _good_text(3)
    return {
        "missing revision": (g[:1] + g[2:], kvfp8.INVALID_ARG),
        "other revision": ([g[0], "revision ckpt-ffff"] + g[2:], kvfp8.INVALID_ARG),
        "bad magic": (["kvfp8-scale-overlay 2"] + g[1:], kvfp8.INVALID_ARG),
        "layer count": (g[:2] + ["layers 4"] + g[3:], kvfp8.INVALID_ARG),
        "missing layer": (g[:-1], kvfp8.INVALID_ARG),
        "duplicate layer": (g[:-1] + [g[-2]], kvfp8.INVALID_ARG),
        "layer out of range": (g[:-1] + ["3 0x1p+0 0x1p+0"], kvfp8.INVALID_ARG),
        "extra field": (g[:-1] + [g[-1] + " 1"], kvfp8.INVALID_ARG),
        "garbage scale": (g[:-1] + ["2 0x1p+0 one"], kvfp8.INVALID_ARG),
        "double space": (g[:-1] + ["2  0x1p+0 0x1p+0"], kvfp8.INVALID_ARG),
        "empty line": (g + [""], kvfp8.INVALID_ARG),
        "zero scale": (g[:-1] + ["2 0x0p+0 0x1p+0"], kvfp8.BAD_SCALE),
        "negative scale": (g[:-1] + ["2 -0x1p+0 0x1p+0"], kvfp8.BAD_SCALE),
        "nan scale": (g[:-1] + ["2 0x1p+0 nan"], kvfp8.BAD_SCALE),
        "inf scale": (g[:-1] + ["2 inf 0x1p+0"], kvfp8.BAD_SCALE),
        "subnormal scale": (g[:-1] + ["2 0x1p-140 0x1p+0"], kvfp8.BAD_SCALE),
        "overflowing scale": (g[:-1] + ["2 0x1p+200 0x1p+0"], kvfp8.BAD_SCALE),
    }


@pytest.mark.parametrize("case", list(_mutations()))
def test_reader_fails_closed(tmp_path, case):
    lines, status = _mutations()[case]
    path = _write(tmp_path, lines)
    k = np.full(3, 7.0, np.float32)
    v = np.full(3, 7.0, np.float32)
    got = kvfp8._lib.kvfp8_scale_overlay_read(path.encode(), REV.encode(), 3, k.ctypes.data, v.ctypes.data)
    assert got == status, kvfp8.last_error()
    assert kvfp8.last_error()
    assert (k == 7.0).all() and (v == 7.0).all()  # untouched: no partial or unit-scale fallback


def test_reader_missing_file_and_empty_file(tmp_path):
    assert _status(kvfp8.scale_overlay_read, str(tmp_path / "absent.txt"), REV, 3) == kvfp8.INVALID_ARG
    (tmp_path / "empty.txt").write_text("")
    assert _status(kvfp8.scale_overlay_read, str(tmp_path / "empty.txt"), REV, 3) == kvfp8.INVALID_ARG


def test_reader_refuses_bad_arguments(tmp_path):
    path = _write(tmp_path, _good_text(3))
    assert _status(kvfp8.scale_overlay_read, path, REV, 0) == kvfp8.INVALID_ARG
    assert _status(kvfp8.scale_overlay_read, path, "", 3) == kvfp8.INVALID_ARG
