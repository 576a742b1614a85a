"""Helpers for GPU parity tests: move a seeded batch to the device, run the
library through its binding, and compare with the oracle on the host."""

import numpy as np
import torch

from oracle import calibrate_amax, new_caches, quant_write

ATOL = 2e-3
RTOL = 1e-2


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def assert_close_attn(gpu_f16: np.ndarray, ref: np.ndarray, what: str = "", strict: bool = False):
    """|gpu - ref| <= 2e-3 + 1e-2 * |ref| elementwise (fp16 output, fp32
    accumulation, against the fp64 oracle). With strict, the largest absolute
    error must also be at most 2e-3 outright: the literal bound, which an fp16
    output can meet wherever |ref| stays below 8 (half an fp16 ulp there is at
    most 2^-9), as in every N(0, 1) workload; the workload with Student-t outlier
    channels, where |ref| reaches tens, keeps the combined rule alone. Prints
    max-abs and max-rel (over |ref| > 1e-3) either way."""
    g = gpu_f16.astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    mabs, mrel = report(gpu_f16, ref)
    print(f"{what}: max abs {mabs:.3g} max rel {mrel:.3g} (|ref| > 1e-3) over {err.size} elements"
          f"{' [strict]' if strict else ''}")
    if strict:
        assert mabs <= ATOL, f"{what}: max abs err {mabs:.3g} above {ATOL} (strict bound)"
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; max abs "
                             f"err {err.max():.3g}; first {idx.tolist()} gpu {g[bad][:5]} ref {ref[bad][:5]}")


def report(gpu_f16, ref):
    g = gpu_f16.astype(np.float64)
    err = np.abs(g - ref)
    big = np.abs(ref) > 1e-3
    rel = (err[big] / np.abs(ref[big])).max() if big.any() else 0.0
    return float(err.max()), float(rel)


class DeviceBatch:
    """A seeded PagedBatch on the GPU with poison-filled caches."""

    def __init__(self, bt, poison=0x7F):
        self.bt = bt
        self.k = dev(bt.k)
        self.v = dev(bt.v)
        self.q = dev(bt.q)
        self.slots = dev(bt.slot_mapping)
        self.block_table = dev(bt.block_table)
        self.seq_lens = dev(bt.seq_lens)
        self.cu_q = dev(bt.cu_q_lens)
        P, D, H = bt.page_size, bt.head_dim, bt.n_kv_heads
        self.k_cache = torch.full((bt.num_pages, H, P, D), poison, dtype=torch.uint8, device="cuda")
        self.v_cache = torch.full((bt.num_pages, H, D, P), poison, dtype=torch.uint8, device="cuda")


def oracle_scales(bt):
    """Oracle K/V scales over the batch's calibration draws (or its own K/V)."""
    ck = bt.calib_k if bt.calib_k is not None else bt.k
    cv = bt.calib_v if bt.calib_v is not None else bt.v
    amax, scale, st = calibrate_amax(np.stack([ck.reshape(-1), cv.reshape(-1)]))
    assert st == 0
    return amax, scale


def oracle_caches(bt, ks, vs, rows=None):
    """Oracle caches with all (or only the listed sequences') tokens written."""
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    if rows is None:
        quant_write(bt.k, bt.v, bt.slot_mapping, ks, vs, kc, vc)
    else:
        for b in rows:
            s0, s1 = int(bt.cu_seq_lens[b]), int(bt.cu_seq_lens[b + 1])
            quant_write(bt.k[s0:s1], bt.v[s0:s1], bt.slot_mapping[s0:s1], ks, vs, kc, vc)
    return kc, vc
