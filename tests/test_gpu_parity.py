"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bit-exact for E4M3 codes, cache bytes, amax and scales; attention within
|gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise (fp16 output, fp32 accumulation).
Every input is a seeded synthetic draw from synth/.
"""

import numpy as np
import pytest
import torch

from oracle import (calibrate_amax, e4m3_decode, e4m3_encode, paged_attention, split_partials,
                    split_reduce)
from synth import make_batch, make_config
from tests.gpu_common import (DeviceBatch, assert_close_attn, dev, oracle_caches, oracle_scales,
                              report)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def sm_of(bt):
    return np.float32(1.0 / np.sqrt(bt.head_dim))


# ----------------------------------------------------------------- codec

def test_device_decode_all_codes(K):
    codes = np.arange(256, dtype=np.uint8)
    got = K.kvfp8_e4m3_decode_f32(dev(codes)).cpu().numpy().astype(np.float64)
    ref = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_device_encode_boundaries_and_random(K):
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    parts = [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
             vals.astype(np.float32),
             np.array([448, 449, 463.9, 464, 464.1, 480, 500, 1e6, np.inf, 0.0, 2 ** -10, 3 * 2 ** -10,
                       2 ** -11, 1e-30, 1e-45], np.float32)]
    rng = np.random.default_rng(0)
    parts.append((rng.standard_normal(500_000) * np.exp2(rng.integers(-14, 12, 500_000))).astype(np.float32))
    x = np.concatenate(parts + [-p for p in parts])
    got = K.kvfp8_e4m3_encode_f32(dev(x)).cpu().numpy()
    assert np.array_equal(got, e4m3_encode(x))
    nan = np.array([np.nan, -np.nan], np.float32)
    assert np.array_equal(K.kvfp8_e4m3_encode_f32(dev(nan)).cpu().numpy(), e4m3_encode(nan))


# ----------------------------------------------------------------- calibration

@pytest.mark.parametrize("which", ["tiny_same_tensors", "decode_calib_set", "ragged_len"])
def test_calibrate_bit_exact(K, which):
    if which == "tiny_same_tensors":
        bt = make_config(1)
        x = np.stack([bt.k.reshape(-1), bt.v.reshape(-1)])
    elif which == "decode_calib_set":
        bt = make_config(2, seq_len_override=64)
        x = np.stack([bt.calib_k.reshape(-1), bt.calib_v.reshape(-1)])
    else:
        rng = np.random.default_rng(3)
        x = (rng.standard_normal((7, 1001)) * 3).astype(np.float16)  # rows not 16-byte multiples
    amax, scale, st = K.kv_calibrate_amax(dev(x))
    ra, rs, rst = calibrate_amax(x)
    assert st == rst == 0
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_calibrate_mixed_workload_48_tensors(K):
    from synth.workloads import make_mixed_calibration
    x = make_mixed_calibration()
    amax, scale, st = K.kv_calibrate_amax(dev(x))
    ra, rs, rst = calibrate_amax(x)
    assert st == rst == 0 and x.shape[0] == 48
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_calibrate_error_statuses(K):
    x = np.zeros((3, 64), dtype=np.float16)
    x[0] = 1.5
    x[2, 7] = np.inf
    amax, scale, st = K.kv_calibrate_amax(dev(x), check=False)
    ra, rs, rst = calibrate_amax(x)
    assert st == rst == K.NONFINITE_INPUT
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    x[2, 7] = 0
    amax, scale, st = K.kv_calibrate_amax(dev(x), check=False)
    assert st == K.BAD_SCALE and calibrate_amax(x)[2] == K.BAD_SCALE
    assert amax.cpu().numpy()[1] == 0 and scale.cpu().numpy()[1] == 0


@pytest.mark.parametrize("pattern", ["rising", "one_outlier", "negative_extremes", "late_nonfinite"])
def test_calibrate_many_blocks(K, pattern):
    """Two 8 Mi-element tensors (hundreds of scan blocks each). A block skips
    its atomic when the maximum folded in so far is not below its own, so the
    patterns put the maximum where every block, one block or the last block
    has to fold it in, and a second call on other data must not see the first."""
    n = 1 << 23
    rng = np.random.default_rng({"rising": 11, "one_outlier": 12, "negative_extremes": 13, "late_nonfinite": 14}[pattern])
    x = rng.standard_normal((2, n)).astype(np.float16)
    if pattern == "rising":
        x = (np.linspace(0.0, 300.0, n, dtype=np.float32)[None, :] * np.array([[1.0], [-0.5]], np.float32)).astype(np.float16)
    elif pattern == "one_outlier":
        x[0, int(rng.integers(n))] = 97.5
        x[1, n - 1] = -311.0
    elif pattern == "negative_extremes":
        x[0, 5] = -65504.0
        x[1, n // 2 + 3] = -60000.0
        x[1, n // 2 + 4] = 59968.0
    else:
        x[0, n - 2] = np.inf
        x[1, n - 7] = np.nan
    for inp in (x, x[:, : n // 4].copy() * np.float16(0.5)):
        amax, scale, st = K.kv_calibrate_amax(dev(inp), check=False)
        ra, rs, rst = calibrate_amax(inp)
        assert st == rst
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32)), (amax, ra)
        assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_calibrate_odd_length_rows(K):
    """Rows of 3,000,001 elements start at every even byte offset modulo 16,
    so each scan block reads a few elements before and after its 16-byte
    aligned middle one by one; the maxima sit in those pieces: a row's first
    element, a row's last, and just past a block's start."""
    n = 3_000_001
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, n)).astype(np.float16)
    x[1, 0] = 200.0
    x[2, n - 1] = -300.0
    x[3, 20480 * 7 + 3] = 250.0
    x[4, n // 2] = -6.0e4
    for inp in (x, x[:4, : n - 6].copy()):
        amax, scale, st = K.kv_calibrate_amax(dev(inp), check=False)
        ra, rs, rst = calibrate_amax(inp)
        assert st == rst == 0
        assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32)), (amax, ra)
        assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_calibrate_more_tensors_than_one_grid_row(K):
    """70,000 tensors of 13 elements: the scan is launched in groups of at
    most 65,535 tensors (the grid's y limit), and a row holds at most one
    aligned 16-byte vector, the rest being read one element per thread. The
    maxima sit in the second group, at its last tensor and at row ends."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((70_000, 13)).astype(np.float16)
    x[65_535, 12] = 123.0
    x[69_999, 0] = -456.0
    amax, scale, st = K.kv_calibrate_amax(dev(x), check=False)
    ra, rs, rst = calibrate_amax(x)
    assert st == rst == 0
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))


# ----------------------------------------------------------------- write

def _gpu_write(K, db, ks, vs):
    K.kv_quant_write(db.k, db.v, db.slots, float(ks), float(vs), db.k_cache, db.v_cache)


@pytest.mark.parametrize("case", ["tiny", "ragged_p16_d128", "p8_d64", "p32", "p64"])
def test_quant_write_bit_exact(K, case):
    bt = {
        "tiny": lambda: make_config(1),
        "ragged_p16_d128": lambda: make_batch([1, 17, 300, 64], [1, 1, 4, 2], 32, 4, 128, 16, seed=41),
        "p8_d64": lambda: make_batch([33, 70], [1, 3], 8, 2, 64, 8, seed=42),
        "p32": lambda: make_batch([100, 31, 64], [1, 1, 1], 16, 2, 128, 32, seed=43),
        "p64": lambda: make_batch([200, 5], [1, 1], 32, 4, 128, 64, seed=44),
    }[case]()
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)


def _slot_pattern(kind, P, num_pages, rng):
    cap = num_pages * P
    if kind == "scattered":  # one token per page here and there (decode-like)
        return rng.permutation(cap)[:300]
    if kind == "scattered_small":  # a decode step's size
        return rng.permutation(cap)[:100]
    if kind == "scattered_large":  # single scattered slots in a call large enough for looping workgroups
        return rng.permutation(cap)[:20000]
    if kind == "runs":  # contiguous runs from arbitrary starts, in random order
        runs, used = [], set()
        while len(runs) < 12:
            st, n = int(rng.integers(0, cap - 300)), int(rng.integers(1, 300))
            if used.isdisjoint(range(st, st + n)):
                used.update(range(st, st + n))
                runs.append(np.arange(st, st + n))
        return np.concatenate(runs)
    if kind == "runs_with_holes":  # one long run with padding and out-of-range slots in it
        s = np.arange(5, 5 + 700)
        s[rng.integers(0, 700, 40)] = -1
        s[rng.integers(0, 700, 3)] = cap + 7
        return s
    # "paged": whole and partial pages in a random page order (a prefill through a block table);
    # "paged_large": the same over most pages of a larger cache
    out = []
    for p in rng.permutation(num_pages)[: (num_pages // 2 if kind == "paged" else num_pages - 8)]:
        out.append(int(p) * P + np.arange(int(rng.integers(1, P + 1))))
    return np.concatenate(out)


@pytest.mark.parametrize("kind", ["scattered_small", "scattered", "runs", "runs_with_holes", "paged", "paged_large",
                                  "scattered_large"])
@pytest.mark.parametrize("D,P", [(128, 4), (128, 16), (128, 64), (64, 8), (64, 32)])
def test_quant_write_slot_patterns(K, kind, D, P):
    """The write stores V in runs of consecutive slots, aligned quads and single
    bytes, with three workgroup shapes chosen by the call's size (up to 256
    tokens; fewer than about four workgroups per CU; more): every slot pattern
    and size gives the oracle's cache bytes exactly."""
    rng = np.random.default_rng([sum(map(ord, kind)), D, P])
    if kind in ("paged_large", "scattered_large"):  # 20,000-24,000 tokens over 8 kv-heads: the large-call shape
        num_pages, hkv = 48000 // P + 8, 8
    else:
        num_pages, hkv = 3000 // P + 8, 2
    slots = _slot_pattern(kind, P, num_pages, rng).astype(np.int64)
    n = slots.shape[0]
    k = (rng.standard_normal((n, hkv, D)) * 2).astype(np.float16)
    v = (rng.standard_normal((n, hkv, D)) * 2).astype(np.float16)
    ks, vs = np.float32(0.02), np.float32(0.015)
    kc_d = torch.full((num_pages, hkv, P, D), 0x7F, dtype=torch.uint8, device="cuda")
    vc_d = torch.full((num_pages, hkv, D, P), 0x7F, dtype=torch.uint8, device="cuda")
    print(f"write {kind} D {D} P {P} tokens {n}", flush=True)
    K.kv_quant_write(dev(k), dev(v), dev(slots), float(ks), float(vs), kc_d, vc_d)
    from oracle import new_caches, quant_write
    kc, vc = new_caches(num_pages, hkv, P, D)
    quant_write(k, v, slots, ks, vs, kc, vc)
    assert np.array_equal(kc_d.cpu().numpy(), kc)
    assert np.array_equal(vc_d.cpu().numpy(), vc)


def test_quant_write_skips_padding_and_saturates(K):
    bt = make_batch([40], [1], 8, 2, 64, 16, seed=45)
    bt.k[7, 0, :8] = np.float16(60000.0)  # far beyond 448 * scale: saturates
    bt.k[5, 1, :4] = np.float16(-0.0)
    slots = bt.slot_mapping.copy()
    slots[::3] = -1
    slots[1] = bt.num_pages * bt.page_size + 5  # past the cache: skipped
    db = DeviceBatch(bt)
    db.slots = dev(slots)
    K.kv_quant_write(db.k, db.v, db.slots, 0.01, 0.02, db.k_cache, db.v_cache)
    from oracle import new_caches, quant_write
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, slots, np.float32(0.01), np.float32(0.02), kc, vc)
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    assert (kc == 0x7E).any()


@pytest.mark.parametrize("n_tok,hkv,D", [(600, 2, 128), (600, 2, 64), (70_000, 1, 128), (131_072, 1, 64)])
def test_quant_write_grouped_nonfinite_and_extremes(K, n_tok, hkv, D):
    """Calls of more than 256 tokens take the grouped write, which encodes two
    codes per convert unless a thread holds a NaN input; NaN of both signs,
    +-Inf, +-65504, -0 and fp16 subnormals are scattered over the call so
    that wavefronts mix both paths. The small sizes run one token per
    thread, the large ones (a grid of at least 1,024 workgroups) two."""
    bt = make_batch([n_tok], [1], 4 * hkv, hkv, D, 16, seed=4700 + n_tok + D)
    rng = np.random.default_rng(n_tok + D)
    specials = np.array([np.nan, -np.nan, np.inf, -np.inf, 65504.0, -65504.0, -0.0, 6e-8, -6e-8, 2.0 ** -24],
                        dtype=np.float16)
    specials[1] = np.frombuffer(np.uint16(0xFE00).tobytes(), np.float16)[0]  # a NaN with the sign bit set
    for arr in (bt.k, bt.v):
        flat = arr.reshape(-1)
        pos = rng.choice(flat.size, size=min(flat.size // 50, 4000), replace=False)
        flat[pos] = specials[rng.integers(0, specials.size, pos.size)]
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, 0.0123, 0.0456, db.k_cache, db.v_cache)
    from oracle import new_caches, quant_write
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, np.float32(0.0123), np.float32(0.0456), kc, vc)
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    assert (kc == 0x7F).any() and (kc == 0xFF).any() and (vc == 0x7E).any() and (vc == 0xFE).any()


# ----------------------------------------------------------------- attention

def _run_decode(K, db, ks, vs, sm, S):
    bt = db.bt
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:  # every partial the reduction reads must have been written
        K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    return K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                    float(ks), float(vs), float(sm), num_splits=S, workspace=ws)


def _run_verify(K, db, ks, vs, sm, S):
    bt = db.bt
    ws = K.workspace(bt.total_q, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:
        K.poison_partials(ws, bt.total_q, bt.n_q_heads, bt.head_dim, S)
    return K.paged_attn_e4m3_verify(db.q, db.cu_q, int(bt.q_lens.max()), db.k_cache, db.v_cache,
                                    db.block_table, db.seq_lens, float(ks), float(vs), float(sm),
                                    num_splits=S, workspace=ws)


DECODE_CASES = {
    "tiny": lambda: make_config(1),
    "d128_p16_ragged": lambda: make_batch([1, 63, 64, 65, 1000, 333], [1] * 6, 32, 4, 128, 16, seed=51),
    "d64_p8": lambda: make_batch([5, 130, 77], [1] * 3, 16, 4, 64, 8, seed=52),
    "d128_p64_g4": lambda: make_batch([700, 64, 129], [1] * 3, 16, 4, 128, 64, seed=53),
    "d128_p32_g16": lambda: make_batch([300, 41], [1] * 2, 32, 2, 128, 32, seed=54),
    "d64_p4_g32": lambda: make_batch([90, 17], [1] * 2, 32, 1, 64, 4, seed=55),
    # more than 64 sequences: the split plan's prefix count runs over several blocks of 64
    "d128_b150_ragged": lambda: make_batch([1 + (37 * i) % 300 for i in range(150)], [1] * 150, 32, 4, 128, 16,
                                           seed=56),
}


@pytest.mark.parametrize("S", [1, 2, 3, 8])
@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_parity(K, case, S):
    bt = DECODE_CASES[case]()
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = sm_of(bt)
    out = _run_decode(K, db, sc[0], sc[1], sm, S).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out, ref, f"{case} S={S}", strict=(case == "tiny"))


APPEND_CASES = {
    # new tokens at a page start, mid-page, the first key, and a tile edge
    "d128_p16": lambda: make_batch([1, 16, 17, 64, 65, 300], [1] * 6, 32, 4, 128, 16, seed=57),
    "d64_p8": lambda: make_batch([9, 130, 8], [1] * 3, 16, 4, 64, 8, seed=58),
    "d128_p64_g4": lambda: make_batch([700, 64, 129], [1] * 3, 16, 4, 128, 64, seed=59),
    # contexts longer than 512 keys per split at page 16: several tiles per wavefront (the
    # instantiation the 4k decode step runs, not the short start-up)
    "d128_p16_long": lambda: make_batch([3000, 1500, 2049, 700, 1], [1] * 5, 32, 4, 128, 16, seed=60),
}


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("case", list(APPEND_CASES))
def test_decode_append_equals_write_then_decode(K, case, S):
    """The fused step writes exactly the bytes kv_quant_write would (every cache
    byte against the oracle) and returns the separate write-then-decode result
    bit for bit."""
    bt = APPEND_CASES[case]()
    _, sc = oracle_scales(bt)
    ks, vs, sm = float(sc[0]), float(sc[1]), float(sm_of(bt))
    name = K.kvfp8_attn_kernel_name(bt.batch, bt.n_q_heads, bt.n_kv_heads, bt.head_dim, bt.page_size,
                                    bt.max_pages, 1, S)
    if case == "d128_p16_long":
        assert name == "attn_split_kernel<128,16,1,8,false>", name
    db = DeviceBatch(bt)
    prior, new = dev(bt.prior_rows()), dev(bt.new_token_rows())
    K.kv_quant_write(db.k[prior].contiguous(), db.v[prior].contiguous(), db.slots[prior].contiguous(), ks, vs,
                     db.k_cache, db.v_cache)
    kc_sep, vc_sep = db.k_cache.clone(), db.v_cache.clone()
    k_new, v_new = db.k[new].contiguous(), db.v[new].contiguous()
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    out = K.paged_attn_e4m3_decode_append(db.q, k_new, v_new, db.k_cache, db.v_cache, db.block_table,
                                          db.seq_lens, ks, vs, sm, num_splits=S, workspace=ws).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm_of(bt))
    assert_close_attn(out, ref, f"append {case} S={S}")
    K.kv_quant_write(k_new, v_new, db.slots[new].contiguous(), ks, vs, kc_sep, vc_sep)
    sep = K.paged_attn_e4m3_decode(db.q, kc_sep, vc_sep, db.block_table, db.seq_lens, ks, vs, sm, num_splits=S,
                                   workspace=ws).cpu().numpy()
    assert np.array_equal(out.view(np.uint16), sep.view(np.uint16))


VERIFY_APPEND_CASES = {
    # new tokens across a split boundary (keys 126..129 at S = 3) and a tile boundary (keys 62..65),
    # a sequence made only of new tokens; 32 rows per kv-head (LDS-staged tiles)
    "edges_g8_p16": lambda: make_batch([130, 66, 4, 300], [4, 4, 4, 3], 32, 4, 128, 16, seed=81),
    # up to 16 rows per kv-head, pages of 8 and 64
    "g4_p8_d64": lambda: make_batch([70, 9, 17], [2, 1, 3], 8, 2, 64, 8, seed=82),
    "g4_p64": lambda: make_batch([700, 64, 129], [4, 2, 3], 16, 4, 128, 64, seed=83),
    # 32 rows per kv-head with pages of 4 (register tiles, no staging)
    "g8_p4_d64": lambda: make_batch([100, 257], [4, 2], 32, 4, 64, 4, seed=84),
    # staged tiles of 32-key pages: at S = 1 the new tokens of the 700-key sequence lie in a wavefront's
    # third tile and those of the 450-key one straddle two wavefronts' second tiles (both stored after
    # the wavefront's first tile has landed)
    "deferred_g8_p32": lambda: make_batch([700, 450, 40], [4, 4, 2], 32, 4, 128, 32, seed=85),
}


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("case", list(VERIFY_APPEND_CASES))
def test_verify_append_equals_write_then_verify(K, case, S):
    """The fused MTP step writes exactly the bytes kv_quant_write would (every
    cache byte against the oracle) and returns the separate write-then-verify
    result bit for bit."""
    bt = VERIFY_APPEND_CASES[case]()
    _, sc = oracle_scales(bt)
    ks, vs, sm = float(sc[0]), float(sc[1]), float(sm_of(bt))
    db = DeviceBatch(bt)
    prior, new = dev(bt.prior_rows()), dev(bt.new_token_rows())
    K.kv_quant_write(db.k[prior].contiguous(), db.v[prior].contiguous(), db.slots[prior].contiguous(), ks, vs,
                     db.k_cache, db.v_cache)
    kc_sep, vc_sep = db.k_cache.clone(), db.v_cache.clone()
    k_new, v_new = db.k[new].contiguous(), db.v[new].contiguous()
    mq = int(bt.q_lens.max())
    ws = K.workspace(bt.total_q, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:
        K.poison_partials(ws, bt.total_q, bt.n_q_heads, bt.head_dim, S)
    out = K.paged_attn_e4m3_verify_append(db.q, k_new, v_new, db.cu_q, mq, db.k_cache, db.v_cache,
                                          db.block_table, db.seq_lens, ks, vs, sm, num_splits=S,
                                          workspace=ws).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm_of(bt))
    assert_close_attn(out, ref, f"verify append {case} S={S}")
    K.kv_quant_write(k_new, v_new, db.slots[new].contiguous(), ks, vs, kc_sep, vc_sep)
    sep = K.paged_attn_e4m3_verify(db.q, db.cu_q, mq, kc_sep, vc_sep, db.block_table, db.seq_lens, ks, vs, sm,
                                   num_splits=S, workspace=ws).cpu().numpy()
    assert np.array_equal(out.view(np.uint16), sep.view(np.uint16))


VERIFY_CASES = {
    "mtp3_small": lambda: make_batch([1024, 70, 4, 300], [4] * 4, 32, 4, 128, 16, seed=61),
    "ragged_q": lambda: make_batch([50, 9, 200, 3], [1, 2, 4, 3], 32, 4, 128, 16, seed=62),
    "d64_p4": lambda: make_batch([100, 257], [4, 2], 8, 2, 64, 4, seed=63),
    "g4_q8": lambda: make_batch([129, 64], [8, 5], 16, 4, 64, 16, seed=64),
    # 32 rows per kv-head with pages of 32 and 64 keys: the LDS-staged verify pipeline
    "p64_q4": lambda: make_batch([700, 64, 129], [4, 2, 3], 32, 4, 128, 64, seed=65),
    "p32_g16_q2": lambda: make_batch([300, 41, 5], [2, 2, 1], 32, 2, 128, 32, seed=66),
}


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("case", list(VERIFY_CASES))
def test_verify_parity(K, case, S):
    bt = VERIFY_CASES[case]()
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = sm_of(bt)
    out = _run_verify(K, db, sc[0], sc[1], sm, S).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out, ref, f"{case} S={S}")


def test_partials_match_oracle_partials(K):
    bt = make_batch([1000, 257, 64, 3], [1, 1, 1, 1], 32, 4, 128, 16, seed=71)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    S = 4
    sm = sm_of(bt)
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                             float(sc[1]), float(sm), num_splits=S, workspace=ws, partials_only=True)
    o, m, l = [t.cpu().numpy().astype(np.float64) for t in K.workspace_views(ws, bt.batch, bt.n_q_heads,
                                                                             bt.head_dim, S)]
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ro, rm, rl = split_partials(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm,
                                S, granule=64)
    assert np.array_equal(np.isneginf(m), np.isneginf(rm))
    fin = np.isfinite(rm)
    np.testing.assert_allclose(m[fin], rm[fin], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(l, rl, rtol=2e-3, atol=1e-5)
    # an empty split writes m = -inf and l = 0 only: its o slot keeps the poison
    scale = np.maximum(rl[..., None], 1.0)
    assert (np.abs(o - ro) <= 2e-3 * scale + 1e-2 * np.abs(ro))[fin].all()
    assert np.isnan(o[~fin]).all()
    # the ragged lengths leave empty splits in the shorter sequences
    assert (~fin).any() and fin[:, :, 1].any()


def test_split_reduce_of_oracle_partials(K):
    bt = make_batch([500, 64, 130], [1, 1, 1], 32, 4, 128, 16, seed=72)
    _, sc = oracle_scales(bt)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    S = 7
    ro, rm, rl = split_partials(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1],
                                sm_of(bt), S, granule=64)
    o32, m32, l32 = ro.astype(np.float32), rm.astype(np.float32), rl.astype(np.float32)
    ref, ref_lse = split_reduce(o32, m32, l32)
    out, lse = K.split_reduce_fp32(dev(o32), dev(m32), dev(l32), with_lse=True)
    assert_close_attn(out.cpu().numpy(), ref, "reduce")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("S", [3, 20, 70])
def test_split_reduce_ignores_o_of_empty_splits(K, S):
    """Empty splits (m = -inf, l = 0) may hold anything in o: before, between
    and after live splits, NaN there must not reach the output."""
    rng = np.random.default_rng(73 + S)
    R, H, D = 3, 4, 128
    m = rng.uniform(-3, 3, (R, H, S)).astype(np.float32)
    l = rng.uniform(0.5, 4, (R, H, S)).astype(np.float32)
    o = rng.standard_normal((R, H, S, D)).astype(np.float32)
    dead = rng.random((R, H, S)) < 0.5
    dead[0, 0, :] = True           # a row with no live split
    dead[1, 1, :] = False
    dead[1, 1, S - 1] = True       # trailing empty split
    dead[2, 2, :] = True
    dead[2, 2, S // 2] = False     # one live split in the middle
    m[dead], l[dead], o[dead] = -np.inf, 0.0, 0.0
    ref, ref_lse = split_reduce(o.astype(np.float64), m, l)  # an empty split's o is 0 by definition
    o[dead] = np.nan
    out, lse = K.split_reduce_fp32(dev(o), dev(m), dev(l), with_lse=True)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all()
    assert (out[0, 0] == 0).all() and np.isneginf(lse[0, 0])
    assert_close_attn(out, ref, f"reduce S={S}")
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-5, atol=1e-5)


def test_split_reduce_all_empty_rows(K):
    o = np.zeros((2, 4, 5, 64), np.float32)
    m = np.full((2, 4, 5), -np.inf, np.float32)
    l = np.zeros((2, 4, 5), np.float32)
    m[1, 2, 3], l[1, 2, 3], o[1, 2, 3] = 1.0, 2.0, 4.0
    out, lse = K.split_reduce_fp32(dev(o), dev(m), dev(l), with_lse=True)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert (out[1, 2] == 2.0).all() and abs(lse[1, 2] - (1 + np.log(2))) < 1e-5


# ----------------------------------------------------------------- invariants

def test_single_token_context_returns_v_for_every_code(K):
    """With one key, the output is v_scale * decode(v): run every non-NaN code
    through the V path (v_scale = 1 so the output is exact in fp16)."""
    bt = make_batch([1, 1], [1, 1], 4, 2, 64, 16, seed=81)
    db = DeviceBatch(bt)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0x00, 0x80], np.uint8)
    codes = codes.reshape(2, 2, 64)  # [sequence, kv-head, dim]
    vc = db.v_cache.cpu().numpy()
    kc = db.k_cache.cpu().numpy()
    for b in range(2):
        page = bt.block_table[b, 0]
        vc[page, :, :, 0] = codes[b]
        kc[page, :, 0, :] = 0x38
    db.v_cache.copy_(dev(vc))
    db.k_cache.copy_(dev(kc))
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, 1.0, 1.0,
                                   0.125).cpu().numpy()
    ref = e4m3_decode(codes)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h].astype(np.float64), ref[b, h // 2])


@pytest.mark.parametrize("D", [64, 128])
def test_every_k_code_reaches_the_scores(K, D):
    """Two keys per sequence: key 0 holds one K code (every non-NaN code, one
    per kv-head) in a single dimension, key 1 is zero; V is 1 for key 0 and 0
    for key 1, so the output is the softmax weight of key 0, a sigmoid of
    q * decode(code) * k_scale * sm_scale. Query magnitudes from 1 to 60000
    put every code, the E4M3 subnormals included, where the weight depends on
    its exact value."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n_kvh = 4
    n_seq = -(-len(codes) // n_kvh)
    codes = np.concatenate([codes, np.zeros(n_seq * n_kvh - len(codes), np.uint8)]).reshape(n_seq, n_kvh)
    bt = make_batch([2] * n_seq, [1] * n_seq, 4 * n_kvh, n_kvh, D, 16, seed=86)
    qmag = np.array([60000.0, 3000.0, 100.0, 1.0], np.float16)
    bt.q[:] = 0
    for h in range(4 * n_kvh):
        bt.q[:, h, 5] = qmag[h % 4]
    kc = np.zeros((bt.num_pages, n_kvh, 16, D), np.uint8)
    vc = np.zeros((bt.num_pages, n_kvh, D, 16), np.uint8)
    for b in range(n_seq):
        page = bt.block_table[b, 0]
        kc[page, :, 0, 5] = codes[b]
        vc[page, :, :, 0] = 0x38  # 1.0
    db = DeviceBatch(bt)
    db.k_cache.copy_(dev(kc))
    db.v_cache.copy_(dev(vc))
    ks, vs, sm = np.float32(0.125), np.float32(1.0), np.float32(0.125)
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(ks),
                                   float(vs), float(sm)).cpu().numpy()
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, ks, vs, sm)
    assert_close_attn(out, ref, f"every K code D={D}")
    # the smallest subnormal code moves the weight well away from 1/2 at q = 60000
    b1, h1 = np.argwhere(codes == 0x01)[0]
    assert out[b1, 4 * h1, 0] > 0.8


def test_page_permutation_bit_identical(K):
    bt = make_batch([300, 77], [1, 1], 32, 4, 128, 16, seed=82)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    out1 = _run_decode(K, db, sc[0], sc[1], sm_of(bt), 2).cpu().numpy()
    relabel = np.random.default_rng(1).permutation(bt.num_pages)
    kc2 = torch.empty_like(db.k_cache)
    vc2 = torch.empty_like(db.v_cache)
    kc2[dev(relabel)] = db.k_cache
    vc2[dev(relabel)] = db.v_cache
    db.k_cache, db.v_cache = kc2, vc2
    db.block_table = dev(np.where(bt.block_table >= 0, relabel[np.maximum(bt.block_table, 0)], -1)
                         .astype(np.int32))
    out2 = _run_decode(K, db, sc[0], sc[1], sm_of(bt), 2).cpu().numpy()
    assert np.array_equal(out1.view(np.uint16), out2.view(np.uint16))


def test_gqa_identical_queries_bit_identical_and_deterministic(K):
    bt = make_batch([500], [1], 32, 4, 128, 16, seed=83)
    bt.q[0, 1] = bt.q[0, 0]
    bt.q[0, 7] = bt.q[0, 0]
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    a = _run_decode(K, db, sc[0], sc[1], sm_of(bt), 3).cpu().numpy()
    b = _run_decode(K, db, sc[0], sc[1], sm_of(bt), 3).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a[0, 0].view(np.uint16), a[0, 1].view(np.uint16))
    assert np.array_equal(a[0, 0].view(np.uint16), a[0, 7].view(np.uint16))


def test_verify_row_equals_decode_of_shorter_sequence(K):
    bt = make_batch([200], [4], 32, 4, 128, 16, seed=84)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = sm_of(bt)
    ver = _run_verify(K, db, sc[0], sc[1], sm, 1).cpu().numpy()
    for i in range(4):
        dec = K.paged_attn_e4m3_decode(db.q[i:i + 1].contiguous(), db.k_cache, db.v_cache, db.block_table,
                                       dev(np.array([200 - 4 + i + 1], np.int32)), float(sc[0]),
                                       float(sc[1]), float(sm)).cpu().numpy()
        err, _ = report(ver[i], dec[0].astype(np.float64))
        assert err <= 2e-3


def test_power_of_two_v_scale_equivariance(K):
    bt = make_batch([123, 64], [1, 1], 32, 4, 128, 16, seed=85)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    a = _run_decode(K, db, sc[0], sc[1], sm_of(bt), 1).cpu().numpy()
    b = _run_decode(K, db, sc[0], np.float32(sc[1] * 2), sm_of(bt), 1).cpu().numpy()
    # exact where the fp16 output is a normal number; an fp16 subnormal rounds at a
    # fixed absolute step, so there doubling and rounding commute only to 2**-24
    normal = np.abs(a) >= np.float16(2.0 ** -14)
    assert np.array_equal(b[normal], a[normal] * np.float16(2))
    assert (np.abs(b[~normal].astype(np.float64) - 2 * a[~normal].astype(np.float64)) <= 2.0 ** -24).all()


# ----------------------------------------------------------------- prefill chunk (query-tiled kernel)

CHUNK_CASES = {
    "chunk_over_prior": lambda: make_batch([700], [200], 32, 4, 128, 16, seed=91),
    "ragged_no_prior": lambda: make_batch([100, 70, 300], [50, 70, 33], 32, 4, 128, 16, seed=92),
    "d64_p4_g4": lambda: make_batch([257, 90], [120, 90], 16, 4, 64, 4, seed=93),
    "p64_g8": lambda: make_batch([1000, 64], [300, 20], 32, 4, 128, 64, seed=94),
    "p8_g16": lambda: make_batch([333], [65], 32, 2, 128, 8, seed=95),
    "mixed_layer_small": lambda: make_batch([1000] * 8 + [1256], [1] * 8 + [256], 32, 4, 128, 16, seed=96),
}


@pytest.mark.parametrize("case", list(CHUNK_CASES))
def test_chunk_parity(K, case):
    bt = CHUNK_CASES[case]()
    assert int(bt.q_lens.max()) * (bt.n_q_heads // bt.n_kv_heads) > 32  # takes the chunk kernel
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = sm_of(bt)
    out = _run_verify(K, db, sc[0], sc[1], sm, 1).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out, ref, case)


def test_chunk_rows_match_split_kernel_rows(K):
    """The same rows computed by the chunk kernel (long q) and by the split
    kernel (one query token at a time) agree within the tolerance."""
    bt = make_batch([400], [96], 32, 4, 128, 16, seed=97)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = sm_of(bt)
    chunk = _run_verify(K, db, sc[0], sc[1], sm, 1).cpu().numpy()
    for i in (0, 31, 32, 95):
        dec = K.paged_attn_e4m3_decode(db.q[i:i + 1].contiguous(), db.k_cache, db.v_cache, db.block_table,
                                       dev(np.array([400 - 96 + i + 1], np.int32)), float(sc[0]),
                                       float(sc[1]), float(sm)).cpu().numpy()
        err, _ = report(chunk[i], dec[0].astype(np.float64))
        assert err <= 2e-3, (i, err)


# ----------------------------------------------------------------- fused reduce, counters, graphs

@pytest.mark.parametrize("S", [16, 17, 64])
def test_many_splits(K, S):
    """Long and short sequences split 16 to 64 ways (many empty splits for the
    short ones), merged by the reduce kernel."""
    bt = make_batch([3000, 1025, 70], [1, 1, 1], 32, 4, 128, 16, seed=101)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = sm_of(bt)
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                   float(sc[1]), float(sm), num_splits=S, workspace=ws).cpu().numpy()
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(out, ref, f"S={S}")


def test_graph_replays_match_eager(K):
    """A captured decode step (write, split attention, reduce) replayed
    several times, with eager work and synchronisations in between, reproduces
    the eager output bit for bit on every replay."""
    bt = make_batch([900, 450, 2000, 64], [1] * 4, 32, 4, 128, 16, seed=102)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    sm = float(sm_of(bt))
    S = 4
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S)
    out = torch.empty_like(db.q)
    new = dev(bt.new_token_rows())
    k_new, v_new, s_new = db.k[new].contiguous(), db.v[new].contiguous(), db.slots[new].contiguous()

    def step():
        K.kv_quant_write(k_new, v_new, s_new, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
        K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                 float(sc[1]), sm, num_splits=S, workspace=ws, out=out)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        _ = (db.q.float() * 2).sum().item()  # unrelated eager work between replays
        step()  # and an eager call sharing the workspace
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_graph_replay_follows_changing_lengths(K):
    """One captured split decode replayed while the context lengths and queries
    change in place between replays (the longest context too, so the split size
    and the work plan change): the work plan is derived on the device from the
    lengths, so every replay must equal an eager call on the same inputs bit for
    bit and match the oracle."""
    bt = make_batch([2000, 2000, 2000, 2000, 2000], [1] * 5, 32, 4, 128, 16, seed=103)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    sm = float(sm_of(bt))
    S = 6
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S)
    out = torch.empty_like(db.q)
    seq_lens = db.seq_lens.clone()
    q = db.q.clone()

    def step():
        K.paged_attn_e4m3_decode(q, db.k_cache, db.v_cache, db.block_table, seq_lens, float(sc[0]), float(sc[1]),
                                 sm, num_splits=S, workspace=ws, out=out)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(104)
    for rep, lens in enumerate(([2000, 1, 700, 1999, 64], [5, 9, 3, 1, 2], [1500, 1500, 1500, 1500, 1500],
                                [64, 128, 2000, 65, 63])):
        lens = np.asarray(lens, np.int32)
        qn = rng.standard_normal(bt.q.shape).astype(np.float16)
        seq_lens.copy_(torch.from_numpy(lens))
        q.copy_(torch.from_numpy(qn))
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(replayed, out), f"replay {rep} differs from the eager call"
        cu = np.arange(bt.batch + 1, dtype=np.int32)
        ref, _ = paged_attention(qn, kc, vc, bt.block_table, lens, cu, sc[0], sc[1], sm)
        assert_close_attn(replayed.cpu().numpy(), ref, f"replay {rep}")


def test_graph_replay_verify_append_follows_lengths(K):
    """A captured MTP verify step with its new tokens appended, replayed while
    the context lengths (and so the new tokens' positions, the split size and
    the work plan) and the queries change in place between replays. The new
    tokens are the ones already cached at those positions, so the appends are
    idempotent and the cache stays the oracle's; every replay equals an eager
    call bit for bit and matches the oracle."""
    B, T = 4, 4
    bt = make_batch([3000] * B, [T] * B, 32, 4, 128, 16, seed=105)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    sm = float(sm_of(bt))
    S = 6
    rows = B * T
    ws = K.workspace(rows, bt.n_q_heads, bt.head_dim, S)
    out = torch.empty_like(db.q)
    seq_lens = db.seq_lens.clone()
    q = db.q.clone()
    k_new = torch.empty((rows, bt.n_kv_heads, bt.head_dim), dtype=torch.float16, device="cuda")
    v_new = torch.empty_like(k_new)

    def step():
        K.paged_attn_e4m3_verify_append(q, k_new, v_new, db.cu_q, T, db.k_cache, db.v_cache, db.block_table,
                                        seq_lens, float(sc[0]), float(sc[1]), sm, num_splits=S, workspace=ws,
                                        out=out)

    def set_inputs(lens, qn):
        tok = np.concatenate([bt.cu_seq_lens[b] + np.arange(L - T, L) for b, L in enumerate(lens)])
        k_new.copy_(torch.from_numpy(bt.k[tok]))
        v_new.copy_(torch.from_numpy(bt.v[tok]))
        seq_lens.copy_(torch.from_numpy(np.asarray(lens, np.int32)))
        q.copy_(torch.from_numpy(qn))

    rng = np.random.default_rng(106)
    set_inputs([3000] * B, bt.q)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep, lens in enumerate(([3000, 4, 1029, 64], [700, 701, 702, 703], [4, 4, 4, 2999], [1234, 3000, 17, 65])):
        qn = rng.standard_normal(bt.q.shape).astype(np.float16)
        set_inputs(lens, qn)
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(replayed, out), f"replay {rep} differs from the eager call"
        assert np.array_equal(db.k_cache.cpu().numpy(), kc) and np.array_equal(db.v_cache.cpu().numpy(), vc)
        ref, _ = paged_attention(qn, kc, vc, bt.block_table, np.asarray(lens, np.int32), bt.cu_q_lens, sc[0], sc[1],
                                 sm)
        assert_close_attn(replayed.cpu().numpy(), ref, f"replay {rep}")


def test_graph_replay_chunk_follows_lengths(K):
    """A captured prefill chunk (the query-tiled chunk kernel: 40 tokens x 8
    heads per kv-head) replayed while the prior context length and the queries
    change in place: every replay equals an eager call bit for bit and matches
    the oracle."""
    T = 40
    bt = make_batch([2000, 2000], [T, T], 32, 4, 128, 16, seed=107)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    sm = float(sm_of(bt))
    out = torch.empty_like(db.q)
    seq_lens = db.seq_lens.clone()
    q = db.q.clone()

    def step():
        K.paged_attn_e4m3_verify(q, db.cu_q, T, db.k_cache, db.v_cache, db.block_table, seq_lens, float(sc[0]),
                                 float(sc[1]), sm, out=out)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(108)
    for rep, lens in enumerate(([2000, 40], [41, 1999], [1000, 1000], [555, 64])):
        lens = np.asarray(lens, np.int32)
        qn = rng.standard_normal(bt.q.shape).astype(np.float16)
        seq_lens.copy_(torch.from_numpy(lens))
        q.copy_(torch.from_numpy(qn))
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(replayed, out), f"replay {rep} differs from the eager call"
        ref, _ = paged_attention(qn, kc, vc, bt.block_table, lens, bt.cu_q_lens, sc[0], sc[1], sm)
        assert_close_attn(replayed.cpu().numpy(), ref, f"replay {rep}")


@pytest.mark.parametrize("S", [1, 3])
def test_decode_sequences_without_keys(K, S):
    """Decode rows whose sequence has no keys (as on a context shard that holds
    none of a sequence's pages) produce zeros, directly and through the split
    partials, and leave the other rows unaffected."""
    bt = make_batch([300, 5, 700, 64], [1] * 4, 32, 4, 128, 16, seed=109)
    _, sc = oracle_scales(bt)
    db = DeviceBatch(bt)
    _gpu_write(K, db, sc[0], sc[1])
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    sm = float(sm_of(bt))
    lens = bt.seq_lens.copy()
    lens[[1, 3]] = 0
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert not ref[[1, 3]].any()
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:
        K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, dev(lens), float(sc[0]),
                                   float(sc[1]), sm, num_splits=S, workspace=ws).cpu().numpy()
    assert not out[[1, 3]].astype(np.float64).any()
    assert_close_attn(out, ref, f"S={S}")
