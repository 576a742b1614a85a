"""Pins of the oracle's paged attention and split algebra (CPU only)."""

import numpy as np
import pytest

from oracle import (calibrate_amax, e4m3_decode, new_caches, paged_attention, quant_write,
                    split_bounds, split_partials, split_reduce)
from synth import make_batch, make_config
from tests import pins


def _written(bt, ks=None, vs=None):
    if ks is None:
        _, sc, st = calibrate_amax(np.stack([bt.k.reshape(-1), bt.v.reshape(-1)]))
        assert st == 0
        ks, vs = sc[0], sc[1]
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, ks, vs, kc, vc)
    return kc, vc, np.float32(ks), np.float32(vs)


def _codes_by_token(bt, kc, vc):
    """Codes of every position in k/v row order, read through the slot mapping."""
    P = bt.page_size
    pages, offs = bt.slot_mapping // P, bt.slot_mapping % P
    return kc[pages, :, offs, :], vc[pages, :, :, offs]


def _attend(bt, kc, vc, ks, vs, sm=None):
    sm = np.float32(1.0 / np.sqrt(bt.head_dim)) if sm is None else sm
    return paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, ks, vs, sm)


def test_brute_force_tiny():
    bt = make_batch([5, 11, 8], [1, 3, 8], 4, 2, 8, 4, seed=21)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(0.3)
    out, _ = _attend(bt, kc, vc, ks, vs, sm)
    kt, vt = _codes_by_token(bt, kc, vc)
    dec1 = lambda c: float(e4m3_decode(np.array([c], np.uint8))[0])
    for b in range(bt.batch):
        s0, s1 = bt.cu_seq_lens[b], bt.cu_seq_lens[b + 1]
        q0, q1 = bt.cu_q_lens[b], bt.cu_q_lens[b + 1]
        ref = pins.brute_force_attention(bt.q[q0:q1].astype(np.float64).tolist(), kt[s0:s1].tolist(),
                                         vt[s0:s1].tolist(), float(ks), float(vs), float(sm),
                                         int(q1 - q0), dec1)
        np.testing.assert_allclose(out[q0:q1], np.array(ref), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cfg", ["tiny", "ragged"])
def test_matches_torch_sdpa_float64(cfg):
    if cfg == "tiny":
        bt = make_config(1)
    else:
        bt = make_batch([1, 64, 65, 200, 33], [1, 4, 1, 7, 33], 8, 2, 32, 16, seed=31)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    out, _ = _attend(bt, kc, vc, ks, vs, sm)
    kt, vt = _codes_by_token(bt, kc, vc)
    ref = pins.sdpa_reference(bt, kt, vt, ks, vs, sm)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_lse_matches_logsumexp():
    bt = make_batch([40, 17], [3, 1], 4, 1, 16, 8, seed=5)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(0.25)
    _, lse = _attend(bt, kc, vc, ks, vs, sm)
    kt, _ = _codes_by_token(bt, kc, vc)
    for b in range(bt.batch):
        s0, s1 = bt.cu_seq_lens[b], bt.cu_seq_lens[b + 1]
        q0, q1 = bt.cu_q_lens[b], bt.cu_q_lens[b + 1]
        L, T = s1 - s0, q1 - q0
        kd = e4m3_decode(kt[s0:s1]) * float(ks)
        for i in range(T):
            for h in range(bt.n_q_heads):
                g = h // (bt.n_q_heads // bt.n_kv_heads)
                s = float(sm) * (kd[:L - T + i + 1, g, :] @ bt.q[q0 + i, h].astype(np.float64))
                ref = np.log(np.sum(np.exp(s - s.max()))) + s.max()
                assert abs(lse[q0 + i, h] - ref) < 1e-12


def test_single_token_context_returns_v():
    bt = make_batch([1, 1], [1, 1], 4, 2, 16, 4, seed=8)
    kc, vc, ks, vs = _written(bt)
    out, _ = _attend(bt, kc, vc, ks, vs)
    _, vt = _codes_by_token(bt, kc, vc)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], e4m3_decode(vt[b, h // 2]) * float(vs))


def test_uniform_keys_give_mean_of_values():
    bt = make_batch([37], [1], 4, 2, 16, 4, seed=9)
    kc, vc, ks, vs = _written(bt)
    kc[:] = 0x3A  # every key code identical -> constant scores
    out, _ = _attend(bt, kc, vc, ks, vs)
    _, vt = _codes_by_token(bt, kc, vc)
    mean = (e4m3_decode(vt) * float(vs)).mean(axis=0)  # [Hkv, D]
    for h in range(4):
        np.testing.assert_allclose(out[0, h], mean[h // 2], rtol=1e-13, atol=1e-15)


def test_physical_page_permutation_invariance():
    bt = make_config(1)
    kc, vc, ks, vs = _written(bt)
    out, _ = _attend(bt, kc, vc, ks, vs)
    rng = np.random.default_rng(1)
    relabel = rng.permutation(bt.num_pages)  # new id of each old page
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[relabel] = kc
    vc2[relabel] = vc
    bt2 = np.where(bt.block_table >= 0, relabel[np.maximum(bt.block_table, 0)], -1).astype(np.int32)
    out2, _ = paged_attention(bt.q, kc2, vc2, bt2, bt.seq_lens, bt.cu_q_lens, ks, vs,
                              np.float32(1 / 8))
    assert np.array_equal(out, out2)


def test_gqa_identical_queries_identical_outputs():
    bt = make_batch([50], [1], 8, 2, 16, 4, seed=10)
    bt.q[0, 1] = bt.q[0, 0]
    bt.q[0, 5] = bt.q[0, 0]
    kc, vc, ks, vs = _written(bt)
    out, _ = _attend(bt, kc, vc, ks, vs)
    assert np.array_equal(out[0, 0], out[0, 1])
    assert not np.allclose(out[0, 0], out[0, 5])  # other group, other keys


def test_verify_row_equals_decode_of_truncated_sequence():
    bt = make_batch([30], [4], 4, 2, 16, 4, seed=12)
    kc, vc, ks, vs = _written(bt)
    out, _ = _attend(bt, kc, vc, ks, vs)
    for i in range(4):
        L = 30 - 4 + i + 1
        o1, _ = paged_attention(bt.q[i:i + 1], kc, vc, bt.block_table, np.array([L]), np.array([0, 1]),
                                ks, vs, np.float32(0.25))
        np.testing.assert_allclose(out[i], o1[0], rtol=1e-13, atol=1e-15)


def test_scale_equivariance():
    bt = make_batch([45, 9], [2, 1], 4, 2, 16, 4, seed=13)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(0.25)
    out, _ = _attend(bt, kc, vc, ks, vs, sm)
    out2, _ = _attend(bt, kc, vc, ks, np.float32(vs * 2), sm)
    assert np.array_equal(out2, out * 2)
    # k_scale * 2 with sm_scale / 2 gives the same scores
    out3, _ = _attend(bt, kc, vc, np.float32(ks * 2), vs, np.float32(sm / 2))
    np.testing.assert_allclose(out3, out, rtol=1e-14, atol=1e-15)


def test_poisoned_slots_never_reach_outputs():
    bt = make_config(1)
    kc, vc, ks, vs = _written(bt)
    out, _ = _attend(bt, kc, vc, ks, vs)
    assert np.isfinite(out).all()
    # the tail of the last page of sequence 1 (257 = 64 * 4 + 1 tokens) is poison
    last = bt.block_table[1, 64]
    assert (kc[last, :, 1:, :] == 0x7F).all() and (vc[last, :, :, 1:] == 0x7F).all()


def test_split_bounds_partition():
    for L in (1, 63, 64, 65, 100, 257, 4096, 32768, 262144):
        for S in (1, 2, 3, 7, 64):
            for Lm in (L, L + 1, 3 * L, 262144):
                b = split_bounds(L, S, max_len=Lm)
                covered = []
                for lo, hi in b:
                    if hi > lo:
                        assert lo % 64 == 0
                        covered.extend(range(lo, hi))
                assert covered == list(range(L))


def test_split_bounds_share_one_size():
    """Every non-empty split but a sequence's last has the same size, set by
    the longest context; the longest sequence uses all S splits."""
    lens = [1024, 4096, 8192, 32768, 100, 1]
    S = 19
    C = -(-32768 // (S * 64)) * 64
    assert C == 1728
    for L in lens:
        b = split_bounds(L, S, max_len=max(lens))
        sizes = [hi - lo for lo, hi in b if hi > lo]
        assert len(sizes) == -(-L // C)
        assert all(x == C for x in sizes[:-1]) and 0 < sizes[-1] <= C
    assert len([1 for lo, hi in split_bounds(32768, S, max_len=32768) if hi > lo]) == S
    with pytest.raises(ValueError):
        split_bounds(100, 2, max_len=99)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 64])
def test_split_reduce_equals_unsplit(S):
    bt = make_batch([100, 257, 64, 3], [1, 4, 2, 1], 8, 2, 16, 4, seed=14)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(0.25)
    out, lse = _attend(bt, kc, vc, ks, vs, sm)
    ws = split_partials(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, ks, vs, sm, S,
                        granule=16)
    o2, lse2 = split_reduce(*ws)
    np.testing.assert_allclose(o2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)
    if S == 1:
        np.testing.assert_allclose(ws[0][:, :, 0, :] / ws[2][:, :, 0, None], out, rtol=1e-12)


def test_split_partials_brute_force():
    bt = make_batch([21], [2], 2, 1, 4, 4, seed=15)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(0.5)
    ws_o, ws_m, ws_l = split_partials(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens,
                                      ks, vs, sm, 3, granule=4)
    kt, vt = _codes_by_token(bt, kc, vc)
    import math
    bounds = [(0, 8), (8, 16), (16, 21)]
    for i in range(2):
        pos = 21 - 2 + i
        for s, (lo, hi) in enumerate(bounds):
            hi = min(hi, pos + 1)
            for h in range(2):
                sc = []
                for j in range(lo, hi):
                    acc = 0.0
                    for d in range(4):
                        acc += float(bt.q[i, h, d]) * float(e4m3_decode(np.array([kt[j, 0, d]]))[0]) * float(ks)
                    sc.append(acc * float(sm))
                m = max(sc)
                assert abs(ws_m[i, h, s] - m) < 1e-12
                w = [math.exp(x - m) for x in sc]
                assert abs(ws_l[i, h, s] - sum(w)) < 1e-12
                for d in range(4):
                    o = sum(w[j - lo] * float(e4m3_decode(np.array([vt[j, 0, d]]))[0]) * float(vs)
                            for j in range(lo, hi))
                    assert abs(ws_o[i, h, s, d] - o) < 1e-12


def test_split_reduce_empty_splits():
    o = np.zeros((1, 1, 3, 4))
    m = np.full((1, 1, 3), -np.inf)
    l = np.zeros((1, 1, 3))
    out, lse = split_reduce(o, m, l)
    assert (out == 0).all() and np.isneginf(lse).all()
    m[0, 0, 1] = 2.0
    l[0, 0, 1] = 4.0
    o[0, 0, 1] = [4.0, 8.0, -4.0, 0.0]
    out, lse = split_reduce(o, m, l)
    assert out[0, 0].tolist() == [1.0, 2.0, -1.0, 0.0]
    assert abs(lse[0, 0] - (2.0 + np.log(4.0))) < 1e-15


@pytest.mark.parametrize("mistake", ["gqa_modulo", "no_causal", "causal_off_by_one", "no_k_scale",
                                     "v_transposed_page"])
def test_pins_catch_planted_attention_mistakes(mistake):
    """A plausible mistake planted in a copy of the oracle's attention must
    make the SDPA pin fail."""
    import oracle.attention as A
    bt = make_batch([1, 64, 65, 200, 33], [1, 4, 1, 7, 33], 8, 2, 32, 16, seed=31)
    kc, vc, ks, vs = _written(bt)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    kt, vt = _codes_by_token(bt, kc, vc)
    ref = pins.sdpa_reference(bt, kt, vt, ks, vs, sm)

    def bad(q_f16, k_cache, v_cache, block_table, seq_lens, cu_q_lens, k_scale, v_scale, sm_scale):
        q = q_f16.astype(np.float64)
        Hq, Hkv = q.shape[1], k_cache.shape[1]
        G = Hq // Hkv
        out = np.zeros_like(q)
        for b in range(len(seq_lens)):
            L = int(seq_lens[b]); q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1]); T = q1 - q0
            kd, vd = A.gather_sequence_kv(k_cache, v_cache, block_table[b], L)
            if mistake == "v_transposed_page":
                # reading the dimension-major V page as if it were token-major
                P = k_cache.shape[2]
                j = np.arange(L)
                as_tok = v_cache.reshape(v_cache.shape[0], Hkv, P, -1)
                vd = e4m3_decode(as_tok[block_table[b][j // P].astype(np.int64), :, j % P, :])
            kd = kd * (1.0 if mistake == "no_k_scale" else float(k_scale))
            vd = vd * float(v_scale)
            for i in range(T):
                pos = L - T + i
                if mistake == "no_causal":
                    pos = L - 1
                if mistake == "causal_off_by_one":
                    pos = max(L - T + i - 1, 0) if T > 1 else L - 1
                for h in range(Hq):
                    g = h % Hkv if mistake == "gqa_modulo" else h // G
                    s = float(sm_scale) * (kd[:pos + 1, g] @ q[q0 + i, h])
                    w = np.exp(s - s.max())
                    out[q0 + i, h] = w @ vd[:pos + 1, g] / w.sum()
        return out

    got = bad(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, ks, vs, sm)
    assert not np.allclose(got, ref, rtol=1e-6, atol=1e-8)
