"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (same split counts). Cache bytes and scales are
compared bit for bit; attention outputs are compared on sampled sequences,
which the oracle recomputes one by one, and checked finite everywhere.
"""

import numpy as np
import pytest
import torch

from oracle import calibrate_amax, paged_attention
from synth import make_config
from synth.workloads import make_mixed_calibration
from tests.gpu_common import DeviceBatch, assert_close_attn, dev, oracle_caches, report

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def _scales_bit_exact(K, ck, cv):
    x = np.stack([ck.reshape(-1), cv.reshape(-1)])
    amax, scale, st = K.kv_calibrate_amax(dev(x))
    ra, rs, rst = calibrate_amax(x)
    assert st == rst == 0
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    return rs


def _sequence_pages(bt, rows):
    pages = []
    for b in rows:
        n = -(-int(bt.seq_lens[b]) // bt.page_size)
        pages.extend(bt.block_table[b, :n].tolist())
    return np.array(sorted(pages))


def _write_all(K, bt, sc):
    db = DeviceBatch(bt)
    K.kv_quant_write(db.k, db.v, db.slots, float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    return db


def _check_cache_bytes(db, bt, sc, rows=None):
    kc, vc = oracle_caches(bt, sc[0], sc[1], rows=rows)
    if rows is None:
        assert np.array_equal(db.k_cache.cpu().numpy(), kc)
        assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    else:
        pg = dev(_sequence_pages(bt, rows))
        assert np.array_equal(db.k_cache[pg].cpu().numpy(), kc[pg.cpu().numpy()])
        assert np.array_equal(db.v_cache[pg].cpu().numpy(), vc[pg.cpu().numpy()])
    return kc, vc


def _decode(K, db, bt, sc, S):
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:
        K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    out = K.paged_attn_e4m3_decode(db.q, db.k_cache, db.v_cache, db.block_table, db.seq_lens, float(sc[0]),
                                   float(sc[1]), float(sm), num_splits=S, workspace=ws)
    return out.cpu().numpy(), sm


def test_decode_4k_full(K):
    bt = make_config(2)
    sc = _scales_bit_exact(K, bt.calib_k, bt.calib_v)
    db = _write_all(K, bt, sc)
    kc, vc = _check_cache_bytes(db, bt, sc)  # every byte of the 128 MiB cache
    assert ((kc & 0x7F) == 0x7E).any() and ((vc & 0x7F) == 0x7E).any()  # saturation exercised
    S = K.default_splits(bt.batch, bt.n_kv_heads, 4096)
    out, sm = _decode(K, db, bt, sc, S)
    assert np.isfinite(out.astype(np.float32)).all()
    rows = [0, 13, 31]
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm, rows=rows)
    assert_close_attn(out[rows], ref[rows], "decode 4k")
    print("decode 4k S=%d max abs %.3g max rel %.3g" % ((S,) + report(out[rows], ref[rows])))


def test_mtp3_verify_full(K):
    bt = make_config(3)
    sc = _scales_bit_exact(K, bt.calib_k, bt.calib_v)
    db = _write_all(K, bt, sc)
    longest = [int(np.argmax(bt.seq_lens)), int(np.argmin(bt.seq_lens))]
    rows = sorted(set(longest + [5]))
    kc, vc = _check_cache_bytes(db, bt, sc, rows=rows)
    S = K.default_splits(bt.batch, bt.n_kv_heads, int(bt.seq_lens.max()), seq_lens=bt.seq_lens,
                                 n_q_heads=bt.n_q_heads, q_len=int(bt.q_lens.max()))
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    ws = K.workspace(bt.total_q, bt.n_q_heads, bt.head_dim, S)
    K.poison_partials(ws, bt.total_q, bt.n_q_heads, bt.head_dim, S)
    out = K.paged_attn_e4m3_verify(db.q, db.cu_q, 4, db.k_cache, db.v_cache, db.block_table, db.seq_lens,
                                   float(sc[0]), float(sc[1]), float(sm), num_splits=S, workspace=ws)
    out = out.cpu().numpy()
    assert np.isfinite(out.astype(np.float32)).all()
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm, rows=rows)
    qrows = np.concatenate([np.arange(bt.cu_q_lens[b], bt.cu_q_lens[b + 1]) for b in rows])
    assert_close_attn(out[qrows], ref[qrows], "mtp3 verify")
    print("mtp3 S=%d contexts %s max abs %.3g max rel %.3g" % ((S, bt.seq_lens[rows].tolist()) +
                                                              report(out[qrows], ref[qrows])))


def test_long_context_256k_64_splits(K):
    bt = make_config(4)
    sc = _scales_bit_exact(K, bt.calib_k, bt.calib_v)
    db = _write_all(K, bt, sc)
    del bt.k, bt.v  # the host copies are not needed any more beyond the sampled sequence
    rows = [2]
    bt2 = make_config(4)  # regenerate (seeded) for the oracle's own write of the sampled sequence
    kc, vc = _check_cache_bytes(db, bt2, sc, rows=rows)
    pages = _sequence_pages(bt2, rows)
    sat = int(((kc[pages] & 0x7F) == 0x7E).sum() + ((vc[pages] & 0x7F) == 0x7E).sum())
    assert sat > 0  # outlier channels drive codes into saturation
    out, sm = _decode(K, db, bt2, sc, 64)
    assert np.isfinite(out.astype(np.float32)).all()
    ref, _ = paged_attention(bt2.q, kc, vc, bt2.block_table, bt2.seq_lens, bt2.cu_q_lens, sc[0], sc[1], sm,
                             rows=rows)
    assert_close_attn(out[rows], ref[rows], "256k")
    print("256k S=64 saturated codes in sampled sequence %d, max abs %.3g max rel %.3g" %
          ((sat,) + report(out[rows], ref[rows])))


def test_mixed_layer_full(K):
    # 48 per-layer scales from 4,096 calibration tokens each, bit-exact
    x = make_mixed_calibration()
    amax, scale, st = K.kv_calibrate_amax(dev(x))
    ra, rs, rst = calibrate_amax(x)
    assert st == rst == 0
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    layer = 0
    sc = rs[2 * layer:2 * layer + 2]
    bt = make_config(5, layer=layer)
    db = DeviceBatch(bt)
    # prior context written first, then this step's 8 + 2,048 new tokens
    prior = dev(bt.prior_rows())
    new = dev(bt.new_token_rows())
    K.kv_quant_write(db.k[prior].contiguous(), db.v[prior].contiguous(), db.slots[prior].contiguous(),
                     float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    K.kv_quant_write(db.k[new].contiguous(), db.v[new].contiguous(), db.slots[new].contiguous(),
                     float(sc[0]), float(sc[1]), db.k_cache, db.v_cache)
    kc, vc = _check_cache_bytes(db, bt, sc)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    # decode rows 0..7 through the split kernel
    S = K.default_splits(8, bt.n_kv_heads, 8192)
    ws = K.workspace(8, bt.n_q_heads, bt.head_dim, S)
    dec = K.paged_attn_e4m3_decode(db.q[:8].contiguous(), db.k_cache, db.v_cache, db.block_table[:8].contiguous(),
                                   db.seq_lens[:8].contiguous(), float(sc[0]), float(sc[1]), float(sm),
                                   num_splits=S, workspace=ws).cpu().numpy()
    # the 2,048-token chunk over 30,000 prior tokens through the chunk kernel
    cu = dev(np.array([0, 2048], np.int32))
    chunk = K.paged_attn_e4m3_verify(db.q[8:].contiguous(), cu, 2048, db.k_cache, db.v_cache,
                                     db.block_table[8:].contiguous(), db.seq_lens[8:].contiguous(),
                                     float(sc[0]), float(sc[1]), float(sm)).cpu().numpy()
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(dec, ref[:8], "mixed decode rows")
    assert_close_attn(chunk, ref[8:], "mixed chunk rows")
    print("mixed layer decode S=%d max abs %.3g / chunk max abs %.3g" %
          (S, report(dec, ref[:8])[0], report(chunk, ref[8:])[0]))
