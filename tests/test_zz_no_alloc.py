"""paged_attn_e4m3_decode_append_noalloc, the decode step whose FP32 split
partials live in the library's static per-GPU scratch, against
paged_attn_e4m3_decode_append with a caller-owned workspace: two calls in a
row on one GPU, the second with a smaller input, each bit for bit equal to the
workspace entry point (cache bytes and output) and within the attention
tolerance of the oracle. Also a split count whose partials exceed the scratch,
refused before any launch.
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention
from synth import make_batch
from tests.gpu_common import DeviceBatch, assert_close_attn, dev, oracle_caches, oracle_scales

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def _step_both_ways(K, bt, S):
    _, sc = oracle_scales(bt)
    ks, vs = float(sc[0]), float(sc[1])
    sm = float(np.float32(1.0 / np.sqrt(bt.head_dim)))
    db = DeviceBatch(bt)
    prior, new = dev(bt.prior_rows()), dev(bt.new_token_rows())
    K.kv_quant_write(db.k[prior].contiguous(), db.v[prior].contiguous(), db.slots[prior].contiguous(), ks, vs,
                     db.k_cache, db.v_cache)
    kc_ws, vc_ws = db.k_cache.clone(), db.v_cache.clone()
    k_new, v_new = db.k[new].contiguous(), db.v[new].contiguous()
    out = torch.full_like(db.q, float("nan"))
    K.paged_attn_e4m3_decode_append_noalloc(db.q, k_new, v_new, db.k_cache, db.v_cache, db.block_table,
                                            db.seq_lens, ks, vs, sm, num_splits=S, out=out)
    ws = K.workspace(bt.batch, bt.n_q_heads, bt.head_dim, S) if S > 1 else None
    if ws is not None:
        K.poison_partials(ws, bt.batch, bt.n_q_heads, bt.head_dim, S)
    ref_out = K.paged_attn_e4m3_decode_append(db.q, k_new, v_new, kc_ws, vc_ws, db.block_table, db.seq_lens, ks,
                                              vs, sm, num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), ref_out.cpu().numpy().view(np.uint16))
    assert torch.equal(db.k_cache, kc_ws) and torch.equal(db.v_cache, vc_ws)
    kc, vc = oracle_caches(bt, sc[0], sc[1])
    assert np.array_equal(db.k_cache.cpu().numpy(), kc)
    assert np.array_equal(db.v_cache.cpu().numpy(), vc)
    ref, _ = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens, sc[0], sc[1], sm)
    assert_close_attn(got, ref, f"noalloc B={bt.batch} S={S}", strict=True)


def test_noalloc_two_calls_second_smaller(K):
    # first call: 24 sequences up to 3,000 keys, 12 splits (24 x 32 x 12 partials: 4.8 MB of the 16 MiB)
    big = make_batch([3000 - 97 * i for i in range(24)], [1] * 24, 32, 4, 128, 16, seed=181)
    _step_both_ways(K, big, 12)
    # second call on the same scratch: 3 sequences, 3 splits, page 64, head_dim 64
    small = make_batch([700, 65, 1], [1] * 3, 16, 4, 64, 64, seed=182)
    _step_both_ways(K, small, 3)
    # and unsplit (no scratch used)
    _step_both_ways(K, small, 1)


def test_noalloc_refuses_partials_beyond_the_scratch(K):
    bt = make_batch([600] * 64, [1] * 64, 32, 4, 128, 16, seed=183)
    S = 128
    assert K.kvfp8_attn_workspace_bytes(bt.batch, bt.n_q_heads, bt.head_dim, S) > K.NOALLOC_SCRATCH_BYTES
    db = DeviceBatch(bt)
    out = torch.full_like(db.q, float("nan"))
    k_new = torch.zeros((bt.batch, bt.n_kv_heads, bt.head_dim), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    with pytest.raises(K.KVFP8Error) as e:
        K.paged_attn_e4m3_decode_append_noalloc(db.q, k_new, k_new, db.k_cache, db.v_cache, db.block_table,
                                                db.seq_lens, 1.0, 1.0, 0.1, num_splits=S, out=out)
    assert e.value.status == K.WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert (db.k_cache == 0x7F).all()  # nothing appended
