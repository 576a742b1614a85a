"""The Python binding's shape checks: the C ABI sees pointers, not buffer
sizes, so the binding refuses (ValueError / TypeError, on the host) an output
of the wrong shape, a block table or context-length vector with the wrong
number of sequences, and a workspace that is not a contiguous fp32 GPU tensor,
before anything is launched: the output buffer keeps its poison."""

import numpy as np
import pytest
import torch

from synth import make_batch
from tests.gpu_common import DeviceBatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


@pytest.fixture(scope="module")
def setup(K):
    bt = make_batch([40, 70, 9], [1, 1, 1], 8, 2, 64, 16, seed=171)
    db = DeviceBatch(bt)
    vb = make_batch([40, 70, 9], [2, 3, 1], 8, 2, 64, 16, seed=172)
    dv = DeviceBatch(vb)
    return bt, db, vb, dv


def _calls(K, bt, db, vb, dv):
    """Every attention wrapper as a function of (out, block_table, seq_lens, workspace)."""
    kf = torch.zeros(db.k_cache.shape, dtype=torch.float16, device="cuda")
    vf = torch.zeros(db.v_cache.shape, dtype=torch.float16, device="cuda")
    k_new = torch.zeros((bt.batch, bt.n_kv_heads, bt.head_dim), dtype=torch.float16, device="cuda")
    kv_new = torch.zeros((vb.total_q, vb.n_kv_heads, vb.head_dim), dtype=torch.float16, device="cuda")
    mq = int(vb.q_lens.max())
    return {
        "decode": (db.q, lambda o, bt_, sl, ws: K.paged_attn_e4m3_decode(
            db.q, db.k_cache, db.v_cache, bt_, sl, 1.0, 1.0, 0.125, num_splits=2, workspace=ws, out=o)),
        "decode_append": (db.q, lambda o, bt_, sl, ws: K.paged_attn_e4m3_decode_append(
            db.q, k_new, k_new, db.k_cache, db.v_cache, bt_, sl, 1.0, 1.0, 0.125, num_splits=2, workspace=ws,
            out=o)),
        "f16_decode": (db.q, lambda o, bt_, sl, ws: K.paged_attn_f16_decode(
            db.q, kf, vf, bt_, sl, 0.125, num_splits=2, workspace=ws, out=o)),
        "verify": (dv.q, lambda o, bt_, sl, ws: K.paged_attn_e4m3_verify(
            dv.q, dv.cu_q, mq, dv.k_cache, dv.v_cache, bt_, sl, 1.0, 1.0, 0.125, num_splits=2, workspace=ws,
            out=o)),
        "verify_append": (dv.q, lambda o, bt_, sl, ws: K.paged_attn_e4m3_verify_append(
            dv.q, kv_new, kv_new, dv.cu_q, mq, dv.k_cache, dv.v_cache, bt_, sl, 1.0, 1.0, 0.125, num_splits=2,
            workspace=ws, out=o)),
        "f16_verify": (dv.q, lambda o, bt_, sl, ws: K.paged_attn_f16_verify(
            dv.q, dv.cu_q, mq, kf, vf, bt_, sl, 0.125, num_splits=2, workspace=ws, out=o)),
    }


@pytest.mark.parametrize("call", ["decode", "decode_append", "f16_decode", "verify", "verify_append", "f16_verify"])
@pytest.mark.parametrize("fault", ["out_shape", "block_table_rows", "seq_lens_rows", "ws_on_host", "ws_dtype",
                                   "ws_strided"])
def test_wrapper_refuses_before_launch(K, setup, call, fault):
    bt, db, vb, dv = setup
    q, fn = _calls(K, bt, db, vb, dv)[call]
    ref = db if call in ("decode", "decode_append", "f16_decode") else dv
    rows = q.shape[0]
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
    ws = K.workspace(rows, q.shape[1], q.shape[2], 2)
    block_table, seq_lens = ref.block_table, ref.seq_lens
    expect = ValueError
    if fault == "out_shape":
        out = torch.full((rows + 1,) + tuple(q.shape[1:]), float("nan"), dtype=torch.float16, device="cuda")
    elif fault == "block_table_rows":
        block_table = torch.cat([block_table, block_table[:1]]).contiguous()
    elif fault == "seq_lens_rows":
        seq_lens = seq_lens[:-1].contiguous()
    elif fault == "ws_on_host":
        ws = ws.cpu()
    elif fault == "ws_dtype":
        ws, expect = ws.to(torch.float16), TypeError
    elif fault == "ws_strided":
        ws = torch.zeros(2 * ws.numel(), dtype=torch.float32, device="cuda")[::2]
    torch.cuda.synchronize()
    with pytest.raises(expect):
        fn(out, block_table, seq_lens, ws)
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "the output was written although the call was refused"


def test_wrappers_accept_the_valid_arguments(K, setup):
    """The same calls with nothing wrong run (so the refusals above come from the faults)."""
    bt, db, vb, dv = setup
    for name, (q, fn) in _calls(K, bt, db, vb, dv).items():
        ref = db if name in ("decode", "decode_append", "f16_decode") else dv
        out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
        ws = K.workspace(q.shape[0], q.shape[1], q.shape[2], 2)
        fn(out, ref.block_table, ref.seq_lens, ws)
        torch.cuda.synchronize()
        assert out.shape == q.shape, name
