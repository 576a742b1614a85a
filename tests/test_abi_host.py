"""Host-side checks of the C ABI (CPU only: no call here reaches a kernel).

Every invalid-argument case is rejected by the library's host validation
before any HIP call, so these run without a GPU. Fake device pointers are
only ever passed together with an argument that is rejected.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from fp8_quantised_paged_amd import kvfp8

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvfp8.h")
L = kvfp8.raw()
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first
MIS = 0x10001


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("kv_quant_write", "kv_calibrate_amax", "paged_attn_e4m3_decode", "paged_attn_e4m3_verify",
              "split_reduce_fp32"):
        assert n in names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(kvfp8.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvfp8.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported
    # nothing else of ours leaks out
    ours = {s for s in exported if s.startswith(("kv", "paged", "split", "_ZN5kvfp8"))}
    assert ours == set(names)


def test_status_strings():
    assert kvfp8.status_str(0) == "KVFP8_OK"
    assert kvfp8.status_str(2) == "KVFP8_BAD_SCALE"
    assert kvfp8.status_str(6) == "KVFP8_HIP_ERROR"
    assert kvfp8.status_str(99) == "KVFP8_UNKNOWN_STATUS"


def test_attn_kernel_name_follows_the_launch_rule():
    """The instantiation each attention call would launch (no launch; the
    device's CU count is the 256 of an MI355X, also the fallback without a GPU)."""
    name = kvfp8.kvfp8_attn_kernel_name
    # decode: one workgroup per (sequence, kv-head, split) and the grid fits one round -> 8 wavefronts
    assert name(32, 32, 4, 128, 16, 256, 1, 2) == "attn_split_kernel<128,16,1,8,false>"
    # at most one 64-key tile per wavefront (splits of <= 512 keys) -> the short start-up
    assert name(32, 8, 1, 128, 16, 256, 1, 8) == "attn_split_kernel<128,16,1,8,true>"
    # more workgroups than compute units -> 4 wavefronts, two workgroups per CU
    assert name(4, 32, 4, 128, 64, 4096, 1, 64) == "attn_split_kernel<128,64,1,4,false>"
    # 32 query rows per kv-head (MTP3 at a GQA group of 8) -> two 16-row blocks
    assert name(16, 32, 4, 128, 16, 2048, 4, 19) == "attn_split_kernel<128,16,2,4,false>"
    # longer chunks -> the query-tiled chunk kernel (one split only)
    assert name(1, 32, 4, 128, 16, 2004, 2048, 1) == "attn_chunk_kernel<128,16>"
    assert name(1, 32, 4, 128, 16, 2004, 2048, 2) == ""
    assert name(32, 32, 4, 128, 16, 256, 1, 2, True) == "attn_split_f16_kernel<128,16,1,8>"
    assert name(1, 32, 4, 128, 16, 2004, 2048, 1, True) == ""
    for bad in ((32, 32, 4, 96, 16, 256, 1, 2), (32, 30, 4, 128, 16, 256, 1, 2), (32, 32, 4, 128, 12, 256, 1, 2),
                (0, 32, 4, 128, 16, 256, 1, 2), (32, 32, 4, 128, 16, 256, 1, 257)):
        assert name(*bad) == "", bad

def test_decode_append_noalloc_rejects_before_any_hip_call():
    """The entry point without a workspace refuses split partials larger than its
    static scratch (KVFP8_WORKSPACE) and a NULL output, before touching the GPU."""
    f = L.paged_attn_e4m3_decode_append_noalloc
    base = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, B=64, hq=32, hkv=4, d=128, p=16,
                mp=64, ks=1.0, vs=1.0, sm=0.1, S=128, out=FAKE)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["sl"], a["B"], a["hq"], a["hkv"], a["d"],
                 a["p"], a["mp"], a["ks"], a["vs"], a["sm"], a["S"], a["out"], None)

    assert kvfp8.kvfp8_attn_workspace_bytes(64, 32, 128, 128) > kvfp8.NOALLOC_SCRATCH_BYTES
    assert call() == kvfp8.WORKSPACE
    assert "static scratch" in kvfp8.last_error()
    assert call(out=None) == kvfp8.INVALID_ARG
    assert call(S=2, ks=float("nan")) == kvfp8.BAD_SCALE
    assert call(S=2, d=96) == kvfp8.UNSUPPORTED
    assert call(S=2, kn=None) == kvfp8.INVALID_ARG
    assert call(S=2, q=MIS) == kvfp8.INVALID_ARG
    assert call(B=0, S=2) == kvfp8.OK

def test_workspace_bytes():
    assert kvfp8.kvfp8_attn_workspace_bytes(32, 32, 128, 4) == 32 * 32 * 4 * 130 * 4
    assert kvfp8.kvfp8_attn_workspace_bytes(4, 32, 128, 64) == 4 * 32 * 64 * 130 * 4
    assert kvfp8.kvfp8_attn_workspace_bytes(0, 32, 128, 4) == 0
    assert kvfp8.kvfp8_attn_workspace_bytes(3, 8, 64, -1) == 0


def write(**kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, n=4, hkv=4, d=128, p=16, pages=10, ks=1.0, vs=1.0, kc=FAKE, vc=FAKE)
    a.update(kw)
    return L.kv_quant_write(a["k"], a["v"], a["slots"], a["n"], a["hkv"], a["d"], a["p"], a["pages"],
                            a["ks"], a["vs"], a["kc"], a["vc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), kvfp8.INVALID_ARG),
    (dict(hkv=0), kvfp8.INVALID_ARG),
    (dict(d=96), kvfp8.UNSUPPORTED),
    (dict(p=12), kvfp8.UNSUPPORTED),
    (dict(p=128), kvfp8.UNSUPPORTED),
    (dict(ks=float("nan")), kvfp8.BAD_SCALE),
    (dict(ks=float("inf")), kvfp8.BAD_SCALE),
    (dict(vs=0.0), kvfp8.BAD_SCALE),
    (dict(vs=-0.5), kvfp8.BAD_SCALE),
    (dict(ks=1e-40), kvfp8.BAD_SCALE),
    (dict(k=None), kvfp8.INVALID_ARG),
    (dict(slots=None), kvfp8.INVALID_ARG),
    (dict(vc=None), kvfp8.INVALID_ARG),
    (dict(k=MIS), kvfp8.INVALID_ARG),
    (dict(kc=MIS), kvfp8.INVALID_ARG),
])
def test_quant_write_rejects(kw, status):
    assert write(**kw) == status
    assert kvfp8.last_error()


def test_quant_write_zero_tokens_is_a_noop():
    assert write(n=0, k=None, v=None) == kvfp8.OK
    # but the scale gate still applies: no unit-scale fallback, even for an empty write
    assert write(n=0, ks=0.0) == kvfp8.BAD_SCALE


def decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, b=2, hq=32, hkv=4, d=128, p=16, mp=8, ks=0.1,
             vs=0.1, sm=0.088, s=1, ws=None, wsb=0, out=FAKE)
    a.update(kw)
    return L.paged_attn_e4m3_decode(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["b"], a["hq"], a["hkv"],
                                    a["d"], a["p"], a["mp"], a["ks"], a["vs"], a["sm"], a["s"], a["ws"],
                                    a["wsb"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), kvfp8.INVALID_ARG),
    (dict(bt=None), kvfp8.INVALID_ARG),
    (dict(sl=None), kvfp8.INVALID_ARG),
    (dict(b=-1), kvfp8.INVALID_ARG),
    (dict(hq=30), kvfp8.INVALID_ARG),
    (dict(hkv=0), kvfp8.INVALID_ARG),
    (dict(mp=0), kvfp8.INVALID_ARG),
    (dict(d=80), kvfp8.UNSUPPORTED),
    (dict(p=128), kvfp8.UNSUPPORTED),
    (dict(s=0), kvfp8.UNSUPPORTED),
    (dict(s=257), kvfp8.UNSUPPORTED),
    (dict(hq=64, hkv=1), kvfp8.UNSUPPORTED),
    (dict(ks=float("nan")), kvfp8.BAD_SCALE),
    (dict(vs=0.0), kvfp8.BAD_SCALE),
    (dict(sm=-1.0), kvfp8.BAD_SCALE),
    (dict(sm=float("inf")), kvfp8.BAD_SCALE),
    (dict(ks=1e-30, sm=1e-20), kvfp8.BAD_SCALE),  # product underflows fp32
    (dict(ks=1e30, sm=1e20), kvfp8.BAD_SCALE),  # product overflows fp32
    (dict(q=MIS), kvfp8.INVALID_ARG),
    (dict(vc=MIS), kvfp8.INVALID_ARG),
    (dict(out=MIS), kvfp8.INVALID_ARG),
    (dict(out=None), kvfp8.INVALID_ARG),
    (dict(s=4), kvfp8.WORKSPACE),
    (dict(s=4, ws=FAKE, wsb=1024), kvfp8.WORKSPACE),
    (dict(s=4, ws=MIS, wsb=1 << 30), kvfp8.INVALID_ARG),
])
def test_decode_rejects(kw, status):
    assert decode(**kw) == status


def test_decode_empty_batch_is_a_noop():
    assert decode(b=0) == kvfp8.OK


def append(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, b=2, hq=32, hkv=4, d=128, p=16, mp=8,
             ks=0.1, vs=0.1, sm=0.088, s=1, ws=None, wsb=0, out=FAKE)
    a.update(kw)
    return L.paged_attn_e4m3_decode_append(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["sl"], a["b"],
                                           a["hq"], a["hkv"], a["d"], a["p"], a["mp"], a["ks"], a["vs"], a["sm"],
                                           a["s"], a["ws"], a["wsb"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), kvfp8.INVALID_ARG),
    (dict(vn=None), kvfp8.INVALID_ARG),
    (dict(kn=MIS), kvfp8.INVALID_ARG),
    (dict(q=None), kvfp8.INVALID_ARG),
    (dict(ks=0.0), kvfp8.BAD_SCALE),
    (dict(d=96), kvfp8.UNSUPPORTED),
    (dict(hq=64, hkv=1), kvfp8.UNSUPPORTED),
    (dict(s=4), kvfp8.WORKSPACE),
])
def test_decode_append_rejects(kw, status):
    assert append(**kw) == status


def test_decode_append_empty_batch_is_a_noop():
    assert append(b=0, kn=None, vn=None) == kvfp8.OK


def verify_append(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, cu=FAKE, tq=8, mq=4, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, b=2, hq=32,
             hkv=4, d=128, p=16, mp=8, ks=0.1, vs=0.1, sm=0.088, s=1, ws=None, wsb=0, out=FAKE)
    a.update(kw)
    return L.paged_attn_e4m3_verify_append(a["q"], a["kn"], a["vn"], a["cu"], a["tq"], a["mq"], a["kc"], a["vc"],
                                           a["bt"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"], a["p"], a["mp"],
                                           a["ks"], a["vs"], a["sm"], a["s"], a["ws"], a["wsb"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), kvfp8.INVALID_ARG),
    (dict(vn=None), kvfp8.INVALID_ARG),
    (dict(vn=MIS), kvfp8.INVALID_ARG),
    (dict(cu=None), kvfp8.INVALID_ARG),
    (dict(mq=0), kvfp8.INVALID_ARG),
    (dict(vs=float("nan")), kvfp8.BAD_SCALE),
    (dict(mq=5), kvfp8.UNSUPPORTED),  # 5 tokens x 8 heads = 40 rows per kv-head
    (dict(s=2), kvfp8.WORKSPACE),
])
def test_verify_append_rejects(kw, status):
    assert verify_append(**kw) == status


def test_verify_append_empty_is_a_noop():
    assert verify_append(tq=0, kn=None, vn=None) == kvfp8.OK


def verify(**kw):
    a = dict(q=FAKE, cu=FAKE, tq=8, mq=4, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, b=2, hq=32, hkv=4, d=128,
             p=16, mp=8, ks=0.1, vs=0.1, sm=0.088, s=1, ws=None, wsb=0, out=FAKE)
    a.update(kw)
    return L.paged_attn_e4m3_verify(a["q"], a["cu"], a["tq"], a["mq"], a["kc"], a["vc"], a["bt"], a["sl"],
                                    a["b"], a["hq"], a["hkv"], a["d"], a["p"], a["mp"], a["ks"], a["vs"],
                                    a["sm"], a["s"], a["ws"], a["wsb"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), kvfp8.INVALID_ARG),
    (dict(tq=-1), kvfp8.INVALID_ARG),
    (dict(mq=0), kvfp8.INVALID_ARG),
    (dict(ks=0.0), kvfp8.BAD_SCALE),
    (dict(d=256), kvfp8.UNSUPPORTED),
    (dict(s=2), kvfp8.WORKSPACE),
    # a long chunk (64 query tokens x 8 heads) goes to the chunk kernel, which takes no splits
    (dict(mq=64, tq=128, s=2, ws=FAKE, wsb=1 << 30), kvfp8.UNSUPPORTED),
])
def test_verify_rejects(kw, status):
    assert verify(**kw) == status


def reduce(**kw):
    a = dict(o=FAKE, m=FAKE, l=FAKE, r=4, hq=32, d=128, s=8, out=FAKE, lse=None)
    a.update(kw)
    return L.split_reduce_fp32(a["o"], a["m"], a["l"], a["r"], a["hq"], a["d"], a["s"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(r=-1), kvfp8.INVALID_ARG),
    (dict(hq=0), kvfp8.INVALID_ARG),
    (dict(d=32), kvfp8.UNSUPPORTED),
    (dict(s=0), kvfp8.UNSUPPORTED),
    (dict(s=300), kvfp8.UNSUPPORTED),
    (dict(o=None), kvfp8.INVALID_ARG),
    (dict(out=None), kvfp8.INVALID_ARG),
    (dict(o=FAKE + 4), kvfp8.INVALID_ARG),
])
def test_split_reduce_rejects(kw, status):
    assert reduce(**kw) == status


def test_split_reduce_zero_rows_is_a_noop():
    assert reduce(r=0, o=None) == kvfp8.OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, -1, 8, FAKE, FAKE), kvfp8.INVALID_ARG),
    ((FAKE, 2, -8, FAKE, FAKE), kvfp8.INVALID_ARG),
    ((FAKE, 2, 8, None, FAKE), kvfp8.INVALID_ARG),
    ((FAKE, 2, 8, FAKE, None), kvfp8.INVALID_ARG),
    ((None, 2, 8, FAKE, FAKE), kvfp8.INVALID_ARG),
    ((MIS, 2, 8, FAKE, FAKE), kvfp8.INVALID_ARG),
    ((FAKE, 0, 8, FAKE, FAKE), kvfp8.OK),
])
def test_calibrate_rejects(args, status):
    assert L.kv_calibrate_amax(*args, None) == status


def test_codec_helpers_reject():
    assert L.kvfp8_e4m3_encode_f32(FAKE, FAKE, -1, None) == kvfp8.INVALID_ARG
    assert L.kvfp8_e4m3_decode_f32(None, FAKE, 5, None) == kvfp8.INVALID_ARG
    assert L.kvfp8_e4m3_decode_f32(FAKE, FAKE, 0, None) == kvfp8.OK


def check_args(bt=FAKE, sl=FAKE, cu=None, b=2, mp=8, p=16, npg=64, tq=0, mq=0, res=FAKE):
    return L.kvfp8_check_paged_args(bt, sl, cu, b, mp, p, npg, tq, mq, res, None)


@pytest.mark.parametrize("kw,status", [
    (dict(b=-1), kvfp8.INVALID_ARG),
    (dict(mp=0), kvfp8.INVALID_ARG),
    (dict(p=0), kvfp8.INVALID_ARG),
    (dict(npg=-1), kvfp8.INVALID_ARG),
    (dict(cu=FAKE, tq=-1), kvfp8.INVALID_ARG),
    (dict(cu=FAKE, mq=-1), kvfp8.INVALID_ARG),
    (dict(bt=None), kvfp8.INVALID_ARG),
    (dict(sl=None), kvfp8.INVALID_ARG),
    (dict(res=None), kvfp8.INVALID_ARG),
    (dict(res=FAKE + 2), kvfp8.INVALID_ARG),
])
def test_check_paged_args_rejects(kw, status):
    assert check_args(**kw) == status


def test_check_paged_args_empty_batch_is_a_noop():
    assert check_args(b=0, bt=None, sl=None, res=None) == kvfp8.OK
