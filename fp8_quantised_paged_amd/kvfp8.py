"""Python binding of libkvfp8.so (argument marshalling only).

Every function has the name of the C entry point it calls. Tensors are
checked for dtype, device, shape and contiguity, then their data pointers and
the current HIP stream go to the library; all computation happens in the
library's HIP kernels. The library must have been built
(``python -m fp8_quantised_paged_amd.build``); importing this module fails
loudly otherwise -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvfp8.so")

OK, INVALID_ARG, BAD_SCALE, NONFINITE_INPUT, WORKSPACE, UNSUPPORTED, HIP_ERROR = range(7)

EXPORTED = (
    "kv_calibrate_amax",
    "kv_quant_write",
    "paged_attn_e4m3_decode",
    "paged_attn_e4m3_decode_append",
    "paged_attn_e4m3_decode_append_noalloc",
    "paged_attn_e4m3_verify",
    "paged_attn_e4m3_verify_append",
    "paged_attn_f16_decode",
    "paged_attn_f16_verify",
    "split_reduce_fp32",
    "kvfp8_attn_workspace_bytes",
    "kvfp8_attn_kernel_name",
    "kvfp8_status_str",
    "kvfp8_last_error",
    "kvfp8_e4m3_encode_f32",
    "kvfp8_e4m3_decode_f32",
    "kvfp8_check_paged_args",
    "kvfp8_scale_overlay_write",
    "kvfp8_scale_overlay_read",
)


class KVFP8Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_str(status)} ({detail})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m fp8_quantised_paged_amd.build` (no fallback path exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "kvfp8_status_str": (ctypes.c_char_p, [I32]),
        "kvfp8_last_error": (ctypes.c_char_p, []),
        "kvfp8_attn_workspace_bytes": (SZ, [I64, I32, I32, I32]),
        "kvfp8_attn_kernel_name": (ctypes.c_char_p, [I32, I32, I32, I32, I32, I32, I32, I32, I32]),
        "kv_calibrate_amax": (I32, [P, I64, I64, P, P, P]),
        "kv_quant_write": (I32, [P, P, P, I64, I32, I32, I32, I64, F32, F32, P, P, P]),
        "paged_attn_e4m3_decode": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, F32, F32, F32,
                                         I32, P, SZ, P, P]),
        "paged_attn_e4m3_decode_append": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, F32,
                                                F32, F32, I32, P, SZ, P, P]),
        "paged_attn_e4m3_decode_append_noalloc": (I32, [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                        F32, F32, F32, I32, P, P]),
        "paged_attn_e4m3_verify": (I32, [P, P, I32, I32, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                         F32, F32, F32, I32, P, SZ, P, P]),
        "paged_attn_e4m3_verify_append": (I32, [P, P, P, P, I32, I32, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                F32, F32, F32, I32, P, SZ, P, P]),
        "paged_attn_f16_decode": (I32, [P, P, P, P, P, I32, I32, I32, I32, I32, I32, F32, I32, P, SZ, P, P]),
        "paged_attn_f16_verify": (I32, [P, P, I32, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, F32, I32,
                                        P, SZ, P, P]),
        "split_reduce_fp32": (I32, [P, P, P, I32, I32, I32, I32, P, P, P]),
        "kvfp8_e4m3_encode_f32": (I32, [P, P, I64, P]),
        "kvfp8_check_paged_args": (I32, [P, P, P, I32, I32, I32, I64, I32, I32, P, P]),
        "kvfp8_e4m3_decode_f32": (I32, [P, P, I64, P]),
        "kvfp8_scale_overlay_write": (I32, [ctypes.c_char_p, ctypes.c_char_p, I32, P, P]),
        "kvfp8_scale_overlay_read": (I32, [ctypes.c_char_p, ctypes.c_char_p, I32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def raw() -> ctypes.CDLL:
    """The loaded C library (for tests that call the ABI directly)."""
    return _lib


def library_path() -> str:
    return _LIB_PATH


def status_str(status: int) -> str:
    return _lib.kvfp8_status_str(int(status)).decode()


def last_error() -> str:
    return _lib.kvfp8_last_error().decode()


def _check(status: int, where: str) -> int:
    if status != OK:
        raise KVFP8Error(status, where, last_error())
    return status


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _check_rows(name: str, out: Optional[torch.Tensor], q: torch.Tensor, block_table: torch.Tensor,
                seq_lens: torch.Tensor, batch: int, workspace: Optional[torch.Tensor]):
    """Shape checks the C ABI cannot make (it sees pointers, not buffer sizes):
    out has q's shape, the block table and the context lengths have one row per
    sequence, and a workspace is a contiguous fp32 GPU tensor."""
    if out is not None and tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"{name}: out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    if block_table.shape[0] != batch:
        raise ValueError(f"{name}: block_table must have {batch} rows (one per sequence), got {block_table.shape[0]}")
    if seq_lens.shape[0] != batch:
        raise ValueError(f"{name}: seq_lens must have {batch} entries (one per sequence), got {seq_lens.shape[0]}")
    if workspace is not None:
        _need(workspace, "workspace", torch.float32)


def kvfp8_attn_workspace_bytes(n_rows: int, n_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(_lib.kvfp8_attn_workspace_bytes(n_rows, n_q_heads, head_dim, num_splits))


def kvfp8_attn_kernel_name(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, page_size: int,
                           max_pages_per_seq: int, max_q_len: int, num_splits: int, f16_kv: bool = False) -> str:
    """Kernel instantiation an attention call with these arguments launches ("" if none)."""
    return _lib.kvfp8_attn_kernel_name(batch, n_q_heads, n_kv_heads, head_dim, page_size, max_pages_per_seq,
                                       max_q_len, num_splits, int(bool(f16_kv))).decode()

VERIFY_ONE_PER_CU_BYTES = 1.2e6  # KV bytes per compute unit up to which verify runs one workgroup per CU


def default_splits(batch: int, n_kv_heads: int, max_seq_len: int, total_keys: Optional[int] = None,
                   cus: int = 256, seq_lens=None, n_q_heads: Optional[int] = None, q_len: int = 1,
                   head_dim: int = 128, kv_elem_bytes: int = 1) -> int:
    """Split count for the split kernel (host-side heuristic).

    Aims for one round of equal-work workgroups over the compute units. Decode
    (at most 16 query rows per kv-head: q_len times the GQA group n_q_heads /
    n_kv_heads) runs 8-wavefront workgroups, one per CU. Verify runs
    4-wavefront workgroups: one per CU while the call's KV bytes (keys x
    n_kv_heads x head_dim x 2 x kv_elem_bytes) stay within
    VERIFY_ONE_PER_CU_BYTES per CU, where start-up and tail dominate, and two
    per CU above it, where the bytes they keep in flight pay off (measured on the
    MTP3 workload: 0.83 MB per CU over E4M3 pages runs fastest at one per CU,
    1.66 MB per CU over fp16 pages at two). All sequences of a call share one
    split size, set by the longest context and the split count, so a shorter
    sequence fills fewer splits. With the context lengths known on the host
    (seq_lens), this returns the split count with the most non-empty splits,
    over all sequences and kv-heads, that still fit in those slots (the
    smallest such count). Otherwise the keys (total_keys, or batch *
    max_seq_len) are divided into that many shares and the longest sequence is
    split into shares of that size. Splits hold at least 512 keys (unless there
    is only one); at most 256 splits."""
    heads = max(1, n_kv_heads)
    group = (n_q_heads // heads) if n_q_heads else 1
    keys = (sum(int(x) for x in seq_lens) if seq_lens is not None
            else (total_keys if total_keys is not None else batch * max_seq_len))
    kv_bytes = keys * heads * head_dim * 2 * kv_elem_bytes
    verify = q_len * group > 16
    slots = 2 * cus if (verify and kv_bytes > VERIFY_ONE_PER_CU_BYTES * cus) else cus
    if seq_lens is not None:
        lens = [int(x) for x in seq_lens]
        lmax = max(lens) if lens else 0
        if lmax <= 0:
            return 1
        best, best_used = 1, 0
        for s in range(1, 257):
            chunk = -(-lmax // (64 * s)) * 64
            if chunk < 512 and s > 1:
                break
            used = sum(-(-L // chunk) for L in lens if L > 0) * heads
            if best_used < used <= slots:  # ties keep the smaller count (fewer empty splits)
                best, best_used = s, used
        return best
    total = (total_keys if total_keys is not None else batch * max_seq_len) * heads
    share = max(512, -(-total // slots))
    s = -(-max(1, max_seq_len) // share)
    return int(max(1, min(s, 256)))


def workspace(n_rows: int, n_q_heads: int, head_dim: int, num_splits: int,
              device="cuda") -> torch.Tensor:
    """An fp32 workspace of the size the attention calls need."""
    nbytes = kvfp8_attn_workspace_bytes(n_rows, n_q_heads, head_dim, num_splits)
    return torch.zeros(max(nbytes // 4, 1), dtype=torch.float32, device=device)


def poison_partials(ws: torch.Tensor, n_rows: int, n_q_heads: int, head_dim: int, num_splits: int):
    """Fill the partials with NaN, so that any partial the reduction uses
    without it having been written shows up in the output."""
    for t in workspace_views(ws, n_rows, n_q_heads, head_dim, num_splits):
        t.fill_(float("nan"))


def workspace_views(ws: torch.Tensor, n_rows: int, n_q_heads: int, head_dim: int, num_splits: int):
    """(ws_o, ws_m, ws_l) views of a workspace, in the layout the library writes."""
    units = n_rows * n_q_heads * num_splits
    o = ws[:units * head_dim].view(n_rows, n_q_heads, num_splits, head_dim)
    m = ws[units * head_dim:units * (head_dim + 1)].view(n_rows, n_q_heads, num_splits)
    l = ws[units * (head_dim + 1):units * (head_dim + 2)].view(n_rows, n_q_heads, num_splits)
    return o, m, l


def kv_calibrate_amax(x: torch.Tensor, amax: Optional[torch.Tensor] = None,
                      scale: Optional[torch.Tensor] = None, check: bool = True
                      ) -> Tuple[torch.Tensor, torch.Tensor, int]:
    """x: fp16 [n_tensors, n_elems]. Returns (amax, scale, status)."""
    _need(x, "x", torch.float16, 2)
    n_t, n_e = x.shape
    amax = torch.empty(n_t, dtype=torch.float32, device=x.device) if amax is None else amax
    scale = torch.empty(n_t, dtype=torch.float32, device=x.device) if scale is None else scale
    _need(amax, "amax", torch.float32, 1)
    _need(scale, "scale", torch.float32, 1)
    st = _lib.kv_calibrate_amax(x.data_ptr(), n_t, n_e, amax.data_ptr(), scale.data_ptr(), _stream())
    if check:
        _check(st, "kv_calibrate_amax")
    return amax, scale, st


def kv_quant_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                   v_scale: float, k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """k, v: fp16 [n_tokens, Hkv, D]; slot_mapping int64 [n_tokens];
    k_cache uint8 [pages, Hkv, P, D]; v_cache uint8 [pages, Hkv, D, P]."""
    _need(k, "k", torch.float16, 3)
    _need(v, "v", torch.float16, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(k_cache, "k_cache", torch.uint8, 4)
    _need(v_cache, "v_cache", torch.uint8, 4)
    n_tok, hkv, d = k.shape
    pages, hkv2, psz, d2 = k_cache.shape
    if v.shape != k.shape or slot_mapping.shape[0] != n_tok:
        raise ValueError("k, v and slot_mapping disagree")
    if (hkv2, d2) != (hkv, d) or tuple(v_cache.shape) != (pages, hkv, d, psz):
        raise ValueError("cache shapes disagree with k/v")
    _check(_lib.kv_quant_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), n_tok, hkv, d,
                               psz, pages, float(k_scale), float(v_scale), k_cache.data_ptr(),
                               v_cache.data_ptr(), _stream()), "kv_quant_write")


def _cache_dims(k_cache, v_cache, q_heads_dim):
    _need(k_cache, "k_cache", torch.uint8, 4)
    _need(v_cache, "v_cache", torch.uint8, 4)
    pages, hkv, psz, d = k_cache.shape
    if tuple(v_cache.shape) != (pages, hkv, d, psz):
        raise ValueError("v_cache must be [pages, Hkv, D, P]")
    if q_heads_dim != d:
        raise ValueError("head_dim of q and caches disagree")
    return hkv, psz, d


def paged_attn_e4m3_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, k_scale: float,
                           v_scale: float, sm_scale: float, num_splits: int = 1,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, partials_only: bool = False
                           ) -> Optional[torch.Tensor]:
    """q: fp16 [B, Hq, D]; block_table int32 [B, max_pages]; seq_lens int32 [B].
    Returns out fp16 [B, Hq, D] (None with partials_only)."""
    _need(q, "q", torch.float16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, hq, d = q.shape
    hkv, psz, _ = _cache_dims(k_cache, v_cache, d)
    if partials_only:
        out = None
    elif out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_e4m3_decode", out, q, block_table, seq_lens, B, workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    _check(_lib.paged_attn_e4m3_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       block_table.data_ptr(), seq_lens.data_ptr(), B, hq, hkv, d, psz,
                                       block_table.shape[1], float(k_scale), float(v_scale),
                                       float(sm_scale), int(num_splits), ws_ptr, ws_bytes, _ptr(out),
                                       _stream()), "paged_attn_e4m3_decode")
    return out


def paged_attn_e4m3_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                                  seq_lens: torch.Tensor, k_scale: float, v_scale: float, sm_scale: float,
                                  num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                                  out: Optional[torch.Tensor] = None, partials_only: bool = False
                                  ) -> Optional[torch.Tensor]:
    """Decode with each sequence's new token appended: k_new, v_new fp16 [B, Hkv, D] are quantised
    into key position seq_lens[b] - 1 (located through the block table), then attended.
    Returns out fp16 [B, Hq, D] (None with partials_only)."""
    _need(q, "q", torch.float16, 3)
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, hq, d = q.shape
    hkv, psz, _ = _cache_dims(k_cache, v_cache, d)
    if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
        raise ValueError(f"k_new/v_new must be [{B}, {hkv}, {d}]")
    if partials_only:
        out = None
    elif out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_e4m3_decode_append", out, q, block_table, seq_lens, B, workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    _check(_lib.paged_attn_e4m3_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                              k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                              seq_lens.data_ptr(), B, hq, hkv, d, psz, block_table.shape[1],
                                              float(k_scale), float(v_scale), float(sm_scale), int(num_splits),
                                              ws_ptr, ws_bytes, _ptr(out), _stream()),
           "paged_attn_e4m3_decode_append")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20  # KVFP8_NOALLOC_SCRATCH_BYTES


def paged_attn_e4m3_decode_append_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                          k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                                          seq_lens: torch.Tensor, k_scale: float, v_scale: float, sm_scale: float,
                                          num_splits: int = 1, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attn_e4m3_decode_append with the split partials in the library's static per-GPU scratch
    (the C call allocates nothing; pass `out` to allocate nothing here either). Returns out."""
    _need(q, "q", torch.float16, 3)
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, hq, d = q.shape
    hkv, psz, _ = _cache_dims(k_cache, v_cache, d)
    if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
        raise ValueError(f"k_new/v_new must be [{B}, {hkv}, {d}]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_e4m3_decode_append_noalloc", out, q, block_table, seq_lens, B, None)
    _check(_lib.paged_attn_e4m3_decode_append_noalloc(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                                      k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                                      seq_lens.data_ptr(), B, hq, hkv, d, psz, block_table.shape[1],
                                                      float(k_scale), float(v_scale), float(sm_scale),
                                                      int(num_splits), out.data_ptr(), _stream()),
           "paged_attn_e4m3_decode_append_noalloc")
    return out

def paged_attn_e4m3_verify(q: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int,
                           k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, k_scale: float, v_scale: float, sm_scale: float,
                           num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, partials_only: bool = False
                           ) -> Optional[torch.Tensor]:
    """q: fp16 [total_q, Hq, D]; cu_q_lens int32 [B+1]."""
    _need(q, "q", torch.float16, 3)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    total_q, hq, d = q.shape
    B = seq_lens.shape[0]
    if cu_q_lens.shape[0] != B + 1:
        raise ValueError("cu_q_lens must have batch + 1 entries")
    hkv, psz, _ = _cache_dims(k_cache, v_cache, d)
    if partials_only:
        out = None
    elif out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_e4m3_verify", out, q, block_table, seq_lens, B, workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    _check(_lib.paged_attn_e4m3_verify(q.data_ptr(), cu_q_lens.data_ptr(), total_q, int(max_q_len),
                                       k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                       seq_lens.data_ptr(), B, hq, hkv, d, psz, block_table.shape[1],
                                       float(k_scale), float(v_scale), float(sm_scale), int(num_splits),
                                       ws_ptr, ws_bytes, _ptr(out), _stream()), "paged_attn_e4m3_verify")
    return out


def paged_attn_e4m3_verify_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  cu_q_lens: torch.Tensor, max_q_len: int, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                                  k_scale: float, v_scale: float, sm_scale: float, num_splits: int = 1,
                                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                                  partials_only: bool = False) -> Optional[torch.Tensor]:
    """MTP verify with the step's new tokens appended: k_new, v_new fp16 [total_q, Hkv, D] (rows in the
    order of q) are quantised into key positions seq_lens[b] - q_len + i (through the block table), then
    attended as paged_attn_e4m3_verify."""
    _need(q, "q", torch.float16, 3)
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    total_q, hq, d = q.shape
    B = seq_lens.shape[0]
    if cu_q_lens.shape[0] != B + 1:
        raise ValueError("cu_q_lens must have batch + 1 entries")
    hkv, psz, _ = _cache_dims(k_cache, v_cache, d)
    if tuple(k_new.shape) != (total_q, hkv, d) or tuple(v_new.shape) != (total_q, hkv, d):
        raise ValueError(f"k_new/v_new must be [{total_q}, {hkv}, {d}]")
    if partials_only:
        out = None
    elif out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_e4m3_verify_append", out, q, block_table, seq_lens, B, workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    _check(_lib.paged_attn_e4m3_verify_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), cu_q_lens.data_ptr(),
                                              total_q, int(max_q_len), k_cache.data_ptr(), v_cache.data_ptr(),
                                              block_table.data_ptr(), seq_lens.data_ptr(), B, hq, hkv, d, psz,
                                              block_table.shape[1], float(k_scale), float(v_scale), float(sm_scale),
                                              int(num_splits), ws_ptr, ws_bytes, _ptr(out), _stream()),
           "paged_attn_e4m3_verify_append")
    return out


def _f16_cache_dims(k_cache, v_cache, q_heads_dim):
    _need(k_cache, "k_cache", torch.float16, 4)
    _need(v_cache, "v_cache", torch.float16, 4)
    pages, hkv, psz, d = k_cache.shape
    if tuple(v_cache.shape) != (pages, hkv, d, psz):
        raise ValueError("v_cache must be [pages, Hkv, D, P]")
    if q_heads_dim != d:
        raise ValueError("head_dim of q and caches disagree")
    return hkv, psz, d


def paged_attn_f16_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float,
                          num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, partials_only: bool = False
                          ) -> Optional[torch.Tensor]:
    """Decode over fp16 K/V pages (k_cache [pages, Hkv, P, D], v_cache [pages, Hkv, D, P]); otherwise
    as paged_attn_e4m3_decode."""
    _need(q, "q", torch.float16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, hq, d = q.shape
    hkv, psz, _ = _f16_cache_dims(k_cache, v_cache, d)
    if partials_only:
        out = None
    elif out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_f16_decode", out, q, block_table, seq_lens, B, workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    _check(_lib.paged_attn_f16_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                      block_table.data_ptr(), seq_lens.data_ptr(), B, hq, hkv, d, psz,
                                      block_table.shape[1], float(sm_scale), int(num_splits), ws_ptr, ws_bytes,
                                      _ptr(out), _stream()), "paged_attn_f16_decode")
    return out


def paged_attn_f16_verify(q: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int,
                          k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, sm_scale: float, num_splits: int = 1,
                          workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          partials_only: bool = False) -> Optional[torch.Tensor]:
    """Multi-query (MTP verify) attention over fp16 K/V pages; otherwise as paged_attn_e4m3_verify
    (at most 32 query rows per kv-head)."""
    _need(q, "q", torch.float16, 3)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    total_q, hq, d = q.shape
    B = seq_lens.shape[0]
    if cu_q_lens.shape[0] != B + 1:
        raise ValueError("cu_q_lens must have batch + 1 entries")
    hkv, psz, _ = _f16_cache_dims(k_cache, v_cache, d)
    if partials_only:
        out = None
    elif out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.float16, 3)
    _check_rows("paged_attn_f16_verify", out, q, block_table, seq_lens, B, workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    _check(_lib.paged_attn_f16_verify(q.data_ptr(), cu_q_lens.data_ptr(), total_q, int(max_q_len),
                                      k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                      seq_lens.data_ptr(), B, hq, hkv, d, psz, block_table.shape[1],
                                      float(sm_scale), int(num_splits), ws_ptr, ws_bytes, _ptr(out), _stream()),
           "paged_attn_f16_verify")
    return out


def split_reduce_fp32(ws_o: torch.Tensor, ws_m: torch.Tensor, ws_l: torch.Tensor,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      with_lse: bool = False):
    """ws_o fp32 [R, Hq, S, D]; ws_m, ws_l fp32 [R, Hq, S]. Returns out (and lse)."""
    _need(ws_o, "ws_o", torch.float32, 4)
    _need(ws_m, "ws_m", torch.float32, 3)
    _need(ws_l, "ws_l", torch.float32, 3)
    R, hq, S, d = ws_o.shape
    if tuple(ws_m.shape) != (R, hq, S) or tuple(ws_l.shape) != (R, hq, S):
        raise ValueError("ws_m / ws_l shapes disagree with ws_o")
    out = torch.empty((R, hq, d), dtype=torch.float16, device=ws_o.device) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((R, hq), dtype=torch.float32, device=ws_o.device)
    _check(_lib.split_reduce_fp32(ws_o.data_ptr(), ws_m.data_ptr(), ws_l.data_ptr(), R, hq, d, S,
                                  out.data_ptr(), _ptr(lse), _stream()), "split_reduce_fp32")
    return (out, lse) if (with_lse or lse is not None) else out


def kvfp8_check_paged_args(block_table: torch.Tensor, seq_lens: torch.Tensor, page_size: int, num_pages: int,
                           cu_q_lens: Optional[torch.Tensor] = None, total_q: int = 0, max_q_len: int = 0,
                           result: Optional[torch.Tensor] = None) -> None:
    """Device check of the attention calls' caller contract (block table, context
    lengths, query offsets); raises KVFP8Error (KVFP8_INVALID_ARG) naming every
    broken rule. block_table int32 [B, max_pages]; seq_lens int32 [B]; cu_q_lens
    int32 [B+1] for verify (None: decode) with total_q, the number of query
    rows, and max_q_len as passed to the verify call. Synchronous."""
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, max_pages = block_table.shape
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens must have one entry per block-table row")
    if cu_q_lens is not None:
        _need(cu_q_lens, "cu_q_lens", torch.int32, 1)
        if cu_q_lens.shape[0] != B + 1:
            raise ValueError("cu_q_lens must have batch + 1 entries")
    if result is None:
        result = torch.empty(4, dtype=torch.int32, device=block_table.device)
    _check(_lib.kvfp8_check_paged_args(block_table.data_ptr(), seq_lens.data_ptr(), _ptr(cu_q_lens), B, max_pages,
                                       int(page_size), int(num_pages), int(total_q), int(max_q_len), result.data_ptr(),
                                       _stream()), "kvfp8_check_paged_args")


def kvfp8_e4m3_encode_f32(x: torch.Tensor) -> torch.Tensor:
    _need(x, "x", torch.float32)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.kvfp8_e4m3_encode_f32(x.data_ptr(), codes.data_ptr(), x.numel(), _stream()),
           "kvfp8_e4m3_encode_f32")
    return codes


def kvfp8_e4m3_decode_f32(codes: torch.Tensor) -> torch.Tensor:
    _need(codes, "codes", torch.uint8)
    x = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(_lib.kvfp8_e4m3_decode_f32(codes.data_ptr(), x.data_ptr(), codes.numel(), _stream()),
           "kvfp8_e4m3_decode_f32")
    return x


def scale_overlay_write(path: str, revision: str, k_scales, v_scales) -> None:
    """Store per-layer K/V scales (host sequences of fp32) for a checkpoint revision."""
    import numpy as np
    k = np.ascontiguousarray(np.asarray(k_scales, dtype=np.float32))
    v = np.ascontiguousarray(np.asarray(v_scales, dtype=np.float32))
    if k.ndim != 1 or k.shape != v.shape:
        raise ValueError("k_scales and v_scales must be 1-D of equal length")
    _check(_lib.kvfp8_scale_overlay_write(os.fsencode(path), revision.encode(), int(k.size),
                                          k.ctypes.data, v.ctypes.data), "kvfp8_scale_overlay_write")


def scale_overlay_read(path: str, revision: str, n_layers: int):
    """Per-layer (k_scales, v_scales) fp32 arrays for `revision`; raises KVFP8Error on anything
    missing, foreign or invalid (no fallback)."""
    import numpy as np
    k = np.zeros(int(n_layers), np.float32)
    v = np.zeros(int(n_layers), np.float32)
    _check(_lib.kvfp8_scale_overlay_read(os.fsencode(path), revision.encode(), int(n_layers), k.ctypes.data,
                                         v.ctypes.data), "kvfp8_scale_overlay_read")
    return k, v
