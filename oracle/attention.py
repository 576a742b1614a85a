"""Paged attention over an E4M3 cache, float64 reference.

Computes scaled dot-product attention of each query row against the keys of
its sequence read through the block table. The pages describe decode, MTP
verify ("Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP", Purpose and
Validation on 4xV100 TP4: MTP3 verifies the drafted tokens of a step) and
mixed catch-up/decode batches ("Integrate calibrated E4M3 QSA KV capacity
path", Changes); all three are the same definition with a different number
of query tokens per sequence. Readings used here (the pages are silent):

* seq_lens[b] counts every key of sequence b including this step's q_lens[b]
  query tokens, which were written to the cache before attending;
* query row i of sequence b (0 <= i < q_lens[b]) sits at position
  seq_lens[b] - q_lens[b] + i and sees keys 0 .. that position (causal,
  aligned to the end);
* query head h reads kv-head h // (Hq / Hkv);
* the key and value of position j are decode(code) * k_scale and
  decode(code) * v_scale -- applying the scale after the dot product instead
  ("Integrate calibrated E4M3 QSA KV capacity path", Changes: the K/V scaling
  is hoisted out of the per-element loops) is equal in exact arithmetic;
* scores are sm_scale * q . k and the softmax is over the visible keys.

A row with no visible key (never produced by the workloads) returns zeros and
log-sum-exp = -inf.
"""

import numpy as np

from .e4m3 import e4m3_decode


def gather_sequence_kv(k_cache, v_cache, block_row, seq_len):
    """Decoded (unscaled) K and V of one sequence as float64 [L, Hkv, D]."""
    page_size = k_cache.shape[2]
    j = np.arange(int(seq_len))
    pages = np.asarray(block_row, dtype=np.int64)[j // page_size]
    offs = j % page_size
    k_codes = k_cache[pages, :, offs, :]  # [L, Hkv, D]
    v_codes = v_cache[pages, :, :, offs]  # [L, Hkv, D]
    return e4m3_decode(k_codes), e4m3_decode(v_codes)


def gather_sequence_kv_f16(k_cache_f16, v_cache_f16, block_row, seq_len):
    """K and V of one sequence from fp16 caches (same layout) as float64 [L, Hkv, D]."""
    page_size = k_cache_f16.shape[2]
    j = np.arange(int(seq_len))
    pages = np.asarray(block_row, dtype=np.int64)[j // page_size]
    offs = j % page_size
    k = np.asarray(k_cache_f16[pages, :, offs, :], dtype=np.float16).astype(np.float64)
    v = np.asarray(v_cache_f16[pages, :, :, offs], dtype=np.float16).astype(np.float64)
    return k, v


def paged_attention_f16(q_f16, k_cache_f16, v_cache_f16, block_table, seq_lens, cu_q_lens, sm_scale,
                        rows=None):
    """The same attention over a cache that stores fp16 values instead of
    E4M3 codes (no K/V scales): the other arm of the pages' comparison of cache
    formats ("Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP", Validation
    on 4xV100 TP4: only kv_cache_dtype differs between the arms)."""
    def kv(b, L):
        return gather_sequence_kv_f16(k_cache_f16, v_cache_f16, block_table[b], L)
    return _attention(q_f16, k_cache_f16.shape[1], kv, seq_lens, cu_q_lens, sm_scale, rows)


def paged_attention(q_f16, k_cache, v_cache, block_table, seq_lens, cu_q_lens,
                    k_scale, v_scale, sm_scale, rows=None):
    """Attention output float64 [total_q, Hq, D] and log-sum-exp [total_q, Hq].

    q_f16: [total_q, Hq, D] query rows, sequence-major (cu_q_lens[b] ..
    cu_q_lens[b+1]-1 belong to sequence b). ``rows`` optionally restricts the
    work to a subset of sequences (others are left as NaN).
    """
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))

    def kv(b, L):
        kd, vd = gather_sequence_kv(k_cache, v_cache, block_table[b], L)
        return kd * ks, vd * vs
    return _attention(q_f16, k_cache.shape[1], kv, seq_lens, cu_q_lens, sm_scale, rows)


def _attention(q_f16, n_kv_heads, kv, seq_lens, cu_q_lens, sm_scale, rows):
    """The definition, given kv(b, L) -> (K, V) float64 [L, Hkv, D] of sequence b."""
    q = np.asarray(q_f16, dtype=np.float16).astype(np.float64)
    total_q, n_q_heads, head_dim = q.shape
    group = n_q_heads // n_kv_heads
    sm = float(np.float32(sm_scale))
    out = np.full((total_q, n_q_heads, head_dim), np.nan)
    lse = np.full((total_q, n_q_heads), np.nan)
    batch = len(seq_lens)
    for b in (range(batch) if rows is None else rows):
        L = int(seq_lens[b])
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        T = q1 - q0
        if T == 0:
            continue
        kd, vd = kv(b, L)
        pos = L - T + np.arange(T)  # position of each query row
        visible = np.arange(L)[None, :] <= pos[:, None]  # [T, L]
        for h in range(n_q_heads):
            g = h // group
            s = sm * (q[q0:q1, h, :] @ kd[:, g, :].T)  # [T, L]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            safe_m = np.where(np.isfinite(m), m, 0.0)
            w = np.where(visible, np.exp(s - safe_m[:, None]), 0.0)
            l = w.sum(axis=1)
            o = w @ vd[:, g, :]
            with np.errstate(invalid="ignore", divide="ignore"):
                out[q0:q1, h, :] = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1.0)[:, None], 0.0)
                lse[q0:q1, h] = np.where(l > 0, safe_m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse
