"""Split-context partials and their reduction, float64 reference.

The pages' decode route writes a split-context temporary output that must be
FP32 ("Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP", Status and
history: the FP32 XQA workspace; "Qualify E4M3 KV with MTP3", Problem and
resulting behavior: the temporary output is allocated in FP32 to match the
native interface). The pages do not give the algebra; the reading used here
is the standard split softmax. For a split covering keys J_s of a row,

    m_s = max_{j in J_s} s_j
    l_s = sum_{j in J_s} exp(s_j - m_s)
    o_s = sum_{j in J_s} exp(s_j - m_s) * v_j        (v_j already scaled)

with s_j the scaled score in natural-log units; an empty split has m_s = -inf,
l_s = 0, o_s = 0. The reduction is

    M = max_s m_s,  w_s = exp(m_s - M),
    O = sum_s w_s o_s / sum_s w_s l_s,  LSE = M + log(sum_s w_s l_s),

which equals the unsplit softmax for any partition of the keys.

Split boundaries (reading; the pages fix only that the split partials are
FP32, not where the splits fall): all sequences of one call share one split
size, set by the longest context of the batch, L_max. Split s of a sequence
with L keys covers [s * C, min((s + 1) * C, L)) with
C = ceil(L_max / (S * granule)) * granule, so every split but the last starts
on a multiple of the granule, the longest sequence uses all S splits, and a
shorter one uses ceil(L / C) of them (the rest are empty). Equal work per
non-empty split is what lets a ragged batch spread over the whole device.
"""

import numpy as np

from .attention import gather_sequence_kv


def split_bounds(seq_len: int, num_splits: int, granule: int = 64, max_len=None):
    """[(start, end)] key ranges of each split (end <= start means empty).

    max_len is the longest context of the batch (seq_len itself when None)."""
    L = int(seq_len)
    Lm = L if max_len is None else int(max_len)
    if Lm < L:
        raise ValueError("max_len must be at least seq_len")
    S = int(num_splits)
    chunk = -(-Lm // (S * granule)) * granule if Lm > 0 else granule
    return [(s * chunk, min((s + 1) * chunk, L)) for s in range(S)]


def split_partials(q_f16, k_cache, v_cache, block_table, seq_lens, cu_q_lens,
                   k_scale, v_scale, sm_scale, num_splits, granule=64, rows=None):
    """Partials (ws_o [total_q, Hq, S, D], ws_m [total_q, Hq, S],
    ws_l [total_q, Hq, S]) in float64."""
    q = np.asarray(q_f16, dtype=np.float16).astype(np.float64)
    total_q, n_q_heads, head_dim = q.shape
    n_kv_heads = k_cache.shape[1]
    group = n_q_heads // n_kv_heads
    S = int(num_splits)
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    sm = float(np.float32(sm_scale))
    ws_o = np.full((total_q, n_q_heads, S, head_dim), np.nan)
    ws_m = np.full((total_q, n_q_heads, S), np.nan)
    ws_l = np.full((total_q, n_q_heads, S), np.nan)
    max_len = int(np.max(seq_lens)) if len(seq_lens) else 0
    for b in (range(len(seq_lens)) if rows is None else rows):
        L = int(seq_lens[b])
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        T = q1 - q0
        if T == 0:
            continue
        kd, vd = gather_sequence_kv(k_cache, v_cache, block_table[b], L)
        kd = kd * ks
        vd = vd * vs
        for i in range(T):
            pos = L - T + i
            for s, (lo, hi) in enumerate(split_bounds(L, S, granule, max_len)):
                hi = min(hi, pos + 1)
                r = q0 + i
                if hi <= lo:
                    ws_m[r, :, s] = -np.inf
                    ws_l[r, :, s] = 0.0
                    ws_o[r, :, s, :] = 0.0
                    continue
                for h in range(n_q_heads):
                    g = h // group
                    sc = sm * (kd[lo:hi, g, :] @ q[r, h, :])
                    m = sc.max()
                    w = np.exp(sc - m)
                    ws_m[r, h, s] = m
                    ws_l[r, h, s] = w.sum()
                    ws_o[r, h, s, :] = w @ vd[lo:hi, g, :]
    return ws_o, ws_m, ws_l


def split_reduce(ws_o, ws_m, ws_l):
    """Combine partials over the split axis; returns (O [R, Hq, D], LSE [R, Hq])."""
    o = np.asarray(ws_o, dtype=np.float64)
    m = np.asarray(ws_m, dtype=np.float64)
    l = np.asarray(ws_l, dtype=np.float64)
    M = m.max(axis=-1)
    safe_M = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(m), np.exp(m - safe_M[..., None]), 0.0)
    den = (w * l).sum(axis=-1)
    num = (w[..., None] * o).sum(axis=-2)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(den[..., None] > 0, num / np.where(den > 0, den, 1.0)[..., None], 0.0)
        lse = np.where(den > 0, safe_M + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return out, lse
