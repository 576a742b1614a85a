"""Independent checks that pin the oracle to something other than itself.

Each check takes the function under test as an argument so that the
planted-mistake tests can hand it a deliberately broken copy and confirm the
check notices. Nothing here imports the HIP library.
"""

from fractions import Fraction
import math

import numpy as np
import torch


# ---------------------------------------------------------------- E4M3 codec

def torch_e4m3_values() -> np.ndarray:
    """Values of all 256 codes as torch's float8_e4m3fn dtype decodes them."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_decode_against_torch(decode) -> bool:
    ours = decode(np.arange(256, dtype=np.uint8))
    ref = torch_e4m3_values()
    same_nan = np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    same_val = np.array_equal(ours[fin], ref[fin])
    same_sign = np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    return bool(same_nan and same_val and same_sign)


def brute_force_encode(values_f32: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code by exhaustive search over the finite codes.

    Magnitudes at or above 448 saturate; ties go to the even code (the code
    whose mantissa LSB is 0); the input's sign is kept, including for values
    that round to zero. Independent of the oracle's binade arithmetic: it
    only uses the 127 non-negative finite code values from the closed form of
    the OCP E4M3 table, built here with plain Python floats.
    """
    mags = []
    for c in range(0x7F):  # 0x00 .. 0x7E
        e, m = c >> 3, c & 7
        mags.append(m / 512.0 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    mags = np.array(mags)
    v = np.asarray(values_f32, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    out = np.empty(v.shape, dtype=np.int64)
    for lo in range(0, v.size, 65536):
        blk = a.reshape(-1)[lo:lo + 65536]
        d = np.abs(blk[:, None] - mags[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # among tied candidates prefer the even code
        even = cand & ((np.arange(0x7F) % 2) == 0)[None, :]
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        pick = np.where(blk >= 448.0, 0x7E, pick)
        out.reshape(-1)[lo:lo + 65536] = pick
    out = out.reshape(v.shape)
    out = np.where(np.isnan(v), 0x7F, out)
    out = out | np.where(np.signbit(v), 0x80, 0)
    return out.astype(np.uint8)


def torch_encode_clamped(values_f32: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn cast after clamping to +-448 (torch does not
    saturate on its own; clamping first is the same as saturating because 448
    is representable)."""
    t = torch.from_numpy(np.asarray(values_f32, dtype=np.float32).copy())
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------- correct rounding f32

def exact_round_f32(num: float, den: float) -> float:
    """fp32 nearest (ties to even) to the exact rational num/den, found by
    comparing exact Fractions of the neighbouring fp32 candidates."""
    q = Fraction(float(num)) / Fraction(float(den))
    approx = np.float32(float(q))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)), np.nextafter(approx, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        if best is None or d < best[0] or (d == best[0] and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = (d, c)
    return float(best[1])


# ---------------------------------------------------------------- attention

def brute_force_attention(q, k_codes_seq, v_codes_seq, k_scale, v_scale, sm_scale, q_len, decode_one):
    """Pure-Python loops over one sequence. k_codes_seq/v_codes_seq are
    [L][Hkv][D] nested lists of codes for positions 0..L-1; q is [T][Hq][D]
    floats; decode_one maps one code to its float value. Returns [T][Hq][D]."""
    L = len(k_codes_seq)
    T = q_len
    Hq = len(q[0])
    Hkv = len(k_codes_seq[0])
    D = len(q[0][0])
    G = Hq // Hkv
    out = []
    for i in range(T):
        pos = L - T + i
        row = []
        for h in range(Hq):
            g = h // G
            scores = []
            for j in range(pos + 1):
                acc = 0.0
                for d in range(D):
                    acc += q[i][h][d] * (decode_one(k_codes_seq[j][g][d]) * k_scale)
                scores.append(acc * sm_scale)
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            o = []
            for d in range(D):
                acc = 0.0
                for j in range(pos + 1):
                    acc += ws[j] * decode_one(v_codes_seq[j][g][d]) * v_scale
                o.append(acc / tot)
            row.append(o)
        out.append(row)
    return out


def sdpa_reference(batch, k_codes_tok, v_codes_tok, k_scale, v_scale, sm_scale):
    """torch scaled_dot_product_attention in float64 on dense K/V.

    k_codes_tok/v_codes_tok are the E4M3 codes of every position in the
    sequence-major token order of ``batch.k`` (obtained from the caches
    through the slot mapping, not the block table). Decoding uses torch's
    float8_e4m3fn dtype; GQA is expanded with repeat_interleave; the causal
    mask is aligned to the end of each sequence.
    """
    Hq = batch.n_q_heads
    Hkv = batch.n_kv_heads
    G = Hq // Hkv
    outs = []
    for b in range(batch.batch):
        s0, s1 = int(batch.cu_seq_lens[b]), int(batch.cu_seq_lens[b + 1])
        q0, q1 = int(batch.cu_q_lens[b]), int(batch.cu_q_lens[b + 1])
        L, T = s1 - s0, q1 - q0
        kc = torch.from_numpy(np.ascontiguousarray(k_codes_tok[s0:s1])).view(torch.float8_e4m3fn)
        vc = torch.from_numpy(np.ascontiguousarray(v_codes_tok[s0:s1])).view(torch.float8_e4m3fn)
        kf = kc.to(torch.float64) * float(np.float32(k_scale))  # [L, Hkv, D]
        vf = vc.to(torch.float64) * float(np.float32(v_scale))
        kf = kf.permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
        vf = vf.permute(1, 0, 2).repeat_interleave(G, dim=0)
        qf = torch.from_numpy(batch.q[q0:q1].astype(np.float64)).permute(1, 0, 2)  # [Hq, T, D]
        pos = torch.arange(T) + (L - T)
        mask = torch.arange(L)[None, :] <= pos[:, None]  # [T, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            qf, kf, vf, attn_mask=mask, scale=float(np.float32(sm_scale)))
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)
