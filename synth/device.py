"""Seeded synthetic K/V drawn directly on the GPU (for workloads whose fp16
values would take too long to draw on the host: the 32k and 256k points).

Same distributions as the host generator: N(0, 1) in fp16, with the batch's
outlier channels replaced by scale * Student-t(df) draws, t = z / sqrt(chi2/df)
built from normal draws. Holds no arithmetic of the method.
"""

import torch


def _student_t(gen, shape, df: int, device):
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(int(df)):
        chi += torch.randn(shape, generator=gen, device=device, dtype=torch.float32) ** 2
    return z / torch.sqrt(chi / df)


def normal_kv(n_tokens: int, n_kv_heads: int, head_dim: int, seed: int, outlier_channels=(),
              outlier_df: int = 3, outlier_scale: float = 8.0, device="cuda", chunk_tokens=1 << 18):
    """fp16 [n_tokens, Hkv, D] on the device, drawn in chunks to bound the
    float32 temporaries."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty((n_tokens, n_kv_heads, head_dim), dtype=torch.float16, device=device)
    ch = torch.as_tensor(list(outlier_channels), dtype=torch.int64, device=device)
    flat = out.view(n_tokens, n_kv_heads * head_dim)
    for t0 in range(0, n_tokens, chunk_tokens):
        t1 = min(n_tokens, t0 + chunk_tokens)
        blk = torch.randn((t1 - t0, n_kv_heads * head_dim), generator=gen, device=device,
                          dtype=torch.float32)
        if ch.numel():
            t = _student_t(gen, (t1 - t0, ch.numel()), outlier_df, device) * outlier_scale
            blk[:, ch] = t.clamp(-65504.0, 65504.0)
        flat[t0:t1] = blk.to(torch.float16)
    return out
