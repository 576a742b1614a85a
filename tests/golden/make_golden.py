"""Writes the stored expected values under tests/golden/ from the oracle only.

The pages print no worked numeric example for this method, so every stored
value here is the oracle's own output on a seeded input, kept so that any
later change to the oracle's arithmetic shows up as a diff that has to be
justified. Run from the repository root:

    python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import (calibrate_amax, e4m3_decode, new_caches, paged_attention,  # noqa: E402
                    quant_write)
from synth import make_config  # noqa: E402


def write_codes(path):
    vals = e4m3_decode(np.arange(256, dtype=np.uint8))
    with open(path, "w") as f:
        f.write("# E4M3 code -> value (float.hex); closed form of the OCP OFP8 E4M3 table\n")
        for c, v in enumerate(vals):
            f.write(f"{c:02x} {float(v).hex() if np.isfinite(v) else 'nan'}\n")


def write_tiny_attention(path):
    bt = make_config(1)
    amax, scale, st = calibrate_amax(np.stack([bt.k.reshape(-1), bt.v.reshape(-1)]))
    kc, vc = new_caches(bt.num_pages, bt.n_kv_heads, bt.page_size, bt.head_dim)
    quant_write(bt.k, bt.v, bt.slot_mapping, scale[0], scale[1], kc, vc)
    sm = np.float32(1.0 / np.sqrt(bt.head_dim))
    out, lse = paged_attention(bt.q, kc, vc, bt.block_table, bt.seq_lens, bt.cu_q_lens,
                               scale[0], scale[1], sm)
    with open(path, "w") as f:
        f.write("# tiny workload (batch 2, contexts 100 and 257, 8/2 heads, head_dim 64, page 4)\n")
        f.write(f"# amax_k amax_v scale_k scale_v\n{float(amax[0]).hex()} {float(amax[1]).hex()} "
                f"{float(scale[0]).hex()} {float(scale[1]).hex()}\n")
        f.write("# row head lse o[0] o[1] o[2] o[63]\n")
        for r in range(out.shape[0]):
            for h in range(out.shape[1]):
                f.write(f"{r} {h} {lse[r, h].hex()} {out[r, h, 0].hex()} {out[r, h, 1].hex()} "
                        f"{out[r, h, 2].hex()} {out[r, h, 63].hex()}\n")


if __name__ == "__main__":
    write_codes(os.path.join(HERE, "e4m3_codes.txt"))
    write_tiny_attention(os.path.join(HERE, "tiny_attention.txt"))
