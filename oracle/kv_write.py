"""Quantising paged cache write, float64 reference.

The pages store the main K/V cache as calibrated E4M3 ("Integrate calibrated
E4M3 QSA KV capacity path", Changes). New tokens are therefore divided by the
layer's scale and encoded before they are stored. Readings used here (the
pages are silent on each):

* the quotient is the correctly rounded float32 quotient fl32(x) / scale, not
  a multiplication by a reciprocal;
* the cache is paged: slot = page * page_size + offset, K pages hold
  [n_kv_heads][page_size][head_dim] bytes (token-major inside a head) and V
  pages hold [n_kv_heads][head_dim][page_size] bytes (dimension-major inside a
  head, so that a run of tokens of one dimension is contiguous);
* a negative slot, or one past the cache, is skipped (padding).
"""

import numpy as np

from .calibrate import quotient_f32
from .e4m3 import e4m3_encode

POISON = 0x7F  # an E4M3 NaN code: unwritten slots must never reach an output


def new_caches(num_pages: int, n_kv_heads: int, page_size: int, head_dim: int, fill: int = POISON):
    """Fresh K and V caches filled with ``fill``."""
    k_cache = np.full((num_pages, n_kv_heads, page_size, head_dim), fill, dtype=np.uint8)
    v_cache = np.full((num_pages, n_kv_heads, head_dim, page_size), fill, dtype=np.uint8)
    return k_cache, v_cache


def quantise(x_f16, scale) -> np.ndarray:
    """E4M3 codes of fl32(x) / scale."""
    x32 = np.asarray(x_f16, dtype=np.float16).astype(np.float32)
    return e4m3_encode(quotient_f32(x32, np.float32(scale)))


def quant_write(k_f16, v_f16, slot_mapping, k_scale, v_scale, k_cache, v_cache):
    """Write the codes of k_f16 / v_f16 [n_tokens, Hkv, D] into the caches
    (in place) at the given slots; returns the caches."""
    num_pages, n_kv_heads, page_size, head_dim = k_cache.shape
    kq = quantise(k_f16, k_scale)
    vq = quantise(v_f16, v_scale)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for t, slot in enumerate(slots):
        if slot < 0 or slot >= num_pages * page_size:
            continue
        page, off = divmod(int(slot), page_size)
        k_cache[page, :, off, :] = kq[t]
        v_cache[page, :, :, off] = vq[t]
    return k_cache, v_cache
