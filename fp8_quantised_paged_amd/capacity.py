"""KV-cache capacity accounting, in bytes.

Only the main K/V cache is stored as E4M3; the indexer's raw and compressed
caches stay FP16 ("[Model][SM70][FP8] Integrate calibrated E4M3 QSA KV capacity
path", Changes). Halving the main cache therefore gives less than twice the
tokens: the pages report 433,401 -> 775,096 tokens (+78.8%) on 4xV100 TP4
("[Model][SM70] Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP", Validation
on 4xV100 TP4) and about 1.83x at the same memory budget (the capacity-path
page, Test Result).

Per token and layer, let M = 2 * n_kv_heads * head_dim bytes be the main cache
in E4M3 (one byte per element, K and V) and X the FP16 side caches. Then

    tokens(E4M3) / tokens(FP16) = (2M + X) / (M + X),   so   X / M = (2 - r) / (r - 1)

for a measured ratio r. The per-layer K/V scales add 8 bytes per layer, not per
token. Capacity is counted in whole pages, as a paged cache allocates it.
"""

from __future__ import annotations

E4M3_BYTES = 1
FP16_BYTES = 2


def main_kv_bytes_per_token(n_kv_heads: int, head_dim: int, elem_bytes: int = E4M3_BYTES) -> int:
    """Bytes of one token's K and V in one layer's main cache."""
    if n_kv_heads <= 0 or head_dim <= 0 or elem_bytes <= 0:
        raise ValueError("n_kv_heads, head_dim and elem_bytes must be positive")
    return 2 * n_kv_heads * head_dim * elem_bytes


def bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int = E4M3_BYTES,
                    side_bytes: int = 0) -> int:
    """Bytes of one token over all layers: main K/V cache plus side_bytes of
    unquantised caches per token and layer."""
    if n_layers <= 0 or side_bytes < 0:
        raise ValueError("n_layers must be positive and side_bytes non-negative")
    return n_layers * (main_kv_bytes_per_token(n_kv_heads, head_dim, elem_bytes) + side_bytes)


def capacity_tokens(budget_bytes: int, n_layers: int, n_kv_heads: int, head_dim: int, page_size: int,
                    elem_bytes: int = E4M3_BYTES, side_bytes: int = 0) -> int:
    """Tokens that fit in budget_bytes when the cache is allocated in pages of
    page_size tokens across all layers (the scales' 8 bytes per layer are taken
    off the budget first)."""
    if page_size <= 0:
        raise ValueError("page_size must be positive")
    usable = budget_bytes - 8 * n_layers
    if usable <= 0:
        return 0
    per_page = page_size * bytes_per_token(n_layers, n_kv_heads, head_dim, elem_bytes, side_bytes)
    return (usable // per_page) * page_size


def capacity_ratio(n_kv_heads: int, head_dim: int, side_bytes: int = 0) -> float:
    """tokens(E4M3 main cache) / tokens(FP16 main cache) at equal budget, ignoring page rounding."""
    m = main_kv_bytes_per_token(n_kv_heads, head_dim, E4M3_BYTES)
    return (2 * m + side_bytes) / (m + side_bytes)


def side_fraction(ratio: float) -> float:
    """X / M implied by a measured capacity ratio r (1 < r <= 2)."""
    if not 1.0 < ratio <= 2.0:
        raise ValueError("a capacity ratio must lie in (1, 2]")
    return (2.0 - ratio) / (ratio - 1.0)
