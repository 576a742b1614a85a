"""KV-capacity accounting (host only). Pins: hand-counted pages, the exact
factor 2 with no side caches, and the pages' two capacity ratios mapped to side
caches and back."""

import pytest

from fp8_quantised_paged_amd import capacity as C

# "[Model][SM70] Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP",
# Validation on 4xV100 TP4: engine-reported tokens, FP16 then E4M3
FP16_TOKENS, E4M3_TOKENS = 433_401, 775_096


def test_hand_counted_pages():
    # 1 MiB + 16 B of scales, 2 layers, 1 kv-head, head_dim 64, pages of 4 tokens:
    # E4M3 128 B per token and layer -> 4 * 2 * 128 = 1,024 B per page -> 1,024 pages
    budget = (1 << 20) + 16
    assert C.capacity_tokens(budget, 2, 1, 64, 4) == 4096
    assert C.capacity_tokens(budget, 2, 1, 64, 4, elem_bytes=C.FP16_BYTES) == 2048
    # one byte short of a page drops the whole page
    assert C.capacity_tokens(budget - 1, 2, 1, 64, 4) == 4092
    assert C.capacity_tokens(16, 2, 1, 64, 4) == 0


def test_no_side_cache_doubles_capacity():
    assert C.capacity_ratio(4, 128) == 2.0
    for P in (4, 16, 64):
        e = C.capacity_tokens(288 * 10**9, 24, 4, 128, P)
        f = C.capacity_tokens(288 * 10**9, 24, 4, 128, P, elem_bytes=C.FP16_BYTES)
        assert e in (2 * f, 2 * f + P)  # page rounding only


def test_pages_ratios_imply_fp16_side_caches():
    r = E4M3_TOKENS / FP16_TOKENS
    x = C.side_fraction(r)
    assert 0.268 < x < 0.269  # side caches hold about 27% of the E4M3 main cache's bytes
    m = C.main_kv_bytes_per_token(4, 128)
    assert C.capacity_ratio(4, 128, side_bytes=x * m) == pytest.approx(r, rel=1e-12)
    # the capacity path page's "approximately 1.83x"
    assert C.side_fraction(1.83) == pytest.approx(0.17 / 0.83, rel=1e-12)
    assert C.side_fraction(2.0) == 0.0


@pytest.mark.parametrize("bad", [1.0, 0.5, 2.01])
def test_side_fraction_rejects_impossible_ratios(bad):
    with pytest.raises(ValueError):
        C.side_fraction(bad)


def test_bytes_per_token():
    assert C.main_kv_bytes_per_token(4, 128) == 1024
    assert C.main_kv_bytes_per_token(4, 128, C.FP16_BYTES) == 2048
    assert C.bytes_per_token(24, 4, 128, side_bytes=100) == 24 * 1124
    with pytest.raises(ValueError):
        C.bytes_per_token(0, 4, 128)
