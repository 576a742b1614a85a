"""Host-side split-count heuristic (default_splits), CPU only.

The kernels take any split count; default_splits picks one that fills the
device with equal-work workgroups. These tests pin its properties against a
brute-force count of the non-empty (sequence, kv-head, split) items, using the
split boundaries of the oracle (shared split size C = ceil(L_max / (64 S)) * 64)."""
import numpy as np
import pytest

from fp8_quantised_paged_amd import kvfp8
from oracle.splits import split_bounds
from synth import make_config


def items(lens, heads, S):
    lmax = max(lens)
    return heads * sum(sum(1 for a, b in split_bounds(L, S, 64, lmax) if b > a) for L in lens if L > 0)


def slots(cus, rows, lens, heads, head_dim=128, elem=1):
    # decode: one workgroup per CU; verify: one per CU up to 1.2 MB of KV per CU, two above
    kv = sum(lens) * heads * head_dim * 2 * elem
    return 2 * cus if (rows > 16 and kv > 1.2e6 * cus) else cus


@pytest.mark.parametrize("seed", range(20))
def test_ragged_choice_is_the_fullest_that_fits(seed):
    rng = np.random.default_rng(4400 + seed)
    B = int(rng.integers(1, 40))
    heads = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 4, 8]))
    q_len = int(rng.choice([1, 4]))
    lens = [int(x) for x in rng.integers(0, 40000, B)]
    lens[0] = max(lens[0], 1)
    cus = int(rng.choice([64, 256]))
    S = kvfp8.default_splits(B, heads, max(lens), cus=cus, seq_lens=lens, n_q_heads=heads * group, q_len=q_len)
    cap = slots(cus, q_len * group, lens, heads)
    lmax = max(lens)
    assert 1 <= S <= 256
    if S > 1:
        assert -(-lmax // (64 * S)) * 64 >= 512  # splits hold at least 512 keys
        assert items(lens, heads, S) <= cap
    # no other admissible count uses more of the slots without exceeding them
    best = items(lens, heads, S) if items(lens, heads, S) <= cap else 0
    for s in range(1, 257):
        if s > 1 and -(-lmax // (64 * s)) * 64 < 512:
            break
        u = items(lens, heads, s)
        assert not (best < u <= cap), f"S={S} uses {best} items, S={s} would use {u} <= {cap}"


def test_uniform_lengths_without_seq_lens():
    # 4k decode: 32 x 4 kv-heads = 128 items per split; one workgroup per CU -> 2 splits
    assert kvfp8.default_splits(32, 4, 4096) == 2
    # 32k decode: the same grid
    assert kvfp8.default_splits(32, 4, 32768) == 2
    # a single sequence is split across the device, at least 512 keys per split
    assert kvfp8.default_splits(1, 1, 1 << 20) == 256
    assert kvfp8.default_splits(1, 1, 1024) == 2
    assert kvfp8.default_splits(4, 4, 100) == 1


def test_mtp3_workload_split_count():
    bt = make_config(3, values=False)
    S = kvfp8.default_splits(bt.batch, bt.n_kv_heads, int(bt.seq_lens.max()), seq_lens=bt.seq_lens,
                             n_q_heads=bt.n_q_heads, q_len=int(bt.q_lens.max()))
    lens = [int(x) for x in bt.seq_lens]
    assert S == 8 and items(lens, bt.n_kv_heads, S) == 220  # 0.83 MB per CU: 220 items over 256 slots (1 per CU)
    # the same workload over fp16 pages: 1.66 MB per CU, two workgroups per CU
    S16 = kvfp8.default_splits(bt.batch, bt.n_kv_heads, int(bt.seq_lens.max()), seq_lens=bt.seq_lens,
                               n_q_heads=bt.n_q_heads, q_len=int(bt.q_lens.max()), kv_elem_bytes=2)
    assert S16 == 19 and items(lens, bt.n_kv_heads, S16) == 496


def test_empty_batch_and_zero_lengths():
    assert kvfp8.default_splits(3, 4, 0, seq_lens=[0, 0, 0]) == 1
    assert kvfp8.default_splits(0, 4, 0, seq_lens=[]) == 1
