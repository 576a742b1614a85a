"""kvfp8_check_paged_args on the GPU: the device check of the attention
calls' caller contract (block table, context lengths, query offsets) against
the rules written out here in numpy, on hand-made violations and on seeded
random tables with planted ones. The check only reads the tables it is given."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    from fp8_quantised_paged_amd import kvfp8
    assert torch.cuda.is_available()
    return kvfp8


def rules(bt, sl, P, num_pages, cu=None, total_q=0, max_q=0):
    """The contract, one sequence at a time: returns {rule: first sequence}."""
    B, maxp = bt.shape
    first = {}
    for b in range(B):
        L = int(sl[b])
        bad_len = L < 0 or L > maxp * P
        if cu is None:
            ql, bad_q = 1, False
        else:
            ql = int(cu[b + 1]) - int(cu[b])
            bad_q = ql < 0 or ql > max_q or (b == 0 and cu[0] != 0) or (b == B - 1 and cu[B] != total_q)
        if cu is not None and not bad_len and not bad_q and ql > L:
            bad_q = True  # a verify row before key 0 (a decode row may see no keys)
        if bad_len:
            first.setdefault("seq_lens", b)
        if bad_q:
            first.setdefault("query", b)
        used = 0 if L <= 0 else -(-min(L, maxp * P) // P)
        if any(not (0 <= int(bt[b, i]) < num_pages) for i in range(used)):
            first.setdefault("block-table", b)
    return first


def run(K, bt, sl, P, num_pages, cu=None, total_q=0, max_q=0):
    """Returns {} on success, else {rule: first sequence} parsed from the error."""
    try:
        K.kvfp8_check_paged_args(torch.from_numpy(np.ascontiguousarray(bt, np.int32)).cuda(),
                                 torch.from_numpy(np.ascontiguousarray(sl, np.int32)).cuda(), P, num_pages,
                                 None if cu is None else torch.from_numpy(np.ascontiguousarray(cu, np.int32)).cuda(),
                                 total_q, max_q)
        return {}
    except K.KVFP8Error as e:
        assert e.status == K.INVALID_ARG, str(e)
        msg = str(e)
        out = {}
        for key, text in (("seq_lens", "seq_lens outside"), ("query", "query rows"),
                          ("block-table", "block-table entry")):
            if text in msg:
                tail = msg.split(text, 1)[1]
                out[key] = int(tail.split("first at sequence", 1)[1].split(")", 1)[0])
        assert out, msg
        return out


def test_valid_decode_and_verify_pass(K):
    P, maxp = 16, 8
    bt = np.arange(4 * maxp, dtype=np.int32).reshape(4, maxp)
    sl = np.array([1, 16, 17, 128], np.int32)
    assert run(K, bt, sl, P, 4 * maxp) == {}
    # verify with zero-length sequences (no rows, no keys) beside ordinary ones
    sl = np.array([0, 5, 0, 70], np.int32)
    cu = np.array([0, 0, 2, 2, 5], np.int32)
    assert run(K, bt, sl, P, 4 * maxp, cu, 5, 3) == {}


def test_each_rule(K):
    P, maxp, npg = 16, 8, 32
    bt = np.arange(4 * maxp, dtype=np.int32).reshape(4, maxp)
    sl = np.array([10, 20, 30, 40], np.int32)
    cases = []
    s = sl.copy(); s[2] = maxp * P + 1; cases.append((bt, s, None, 0, 0, {"seq_lens": 2}))
    s = sl.copy(); s[1] = -3; cases.append((bt, s, None, 0, 0, {"seq_lens": 1}))
    s = sl.copy(); s[3] = 0; cases.append((bt, s, None, 0, 0, {}))  # a decode sequence with no keys
    b = bt.copy(); b[1, 1] = npg; cases.append((b, sl, None, 0, 0, {"block-table": 1}))
    b = bt.copy(); b[2, 0] = -1; cases.append((b, sl, None, 0, 0, {"block-table": 2}))
    b = bt.copy(); b[1, 2] = 10 ** 6; cases.append((b, sl, None, 0, 0, {}))  # past seq 1's last page: never read
    cu = np.array([0, 1, 2, 6, 10], np.int32)
    cases.append((bt, sl, cu, 10, 4, {}))
    c = cu.copy(); c[0] = 1; cases.append((bt, sl, c, 10, 4, {"query": 0}))
    cases.append((bt, sl, cu, 9, 4, {"query": 3}))                            # cu_q_lens[batch] != total_q
    cases.append((bt, sl, cu, 10, 3, {"query": 2}))                           # q_len above max_q_len
    c = cu.copy(); c[2] = 0; cases.append((bt, sl, c, 10, 6, {"query": 1}))   # decreasing offsets
    s = sl.copy(); s[2] = 3; cases.append((bt, s, cu, 10, 4, {"query": 2}))   # more rows than keys
    b = bt.copy(); b[0, 0] = npg + 5; s = sl.copy(); s[3] = 4096
    cases.append((b, s, cu, 10, 4, {"seq_lens": 3, "block-table": 0}))
    for i, (b, s, c, tq, mq, want) in enumerate(cases):
        assert rules(b, s, P, npg, c, tq, mq) == want, f"case {i}: the rules disagree with the expectation"
        assert run(K, b, s, P, npg, c, tq, mq) == want, f"case {i}"


@pytest.mark.parametrize("seed", range(6))
def test_random_tables_match_the_rules(K, seed):
    rng = np.random.default_rng(7700 + seed)
    B = int(rng.integers(1, 300))
    P = int(rng.choice([4, 8, 16, 32, 64]))
    maxp = int(rng.integers(1, 40))
    npg = B * maxp
    bt = rng.permutation(npg).astype(np.int32).reshape(B, maxp)
    verify = seed % 2 == 1
    ql = rng.integers(0, 5, B) if verify else np.ones(B, np.int64)
    sl = np.minimum(ql + rng.integers(0, maxp * P, B), maxp * P).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32) if verify else None
    total_q = int(cu[-1]) if verify else 0
    assert run(K, bt, sl, P, npg, cu, total_q, 4) == {} == rules(bt, sl, P, npg, cu, total_q, 4)
    # plant violations at random places
    for _ in range(int(rng.integers(1, 4))):
        kind = int(rng.integers(0, 3))
        b = int(rng.integers(0, B))
        if kind == 0:
            sl[b] = maxp * P + int(rng.integers(1, 50))
        elif kind == 1:
            bt[b, int(rng.integers(0, maxp))] = int(rng.choice([-7, npg, npg + 1000]))
        elif verify:
            cu[b + 1:] += 6
        else:
            sl[b] = -1
    want = rules(bt, sl, P, npg, cu, total_q, 4)
    assert run(K, bt, sl, P, npg, cu, total_q, 4) == want


def test_large_table_grid_stride(K):
    """More entries than the check's grid has threads: a violation in the last
    entry read is still found."""
    B, maxp, P = 600, 3000, 16
    npg = B * maxp
    bt = np.arange(npg, dtype=np.int32).reshape(B, maxp)
    sl = np.full(B, maxp * P, np.int32)
    assert run(K, bt, sl, P, npg) == {}
    bt[B - 1, maxp - 1] = npg
    assert run(K, bt, sl, P, npg) == {"block-table": B - 1}
