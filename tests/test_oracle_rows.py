"""Pins of the oracle's speculative multi-row resolve (``Cache.resolve_rows``) -- CPU only.

"HiSparse 深度解析" (gentlecold.top) §6.5 comparison table and "HiSparse local
KV offload architecture" (docs.vllm.ai), speculative decoding: the verification
rows of one step are resolved together as the union of their selections, in
first-reference order; rows that select the same position share its slot and
no row evicts a slot another row reads.  Pinned by the one-row special case, by
identical rows, by a three-step example worked by hand (tests/golden), by the union's
order against numpy's first-occurrence indices, and by the independent list model run on a
union built here with a dictionary.
"""
import numpy as np
import pytest

import oracle
from oracle.brute import ListCache

REC = 16


def host_for(n_pos, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n_pos, REC), dtype=np.uint8)


def test_one_row_is_the_plain_resolve():
    rng = np.random.default_rng(2)
    U, B, k = 100, 20, 8
    host = host_for(U)
    a, b = oracle.Cache(B, U, REC), oracle.Cache(B, U, REC)
    for t in range(30):
        sel = rng.choice(U, size=k, replace=False)
        ra = a.resolve(sel, U, host)
        rb = b.resolve_rows(sel[None], U, host)
        assert np.array_equal(ra[0], rb[0][0]) and ra[1:3] == rb[1:3] and rb[6] == k
        assert np.array_equal(ra[3], rb[4]) and np.array_equal(ra[4], rb[5])
    for key in ("slot_pos", "stamp", "lru"):
        assert np.array_equal(a.export()[key], b.export()[key])


def test_identical_rows_share_every_slot():
    rng = np.random.default_rng(3)
    U, B, k = 100, 20, 8
    host = host_for(U)
    a, b = oracle.Cache(B, U, REC), oracle.Cache(B, U, REC)
    for t in range(20):
        sel = rng.choice(U, size=k, replace=False)
        ra = a.resolve(sel, U, host)
        rb = b.resolve_rows(np.stack([sel] * 4), U, host)
        assert all(np.array_equal(ra[0], row) for row in rb[0])
        assert rb[6] == k and ra[2] == rb[2]
    assert np.array_equal(a.export()["lru"], b.export()["lru"])


def union_first_reference(rows):
    seen, uni, idx = {}, [], []
    for row in rows:
        r_idx = []
        for p in row:
            p = int(p)
            if p not in seen:
                seen[p] = len(uni)
                uni.append(p)
            r_idx.append(seen[p])
        idx.append(r_idx)
    return uni, idx


@pytest.mark.parametrize("newest", [False, True])
def test_matches_list_model_on_the_union(newest):
    rng = np.random.default_rng(11 + newest)
    for trial in range(400):
        U = int(rng.integers(6, 24))
        k = int(rng.integers(1, 5))
        Q = int(rng.integers(1, 5))
        B = int(rng.integers(Q * k, Q * k + 4))
        host = host_for(U + 1, seed=trial)
        c = oracle.Cache(B, U + 1, REC, newest_slot=newest)
        lc = ListCache(B, newest_slot=newest)
        for t in range(int(rng.integers(1, 7))):
            if newest:
                nw = int(rng.integers(0, U))
                c.append(nw, host[nw], None)
                lc.append(nw)
            base = rng.choice(U, size=k, replace=False)
            rows = [base]
            for q in range(1, Q):  # verification rows overlap the first
                keep = rng.random(k) < 0.6
                fresh = [p for p in rng.permutation(U) if p not in base[keep]][: k - keep.sum()]
                rows.append(rng.permutation(np.concatenate([base[keep], fresh]).astype(np.int64)))
            rows = np.stack(rows).astype(np.int32)
            got = c.resolve_rows(rows, U, host)
            uni, idx = union_first_reference(rows)
            lo, lh, lm, lplan = lc.resolve(uni)
            exp = np.array([[lo[u] for u in r] for r in idx])
            assert np.array_equal(got[0], exp), (trial, t)
            assert (got[1], got[2], got[6]) == (lh, lm, len(uni))
            assert list(zip(got[4].tolist(), got[5].tolist())) == lplan
            assert c.export()["lru"].tolist() == lc.order
            # every row reads its own records afterwards
            for q in range(Q):
                for i in range(k):
                    assert np.array_equal(c.hot[got[0][q, i]], host[rows[q, i]])


def _golden_steps(path):
    """(B, positions, [(rows, slots, counts, plan, lru)]) from a worked example file."""
    B = U = None
    steps, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(" ")
        if key == "B":
            B = int(val)
        elif key == "positions":
            U = int(val)
        elif key == "step":
            cur = {"rows": [[int(x) for x in r.split(",")] for r in val.split(" ", 1)[1].split(";")]}
            steps.append(cur)
        elif key == "expect_slots":
            cur["slots"] = [[int(x) for x in r.split(",")] for r in val.split(";")]
        elif key == "expect_counts":
            cur["counts"] = [int(x) for x in val.split()]
        elif key == "expect_plan":
            cur["plan"] = [tuple(int(y) for y in x.split(":")) for x in val.split()]
        elif key == "expect_lru":
            cur["lru"] = [int(x) for x in val.split()]
    return B, U, steps


def test_worked_example_by_hand():
    """Three steps of overlapping rows from an empty buffer, the expected slots, counts, plan
    and LRU order worked out by hand from the union and stamp rules (tests/golden)."""
    import os
    B, U, steps = _golden_steps(os.path.join(os.path.dirname(__file__), "golden", "rows_union_example.txt"))
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    for n, st in enumerate(steps):
        got = c.resolve_rows(np.array(st["rows"], dtype=np.int32), U, host)
        assert got[0].tolist() == st["slots"], n
        assert [got[1], got[2], got[6]] == st["counts"], n
        assert list(zip(got[4].tolist(), got[5].tolist())) == st["plan"], n
        assert c.export()["lru"].tolist() == st["lru"], n


def test_union_order_is_the_order_of_first_occurrence():
    """From an empty buffer every union entry misses, so the miss plan lists the union in the
    order the call resolved it: the positions sorted by the index of their first occurrence in
    the rows laid end to end (numpy's unique gives those indices)."""
    rng = np.random.default_rng(29)
    for trial in range(200):
        U = int(rng.integers(8, 40))
        k = int(rng.integers(1, 6))
        Q = int(rng.integers(1, 5))
        rows = np.stack([rng.choice(U, size=k, replace=False) for _ in range(Q)]).astype(np.int32)
        flat = rows.reshape(-1)
        _, first = np.unique(flat, return_index=True)
        want = flat[np.sort(first)]
        c = oracle.Cache(Q * k, U, REC)
        got = c.resolve_rows(rows, U, host_for(U, seed=trial))
        assert got[1] == 0 and got[2] == want.size == got[6], trial
        assert np.array_equal(got[4], want), trial
        # the victims of an empty buffer are the slots in index order
        assert np.array_equal(got[5], np.arange(want.size)), trial


def test_duplicates_and_capacity():
    U, B = 50, 6
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    c.resolve_rows([[1, 2, 3]], U, host)
    before = c.export()
    with pytest.raises(oracle.OracleError) as e:  # a duplicate inside one row
        c.resolve_rows([[4, 5, 6], [7, 8, 7]], U, host)
    assert e.value.code == oracle.ERR_DUP
    with pytest.raises(oracle.OracleError) as e:  # the union does not fit B
        c.resolve_rows([[4, 5, 6], [7, 8, 9], [10, 1, 2]], U, host)
    assert e.value.code == oracle.ERR_CAPACITY
    with pytest.raises(oracle.OracleError) as e:
        c.resolve_rows([[4, 5, 60]], U, host)
    assert e.value.code == oracle.ERR_RANGE
    after = c.export()
    for key in ("slot_pos", "stamp", "lru", "step"):
        assert np.array_equal(before[key], after[key])
    # repeats across rows are not errors
    out = c.resolve_rows([[4, 5, 1], [1, 4, 9]], U, host)[0]
    assert out[0, 0] == out[1, 1] and out[0, 2] == out[1, 0]


def test_rows_with_resident_tier():
    U, B, shift = 64, 8, 2
    host = host_for(U)
    rt = np.full(U >> shift, -1, np.int32)
    rt[3] = 2  # positions 12..15 resident at rows 8..11
    a, b = oracle.Cache(B, U, REC), oracle.Cache(B, U, REC)
    rows = np.array([[12, 1, 2], [2, 13, 5]], np.int32)
    got = a.resolve_rows(rows, U, host, rt, shift, 64)
    uni, idx = union_first_reference(rows)
    ref = b.resolve_tiered(uni, U, rt, shift, 64, host)
    assert np.array_equal(got[0], np.array([[ref[0][u] for u in r] for r in idx]))
    assert got[3] == 2 and got[0][0, 0] == B + 1 + 8 and got[0][1, 1] == B + 1 + 9
