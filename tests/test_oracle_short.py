"""Pins of the oracle's short-sequence fast path -- CPU only.

"HiSparse 深度解析" (gentlecold.top) §5.4 and §5.5: while a request's context
fits the device buffer, its tokens sit in the buffer in order and the kernel
returns the positions' own slots at once, with no host IO.  Reading used here:
admission stages the first tokens into slots 0 .. ctx-1, appends extend that
while they fit, the LRU is not touched meanwhile, and once the context exceeds
B the normal path starts from "slots 0 .. B-1 hold positions 0 .. B-1, never
used".  Pinned by these definitions and, after the switch, by the independent
list model started from that state.
"""
import numpy as np
import pytest

import oracle
from oracle.brute import ListCache

REC = 16


def host_for(n_pos, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n_pos, REC), dtype=np.uint8)


def test_fast_path_returns_positions_and_changes_nothing():
    B, U = 16, 64
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    c.admit_short(10, host)
    st0 = c.export()
    assert st0["slot_pos"].tolist() == list(range(10)) + [-1] * 6
    for sel in ([3, 1, 9], [0, 5, 2, 8], [9]):
        out, hits, misses, _, _ = c.resolve(sel, 10, host)
        assert out.tolist() == sel and (hits, misses) == (len(sel), 0)
        for i, p in enumerate(sel):
            assert np.array_equal(c.hot[out[i]], host[p])
    st = c.export()
    for key in ("slot_pos", "stamp", "lru", "step"):
        assert np.array_equal(st[key], st0[key])
    # the pages' fast path checks nothing but the range
    assert c.resolve([2, 2], 10, host)[0].tolist() == [2, 2]
    with pytest.raises(oracle.OracleError) as e:
        c.resolve([2, 10], 10, host)
    assert e.value.code == oracle.ERR_RANGE


def test_admission_needs_an_empty_cache_and_a_short_context():
    host = host_for(64)
    c = oracle.Cache(8, 64, REC)
    with pytest.raises(oracle.OracleError):
        c.admit_short(9, host)
    c.resolve([1, 2], 64, host)
    with pytest.raises(oracle.OracleError):
        c.admit_short(4, host)


def test_switch_to_the_normal_path_matches_the_list_model():
    """Appends keep tokens in order while they fit; past B the cache behaves like the list
    model started from slots 0..B-1 holding 0..B-1 in slot order.  (A short request grows
    only by appends, so the switch always finds the B slots full.)"""
    newest = True
    rng = np.random.default_rng(5)
    for trial in range(150):
        B = int(rng.integers(4, 12))
        k = int(rng.integers(1, B + 1))
        ctx0 = int(rng.integers(k, B + 1))
        U = B + 20
        host = host_for(U + 1, seed=trial)
        c = oracle.Cache(B, U + 1, REC, newest_slot=True)
        c.admit_short(ctx0, host)
        lc = None
        ctx = ctx0
        for t in range(12):
            if newest:  # a decode step appends one token
                c.append(ctx, host[ctx], None)
                ctx += 1
            sel = rng.choice(ctx, size=min(k, ctx), replace=False).tolist()
            res = c.resolve(sel, ctx, host)
            if ctx <= B:
                assert res[0].tolist() == sel
                continue
            if lc is None:  # the first normal step: the state the short phase left
                lc = ListCache(B, newest_slot=True)
                lc.holds = list(range(B))
                lc.order = list(range(B))
                if newest:
                    lc.append(ctx - 1)
            elif newest:
                lc.append(ctx - 1)
            exp = lc.resolve(sel)
            assert res[0].tolist() == exp[0] and (res[1], res[2]) == (exp[1], exp[2]), (trial, t)
            assert c.export()["lru"].tolist() == lc.order
            for i, p in enumerate(sel):
                assert np.array_equal(c.hot[res[0][i]], host[p])


def test_fast_path_precedes_the_resident_tier_and_serves_rows():
    B, U, shift = 16, 64, 2
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    c.admit_short(12, host)
    rt = np.full(U >> shift, -1, np.int32)
    rt[1] = 3
    out, hits, misses, res, _, _ = c.resolve_tiered([5, 1, 9], 12, rt, shift, 64, host)
    assert out.tolist() == [5, 1, 9] and (hits, misses, res) == (3, 0, 0)
    rows = c.resolve_rows([[1, 2, 3], [3, 4, 1]], 12, host)
    assert rows[0].tolist() == [[1, 2, 3], [3, 4, 1]] and rows[1] == 4 and rows[6] == 4
