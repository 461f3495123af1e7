"""Pins of the oracle's resident-first resolve (``Cache.resolve_tiered``) -- CPU only.

"HiSparse 深度解析" (gentlecold.top) §6.5 and "HiSparse local KV offload
architecture" (docs.vllm.ai), "Hot lookup and LRU": each selected position is
looked up in the resident pages first, then in the hot slots, then fetched from
host; a call whose selection is entirely resident returns before any hot-LRU
work.  Pinned by the special case without resident pages (plain resolve), by the
all-resident invariants, and by the independent list model run on the entries
the resident tier does not serve.
"""
import numpy as np
import pytest

import oracle
from oracle.brute import ListCache

REC = 16


def host_for(n_pos, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n_pos, REC), dtype=np.uint8)


def random_table(rng, n_pages, frac, pool_pages):
    rt = np.full(n_pages, -1, np.int32)
    pick = np.nonzero(rng.random(n_pages) < frac)[0]
    rt[pick] = rng.permutation(pool_pages)[: pick.size]
    return rt


def test_no_resident_pages_is_the_plain_resolve():
    rng = np.random.default_rng(1)
    U, B, k, shift = 200, 24, 10, 3
    host = host_for(U)
    a, b = oracle.Cache(B, U, REC), oracle.Cache(B, U, REC)
    rt = np.full(U >> shift, -1, np.int32)
    for t in range(40):
        sel = rng.choice(U, size=k, replace=False)
        ra = a.resolve(sel, U, host)
        rb = b.resolve_tiered(sel, U, rt, shift, 1 << 20, host)
        assert np.array_equal(ra[0], rb[0]) and ra[1:3] == rb[1:3] and rb[3] == 0
        assert np.array_equal(ra[3], rb[4]) and np.array_equal(ra[4], rb[5])
    ea, eb = a.export(), b.export()
    for key in ("slot_pos", "stamp", "lru", "step"):
        assert np.array_equal(ea[key], eb[key])


def test_all_resident_returns_rows_and_changes_nothing():
    U, B, shift = 256, 16, 2
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    c.resolve([5, 9, 17, 33], U, host)
    before, pt = c.export(), c.page_table.copy()
    rt = np.full(U >> shift, -1, np.int32)
    rt[2] = 7      # positions 8..11 on resident page 7: rows 28..31
    rt[4] = 0      # positions 16..19 on resident page 0: rows 0..3
    sel = [9, 16, 11, 19, 9]  # resident throughout, one position twice
    out, hits, misses, res, ppos, pslot = c.resolve_tiered(sel, U, rt, shift, 32, host)
    assert out.tolist() == [B + 1 + 29, B + 1 + 0, B + 1 + 31, B + 1 + 3, B + 1 + 29]
    assert (hits, misses, res) == (0, 0, 5) and ppos.size == 0
    after = c.export()
    for key in ("slot_pos", "stamp", "lru", "step"):
        assert np.array_equal(before[key], after[key])
    assert np.array_equal(pt, c.page_table)


def test_errors():
    U, B, shift = 64, 8, 2
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    c.resolve([1, 2], U, host)
    before = c.export()
    rt = np.full(U >> shift, -1, np.int32)
    rt[3] = 4  # rows 16..19, beyond a pool of 16 rows
    with pytest.raises(oracle.OracleError) as e:
        c.resolve_tiered([13, 1], U, rt, shift, 16, host)
    assert e.value.code == oracle.ERR_RESIDENT
    rt[3] = 1
    with pytest.raises(oracle.OracleError) as e:  # a duplicate is caught once any entry is not resident
        c.resolve_tiered([13, 1, 13], U, rt, shift, 16, host)
    assert e.value.code == oracle.ERR_DUP
    with pytest.raises(oracle.OracleError) as e:
        c.resolve_tiered([13, 70], U, rt, shift, 16, host)
    assert e.value.code == oracle.ERR_RANGE
    after = c.export()
    for key in ("slot_pos", "stamp", "lru", "step"):
        assert np.array_equal(before[key], after[key])


@pytest.mark.parametrize("newest", [False, True])
def test_matches_list_model_on_the_non_resident_entries(newest):
    """The resident tier answers first; the list model sees only the other entries."""
    rng = np.random.default_rng(7 + newest)
    for trial in range(300):
        U = int(rng.integers(8, 40))
        shift = int(rng.integers(0, 3))
        n_pages = (U + (1 << shift) - 1) >> shift
        pool_pages = n_pages + 2
        k = int(rng.integers(1, 7))
        B = int(rng.integers(k, k + 5))
        host = host_for(U + 1, seed=trial)
        c = oracle.Cache(B, U + 1, REC, newest_slot=newest)
        lc = ListCache(B, newest_slot=newest)
        for t in range(int(rng.integers(1, 9))):
            rt = random_table(rng, n_pages + 1, float(rng.uniform(0, 0.7)), pool_pages)
            nw = None
            if newest:
                nw = int(rng.integers(0, U))
                c.append(nw, host[nw], None)
                lc.append(nw)
            sel = rng.choice(U, size=k, replace=False)
            res_rows = pool_pages << shift
            got = c.resolve_tiered(sel, U, rt, shift, res_rows, host)
            # independent composition: resident rows by definition, the rest through the list model
            page = sel >> shift
            is_res = rt[page] >= 0
            exp = np.empty(k, np.int64)
            exp[is_res] = B + 1 + (rt[page[is_res]].astype(np.int64) << shift) + (sel[is_res] & ((1 << shift) - 1))
            if is_res.all():
                assert got[0].tolist() == exp.tolist() and got[1:4] == (0, 0, k)
                continue
            lo, lh, lm, lplan = lc.resolve(sel[~is_res].tolist())
            exp[~is_res] = lo
            assert got[0].tolist() == exp.tolist(), (trial, t)
            assert (got[1], got[2], got[3]) == (lh, lm, int(is_res.sum()))
            assert list(zip(got[4].tolist(), got[5].tolist())) == lplan
            assert c.export()["lru"].tolist() == lc.order
            # bytes: every hot entry holds its position's record
            for i in np.nonzero(~is_res)[0]:
                assert np.array_equal(c.hot[got[0][i]], host[sel[i]]) or got[0][i] == B


def test_slot_of_a_resident_position_is_evictable():
    """A hot slot whose position is now served by the resident tier is not selected through
    the LRU: it is the first victim when it is the least recent."""
    U, B, shift = 64, 2, 0
    host = host_for(U)
    c = oracle.Cache(B, U, REC)
    rt = np.full(U, -1, np.int32)
    c.resolve_tiered([3, 4], U, rt, shift, 64, host)   # slot 0 <- 3, slot 1 <- 4
    c.resolve_tiered([4], U, rt, shift, 64, host)      # 4 hit: slot 0 (holding 3) is least recent
    rt[4] = 9                                           # position 4 becomes resident
    out = c.resolve_tiered([3, 4, 5], U, rt, shift, 64, host)[0]
    # 3 hits slot 0; 4 is resident (row 9); 5 takes slot 1 although 4 is selected
    assert out.tolist() == [0, B + 1 + 9, 1]
    assert c.export()["slot_pos"].tolist() == [3, 5]
