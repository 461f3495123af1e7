"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test names the passage or the closed form it checks.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth
from oracle.brute import ListCache

REC = 16  # small records keep the byte checks cheap


def host_for(n_pos, rec=REC, seed=0):
    """Distinct bytes per position so that a wrong copy is always visible."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n_pos, rec), dtype=np.uint8)


def check_invariants(cache, sel, out, hits, misses, host, ctx, prev_sel=None, prev_newest=None):
    B = cache.B
    st = cache.export()
    pt = cache.page_table
    k = len(sel)
    assert hits + misses == k
    # slot_pos and page_table are mutual inverses over occupied slots
    occ = st["slot_pos"] >= 0
    assert occ.sum() <= B
    assert np.all(pt[st["slot_pos"][occ]] == np.nonzero(occ)[0])
    assert (pt >= 0).sum() == occ.sum()
    # every selected position is resident after the step, in the slot published for it
    for i, p in enumerate(sel):
        if out[i] == B:
            assert st["newest_pos"] == p
        else:
            assert pt[p] == out[i]
        assert np.array_equal(cache.hot[out[i]], host[p])
    # LRU order is the (stamp, slot) order and a permutation of the slots
    assert sorted(st["lru"].tolist()) == list(range(B))
    keys = [(st["stamp"][s], s) for s in st["lru"]]
    assert keys == sorted(keys)
    if prev_sel is not None and B >= k:
        resident_before = set(prev_sel) - ({prev_newest} if prev_newest is not None else set())
        assert misses <= len(set(sel) - resident_before)


# --- worked examples printed on the pages ---------------------------------------

def test_example_a_resolve_walkthrough(golden):
    """gentlecold.top §3.5: B=8, k=4 walk-through; exact slots and new LRU order."""
    g = dict(golden("example_a.txt"))
    B = int(g["B"][0])
    before_tokens = [int(x) for x in g["before_tokens"]]
    newest = int(g["newest"][0])
    sel = [int(x) for x in g["selection"]]
    host = host_for(64)
    c = oracle.Cache(B, 64, REC, newest_slot=True)
    # reach the printed state: two k=4 steps fill s0..s3 then s4..s7 (empty slots first)
    c.resolve(before_tokens[:4], newest, host)
    c.resolve(before_tokens[4:], newest, host)
    st = c.export()
    assert st["lru"].tolist() == [int(x) for x in g["before_lru"]]
    assert st["slot_pos"].tolist() == before_tokens
    c.append(newest, host[newest], None)
    out, hits, misses, ppos, pslot = c.resolve(sel, newest + 1, host)
    assert out.tolist() == [int(x) for x in g["expect_slots"]]
    assert hits == int(g["expect_hits"][0]) and misses == int(g["expect_misses"][0])
    assert c.export()["lru"].tolist() == [int(x) for x in g["expect_lru"]]
    assert ppos.tolist() == [25] and pslot.tolist() == [0]


def test_example_b_capacity(golden):
    """notes.kuangjux.top §5: {1,4,8},{1,5,8},{1,4,8}: B=3 misses at step 3, B=4 does not."""
    rows = golden("example_b.txt")
    sels = [[int(x) for x in v] for k, v in rows if k == "selection"]
    cases = [(int(v[0]), [int(x) for x in v[2:]]) for k, v in rows if k == "B"]
    assert len(cases) == 2
    host = host_for(16)
    for B, expect in cases:
        c = oracle.Cache(B, 16, REC)
        got = [c.resolve(s, 16, host)[2] for s in sels]
        assert got == expect, (B, got)
        lc = ListCache(B)
        assert [lc.resolve(s)[2] for s in sels] == expect


# --- closed forms ---------------------------------------------------------------

def stack_distance_misses(seq, B):
    """Mattson et al. (1970): under LRU with B entries a reference misses iff it is
    the first reference or more than B-1 distinct others came since its last use."""
    res = []
    for t, p in enumerate(seq):
        prev = [u for u in range(t) if seq[u] == p]
        if not prev:
            res.append(1)
        else:
            distinct = len(set(seq[prev[-1] + 1:t]))
            res.append(1 if distinct + 1 > B else 0)
    return res


@pytest.mark.parametrize("B", [1, 2, 3, 5, 8])
def test_k1_is_textbook_lru(B):
    """k=1: the per-step misses equal the stack-distance test for every B."""
    rng = np.random.default_rng(B)
    for trial in range(30):
        seq = rng.integers(0, 12, size=40).tolist()
        host = host_for(12)
        c = oracle.Cache(B, 12, REC)
        got = [c.resolve([p], 12, host)[2] for p in seq]
        assert got == stack_distance_misses(seq, B)


def test_b_equals_k_closed_form():
    """B=k: the buffer holds exactly S_t, so misses_1 = k and misses_t = |S_t \\ S_{t-1}|."""
    w = synth.WORKLOADS["tiny"]
    for r in range(3):
        tr = synth.selection_trace(w, r, 0)
        host = host_for(w.ctx)
        c = oracle.Cache(w.k, w.ctx, REC)
        for t in range(tr.shape[0]):
            out, hits, misses, _, _ = c.resolve(tr[t], w.ctx, host)
            expect = w.k if t == 0 else len(set(tr[t]) - set(tr[t - 1]))
            assert misses == expect


def test_large_buffer_only_compulsory_misses():
    """B >= |union of all selections|: each distinct position misses exactly once."""
    w = synth.WORKLOADS["tiny"].scaled(ctx=600)
    tr = synth.selection_trace(w, 0, 0)
    distinct = len(np.unique(tr))
    host = host_for(w.ctx)
    c = oracle.Cache(distinct + 3, w.ctx, REC)
    seen, total = set(), 0
    for t in range(tr.shape[0]):
        _, _, misses, ppos, _ = c.resolve(tr[t], w.ctx, host)
        assert set(ppos.tolist()).isdisjoint(seen)
        seen |= set(ppos.tolist())
        total += misses
    assert total == distinct


def test_first_step_fills_empty_slots_in_list_order():
    """Admission leaves every slot empty (gentlecold.top §5.3); empty slots go first,
    lowest index first, to the misses in list order: out = 0, 1, ..., k-1."""
    rng = np.random.default_rng(3)
    host = host_for(500)
    for B in (8, 13, 64):
        c = oracle.Cache(B, 500, REC)
        sel = rng.choice(500, size=min(B, 8), replace=False)
        out, hits, misses, ppos, pslot = c.resolve(sel, 500, host)
        assert out.tolist() == list(range(sel.size)) and misses == sel.size
        assert ppos.tolist() == sel.tolist() and pslot.tolist() == list(range(sel.size))


# --- brute force against the independent list model ----------------------------

def run_both(seqs, B, universe, newest=None):
    host = host_for(universe + 1)
    c = oracle.Cache(B, universe + 1, REC, newest_slot=newest is not None)
    lc = ListCache(B, newest_slot=newest is not None)
    for t, sel in enumerate(seqs):
        if newest is not None and newest[t] is not None:
            c.append(newest[t], host[newest[t]], None)
            lc.append(newest[t])
        a = c.resolve(sel, universe + 1, host)
        b = lc.resolve(sel)
        assert a[0].tolist() == b[0] and a[1] == b[1] and a[2] == b[2], (seqs, B, t)
        assert list(zip(a[3].tolist(), a[4].tolist())) == b[3]
        assert c.export()["lru"].tolist() == lc.order


@pytest.mark.parametrize("k", [1, 2])
def test_exhaustive_tiny_traces(k):
    """Every ordered selection sequence over 4 positions, 4 steps, B in k..k+3."""
    universe = 4
    sels = list(itertools.permutations(range(universe), k))
    for B in range(k, k + 4):
        for seqs in itertools.product(sels, repeat=4 if k == 1 else 3):
            run_both([list(s) for s in seqs], B, universe)


def test_random_traces_against_list_model():
    rng = np.random.default_rng(11)
    for trial in range(1500):
        universe = int(rng.integers(4, 14))
        k = int(rng.integers(1, min(6, universe) + 1))
        B = int(rng.integers(k, k + 5))
        steps = int(rng.integers(1, 9))
        seqs = [rng.choice(universe, size=k, replace=False).tolist() for _ in range(steps)]
        run_both(seqs, B, universe)


def test_random_traces_with_newest_slot():
    """With the reserved newest slot (gentlecold.top §3.4, §5.2): the newest position
    binds to slot B and stays out of the LRU; the previous newest lives on host only."""
    rng = np.random.default_rng(12)
    for trial in range(800):
        universe = int(rng.integers(6, 14))
        k = int(rng.integers(1, 5))
        B = int(rng.integers(k, k + 4))
        steps = int(rng.integers(1, 8))
        seqs, newest = [], []
        for t in range(steps):
            nw = int(rng.integers(0, universe))
            sel = rng.choice(universe, size=k, replace=False).tolist()
            if rng.random() < 0.6 and nw not in sel:
                sel[int(rng.integers(0, k))] = nw
            seqs.append(sel)
            newest.append(nw)
        run_both(seqs, B, universe, newest)


def test_newest_position_also_in_an_lru_slot():
    """Corner case the pages leave open: appending a position that an LRU slot
    already holds.  Reading: the newest slot serves it and the LRU slot counts as
    not selected (evictable), in both models."""
    for seqs, newest in [([[1, 2], [2, 3], [1, 2]], [None, 2, 2]),
                         ([[0, 1, 2], [2, 4, 5], [5, 0, 2]], [None, 2, 5])]:
        for B in (2, 3, 4, 6):
            if B >= len(seqs[0]):
                run_both(seqs, B, 8, newest)


# --- invariants over synthetic workloads ----------------------------------------

@pytest.mark.parametrize("B", [64, 96, 128, 256])
def test_invariants_tiny(B):
    w = synth.WORKLOADS["tiny"]
    tr = synth.selection_trace(w, 0, 0)
    host = host_for(w.ctx, seed=5)
    c = oracle.Cache(B, w.ctx, REC)
    prev = None
    for t in range(tr.shape[0]):
        out, hits, misses, _, _ = c.resolve(tr[t], w.ctx, host)
        check_invariants(c, tr[t], out, hits, misses, host, w.ctx, prev)
        prev = tr[t]


def test_invariants_with_append():
    """The long-request trace model scaled down: one token appended per step,
    written through, and always selected."""
    w = synth.WORKLOADS["long"].scaled(ctx=3000, k=64, B=128, steps=40)
    tr = synth.selection_trace(w, 0, 3)
    lmax = w.max_positions()
    host = host_for(lmax, seed=6)
    new_rec = host_for(lmax, seed=7)
    c = oracle.Cache(w.B, lmax, REC, newest_slot=True)
    prev, prev_newest = None, None
    for t in range(w.steps):
        p = w.ctx + t
        c.append(p, new_rec[p], host)
        assert np.array_equal(host[p], new_rec[p])
        assert p in set(tr[t].tolist())
        out, hits, misses, _, _ = c.resolve(tr[t], p + 1, host)
        check_invariants(c, tr[t], out, hits, misses, host, p + 1, prev, prev_newest)
        prev, prev_newest = tr[t], p


def test_miss_rate_falls_with_buffer_size_on_average():
    """Averaged over caches the miss count falls as B grows (not a per-trace
    invariant: a single trace can miss more with a larger buffer)."""
    w = synth.WORKLOADS["tiny"]
    totals = []
    for B in (64, 128, 256):
        tot = 0
        for r in range(6):
            tr = synth.selection_trace(w, r, 0)
            host = host_for(w.ctx)
            c = oracle.Cache(B, w.ctx, REC)
            tot += sum(c.resolve(tr[t], w.ctx, host)[2] for t in range(tr.shape[0]))
        totals.append(tot)
    assert totals[0] > totals[1] > totals[2]


# --- error handling ---------------------------------------------------------------

def test_errors_leave_state_unchanged():
    host = host_for(100)
    c = oracle.Cache(8, 100, REC)
    c.resolve([1, 2, 3], 100, host)
    before = c.export()
    pt_before = c.page_table.copy()
    with pytest.raises(oracle.OracleError) as e:
        c.resolve([4, 5, 4], 100, host)
    assert e.value.code == oracle.ERR_DUP
    with pytest.raises(oracle.OracleError) as e:
        c.resolve([4, 99], 50, host)
    assert e.value.code == oracle.ERR_RANGE
    with pytest.raises(oracle.OracleError) as e:
        c.resolve([4, -1, 4], 100, host)
    assert e.value.code == oracle.ERR_RANGE | oracle.ERR_DUP
    with pytest.raises(oracle.OracleError) as e:
        c.resolve(list(range(9)), 100, host)
    assert e.value.code == oracle.ERR_CAPACITY
    after = c.export()
    for key in ("slot_pos", "stamp", "lru"):
        assert np.array_equal(before[key], after[key])
    assert after["step"] == before["step"]
    assert np.array_equal(pt_before, c.page_table)


# --- blocks and shared layers ---------------------------------------------------

def test_block_expansion():
    """gentlecold.top §5.5: block ids expand to token positions; list order of blocks
    kept, tokens ascending within a block."""
    out = oracle.expand_blocks([3, 0, 7], 4)
    assert out.tolist() == [12, 13, 14, 15, 0, 1, 2, 3, 28, 29, 30, 31]


def test_shared_layer_lockstep():
    """gentlecold.top §3.6: a shared layer follows the anchor's plan with its own
    records; afterwards each occupied slot holds that layer's record of the position
    the anchor's slot holds."""
    w = synth.WORKLOADS["tiny"]
    tr = synth.selection_trace(w, 0, 0)
    host_a, host_s = host_for(w.ctx, seed=1), host_for(w.ctx, seed=2)
    c = oracle.Cache(w.B, w.ctx, REC)
    hot_s = np.zeros((w.B + 1, REC), np.uint8)
    for t in range(tr.shape[0]):
        out, _, _, ppos, pslot = c.resolve(tr[t], w.ctx, host_a)
        oracle.replay(ppos, pslot, host_s, hot_s, REC)
        st = c.export()
        occ = np.nonzero(st["slot_pos"] >= 0)[0]
        assert np.array_equal(hot_s[occ], host_s[st["slot_pos"][occ]])
        for i, p in enumerate(tr[t]):
            assert np.array_equal(hot_s[out[i]], host_s[p])


# --- attention --------------------------------------------------------------------

def bf16_bytes(x):
    import torch
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000).astype(np.float32)
    u = bf16_bytes(x)
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.attention.bf16_to_f64(u), ref)


def random_slots_case(rng, H=16, D=576, S=40, k=12):
    hot = np.stack([bf16_bytes(rng.standard_normal(D)).view(np.uint8) for _ in range(S)])
    q = bf16_bytes(rng.standard_normal((H, D)))
    slots = rng.choice(S, size=k, replace=False)
    return q, hot, slots


def test_attention_zero_query_is_mean_of_values():
    """q = 0: every score is 0, softmax is uniform, o = mean of the value rows."""
    rng = np.random.default_rng(1)
    q, hot, slots = random_slots_case(rng)
    q[:] = 0
    o = oracle.attention.sparse_decode_attention(q, hot, slots, 576 ** -0.5)
    V = oracle.attention.bf16_to_f64(hot[slots].view(np.uint16))[:, :512]
    assert np.allclose(o, V.mean(axis=0)[None, :].repeat(16, 0), rtol=0, atol=1e-13)


def test_attention_single_entry_returns_its_value():
    rng = np.random.default_rng(2)
    q, hot, slots = random_slots_case(rng, k=1)
    o = oracle.attention.sparse_decode_attention(q, hot, slots, 0.1)
    V = oracle.attention.bf16_to_f64(hot[slots[0]].view(np.uint16))[:512]
    assert np.allclose(o, V[None, :], rtol=0, atol=1e-15)


def test_attention_matches_library_sdpa():
    """Against torch's scaled_dot_product_attention in float64 (a library routine)."""
    import torch
    rng = np.random.default_rng(3)
    q, hot, slots = random_slots_case(rng, k=30)
    scale = 576 ** -0.5
    o = oracle.attention.sparse_decode_attention(q, hot, slots, scale)
    Q = torch.from_numpy(oracle.attention.bf16_to_f64(q))[None, :, None, :]
    KV = torch.from_numpy(oracle.attention.bf16_to_f64(hot[slots].view(np.uint16)))
    K = KV[None, None].expand(1, 16, -1, -1)
    V = KV[:, :512][None, None].expand(1, 16, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, :, 0, :]
    assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_attention_invariant_to_entry_order():
    rng = np.random.default_rng(4)
    q, hot, slots = random_slots_case(rng, k=20)
    a = oracle.attention.sparse_decode_attention(q, hot, slots, 0.05)
    b = oracle.attention.sparse_decode_attention(q, hot, slots[::-1].copy(), 0.05)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
