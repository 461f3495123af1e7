"""Pins of the offline policy comparator (oracle/policies.py) -- CPU only.

Pinned by textbook page-replacement results, by an exhaustive search for the
optimum on tiny traces, by the closed form of the B = k policy, and by the C
stamp oracle's LRU on the seeded workloads.
"""
from __future__ import annotations

import itertools
from functools import lru_cache

import numpy as np
import pytest

import oracle
import synth
from oracle import policies
from synth.traces import selection_trace

# Silberschatz, Galvin & Gagne, "Operating System Concepts", chapter on virtual
# memory: this reference string with 3 frames gives 15 faults under FIFO, 12
# under LRU and 9 under the optimal algorithm.
TEXTBOOK = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]
# Belady, Nelson & Shedler (1969), "An anomaly in space-time characteristics of
# certain programs running in a paging machine": FIFO on this string faults 9
# times with 3 frames and 10 times with 4.
ANOMALY = [1, 2, 3, 4, 1, 2, 5, 1, 2, 3, 4, 5]


def single(seq):
    return [[p] for p in seq]


@pytest.mark.parametrize("policy,faults", [("fifo", 15), ("lru", 12), ("belady", 9)])
def test_textbook_reference_string(policy, faults):
    assert policies.simulate(single(TEXTBOOK), 3, policy).sum() == faults


def test_belady_anomaly_fifo():
    assert policies.simulate(single(ANOMALY), 3, "fifo").sum() == 9
    assert policies.simulate(single(ANOMALY), 4, "fifo").sum() == 10
    # LRU is a stack algorithm: more frames never fault more on a single-entry string
    assert policies.simulate(single(ANOMALY), 4, "lru").sum() <= policies.simulate(single(ANOMALY), 3, "lru").sum()


def test_fifo_evicts_in_insertion_order():
    # step 1 fills 1, 2, 3 in selection order; 4 then replaces 1 (first in), so 3 stays resident
    assert list(policies.simulate([[1, 2, 3], [4], [3], [1]], 3, "fifo")) == [3, 1, 0, 1]
    # a hit does not refresh FIFO age: 1 is hit at step 2 and still evicted at step 3,
    # where LRU evicts 2 instead
    assert list(policies.simulate([[1, 2], [1], [3], [1]], 2, "fifo")) == [2, 0, 1, 1]
    assert list(policies.simulate([[1, 2], [1], [3], [1]], 2, "lru")) == [2, 0, 1, 0]


def brute_min_misses(trace, B):
    """Fewest misses over every choice of victims (resident sets only; slots do not matter)."""
    sels = [frozenset(s) for s in trace]

    @lru_cache(maxsize=None)
    def best(t, resident):
        if t == len(sels):
            return 0
        s = sels[t]
        miss = s - resident
        free = B - len(resident)
        need = len(miss) - free
        if need <= 0:
            return len(miss) + best(t + 1, resident | miss)
        out = None
        for ev in itertools.combinations(sorted(resident - s), need):
            v = best(t + 1, (resident - frozenset(ev)) | miss)
            out = v if out is None else min(out, v)
        return len(miss) + out

    return best(0, frozenset())


def random_traces(n, universe, k, steps, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        yield [list(rng.choice(universe, size=k, replace=False)) for _ in range(steps)]


@pytest.mark.parametrize("k,B", [(1, 2), (2, 3), (2, 4), (3, 4), (3, 5)])
def test_belady_is_optimal_on_tiny_traces(k, B):
    for tr in random_traces(60, 7, k, 6, seed=100 * k + B):
        assert policies.simulate(tr, B, "belady").sum() == brute_min_misses(tr, B), tr


def test_belady_never_worse_than_online_policies():
    for tr in random_traces(40, 40, 8, 30, seed=5):
        for B in (8, 12, 16):
            opt = policies.simulate(tr, B, "belady").sum()
            for pol in ("fifo", "random", "lru"):
                assert opt <= policies.simulate(tr, B, pol, seed=3).sum()


def test_topk_closed_form():
    w = synth.WORKLOADS["tiny"]
    tr = selection_trace(w, 0, 0, 32)
    ms = policies.simulate(list(tr), w.B, "topk")
    assert ms[0] == w.k
    for t in range(1, len(tr)):
        assert ms[t] == np.setdiff1d(tr[t], tr[t - 1]).size


def test_every_policy_holds_the_selection():
    # with B >= distinct positions, each position misses exactly once under every policy
    for tr in random_traces(10, 30, 5, 12, seed=9):
        distinct = len({p for s in tr for p in s})
        for pol in ("fifo", "random", "lru", "belady"):
            assert policies.simulate(tr, 30, pol).sum() == distinct


def test_random_is_seeded():
    tr = next(random_traces(1, 50, 6, 40, seed=2))
    a = policies.simulate(tr, 9, "random", seed=7)
    assert np.array_equal(a, policies.simulate(tr, 9, "random", seed=7))


def oracle_misses(tr, B, newest=None, lmax=None):
    """Per-step misses and the final slot map of the C stamp oracle."""
    lmax = lmax or int(max(max(s) for s in tr)) + 2
    c = oracle.Cache(B, lmax, 16, newest_slot=newest is not None)
    host = np.zeros((lmax, 16), np.uint8)
    out = []
    for t, s in enumerate(tr):
        if newest is not None:
            c.append(newest[t], np.zeros(16, np.uint8), host)
        res = c.resolve(np.asarray(s, np.int32), lmax, host)
        out.append(res[2])
    return np.array(out), c.export()["slot_pos"]


@pytest.mark.parametrize("name", ["tiny", "long", "capacity"])
def test_lru_matches_stamp_oracle(name):
    w = synth.WORKLOADS[name]
    if name != "tiny":
        w = w.scaled()
    steps = min(w.steps, 24)
    for r, l, tr, newest in policies.workload_traces(w, requests=[0], layers=[0], steps=steps):
        lmax = w.max_positions(steps)
        got, holds = policies.simulate(tr, w.B, "lru", newest, return_slots=True)
        exp, slot_pos = oracle_misses(tr, w.B, newest, lmax)
        assert np.array_equal(got, exp)
        assert np.array_equal(holds, slot_pos)


def test_compare_rows_are_ordered():
    w = synth.WORKLOADS["tiny"]
    rows = policies.compare(w, [("topk", w.k), ("lru", 2 * w.k), ("belady", 2 * w.k)])
    rate = {p: r for p, _, r, _ in rows}
    assert rate["belady"] <= rate["lru"] <= rate["topk"]
