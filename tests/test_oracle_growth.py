"""Pins of oracle.growth (device memory of an on-demand hot buffer) without a GPU: a closed form
on chunk-aligned layer regions, a byte-level brute force on small random layouts, and the
whole range when every request holds all B slots."""
import numpy as np

from oracle import growth


def test_closed_form_on_chunk_aligned_regions():
    """When each layer's region (B + 1 records) is a whole number of chunks and a record does not
    straddle a chunk, a request of capacity c holds ceil(c * rec / chunk) chunks of each layer
    below its newest slot, plus the chunk of the newest slot (unless those overlap)."""
    rec, chunk = 64, 256
    B = 4 * chunk // rec * 3 - 1          # (B + 1) * rec = 12 chunks
    assert (B + 1) * rec % chunk == 0
    for L in (1, 3):
        for cap in (0, 1, 4, 5, 40, B - 4):
            per_layer = -(-cap * rec // chunk) + 1
            assert growth.backed_bytes({0: cap}, L, B, rec, chunk) == L * per_layer * chunk, (L, cap)
        # two requests: disjoint regions, so the counts add up
        assert growth.backed_bytes({0: 7, 1: 9}, L, B, rec, chunk) == \
            growth.backed_bytes({0: 7}, L, B, rec, chunk) + growth.backed_bytes({1: 9}, L, B, rec, chunk)


def test_brute_force_bytes():
    """Every byte a grown request holds marked in an array; the chunks that contain a marked
    byte, counted, on random small layouts (records straddling chunks, regions sharing them)."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        R, L = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        rec = 16 * int(rng.integers(1, 9))
        B = int(rng.integers(1, 40))
        chunk = 16 * int(rng.integers(1, 20))
        total = R * L * (B + 1) * rec
        caps = {r: int(rng.integers(0, B + 1)) for r in range(R) if rng.random() < 0.8}
        held = np.zeros(total, bool)
        for r, cap in caps.items():
            for l in range(L):
                region = (r * L + l) * (B + 1) * rec
                held[region:region + cap * rec] = True
                held[region + B * rec:region + (B + 1) * rec] = True
        n_chunks = -(-total // chunk)
        padded = np.zeros(n_chunks * chunk, bool)
        padded[:total] = held
        want = int(padded.reshape(n_chunks, chunk).any(axis=1).sum()) * chunk
        assert growth.backed_bytes(caps, L, B, rec, chunk) == want, (R, L, rec, B, chunk, caps)


def test_full_capacity_is_the_whole_range():
    R, L, B, rec, chunk = 3, 2, 100, 1152, 65536
    total = R * L * (B + 1) * rec
    assert growth.backed_bytes({r: B for r in range(R)}, L, B, rec, chunk) == -(-total // chunk) * chunk


def test_growth_is_monotone():
    R, L, B, rec, chunk = 2, 3, 256, 1152, 65536
    prev = 0
    for cap in range(0, B + 1, 7):
        cur = growth.backed_bytes({0: cap, 1: cap // 2}, L, B, rec, chunk)
        assert cur >= prev
        prev = cur
