"""Device memory of an on-demand hot buffer, as a plain set computation.

TEST INFRASTRUCTURE (like the rest of ``oracle``): used by ``tests/`` only.

"HiSparse 深度解析" (gentlecold.top) §5.4: the device buffer grows on demand
(``_grow_device_buffers``), so a short request does not hold all B slots from
the start; §5.3: a request longer than B gets the full B.  Reading used here
(the library's layout): the hot buffer is the fixed address range
[R][L][B+1][record_bytes]; a request grown to capacity c holds, in every layer,
its slots 0 .. c-1 and its newest slot B; device memory is committed in whole
chunks of ``chunk`` bytes of that range (a chunk may serve two neighbouring
layers or requests), and never released before teardown.  So the memory in
use is the number of distinct chunks that contain a held byte, times the chunk
size.
"""
from __future__ import annotations


def held_ranges(r: int, cap: int, L: int, B: int, rec: int):
    """Byte ranges [lo, hi) of the hot range that request r holds at capacity cap (every layer's
    slots 0 .. cap-1 and its newest slot B)."""
    out = []
    for l in range(L):
        base = ((r * L) + l) * (B + 1) * rec
        if cap > 0:
            out.append((base, base + cap * rec))
        out.append((base + B * rec, base + (B + 1) * rec))
    return out


def backed_bytes(caps: dict, L: int, B: int, rec: int, chunk: int) -> int:
    """Device bytes behind the hot buffer when request r has been grown to caps[r] (requests
    never grown are absent): the chunks that contain a held byte."""
    chunks = set()
    for r, cap in caps.items():
        for lo, hi in held_ranges(r, cap, L, B, rec):
            chunks.update(range(lo // chunk, (hi - 1) // chunk + 1))
    return len(chunks) * chunk
