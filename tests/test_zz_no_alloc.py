"""hs_sparse_attn_static: the attention call that allocates nothing (its chunk partials in a
file-scope device array of the library) against hs_sparse_attn on the same handle, inputs
and slots -- the same kernels, so the outputs must agree bit for bit.  Two calls in a row, the
second with a smaller input (fewer requests, a shorter selection, fewer heads), then the first
shape again; also the size limit and a skipped (padded) request."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_kv_cache_amd as hk  # noqa: E402
import synth  # noqa: E402

SCALE = 576 ** -0.5


def log(msg):
    print(msg, flush=True)


class Case:
    """A handle whose hot slots hold records, one resolved selection per request, queries."""

    def __init__(self, R, k, B, heads, steps=3, seed_w="batched", ctx=8192):
        w = synth.WORKLOADS[seed_w].scaled(R=R, L=1, k=k, B=B, ctx=ctx)
        self.R, self.k, self.heads = R, k, heads
        self.c = hk.HiSparse(hk.make_config(R, 1, ctx, k, B))
        for r in range(R):
            synth.fill_request(self.c.host_pool_address(r), r, 1, ctx, ctx)
        tr = np.stack([synth.selection_trace(w, r, 0, steps) for r in range(R)], axis=1)  # [steps][R][k]
        d_ctx = torch.full((R,), ctx, dtype=torch.int32, device="cuda")
        self.slots = torch.empty((R, k), dtype=torch.int32, device="cuda")
        st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device="cuda")
        for t in range(steps):  # a few steps, so that hits and misses both feed the slots
            sel = torch.from_numpy(tr[t]).cuda()
            hk.hs_resolve(self.c.h, 0, sel.data_ptr(), d_ctx.data_ptr(), self.slots.data_ptr(), st.data_ptr(),
                          0, 0, 0)
        torch.cuda.synchronize()
        assert not st[:, 2].any()
        self.q = torch.from_numpy(synth.queries(R, 1, 7, heads=heads)[:, 0].view(np.int16)).cuda()

    def run(self, static, num_reqs=None):
        out = torch.full((self.R, self.heads, 512), -3.0, dtype=torch.float32, device="cuda")
        nr = torch.tensor([num_reqs], dtype=torch.int32, device="cuda") if num_reqs is not None else None
        fn = hk.hs_sparse_attn_static if static else hk.hs_sparse_attn
        fn(self.c.h, 0, self.q.data_ptr(), self.heads, 512, self.slots.data_ptr(), out.data_ptr(), SCALE,
           nr.data_ptr() if nr is not None else 0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        return out

    def close(self):
        self.c.close()


def check(case, num_reqs=None):
    ref = case.run(False, num_reqs)
    got = case.run(True, num_reqs)
    assert torch.isfinite(ref[: num_reqs or case.R]).all()
    assert torch.equal(got, ref), float((got - ref).abs().max())


def test_static_matches_workspace_call_big_then_small():
    big = Case(R=32, k=2048, B=4096, heads=16)   # 32 x 8 chunks: 256 partial records
    small = Case(R=3, k=300, B=512, heads=5)     # 3 x 5 chunks
    try:
        log("R=32 k=2048 heads=16")
        check(big)
        log("R=3 k=300 heads=5 (smaller, right after)")
        check(small)
        log("R=32 again, then 20 of 32 requests (the rest skipped and untouched)")
        check(big)
        check(big, num_reqs=20)
    finally:
        big.close()
        small.close()


def test_static_size_limit_is_an_error():
    """More partial records than the static array holds: HS_EINVAL, nothing enqueued."""
    case = Case(R=300, k=2048, B=2048, heads=1, steps=1, ctx=4096)  # 300 requests x 2 chunks
    try:
        with pytest.raises(hk.HsError) as e:
            case.run(True)
        assert e.value.code == hk.HS_EINVAL and "static scratch" in str(e.value)
        ref = case.run(False)  # the workspace call still works
        assert torch.isfinite(ref).all()
    finally:
        case.close()
