"""The measurement probes: the scattered-record gather reads exactly the indexed records."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_kv_cache_amd as hk  # noqa: E402


@pytest.mark.parametrize("rec,n", [(1152, 1000), (656, 37), (16, 1)])
def test_host_record_gather(rec, n):
    print("gather rec=%d n=%d" % (rec, n), flush=True)
    nsrc = 4096
    rng = np.random.Generator(np.random.PCG64(rec + n))
    src = torch.from_numpy(rng.integers(0, 256, size=(nsrc, rec), dtype=np.uint8)).pin_memory()
    idx = rng.integers(0, nsrc, size=n).astype(np.int32)
    idx[::7] = -1          # skipped
    idx[3::11] = nsrc      # skipped
    dst = torch.full((n, rec), 0xAB, dtype=torch.uint8, device="cuda")
    d_idx = torch.from_numpy(idx).cuda()
    hk.hs_probe_host_records(src.data_ptr(), nsrc, rec, d_idx.data_ptr(), n, dst.data_ptr(), 64, 0)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    ok = (idx >= 0) & (idx < nsrc)
    assert np.array_equal(got[ok], src.numpy()[idx[ok]])
    assert (got[~ok] == 0xAB).all()


def test_host_record_gather_rejects_bad_sizes():
    src = torch.empty(1024, dtype=torch.uint8).pin_memory()
    d = torch.empty(1024, dtype=torch.uint8, device="cuda")
    i = torch.zeros(1, dtype=torch.int32, device="cuda")
    for rec in (0, 8, 24, 32768):
        with pytest.raises(hk.HsError):
            hk.hs_probe_host_records(src.data_ptr(), 1, rec, i.data_ptr(), 1, d.data_ptr(), 1, 0)
    with pytest.raises(hk.HsError):
        hk.hs_probe_host_records(src.data_ptr(), 1, 16, i.data_ptr(), 1, d.data_ptr(), 0, 0)
