"""The benchmark's host-side contract (no GPU): one GPU only, and the committed HBM-traffic
figures are used only while the kernel sources they were taken from are unchanged."""
import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def _profile(tmp_path, source_text, recorded_text):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text(source_text)
    digest = hashlib.sha256(recorded_text.encode()).hexdigest()
    (tmp_path / "profiles" / "kern_long_traffic.txt").write_text(
        "# HBM traffic per launch\nbytes_per_launch: 123456\nsource_files: k.hip\nsource_sha256: %s\n" % digest)


def test_traffic_used_while_sources_unchanged(tmp_path, monkeypatch):
    _profile(tmp_path, "kernel v1", "kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profile_traffic("kern") == 123456.0


def test_traffic_nulled_when_sources_change(tmp_path, monkeypatch):
    _profile(tmp_path, "kernel v2", "kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profile_traffic("kern") is None
    assert bench.profile_traffic("missing") is None


def test_committed_profiles_name_existing_sources():
    """Every committed traffic summary names source files that exist and a command that runs
    committed files only (bench.py)."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith(".txt")]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "rocprofv3" in text and "bench.py" in text, n
        assert "_work" not in text, n
        for line in text.splitlines():
            if line.startswith("source_files:"):
                for src in line.split(":", 1)[1].split():
                    assert os.path.exists(os.path.join(ROOT, src)), (n, src)


def test_precomputed_addresses_match_the_views():
    """bench.addr(t, i, ...) is the address of the view t[i, ...], for every buffer shape and
    index the timed loop uses (contiguous and permuted-then-contiguous tensors, leading
    indices only)."""
    import torch
    steps, L, R, k = 5, 3, 2, 7
    tensors = [
        torch.zeros((steps, L, R, k), dtype=torch.int32),          # selections
        torch.zeros((steps, L, R, 6), dtype=torch.int32),            # stats
        torch.zeros((steps, R), dtype=torch.int32),                # context lengths
        torch.zeros((steps, R, L, 9), dtype=torch.uint8),          # new records
        torch.zeros((steps, R, L, 3, 5), dtype=torch.int16).permute(0, 2, 1, 3, 4).contiguous(),  # queries
        torch.zeros((L, R, 3, 6), dtype=torch.float32),            # outputs
    ]
    for t in tensors:
        for i in range(t.shape[0]):
            assert bench.addr(t, i) == t[i].data_ptr()
            if t.dim() > 2:
                for j in range(t.shape[1]):
                    assert bench.addr(t, i, j) == t[i, j].data_ptr()
