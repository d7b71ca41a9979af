"""Host-side checks of bench.py's contract (no GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_traffic_needs_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (tmp_path / "decode_megakernel_wg_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "decode_megakernel_wg_amd" / "csrc" / "k.hip").write_text("kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()
    (prof / "mk_persistent_b1_8k_hbm_counters.md").write_text(
        f"Kernel source hash (sha256 ...): `{h}`\n\n| traffic_bytes_per_launch | 123456 |\n")
    assert bench.counter_traffic("b1_8k") == 123456
    (tmp_path / "decode_megakernel_wg_amd" / "csrc" / "k.hip").write_text("kernel v2")
    assert bench.counter_traffic("b1_8k") is None
    assert bench.counter_traffic("long_64k") is None
