"""Host logic of bench.py, without a GPU: the algorithmic flop and byte counts per
token-head, the rule that a committed counter summary is used only for the kernel sources it
was taken on, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_counts():
    # 5 C d + 6 d^2 at C = 64, d = 128: A and Aqk, the solve for both right-hand sides,
    # Aqk U', and the three state products
    assert bench.flops_per_token_head() == 5 * 64 * 128 + 6 * 128 * 128 == 139264
    # minimal bytes: q, k, g, v and beta in bf16 read once, a bf16-sized o written once
    assert bench.bytes_per_token_head() == 4 * 128 * 2 + 2 + 128 * 2 == 1282
    # the same with the fp32 o the library writes
    assert bench.bytes_per_token_head(out_bytes=4) == 1538
    # S0 read and S_T written once, fp32: 128 KiB per (sequence, head)
    assert bench.state_bytes(1, 16) == 16 * 2 * 4 * 128 * 128


def test_traffic_needs_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x_traffic.txt").write_text("# comment = 1\nkernel_src_sha = abc123\n"
                                        "hbm_bytes_per_launch = 4096\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("x_traffic.txt", "abc123") == 4096.0
    assert bench.read_traffic("x_traffic.txt", "other") is None
    assert bench.read_traffic("missing.txt", "abc123") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
