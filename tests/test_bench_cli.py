"""bench.py's host-side contract, on the CPU: a request for more than one GPU exits with a
message (the library has no multi-GPU path), and the algorithmic byte counts of a call follow
the arena's formats (per quantized token-head: the planes read plus one metadata pair per token
and one per channel per group)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_byte_counts_follow_the_formats():
    G, H, D, nq, nt, m = 128, 32, 128, 131072, 70, 7
    tail_io = H * (nt * 4 * D)
    # draft: both upper planes (D/2 bytes each), fp32 pairs: 8 B per token + 8 B per channel / G
    assert bench.draft_bytes(nq, nt, H, D) == H * nq * (D + 8 + 8 * D // G) + tail_io + H * 6 * D
    assert bench.draft_bytes(nq, nt, H, D, mb=4) == \
        H * nq * (D + 4 + 4 * D // G) + tail_io + H * 6 * D
    # verify: all four planes, m queries in and out
    assert bench.verify_bytes(nq, nt, H, D, m) == \
        H * nq * (2 * D + 8 + 8 * D // G) + tail_io + m * H * 6 * D
    assert bench.draft_bytes(nq, nt, H, D) - bench.draft_bytes(nq, nt, H, D, mb=4) == \
        H * nq * 4 * (1 + D // G)
