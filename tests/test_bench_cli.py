"""bench.py's contract pieces that need no GPU: the one-GPU guard and the
algorithmic byte accounting its roofline divides by."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_algorithmic_bytes_per_element():
    import bench
    N, W, k, L = 1_000_000, 4, 10_000, 3
    rows = L * 8192 * 4  # the histogram rows the dense pass zeroes
    # dense pass: W bf16 gradients and W fp32 residuals read, W residuals
    # written, m read, a 16-bit key written, one mask bit read; W sparse
    # entries and the m stash written per masked element
    dense, step = bench.alg_bytes(N, W, k, L, fused=False)
    assert dense == N * (2 * W + 4 * W + 4 * W + 4 + 2 + 1 / 8) + k * (4 * W + 4) + rows
    # the step adds the key's read by the selection and the next mask's bits,
    # and per masked element the buffers' reads, idx / m-stash / x reads and
    # x / m / v / next-idx writes
    assert step == N * (10 * W + 4 + 2 + 2 + 1 / 8 + 1 / 8) + k * (4 * W + 4 * W + 7 * 4) + rows
    # with the update in the dense pass: per masked element the W sparse
    # entries written, x read and x / m / v written; the step adds the
    # next mask's idx
    dense, step = bench.alg_bytes(N, W, k, L, fused=True)
    assert dense == N * (2 * W + 4 * W + 4 * W + 4 + 2 + 1 / 8) + k * (4 * W + 4 + 3 * 4) + rows
    assert step == N * (10 * W + 4 + 2 + 2 + 1 / 8 + 1 / 8) + k * (4 * W + 4 + 3 * 4 + 4) + rows
    assert bench.fused_update(64 * 32, 64) and bench.fused_update(64 * 32 - 1, 64)
    assert not bench.fused_update(64 * 32, 64, on=False)
    assert not bench.streams_whole(64 * 32, 64) and bench.streams_whole(64 * 32 - 1, 64)
    assert bench.dense_kernel_name(8, True, True, True) == "k_ef_compact<8, false, 4> (with the update)"
    assert bench.dense_alg_bytes(N, W) == N * (2 * W + 4 + 4 + 4 + 4 + 4)


def test_source_hash_is_stable():
    import bench
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_source_hash() == h
