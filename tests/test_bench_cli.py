"""bench.py's command-line contract that holds without a GPU: more than one
GPU is refused with a message, and the FLOP convention and the per-kernel
algorithmic work it reports follow the page's counts."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_convention():
    import bench
    B, H, L, D, R = 2, 12, 8192, 64, 512
    # BH(14 L^2 D + 16 L R D) = forward BH(4L^2D + 4LRD) + backward BH(10L^2D + 12LRD)
    assert bench.flops_fwd_bwd(B, H, L, D, R) == B * H * (4 * L * L * D + 4 * L * R * D) + \
        B * H * (10 * L * L * D + 12 * L * R * D)
    assert abs(bench.flops_fwd_bwd(B, H, L, D, R) - 1.5462e12) / 1.5462e12 < 1e-4
    per, rel = B * H * L * L * D, B * H * L * R * D
    assert bench.kernel_algorithmic_flops("fwd", B, H, L, D, R) == 4 * per
    assert bench.kernel_algorithmic_flops("bwd_dkv", B, H, L, D, R) == 8 * per + 2 * rel
    assert bench.kernel_algorithmic_flops("bwd_dq", B, H, L, D, R) == 6 * per + 2 * rel
    assert bench.kernel_algorithmic_flops("delta", B, H, L, D, R) is None


def test_latency_distribution_fields():
    import bench
    d = bench.dist([5.0, 1.0, 3.0, 2.0, 4.0])
    assert d == {"n": 5, "min": 1.0, "p10": 1.0, "median": 3.0, "p90": 5.0}
