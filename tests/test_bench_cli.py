"""Host-side checks of the benchmark script (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_recorded_traffic_is_tied_to_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    digest = bench.kernel_source_digest()
    assert len(digest) == 64
    workload = "kimi_k2_experts_648x2048x7168_bf16_gaussian_plus_rank32_spike"
    rec = bench.recorded_traffic("gemm_rect", workload)
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_k2_experts_648x2048x7168.md")) as f:
        text = f.read()
    if digest in text:
        # the committed counters were taken on these sources: the bench reports them
        assert rec is not None and rec[0] > 0
    else:
        assert rec == (None, None)
