"""bench.py's command line on the CPU: it measures one GPU only, so any
request for more GPUs (the flag or a launcher's WORLD_SIZE) stops before
anything is imported or allocated, with a message and exit status 2."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          timeout=120, env=e)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_launcher_world_size_is_refused():
    r = _run(["--gpus", "1"], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_workloads():
    r = _run(["--help"])
    assert r.returncode == 0
    for word in ("--layer", "fc1", "nf4_fc1", "--launch", "--settle-ms", "--tokens"):
        assert word in r.stdout


def test_traffic_entries_cover_their_own_workload_only():
    """The HBM traffic a bench line reports belongs to one workload shape:
    other shapes of the same kernel (1024 tokens, QKV) report none, and every
    entry names a kernel source that exists."""
    sys.path.insert(0, ROOT)
    import bench
    for name, t in bench.TRAFFIC.items():
        assert os.path.exists(os.path.join(ROOT, "w4a4_rank_corrected_quantize_amd", "csrc", t["source"])), name
        assert t["bytes"] > 0
    for other in ("mx1k_fc1", "mx1k_qkv", "qkv", "mx_qkv", "fc2", "nf4_qkv"):
        assert bench.measured_traffic(other) is None
