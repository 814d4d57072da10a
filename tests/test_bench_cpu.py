"""bench.py's host-side contract without a GPU: it measures one GPU only and says so for any
other count, and the recorded counter traffic is used only for the sources it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_recorded_traffic_needs_a_matching_record():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.recorded_traffic("no-such-workload", "decode_kernel") is None
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
