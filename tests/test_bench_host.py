"""Host-side checks of bench.py (no GPU needed)."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_refuses_multi_rank_launch():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_is_well_formed():
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    t = bench.measured_traffic()
    # null when the attention kernel changed since the counters were taken,
    # else read + written bytes of one sparse launch
    assert t is None or (isinstance(t, int) and t > 0)
