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


def test_cpu_baseline_times_every_phase():
    """The oracle baseline on the tiny workload: discovery, selection and late
    phases each timed, a single-thread sample, and the CPU model."""
    sys.path.insert(0, ROOT)
    import bench
    from wise_inputs import CONFIGS
    r = bench.cpu_baseline(CONFIGS["tiny"], 2, 5.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
    ph = r["phases"]
    assert ph["discovery_tflops"] > 0 and ph["late_tflops"] > 0 and ph["select_ms_per_head"] >= 0
    assert r["single_thread"]["threads"] == 1 and r["single_thread"]["late_tflops"] > 0
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert "2 selections" in r["sample"]


def test_quartiles():
    sys.path.insert(0, ROOT)
    import bench
    q = bench.quartiles([4.0, 1.0, 3.0, 2.0, 5.0])
    assert q == {"median": 3.0, "iqr": [2.0, 4.0]}
