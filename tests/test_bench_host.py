"""Host-side checks of bench.py's contract (no GPU): one GPU only, and the
FLOP / byte accounting it reports."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_flop_and_byte_accounting():
    # 4 B H N^2 d, halved for causal; the headline workload's figures
    assert bench.attention_flops(4, 16, 4096, 64, True) == 137438953472
    assert bench.attention_flops(1, 32, 8192, 128, False) == 1099511627776
    assert bench.bwd_flops(4, 16, 4096, 64, True) == 2.5 * 137438953472
    # Q, K, V, O once plus the fp32 lse; K and V with H_kv heads
    assert bench.algorithmic_bytes(4, 16, 4096, 64, 2) == 135266304
    assert bench.algorithmic_bytes(4, 16, 4096, 64, 2, H_kv=4) == \
        2 * 4 * (16 + 4) * 4096 * 64 * 2 + 4 * 4 * 16 * 4096


def test_traffic_is_tied_to_the_kernel_sources():
    """roofline.traffic comes from committed counters only while the kernel
    sources hash as they did when the counters were taken."""
    import json
    with open(bench.COUNTER_FILE) as f:
        data = json.load(f)
    entry = data["c3_bf16_causal"]
    got = bench.measured_traffic("c3_bf16_causal")
    if entry["kernel_source_sha"] == bench.kernel_source_hash():
        assert got == entry["hbm_bytes_per_launch"]
    else:
        assert got is None
    assert bench.measured_traffic("no_such_workload") is None


def test_device_state_degrades_to_nulls_without_a_device():
    """The clock / power sampler runs outside the timed region and must never
    fail a bench run: without a GPU (or without amdsmi) every field is None,
    and the function returns without calling the step; the timed-region
    clock sampler then collects nothing."""
    calls = []
    smi = bench._NoSmi()
    state = bench.device_state_under_load(smi, lambda: calls.append(1), seconds=0.05)
    assert set(state) == {"gfx_clock_mhz", "socket_power_w", "hotspot_c", "limit_fracs"}
    assert all(v is None for v in state.values()) and not calls
    with bench.ClockSampler(smi) as clk:
        pass
    assert clk.window(0.0, 1e30) == (None, 0) and clk.samples == []


def test_clock_window_picks_readings_by_host_time():
    clk = bench.ClockSampler(bench._NoSmi())
    clk.samples = [(1.0, 2100.0), (2.0, 1900.0), (3.0, 1800.0), (4.0, 1850.0), (9.0, 2400.0)]
    assert clk.window(2.0, 4.0) == (1850.0, 3)
    assert clk.window(5.0, 8.0) == (None, 0)


def test_limit_fractions():
    v0 = {"ticks": 100, "ppt_pwr": 10, "socket_thrm": 0}
    v1 = {"ticks": 300, "ppt_pwr": 110, "socket_thrm": 50}
    assert bench._Smi.limit_fracs(v0, v1) == {"ppt_pwr": 0.5, "socket_thrm": 0.25}
    assert bench._Smi.limit_fracs(v0, v0) is None


def test_every_pass_has_its_runner():
    """Each --pass of bench.py resolves to a function of the module (a run on
    the GPU is the only other place that would notice a missing one)."""
    for name in ("run_bwd", "run_unfused", "_time_calls", "median_launch_ms", "parity_stats",
                 "cpu_baseline", "cpu_baseline_bwd", "device_state_under_load"):
        assert callable(getattr(bench, name, None)), name
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    defined = set()
    for n in ast.walk(tree):
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            defined.add(n.name)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
            defined.add(n.id)
        elif isinstance(n, ast.arg):
            defined.add(n.arg)
        elif isinstance(n, ast.alias):
            defined.add((n.asname or n.name).split(".")[0])
    called = {n.func.id for n in ast.walk(tree)
              if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    import builtins
    missing = {c for c in called if c not in defined and not hasattr(builtins, c)}
    assert not missing, missing
