"""Benchmark of the fused attention forward on one MI355X.

A step is one attention forward (one launch of the fused kernel) over the
workload's synthetic inputs, which are resident in HBM before timing starts.
Default workload: bf16, causal, B=4, H=16, N=4096, d=64.

Prints ONE JSON line with the attention TFLOPS, its roofline fraction and
the CPU fp64 oracle timed on a bounded sample of the same workload.
``--pass bwd`` times the backward pass (dQ, dK, dV) instead: one step is one
attn_bwd call (its three or four kernels) with q, k, v, o, lse and dO
resident.
``--pass unfused`` times the unfused three-kernel forward (S, softmax, P V
with N x N buffers) and, on the same inputs, the fused kernel, and reports
what fusion gains.

FLOP convention (every page's): 4*B*H*N^2*d per forward, halved for causal —
checked against the figures printed in "Flash Attention（二）v2版本朴素实现
cuda core", section 4.1, and in the final table of "Flash Attention CUDA
Kernel 优化: 从 56 到 986 TFLOPS on B300 — G7: 回归 1CTA".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth.
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0

DTYPE_NAME = {"torch.bfloat16": "bf16", "torch.float16": "fp16", "torch.float32": "fp32"}

# Work of the CPU baseline: the multi-core sample (whole (b,h) slices; all 64
# of the headline workload, ~5-15 s on 16 cores) and the single-thread one.
CPU_FLOPS = 150e9
PER_CORE_FLOPS = 2e9

COUNTER_FILE = os.path.join(ROOT, "profiles", "attn_fwd_hbm_counters.txt")
# Sources of the kernel the committed counters were taken on (the bf16 /
# fp16 forward, its launcher and the entry point).
KERNEL_SOURCES = ["exact_attention_15_amd/csrc/fwd_mfma16.hip",
                  "exact_attention_15_amd/csrc/fwd_order.h",
                  "exact_attention_15_amd/csrc/mfma_common.h",
                  "exact_attention_15_amd/csrc/attn_api.hip",
                  "exact_attention_15_amd/csrc/attn_internal.h"]


def attention_flops(B, H, N, d, causal) -> float:
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def algorithmic_bytes(B, H, N, d, elem_bytes, H_kv=None) -> int:
    """Q, K, V read once, O written once, plus the fp32 lse row statistic
    (K and V have H_kv heads under grouped-query attention)."""
    H_kv = H if H_kv is None else H_kv
    return 2 * B * (H + H_kv) * N * d * elem_bytes + 4 * B * H * N


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, or None when absent or taken on other kernel sources."""
    if not os.path.exists(COUNTER_FILE):
        return None
    with open(COUNTER_FILE) as f:
        data = json.load(f)
    entry = data.get(workload)
    if not entry or entry.get("kernel_source_sha") != kernel_source_hash():
        return None
    return entry["hbm_bytes_per_launch"]


def bwd_flops(B, H, N, d, causal) -> float:
    """Five N x N x d products (dV, dP, dQ, dK and the recomputed S): 2.5x the
    forward's two, halved for causal — the convention that sets backward
    FLOPs against the forward's. The dQ kernel's second S and dP products
    are not counted."""
    return 2.5 * attention_flops(B, H, N, d, causal)


def cpu_baseline(w, q, k, v, n_slices: int):
    import numpy as np
    import oracle

    oracle.build() if not os.path.exists(oracle.LIB_PATH) else None
    threads = len(os.sched_getaffinity(0))
    rows = np.arange(n_slices * w.N, dtype=np.int64)   # every row of the first slices
    t0 = time.perf_counter()
    oracle.attn_fwd_ref_rows(q, k, v, w.causal, w.scale, rows, num_threads=threads)
    dt = time.perf_counter() - t0
    flops = attention_flops(1, n_slices, w.N, w.d, w.causal)
    # One core: the last rows of slice 0 (they see every key), single-threaded,
    # about PER_CORE_FLOPS of the rows' own products (4 d FLOP per visible key).
    rows1, flops1 = [], 0.0
    for i in range(w.N - 1, -1, -1):
        rows1.append(i)
        flops1 += 4.0 * w.d * (i + 1 if w.causal else w.N)
        if flops1 >= PER_CORE_FLOPS:
            break
    t1 = time.perf_counter()
    oracle.attn_fwd_ref_rows(q, k, v, w.causal, w.scale, np.array(rows1, dtype=np.int64),
                             num_threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{n_slices} of {w.B * w.H} (b,h) slices, all {w.N} rows each "
                      f"({flops / 1e9:.1f} GFLOP by the same convention), {dt:.2f} s wall",
            "per_core_value": flops1 / dt1 / 1e12,
            "per_core_sample": f"the last {len(rows1)} rows of slice 0 on one thread "
                               f"({flops1 / 1e9:.2f} GFLOP), {dt1:.2f} s wall"}


def cpu_baseline_bwd(w, q, k, v, dout, n_kv: int):
    """The oracle's backward on the first n_kv K/V slices (each with its query
    heads), timed on the host cores."""
    import oracle

    oracle.build() if not os.path.exists(oracle.LIB_PATH) else None
    threads = len(os.sched_getaffinity(0))
    G = w.H // w.kv_heads
    dt = 0.0
    for s in range(n_kv):
        b, hk = divmod(s, w.kv_heads)
        hs = slice(hk * G, (hk + 1) * G)
        sub = tuple(t.contiguous() for t in (q[b:b + 1, hs], k[b:b + 1, hk:hk + 1],
                                             v[b:b + 1, hk:hk + 1], dout[b:b + 1, hs]))
        t0 = time.perf_counter()
        oracle.attn_bwd_ref(*sub, w.causal, w.scale, num_threads=threads)
        dt += time.perf_counter() - t0
    flops = bwd_flops(1, n_kv * G, w.N, w.d, w.causal)
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"backward of {n_kv} of {w.B * w.kv_heads} K/V slices with their "
                      f"{G} query head(s) each, all {w.N} rows "
                      f"({flops / 1e9:.1f} GFLOP by the same convention), {dt:.2f} s wall"}


def run_bwd(args, name, w):
    """Backward-pass bench line (``--pass bwd``)."""
    import numpy as np
    import torch

    import exact_attention_15_amd as ea
    from exact_attention_15_amd.inputs import workload_dout, workload_inputs

    dt_name = DTYPE_NAME[str(w.dtype)]
    ea.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = workload_inputs(w)
    dout = workload_dout(w)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    o, lse = ea.fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    G = w.H // w.kv_heads
    out = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
           torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev))

    parity = None
    if not args.no_check:
        # First K/V slice: o / lse from the oracle, gradients against the
        # oracle's, within the first-order rounding bound of the parity tests.
        import oracle
        sub = tuple(t.contiguous() for t in (q[:1, :G], k[:1, :1], v[:1, :1], dout[:1, :G]))
        o_r, l_r = oracle.attn_fwd_ref(sub[0], sub[1], sub[2], w.causal, w.scale)
        o[:1, :G] = torch.from_numpy(o_r).to(w.dtype).to(dev)
        lse[:1, :G] = torch.from_numpy(l_r).to(torch.float32).to(dev)
        grads = ea.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, out=out)
        torch.cuda.synchronize()
        ref = oracle.attn_bwd_ref(*sub, w.causal, w.scale, error_scales=True)
        u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -12}[dt_name]
        s_half = {"bf16": 2.0 ** -134, "fp16": 2.0 ** -25, "fp32": 2.0 ** -150}[dt_name]
        worst = 0.0
        for got, r, e, z in zip((grads[0][:1, :G], grads[1][:1, :1], grads[2][:1, :1]),
                                ref[:3], ref[3:6], ref[6:9]):
            diff = np.abs(got.cpu().double().numpy() - r)
            bound = 2 * ((u + (G * w.N / 16 + 32) * 2.0 ** -24) * (e + np.abs(r)) +
                         s_half * (z + 1))
            worst = max(worst, float((diff / bound).max()))
        parity = worst
        if not worst <= 1.0:
            print(f"bench.py: backward parity gate failed: err/bound {worst:.3f}", file=sys.stderr)
            sys.exit(1)

    for _ in range(args.warmup):
        ea.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        ea.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, out=out)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / args.steps
    flops = bwd_flops(w.B, w.H, w.N, w.d, w.causal)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dt_name]
    line = {
        "metric": "attention bwd TFLOPS (dQ, dK, dV; 2.5x forward FLOPs); % of MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic (seeded i.i.d. N(0,1) inputs and dO rounded to the dtype)",
        "config": {"workload": w.describe().replace("fwd", "bwd"), "name": name, "B": w.B,
                   "H": w.H, "H_kv": w.kv_heads, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.scale},
        "pct_of_peak": round(100 * tflops / peak, 2),
        # One attn_bwd call (three kernels) is the unit timed here.
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": None},
        "parity_err_over_bound_slice0": parity,
        "wall_s_timed_region": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        n_kv = max(1, min(args.cpu_slices or 4, w.B * w.kv_heads))
        line["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, dout, n_kv)
    print(json.dumps(line), flush=True)


def median_launch_ms(fn, n: int = 200) -> float:
    """Median of n launches, each bracketed by its own pair of HIP events
    (outside the timed region)."""
    import torch
    stream = torch.cuda.current_stream()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for e0, e1 in pairs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
    return ts[n // 2]


class _Smi:
    """Read-only amdsmi queries for the current device; every method returns
    None where amdsmi is missing or refuses the query."""

    # Accumulated throttle counters of amdsmi_get_violation_status, each a
    # count of firmware ticks (acc_counter) spent under that limit.
    LIMITS = {"ppt_pwr": "acc_ppt_pwr", "socket_thrm": "acc_socket_thrm",
              "prochot_thrm": "acc_prochot_thrm", "vr_thrm": "acc_vr_thrm",
              "hbm_thrm": "acc_hbm_thrm", "gfx_clk_below_host_limit": "acc_gfx_clk_below_host_limit"}

    def __init__(self):
        import torch
        self.ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.h = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
            self.ok = True
        except Exception:
            pass

    def _try(self, f, *a):
        if not self.ok:
            return None
        try:
            return f(*a)
        except Exception:
            return None

    def clock_mhz(self):
        info = self._try(self.amdsmi.amdsmi_get_clock_info, self.h, self.amdsmi.AmdSmiClkType.GFX) \
            if self.ok else None
        clk = info.get("clk") if isinstance(info, dict) else None
        return float(clk) if isinstance(clk, (int, float)) and clk > 0 else None

    def socket_power_w(self):
        pw = self._try(self.amdsmi.amdsmi_get_power_info, self.h) if self.ok else None
        sp = pw.get("socket_power") if isinstance(pw, dict) else None
        return float(sp) if isinstance(sp, (int, float)) and sp > 0 else None

    def power_cap_w(self):
        cap = self._try(self.amdsmi.amdsmi_get_power_cap_info, self.h) if self.ok else None
        c = cap.get("power_cap") if isinstance(cap, dict) else None
        return round(c / 1e6, 1) if isinstance(c, (int, float)) and c > 0 else None   # microwatts

    def hotspot_c(self):
        if not self.ok:
            return None
        a = self.amdsmi
        t = self._try(a.amdsmi_get_temp_metric, self.h, a.AmdSmiTemperatureType.HOTSPOT,
                      a.AmdSmiTemperatureMetric.CURRENT)
        return float(t) if isinstance(t, (int, float)) else None

    def violations(self):
        v = self._try(self.amdsmi.amdsmi_get_violation_status, self.h) if self.ok else None
        if not isinstance(v, dict) or not isinstance(v.get("acc_counter"), int):
            return None
        out = {"ticks": v["acc_counter"]}
        for name, key in self.LIMITS.items():
            if isinstance(v.get(key), int):
                out[name] = v[key]
        return out

    @staticmethod
    def limit_fracs(v0, v1):
        """Share of the ticks between two violation readings spent under each limit."""
        if not v0 or not v1 or v1["ticks"] <= v0["ticks"]:
            return None
        dt = v1["ticks"] - v0["ticks"]
        return {k: round((v1[k] - v0[k]) / dt, 3) for k in v1 if k != "ticks" and k in v0}

    def close(self):
        self._try(self.amdsmi.amdsmi_shut_down) if self.ok else None


def device_state_under_load(smi, fn, seconds: float = 2.0, ms_per_call: float = 0.1):
    """GFX clock (MHz), socket power (W) and hotspot temperature, medians of
    amdsmi readings taken while launches of fn keep the GPU busy, and the
    share of that time the firmware held the clock down under each of its
    limits (package power, socket / VR / HBM temperature, PROCHOT, below the
    host's clock limit). amdsmi's readings trail the load by up to about a
    second, so launches run without a break for `seconds` and only the
    second half counts; each reading is taken with ~25 ms of launches queued
    and kept only while the stream still has work pending."""
    import torch
    state = {"gfx_clock_mhz": None, "socket_power_w": None, "hotspot_c": None,
             "limit_fracs": None}
    if not smi.ok:
        return state
    clocks, powers, temps, v0 = [], [], [], None
    stream = torch.cuda.current_stream()
    per_sample = max(10, int(25.0 / max(ms_per_call, 1e-3)))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(per_sample):
            fn()
        if time.perf_counter() - t0 < seconds / 2:
            continue
        if v0 is None:
            v0 = smi.violations()
        clk, sp, tc = smi.clock_mhz(), smi.socket_power_w(), smi.hotspot_c()
        if not stream.query():
            clocks += [clk] if clk else []
            powers += [sp] if sp else []
            temps += [tc] if tc is not None else []
    v1 = smi.violations()
    torch.cuda.synchronize()
    med = lambda xs: sorted(xs)[len(xs) // 2] if xs else None   # noqa: E731
    state.update(gfx_clock_mhz=med(clocks), socket_power_w=med(powers), hotspot_c=med(temps),
                 limit_fracs=smi.limit_fracs(v0, v1))
    return state


class ClockSampler:
    """Polls the GFX clock from a second thread (amdsmi calls release the
    interpreter lock), one reading every ~0.5 ms with its host time, so
    that the readings inside any host-time window (the timed region) can be
    picked afterwards. It is started before the warm-up: no amdsmi call then
    separates the warm-up from the timed region (an idle gap of a few ms
    there measurably slows the first launches after it)."""

    def __init__(self, smi):
        import threading
        self.smi, self.samples, self._stop = smi, [], threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True) if smi.ok else None

    def _run(self):
        while not self._stop.wait(0.0005):
            c = self.smi.clock_mhz()
            if c:
                self.samples.append((time.perf_counter(), c))

    def __enter__(self):
        if self._t:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()
        return False

    def window(self, t0, t1):
        """(median, count) of the readings taken between host times t0, t1."""
        xs = sorted(c for t, c in self.samples if t0 <= t <= t1)
        return (xs[len(xs) // 2] if xs else None), len(xs)


def _time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, time.perf_counter() - t_wall


def run_unfused(args, name, w):
    """Unfused-versus-fused comparison line (``--pass unfused``)."""
    import numpy as np
    import torch

    import exact_attention_15_amd as ea
    from exact_attention_15_amd.inputs import workload_inputs

    dt_name = DTYPE_NAME[str(w.dtype)]
    elem = 4 if dt_name == "fp32" else 2
    ea.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = workload_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    ws = torch.empty(ea.unfused_workspace_bytes(w.B, w.H, w.N, ea.dtype_code(w.dtype)),
                     dtype=torch.uint8, device=dev)
    o, lse = ea.fwd_unfused(qd, kd, vd, causal=w.causal, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    parity = None
    if not args.no_check:
        import oracle
        rng = np.random.default_rng(1)
        rows = np.unique(np.concatenate([np.arange(8), rng.integers(0, w.B * w.H * w.N, 56)]))
        o_ref, _ = oracle.attn_fwd_ref_rows(q, k, v, w.causal, w.scale, rows)
        parity = float(np.abs(o.cpu().double().numpy().reshape(-1, w.d)[rows] - o_ref).max())
        if not parity <= (1e-4 if elem == 4 else 2e-2):
            print(f"bench.py: unfused parity gate failed: {parity:.3e}", file=sys.stderr)
            sys.exit(1)
    steps = max(1, args.steps // 10)
    ms_u, t_wall = _time_calls(lambda: ea.fwd_unfused(qd, kd, vd, causal=w.causal,
                                                      scale=w.scale, workspace=ws),
                               steps, max(1, args.warmup // 10))
    out = (torch.empty_like(qd), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev))
    ms_f, _ = _time_calls(lambda: ea.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=out),
                          args.steps, args.warmup)
    flops = attention_flops(w.B, w.H, w.N, w.d, w.causal)
    tflops = flops / (ms_u * 1e-3) / 1e12
    ld = (w.N + 63) // 64 * 64
    # The method's own traffic: S written and read (fp32), P written and read
    # (in the input type), plus Q, K, V read and O, lse written.
    mbytes = (w.B * w.H * w.N * ld * (4 + 4 + 2 * elem)
              + algorithmic_bytes(w.B, w.H, w.N, w.d, elem))
    gbs = mbytes / (ms_u * 1e-3) / 1e9
    line = {
        "metric": "unfused attention fwd TFLOPS (S, softmax, P V as three kernels)",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(1, args.warmup // 10),
        "ms_per_step": round(ms_u, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic (seeded i.i.d. N(0,1) inputs rounded to the dtype)",
        "config": {"workload": w.describe() + " (unfused)", "name": name, "B": w.B, "H": w.H,
                   "N": w.N, "d": w.d, "causal": w.causal, "scale": w.scale},
        # The unfused path is bound by its N x N traffic.
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "fused_ms_per_step": round(ms_f, 5),
        "fused_tflops": round(flops / (ms_f * 1e-3) / 1e12, 2),
        "fusion_speedup": round(ms_u / ms_f, 2),
        "parity_o_max_abs_sampled": parity,
        "wall_s_timed_region": round(t_wall, 4),
    }
    print(json.dumps(line), flush=True)


class _NoSmi(_Smi):
    def __init__(self):
        self.ok = False


def parity_stats(w, q, k, v, o, lse, n_rows: int = 2048):
    """O and lse against the oracle on sampled rows (the first 8 and n_rows
    drawn at random): O max-abs and mean-abs error, the noise-to-signal
    ratio ||O - O_ref|| / ||O_ref|| and the lse max-abs error."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(8), rng.integers(0, w.B * w.H * w.N, n_rows)]))
    o_ref, l_ref = oracle.attn_fwd_ref_rows(q, k, v, w.causal, w.scale, rows)
    o_got = o.cpu().double().numpy().reshape(-1, w.d)[rows]
    l_got = lse.cpu().double().numpy().reshape(-1)[rows]
    diff = np.abs(o_got - o_ref)
    return {"rows": int(len(rows)), "o_max_abs": float(diff.max()),
            "o_mean_abs": float(diff.mean()),
            "o_nsr": float(np.linalg.norm(o_got - o_ref) / np.linalg.norm(o_ref)),
            "lse_max_abs": float(np.abs(l_got - l_ref).max())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # The GPU needs ~1000 back-to-back launches (a few hundred ms) to reach
    # its sustained clocks; fewer warm-up launches time a ramping clock.
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd", "unfused"], default="fwd",
                    help="time the forward (default), the backward pass, or the unfused "
                         "forward against the fused one")
    ap.add_argument("--cpu-slices", type=int, default=None,
                    help="slices the CPU oracle baseline runs on: (b,h) slices for the forward "
                         "(default: as many as fit 150 GFLOP, all 64 of the headline workload), "
                         "K/V slices for the backward (default 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled parity gate")
    ap.add_argument("--no-device-state", action="store_true",
                    help="skip the ~2 s of extra launches that sample clock and power "
                         "(for runs under a counter profiler, which serialises every launch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by (b,h) slices with no exchange, but no multi-GPU run exists)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 3}))
        return

    import exact_attention_15_amd as ea
    from exact_attention_15_amd.inputs import HEADLINE, WORKLOADS, workload_inputs

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    if args.pass_ == "bwd":
        run_bwd(args, name, w)
        return
    if args.pass_ == "unfused":
        run_unfused(args, name, w)
        return
    dt_name = DTYPE_NAME[str(w.dtype)]
    ea.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    q, k, v = workload_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    out = (o, lse)
    # One step is one attn_fwd_gqa call. The wrapper's checks run once
    # (through ea.fwd, whose result the parity gate reads); the timed calls
    # pass the same validated pointers straight to the C entry point, so the
    # host enqueues each launch in a few microseconds and the GPU does not
    # wait on Python between launches.
    ea.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=out)
    torch.cuda.synchronize()
    lib = ea.load_library()
    c_args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
              w.kv_heads, w.N, w.d, int(w.causal), w.scale, ea.dtype_code(w.dtype),
              torch.cuda.current_stream(dev).cuda_stream)

    def step_fn():
        rc = lib.attn_fwd_gqa(*c_args)
        if rc != 0:
            raise ea.AttnError(rc, ea.strerror(rc), "attn_fwd_gqa")

    # Parity gate on the first launch, before anything is timed: sampled rows
    # against the oracle, with the error statistics reported in the line.
    errs = None
    if not args.no_check:
        errs = parity_stats(w, q, k, v, o, lse)
        tol = 1e-4 if dt_name == "fp32" else 2e-2
        if not errs["o_max_abs"] <= tol:
            print(f"bench.py: parity gate failed: O max-abs {errs['o_max_abs']:.3e} > {tol}",
                  file=sys.stderr)
            sys.exit(1)

    # Per-launch median and the device's sustained state under this load
    # (clock, power, temperature, throttle shares), measured before the
    # warm-up: the GPU then enters the warm-up and the timed region already
    # at its sustained clock.
    smi = _Smi()
    ms_median = median_launch_ms(step_fn)
    dev_state = (device_state_under_load(smi, step_fn, ms_per_call=ms_median)
                 if not args.no_device_state else
                 dict.fromkeys(("gfx_clock_mhz", "socket_power_w", "hotspot_c", "limit_fracs")))

    # Warm-up, then the timed region: barrier-equivalent sync, K launches
    # bracketed by HIP events recorded on the stream the kernels run on, sync.
    # A second thread reads the GFX clock meanwhile.
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with ClockSampler(smi if not args.no_device_state else _NoSmi()) as clk:
        for _ in range(args.warmup):
            step_fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(args.steps):
            step_fn()
        stop.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    t_wall = t1 - t0
    ms = start.elapsed_time(stop) / args.steps
    clk_timed, clk_n = clk.window(t0, t1)
    power_cap = smi.power_cap_w()
    smi.close()

    flops = attention_flops(w.B, w.H, w.N, w.d, w.causal)
    tflops = flops / (ms * 1e-3) / 1e12
    elem = 4 if dt_name == "fp32" else 2
    abytes = algorithmic_bytes(w.B, w.H, w.N, w.d, elem, w.kv_heads)
    peak = PEAK_TFLOPS[dt_name]
    traffic = measured_traffic(name)
    lf = dev_state["limit_fracs"] or {}

    # The headline workload carries the headline metric's name; the others
    # the same measure, named for their own dtype (config names the shape).
    metric = ("attention fwd TFLOPS (bf16, causal, N=4096 d=64); % of MFMA peak" if name == HEADLINE
              else f"attention fwd TFLOPS ({dt_name}); % of MFMA peak")
    line = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic (seeded i.i.d. N(0,1) inputs rounded to the dtype)",
        "config": {"workload": w.describe(), "name": name, "B": w.B, "H": w.H,
                   "H_kv": w.kv_heads, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.scale},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic},
        "ms_median_launch": round(ms_median, 5),
        "gfx_clock_mhz_timed_region": clk_timed,
        "gfx_clock_samples_timed_region": clk_n,
        "gfx_clock_mhz_under_load": dev_state["gfx_clock_mhz"],
        "socket_power_w_under_load": dev_state["socket_power_w"],
        "hotspot_c_under_load": dev_state["hotspot_c"],
        "power_cap_w": power_cap,
        "power_limited_frac_under_load": lf.get("ppt_pwr"),
        "limit_fracs_under_load": dev_state["limit_fracs"],
        "algorithmic_gb_s": round(abytes / (ms * 1e-3) / 1e9, 1),
        "exp_per_s": (w.B * w.H * w.N * w.N / (2 if w.causal else 1)) / (ms * 1e-3),
        "parity_sampled": errs,
        "wall_s_timed_region": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        per_slice = attention_flops(1, 1, w.N, w.d, w.causal)
        n_sl = max(1, min(args.cpu_slices or int(CPU_FLOPS // per_slice), w.B * w.H))
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, n_sl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
