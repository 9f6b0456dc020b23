"""GPU parity: the HIP path against the CPU fp64 oracle, through the C ABI.

Bars (max-abs over every compared element, oracle run on the same rounded
inputs):
  O    fp32 <= 1e-4, fp16/bf16 <= 2e-2
  lse  fp32 <= 1e-4; fp16/bf16 <= u + N s/2 + (N/16 + 32) 2^-24 + 1e-5
The lse bound follows from the arithmetic: the kernels sum the probabilities
after rounding them to the P.V operand type, whose rounding error is at most
u|p| + s/2 (unit roundoff u = 2^-8 bf16, 2^-11 fp16; subnormal spacing
s = 2^-24 fp16, 2^-133 bf16). The largest probability of a row is >= 1, so
l >= 1 and ln(l) moves by at most u + N s/2; the fp32 row sum adds one
rounding per accumulator update, and 1e-5 covers the fp32 scores and the
hardware exp2's zero for every p below 2^-126 (no subnormal results: at most
N 2^-126 more).

Small shapes are checked element by element on every output; the full-size
workloads (in the launch configuration the bench times) on every row, or on
every row of eight whole slices for the three d = 128, N = 8192 workloads.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_15_amd.inputs import (WORKLOADS, make_dout, make_qkv, make_qkv_device,
                                           make_structured_qkv,
                                           workload_inputs)

pytestmark = pytest.mark.gpu

O_TOL = {torch.float32: 1e-4, torch.float16: 2e-2, torch.bfloat16: 2e-2}
_U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
_S = {torch.float16: 2.0 ** -24, torch.bfloat16: 2.0 ** -133}


def lse_tol(dtype, n):
    if dtype == torch.float32:
        return 1e-4
    return _U[dtype] + n * _S[dtype] / 2 + (n / 16 + 32) * 2.0 ** -24 + 1e-5


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.load_library()
    return ea


def _run_gpu(ea, q, k, v, causal, scale):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = ea.fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def _check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what, n):
    err_o = np.abs(o_gpu - o_ref)
    err_l = np.abs(lse_gpu - lse_ref)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), what
    mo, ml = float(err_o.max()), float(err_l.max())
    # noise-to-signal ratio ||O - O_ref|| / ||O_ref||
    nsr = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    print(f"{what}: O max-abs {mo:.3e} mean-abs {float(err_o.mean()):.3e} NSR {nsr:.2e}; "
          f"lse max-abs {ml:.3e}", flush=True)
    assert mo <= O_TOL[dtype], (what, mo)
    assert ml <= lse_tol(dtype, n), (what, ml)


SWEEP_N = [1, 2, 3, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 257]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_sweep_small(ea, oracle_lib, dtype, d, causal):
    """Every output element, N across tile edges and ragged tails."""
    for n in SWEEP_N:
        q, k, v = make_qkv(2, 2, n, d, dtype, seed=7000 + n + d)
        scale = ea.default_scale(d)
        o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, causal, scale)
        o, lse = _run_gpu(ea, q, k, v, causal, scale)
        _check(o, lse, o_ref, lse_ref, dtype, f"N={n} d={d} {dtype} causal={causal}", n)


GQA_HEADS = [(4, 1), (4, 2), (6, 3), (8, 2), (16, 4)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_gqa_small(ea, oracle_lib, dtype, d, causal):
    """Grouped-query and multi-query attention, every output element, with
    B = 2 so that both the head grouping and the batch offset of K/V matter;
    the GPU result with shared K/V heads is also bit-identical to the
    multi-head launch on K/V expanded to one head per query head."""
    for (H, H_kv), n in zip(GQA_HEADS, [1, 65, 130, 200, 257]):
        q, k, v = make_qkv(2, H, n, d, dtype, seed=8000 + 7 * H + H_kv + n, H_kv=H_kv)
        scale = ea.default_scale(d)
        o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, causal, scale)
        o, lse = _run_gpu(ea, q, k, v, causal, scale)
        _check(o, lse, o_ref, lse_ref, dtype,
               f"GQA H={H} H_kv={H_kv} N={n} d={d} {dtype} causal={causal}", n)
        G = H // H_kv
        ke = k.repeat_interleave(G, dim=1).contiguous()
        ve = v.repeat_interleave(G, dim=1).contiguous()
        o2, lse2 = _run_gpu(ea, q, ke, ve, causal, scale)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def _sample_rows(B, H, N, rng, n_random=192):
    BH = B * H
    rows = set()
    for i in list(range(min(N, 40))) + list(range(max(0, N - 40), N)):
        rows.add(i)                          # slice 0: head and tail
        rows.add((BH - 1) * N + i)           # last slice
    mid = BH // 2
    for t in (127, 128, 129, 255, 256, 1023, 1024, N // 2, N - 129, N - 128):
        if 0 <= t < N:
            rows.add(mid * N + t)
    rows.update(rng.integers(0, BH * N, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)


# Full-size workloads compared on every row, except the three d = 128,
# N = 8192 ones with 32 slices (the oracle needs ~1.5-3 s of 16 cores per
# slice there): these compare every row of 8 whole (b,h) slices, one on each
# of the 8 XCDs (slice s runs on XCD s mod 8), spread from the first slice
# to the last.
_SLICE_PICKS = {"c4_bf16_d128_causal": [0, 9, 18, 27, 4, 13, 22, 31],
                "c4_bf16_d128": [0, 9, 18, 27, 4, 13, 22, 31],
                "g2_bf16_d128_mqa": [0, 9, 18, 27, 4, 13, 22, 31]}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(ea, oracle_lib, name):
    """Full-size workloads in the launch configuration the bench times:
    every output row against the oracle, or every row of whole slices where
    the oracle's cost rules out the rest."""
    w = WORKLOADS[name]
    print(f"workload {name}: {w.describe()}", flush=True)
    q, k, v = workload_inputs(w)
    o, lse = _run_gpu(ea, q, k, v, w.causal, w.scale)
    picks = _SLICE_PICKS.get(name)
    if picks is None:
        o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, w.causal, w.scale)
        _check(o, lse, o_ref, lse_ref, w.dtype, f"{name} (every row)", w.N)
        return
    rows = np.concatenate([s * w.N + np.arange(w.N) for s in picks]).astype(np.int64)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, w.causal, w.scale, rows)
    _check(o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, w.dtype,
           f"{name} (every row of slices {picks})", w.N)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_attn_fwd_entry_point(ea, oracle_lib, dtype, d, causal):
    """attn_fwd itself, the multi-head entry point, called through the C ABI
    with raw device pointers and torch's current stream: every element
    against the oracle at a ragged N, and bit-identical to attn_fwd_gqa with
    H_kv = H (the path the Python wrapper takes)."""
    lib = ea.load_library()
    B, H, n = 2, 3, 333
    q, k, v = make_qkv(B, H, n, d, dtype, seed=7700 + d + int(causal))
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    scale = ea.default_scale(d)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, n, d, int(causal), scale, ea.dtype_code(dtype), stream)
    assert rc == 0, ea.strerror(rc)
    o2, lse2 = ea.fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, causal, scale)
    _check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, dtype,
           f"attn_fwd N={n} d={d} {dtype} causal={causal}", n)


def test_attn_fwd_entry_point_two_query_blocks(ea, oracle_lib):
    """attn_fwd on a non-causal d = 64 grid that takes the two-query-block
    kernel (2*64 slices x 2 tiles of 512 rows = 256 items), ragged N."""
    lib = ea.load_library()
    B, H, n, d = 2, 64, 1000, 64
    q, k, v = make_qkv(B, H, n, d, torch.bfloat16, seed=7750)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    scale = ea.default_scale(d)
    rc = lib.attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, n, d, 0, scale, ea.ATTN_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, ea.strerror(rc)
    o2, lse2 = ea.fwd(qd, kd, vd, causal=False, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    rows = _sample_rows(B, H, n, np.random.default_rng(7750), n_random=96)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, False, scale, rows)
    _check(o.cpu().double().numpy().reshape(-1, d)[rows], lse.cpu().double().numpy().reshape(-1)[rows],
           o_ref, lse_ref, torch.bfloat16, f"attn_fwd two query blocks ({len(rows)} sampled rows)", n)


def wrap_slices(n_slices, slice_elems, elem_bytes, group=1):
    """Query slices whose data (or whose K/V slice's data, with `group` query
    heads per K/V head) ends just before or starts at an offset where 32-bit
    arithmetic would wrap: 2^31 bytes, 2^32 bytes, 2^31 elements; and the
    first and last slice."""
    picks = {0, n_slices - 1}
    for lim in (2 ** 31 // elem_bytes, 2 ** 32 // elem_bytes, 2 ** 31):
        first = -(-lim // slice_elems)   # first slice starting at or past lim
        for t in (first - 1, first):
            for h in (t, t * group, t * group + group - 1):
                if 0 <= h < n_slices:
                    picks.add(h)
    return sorted(picks)


LARGE = [   # (dtype, d, causal, H, H_kv) at B = 1, N = 1024: Q holds more than 2^31 elements
    (torch.bfloat16, 64, True, 32800, 32800),    # one query block per wave
    (torch.bfloat16, 64, False, 32800, 32800),   # two query blocks per wave
    (torch.float16, 128, False, 16400, 8200),    # d = 128, two query heads per K/V head
    (torch.float32, 64, True, 32800, 32800),
]


@pytest.mark.parametrize("dtype,d,causal,H,H_kv", LARGE,
                         ids=["bf16-d64-causal", "bf16-d64", "f16-d128-gqa2", "f32-d64-causal"])
def test_offsets_past_2_31_elements(ea, oracle_lib, dtype, d, causal, H, H_kv):
    """Q, K, V, O of more than 2^31 elements (4.3-8.6 GB each): every slice
    is addressed with 64-bit offsets. Inputs are drawn on the device; the
    slices on both sides of every 32-bit wrap point (bytes and elements, of
    Q/O and of K/V) and the first and last are checked on every element
    against the oracle."""
    N = 1024
    assert H * N * d > 2 ** 31
    G = H // H_kv
    q, k, v = make_qkv_device(1, H, N, d, dtype, seed=31, H_kv=H_kv)
    scale = ea.default_scale(d)
    o, lse = ea.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    picks = sorted(set(wrap_slices(H, N * d, q.element_size())) |
                   set(wrap_slices(H, N * d, q.element_size(), G)))
    print(f"{dtype} d={d} causal={causal} H={H} H_kv={H_kv}: slices {picks}", flush=True)
    for h in picks:
        kh = h // G
        qs, ks, vs = (t[:, a:a + 1].cpu() for t, a in ((q, h), (k, kh), (v, kh)))
        o_ref, lse_ref = oracle_lib.attn_fwd_ref(qs, ks, vs, causal, scale)
        _check(o[:, h:h + 1].cpu().to(torch.float64).numpy(),
               lse[:, h:h + 1].cpu().to(torch.float64).numpy(), o_ref, lse_ref, dtype,
               f"slice {h} (Q offset {h * N * d} elements)", N)
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_two_query_block_kernel(ea, oracle_lib, dtype):
    """The non-causal d = 64 kernel with two 32-row query blocks per wave,
    which the launcher takes only when its 512-row items cover every compute
    unit (here 2*64 slices x 2 tiles = 256 items, N ragged past a tile):
    sampled rows against the oracle."""
    q, k, v = make_qkv(2, 64, 1000, 64, dtype, seed=5200)
    o, lse = _run_gpu(ea, q, k, v, False, ea.default_scale(64))
    rows = _sample_rows(2, 64, 1000, np.random.default_rng(5200), n_random=96)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, False, ea.default_scale(64), rows)
    _check(o.reshape(-1, 64)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype,
           f"two query blocks N=1000 {dtype} ({len(rows)} sampled rows)", 1000)


@pytest.mark.parametrize("dtype,d,n,causal", [
    (torch.bfloat16, 64, 131072, True),
    (torch.float16, 128, 65535, False),
    (torch.float16, 64, 40000, True),    # past the fp16 first pass's 32768 keys
    (torch.float16, 64, 32768, False),   # the fp16 first pass's longest rows
    (torch.float32, 64, 32768, True),
], ids=["bf16-d64-128k-causal", "f16-d128-64k-ragged", "f16-d64-40k-causal", "f16-d64-32k",
        "f32-d64-32k-causal"])
def test_long_sequence(ea, oracle_lib, dtype, d, n, causal):
    """Sequence lengths far past the workloads (one slice): positions and
    offsets stay exact; sampled rows across the whole range, the last rows
    (which see every key) included."""
    q, k, v = make_qkv(1, 1, n, d, dtype, seed=5100 + d)
    o, lse = _run_gpu(ea, q, k, v, causal, ea.default_scale(d))
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n),
                                     rng.integers(0, n, 48)])).astype(np.int64)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, causal, ea.default_scale(d), rows)
    _check(o.reshape(-1, d)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, dtype,
           f"N={n} d={d} {dtype} causal={causal} ({len(rows)} sampled rows)", n)


@pytest.mark.parametrize("kind", ["rising", "spikes"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_two_query_block_running_max(ea, oracle_lib, kind, dtype):
    """The two-query-block kernel (non-causal, d = 64, 512-row items on
    every compute unit: 128 slices x 2 tiles) on score rows whose maximum
    moves on every key tile (rising) or jumps past fp32's exp2 range inside
    one tile (spikes): sampled rows, the first and last included, against
    the oracle."""
    B, H, n, d = 1, 128, 1000, 64
    q, k, v = make_structured_qkv(kind, B, H, n, d, dtype, seed=5300)
    scale = ea.default_scale(d)
    o, lse = _run_gpu(ea, q, k, v, False, scale)
    rows = _sample_rows(B, H, n, np.random.default_rng(5300), n_random=96)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, False, scale, rows)
    err_o = float(np.abs(o.reshape(-1, d)[rows] - o_ref).max())
    err_l = float(np.abs(lse.reshape(-1)[rows] - lse_ref).max())
    tol_l = lse_tol(dtype, n) + _score_term(q, k, scale)
    print(f"two query blocks {kind} {dtype} ({len(rows)} sampled rows): O max-abs {err_o:.3e}, "
          f"lse max-abs {err_l:.3e} (bound {tol_l:.3e})", flush=True)
    assert np.all(np.isfinite(o)) and err_o <= O_TOL[dtype], err_o
    assert err_l <= tol_l, err_l


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_first_pass_modes_are_bit_identical(ea, dtype):
    """At d = 64 the automatic choice (first pass without the per-tile
    overflow test), the exact pass alone and the first pass at any length
    (attn_debug_set_fwd_first_pass 0, 1, 2) give the same bits: on each
    d = 64 kernel (one and two query blocks, causal and not, ragged N, a
    grouped-query shape), at an fp16 length past the automatic first pass's
    32768 keys, on flat fp16 rows of exactly 32768 keys (every P = 1, so
    l = 2^15 sits on the first pass's l <= 2^15 check; O must be the mean
    of V and lse ln N), and on the full-size headline workload."""
    cases = [(1, 8, 8, 1000, True), (1, 128, 128, 1000, False), (2, 4, 4, 777, False),
             (1, 32, 32, 8192, True), (2, 16, 4, 640, True), (1, 2, 2, 33000, False)]
    try:
        for B, H, H_kv, n, causal in cases:
            q, k, v = (t.cuda() for t in make_qkv(B, H, n, 64, dtype, seed=8900 + n, H_kv=H_kv))
            outs = []
            for mode in (0, 1, 2):
                ea.debug_set_fwd_first_pass(mode)
                outs.append(ea.fwd(q, k, v, causal=causal))
            torch.cuda.synchronize()
            same = all(torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1]) for o, l in outs[1:])
            print(f"{dtype} B{B} H{H}/{H_kv} N{n} causal={causal}: modes 0/1/2 identical={same}", flush=True)
            assert same, (B, H, H_kv, n, causal)
        if dtype == torch.float16:
            n = 32768
            q, k, v = (t.cuda() for t in make_qkv(1, 2, n, 64, dtype, seed=8950))
            q.zero_()
            outs = []
            for mode in (0, 1, 2):
                ea.debug_set_fwd_first_pass(mode)
                outs.append(ea.fwd(q, k, v))
            torch.cuda.synchronize()
            same = all(torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1]) for o, l in outs[1:])
            mean_v = v.double().mean(dim=2, keepdim=True).expand(-1, -1, n, -1)
            o_err = float((outs[0][0].double() - mean_v).abs().max())
            lse_err = float((outs[0][1].double() - math.log(n)).abs().max())
            print(f"flat f16 N{n}: modes identical={same}, O vs mean of V {o_err:.2e}, "
                  f"lse vs ln N {lse_err:.2e}", flush=True)
            assert same and o_err <= O_TOL[dtype] and lse_err <= 1e-5
        if dtype == torch.bfloat16:
            w = WORKLOADS["c3_bf16_causal"]
            q, k, v = (t.cuda() for t in workload_inputs(w))
            outs = []
            for mode in (0, 1):
                ea.debug_set_fwd_first_pass(mode)
                outs.append(ea.fwd(q, k, v, causal=w.causal, scale=w.scale))
            torch.cuda.synchronize()
            same = torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
            print(f"c3_bf16_causal: first pass and exact pass identical={same}", flush=True)
            assert same
    finally:
        ea.debug_set_fwd_first_pass()


@pytest.mark.parametrize("kind", ["random", "spikes"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_causal_two_query_block_kernel(ea, oracle_lib, kind, dtype):
    """Under a causal mask the launcher takes two query blocks per wave from
    8192 keys on (B1 H32 N8192: 512 items of 512 rows): i.i.d. inputs, and
    spike rows whose maximum jumps past fp32's exp2 range inside one tile
    (their items take the exact pass); sampled rows of the first, middle
    and last slice (item and diagonal boundaries included) and random ones
    against the oracle."""
    B, H, n, d = 1, 32, 8192, 64
    if kind == "random":
        q, k, v = make_qkv(B, H, n, d, dtype, seed=5400)
    else:
        q, k, v = make_structured_qkv("spikes", B, H, n, d, dtype, seed=5400)
    scale = ea.default_scale(d)
    o, lse = _run_gpu(ea, q, k, v, True, scale)
    rows = _sample_rows(B, H, n, np.random.default_rng(5400), n_random=64)
    rows = np.unique(np.concatenate([rows, (H // 2) * n + np.array([511, 512, 4095, 4096, 8190])]))
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, True, scale, rows)
    err_o = float(np.abs(o.reshape(-1, d)[rows] - o_ref).max())
    err_l = float(np.abs(lse.reshape(-1)[rows] - lse_ref).max())
    tol_l = lse_tol(dtype, n) + _score_term(q, k, scale)
    print(f"causal two query blocks {kind} {dtype} ({len(rows)} sampled rows): O max-abs {err_o:.3e}, "
          f"lse max-abs {err_l:.3e} (bound {tol_l:.3e})", flush=True)
    assert np.all(np.isfinite(o)) and err_o <= O_TOL[dtype], err_o
    assert err_l <= tol_l, err_l


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_forced_variants_are_bit_identical(ea, dtype):
    """Every forward variant computes each row with the same arithmetic in
    the same order: forcing one or two query blocks per wave, or the
    tile-major or XCD-major work order (attn_debug_set_fwd_variant), gives
    the automatic choice's output bit for bit, on shapes where the
    automatic choice is the other variant: d = 64 non-causal with 256
    512-row items (automatic: two blocks, XCD-major), a small non-causal
    shape (one block), and causal shapes with 8 K/V slices (tile-major),
    multi-head and grouped-query."""
    cases = [(2, 64, 64, 1000, 64, False, [(1, 0), (0, 1), (1, 1)]),
             (1, 2, 2, 300, 64, False, [(2, 0)]),
             (1, 8, 8, 700, 64, True, [(0, 2), (2, 2)]),
             (2, 16, 4, 640, 64, True, [(0, 2)]),
             (1, 8, 8, 520, 128, False, [(0, 1), (2, 1)]),
             (1, 8, 8, 520, 128, True, [(0, 2)])]
    try:
        for B, H, H_kv, n, d, causal, forced in cases:
            q, k, v = (t.cuda() for t in make_qkv(B, H, n, d, dtype, seed=8800 + n, H_kv=H_kv))
            ea.debug_set_fwd_variant()
            o_auto, lse_auto = ea.fwd(q, k, v, causal=causal)
            for qb, order in forced:
                ea.debug_set_fwd_variant(qb, order)
                o, lse = ea.fwd(q, k, v, causal=causal)
                torch.cuda.synchronize()
                print(f"B{B} H{H}/{H_kv} N{n} d{d} causal={causal} forced (qb={qb}, order={order}): "
                      f"identical={torch.equal(o, o_auto) and torch.equal(lse, lse_auto)}", flush=True)
                assert torch.equal(o, o_auto) and torch.equal(lse, lse_auto), (B, H, n, d, causal, qb, order)
    finally:
        ea.debug_set_fwd_variant()


@pytest.mark.parametrize("dtype,spike", [(torch.bfloat16, 4.0), (torch.float16, 1.0)],
                         ids=["bf16", "f16"])
def test_exact_pass_keeps_bits_across_variants(ea, oracle_lib, dtype, spike):
    """At d = 64 a first pass runs without the per-tile overflow test and
    hands a work item to the exact pass when some row's l exceeds the
    threshold T (2^64 bf16, 2^15 fp16). Here one key (index 700) has a
    score of 192 spike / 8 nats (~96 bf16, ~24 fp16) for the query rows
    300-310 only, far past T against their base, so their items take the
    exact pass, and of spike / 8 (u . q) for the others (u . q ~ N(0, 64):
    P up to ~2^22 against their base for bf16, ~2^6 for fp16, within T).
    With one query block per wave (256-row items) rows 0-255 stay in the
    first pass; with two (512-row items) they share an item with the
    spiking rows and are computed by the exact pass: both must give the
    same bits, and every row must match the oracle."""
    B, H, n, d = 1, 2, 1024, 64
    g = torch.Generator(device="cpu")
    g.manual_seed(9100)
    q = torch.randn((B, H, n, d), generator=g)
    k = torch.randn((B, H, n, d), generator=g)
    v = torch.randn((B, H, n, d), generator=g)
    u = torch.randint(0, 2, (d,), generator=g).to(torch.float32) * 2.0 - 1.0
    q[:, :, 300:311] = 3.0 * u + 0.25 * torch.randn((B, H, 11, d), generator=g)
    k[:, :, 700] = spike * u
    q, k, v = (t.to(dtype) for t in (q, k, v))
    scale = ea.default_scale(d)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    try:
        outs = []
        for qb in (1, 2):
            ea.debug_set_fwd_variant(qb, 0)
            outs.append(ea.fwd(qd, kd, vd, causal=False, scale=scale))
        torch.cuda.synchronize()
    finally:
        ea.debug_set_fwd_variant()
    (o1, l1), (o2, l2) = outs
    same = torch.equal(o1, o2) and torch.equal(l1, l2)
    print(f"{dtype}: one vs two query blocks around the exact pass: identical={same}", flush=True)
    assert same
    o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, False, scale)
    _check(o1.cpu().to(torch.float64).numpy(), l1.cpu().to(torch.float64).numpy(), o_ref, lse_ref,
           dtype, f"{dtype} d=64 spiking rows 300-310", n)
    assert float(lse_ref[0, :, 300:311].min()) > 20.0 * spike   # the spiking rows


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16],
                         ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_invariants_on_gpu(ea, dtype, causal):
    """Constant V gives that constant; Q = 0 gives the (prefix) mean of V
    with lse = ln|J_i|; the unit-basis probe V[k][0] = 1 reads column k of
    P, whose rows then sum to 1."""
    B, H, N, d = 1, 2, 200, 64
    q, k, v = make_qkv(B, H, N, d, dtype, seed=31)
    tol = O_TOL[dtype]
    c = 0.375
    o, _ = _run_gpu(ea, q, k, torch.full_like(v, c), causal, 0.125)
    assert np.abs(o - c).max() <= tol

    o, lse = _run_gpu(ea, torch.zeros_like(q), k, v, causal, 0.125)
    vv = v.to(torch.float64).numpy()
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = (np.cumsum(vv, axis=2) / np.arange(1, N + 1)[:, None]) if causal else \
        np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    assert np.abs(o - mean).max() <= tol
    assert np.abs(lse - np.log(cnt)).max() <= lse_tol(dtype, N)

    n = 70
    q2, k2, _ = make_qkv(1, 1, n, d, dtype, seed=32)
    cols = []
    for kk in range(n):
        vb = torch.zeros(1, 1, n, d, dtype=dtype)
        vb[0, 0, kk, 0] = 1.0
        o, _ = _run_gpu(ea, q2, k2, vb, causal, 0.125)
        assert np.abs(o[..., 1:]).max() == 0.0
        cols.append(o[0, 0, :, 0])
    p = np.stack(cols, axis=1)
    assert np.abs(p.sum(1) - 1).max() <= 2 * tol
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0.0)


def _score_term(q, k, scale):
    """lse error allowance for the fp32 scores, in nats: the kernel's score
    is an fp32 sum of d products, then one fma with the fp32 constant
    scale*log2(e) and one exp2, so its error is at most about
    scale (d + 2) 2^-24 max_ij sum_c |q_ic k_jc| (plus 2^-20 for the exp2
    argument's own rounding); the lse moves by at most that much."""
    qa = q.to(torch.float64).abs()
    ka = k.to(torch.float64).abs()
    m = float(torch.matmul(qa, ka.transpose(-1, -2)).max())
    d = q.shape[-1]
    return scale * (d + 2) * 2.0 ** -24 * m + 2.0 ** -20


@pytest.mark.parametrize("kind", ["rising", "falling", "wide", "spikes"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_running_max_paths(ea, oracle_lib, kind, dtype, d, causal):
    """Score rows shaped to drive the online softmax's running maximum:
    rising rows move it by ~8 nats on every full 64-key tile (the accumulator
    is rescaled on every tile), falling rows fix it in the first tile, wide
    rows (score std ~4) make it jump irregularly, and spike rows make it
    jump by ~100 nats inside one tile, so that the probabilities against the
    old maximum overflow fp32 and the kernel must notice and redo the tile.
    N = 300 spans five key tiles with a ragged tail."""
    n = 300
    q, k, v = make_structured_qkv(kind, 1, 2, n, d, dtype, seed=4100 + d)
    scale = ea.default_scale(d)
    o, lse = _run_gpu(ea, q, k, v, causal, scale)
    o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, causal, scale)
    err_o = float(np.abs(o - o_ref).max())
    err_l = float(np.abs(lse - lse_ref).max())
    tol_l = lse_tol(dtype, n) + _score_term(q, k, scale)
    print(f"{kind} d={d} {dtype} causal={causal}: O max-abs {err_o:.3e}, lse max-abs "
          f"{err_l:.3e} (bound {tol_l:.3e})", flush=True)
    assert np.all(np.isfinite(o)) and err_o <= O_TOL[dtype], err_o
    assert err_l <= tol_l, err_l


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_nonfinite_inputs_return_normally(ea, dtype):
    """NaN and infinite inputs are outside the contract (the results are not
    specified), but the calls return ATTN_OK and the stream stays usable:
    no address in any kernel depends on the data. Rows of a slice whose
    inputs are all finite still match the clean run."""
    q, k, v = (t.cuda() for t in make_qkv(2, 2, 300, 64, dtype, seed=77))
    dout = make_dout(2, 2, 300, 64, dtype, seed=77).cuda()
    o_clean, lse_clean = ea.fwd(q, k, v, causal=True)
    qb, kb, vb = q.clone(), k.clone(), v.clone()
    qb[0, 0, 5, 3] = float("nan")
    kb[0, 1, 7, 0] = float("inf")
    vb[0, 0, 11, 2] = float("-inf")
    o, lse = ea.fwd(qb, kb, vb, causal=True)
    dq, dk, dv = ea.bwd(qb, kb, vb, o, lse, dout, causal=True)
    o_u, _ = ea.fwd_unfused(qb, kb, vb, causal=True)
    torch.cuda.synchronize()
    # batch 1 holds no non-finite input: its slices are unaffected
    assert torch.equal(o[1], o_clean[1]) and torch.equal(lse[1], lse_clean[1])
    assert torch.isfinite(dq[1].float()).all() and torch.isfinite(dk[1].float()).all()
    o2, _ = ea.fwd(q, k, v, causal=True)   # the stream still works
    torch.cuda.synchronize()
    assert torch.equal(o2, o_clean)
    del o_u, dv


def test_deterministic(ea):
    """No atomics on the path: repeated runs are bitwise identical."""
    w = WORKLOADS["c3_bf16_causal"]
    q, k, v = (t.cuda() for t in make_qkv(1, 4, 1000, 64, torch.bfloat16, seed=5))
    o1, l1 = ea.fwd(q, k, v, causal=True)
    o2, l2 = ea.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    del w


def test_stream_and_out_buffers(ea):
    """Launch on a non-default stream into preallocated outputs."""
    q, k, v = (t.cuda() for t in make_qkv(1, 2, 300, 128, torch.bfloat16, seed=6))
    ref_o, ref_l = ea.fwd(q, k, v, causal=False)
    s = torch.cuda.Stream()
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 300, device="cuda", dtype=torch.float32)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ea.fwd(q, k, v, causal=False, out=(o, lse))
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
