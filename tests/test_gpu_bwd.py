"""GPU parity of the backward pass (dQ, dK, dV) against the CPU fp64 oracle,
through the C ABI.

Inputs o and lse are the oracle's exact forward values rounded to their
storage types (o to the input dtype, lse to fp32), so the comparison
isolates the backward kernels' arithmetic. The bound per gradient element,
from the error analysis of that arithmetic (first order):
    |g - g_ref| <= 2 [(u + n_acc 2^-24) (e + |g_ref|) + (s/2) (z + 1)]
Rounding x to the 16-bit type errs by at most u|x| + s/2: u its unit
roundoff (2^-8 bf16, 2^-11 fp16), s its subnormal spacing (2^-24 fp16,
2^-133 bf16); fp32 rounds nothing below fp32 (u = 0). To u is added the
relative error of p from the fp32 scores, |ds| <= d 2^-24 scale
max_ij sum_c |q_ic k_jc| (computed from the inputs), and 2^-22 for exp2. p and ds are rounded to it as matrix-core operands, o was
rounded to it, and the output is rounded to it; e and z are the oracle's
error scales of the element (the sums of the magnitudes those roundings
perturb, relatively and absolutely); n_acc = G N / 16 + 32 bounds the fp32
accumulator updates behind one element; the factor 2 covers second-order
terms. Small shapes compare every element; full-size workloads
compare every element of sampled K/V slices (the oracle recomputes those
slices alone: slices are independent) and check identities on all others.
"""
import numpy as np
import pytest
import torch

from exact_attention_15_amd.inputs import WORKLOADS, make_dout, make_dout_device, make_qkv, \
    make_qkv_device, make_structured_qkv, workload_dout, workload_inputs

pytestmark = pytest.mark.gpu

U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8, torch.float32: 0.0}
SUB = {torch.float16: 2.0 ** -24, torch.bfloat16: 2.0 ** -133, torch.float32: 2.0 ** -149}


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.load_library()
    return ea


def _fwd_stats(oracle_lib, q, k, v, causal, scale):
    o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, causal, scale)
    return torch.from_numpy(o_ref).to(q.dtype), torch.from_numpy(lse_ref).to(torch.float32)


def _score_term(q, k, scale):
    """d 2^-24 scale max_ij sum_c |q_ic k_jc| + 2^-22: the relative error of p
    that the fp32 scores and exp2 can cause."""
    G = q.shape[1] // k.shape[1]
    qa = q.to(torch.float64).abs()
    ka = k.to(torch.float64).abs().repeat_interleave(G, dim=1)
    m = float(torch.matmul(qa, ka.transpose(-1, -2)).max())
    return q.shape[-1] * 2.0 ** -24 * float(scale) * m + 2.0 ** -22


def _flush_terms(q, k, v, dout, scale):
    """Absolute error that the kernels' exp2 adds by returning 0 for every p
    below 2^-126 (the hardware instruction has no subnormal results): a lost
    p_ij moves ds_ij = p_ij (dp_ij - D_i) by at most 2^-126 |dO_i|_1 2 max|v|
    (|dp_ij| and |D_i| are each at most |dO_i|_1 max|v|, o_i being a convex
    combination of the rows of v) and dv_j by 2^-126 |dO_ic|. Summed over
    every row and key, masked or not, so an upper bound under a causal mask
    too. Returns (fq, fk, fv) shaped like dq, dk, dv."""
    G = q.shape[1] // k.shape[1]
    qa, ka, da = (t.to(torch.float64).abs() for t in (q, k, dout))
    g = da.sum(-1, keepdim=True)                                   # [B,H,N,1]
    c = 2.0 ** -126 * 2.0 * float(v.to(torch.float64).abs().max()) * float(scale)
    ksum = ka.sum(2, keepdim=True).repeat_interleave(G, dim=1)     # [B,H,1,d]
    fq = c * g * ksum
    B, H, N, d = q.shape
    fk = c * (g * qa).sum(2, keepdim=True).reshape(B, H // G, G, 1, d).sum(2)
    fv = 2.0 ** -126 * da.sum(2, keepdim=True).reshape(B, H // G, G, 1, d).sum(2)
    return tuple(np.broadcast_to(t.numpy(), s) for t, s in
                 ((fq, q.shape), (fk, k.shape), (fv, v.shape)))


def _check(got, ref, err, zerr, dtype, n_acc, what, u_s, flush=0.0):
    got = got.to(torch.float64).cpu().numpy() if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(got)), what
    bound = 2 * ((U[dtype] + u_s + n_acc * 2.0 ** -24) * (err + np.abs(ref)) +
                 SUB[dtype] / 2 * (zerr + 1) + flush)
    diff = np.abs(got - ref)
    ratio = float((diff / np.maximum(bound, 1e-300)).max())
    print(f"{what}: max-abs {float(diff.max()):.3e}, max err/bound {ratio:.3f}", flush=True)
    assert np.all(diff <= bound), (what, ratio)


def _bwd_and_check(ea, oracle_lib, q, k, v, dout, causal, scale, what):
    o, lse = _fwd_stats(oracle_lib, q, k, v, causal, scale)
    dq, dk, dv = ea.bwd(*(t.cuda() for t in (q, k, v, o, lse, dout)), causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv, eq, ek, ev, zq, zk, zv = oracle_lib.attn_bwd_ref(q, k, v, dout, causal, scale,
                                                                 error_scales=True)
    n_acc = (q.shape[1] // k.shape[1]) * q.shape[2] / 16 + 32
    u_s = _score_term(q, k, scale)
    fq, fk, fv = _flush_terms(q, k, v, dout, scale)
    _check(dq, rq, eq, zq, q.dtype, n_acc, what + " dq", u_s, fq)
    _check(dk, rk, ek, zk, q.dtype, n_acc, what + " dk", u_s, fk)
    _check(dv, rv, ev, zv, q.dtype, n_acc, what + " dv", u_s, fv)


SWEEP = [(1, 2, 2), (2, 4, 1), (17, 2, 2), (64, 4, 2), (65, 2, 2), (127, 6, 3), (128, 2, 2),
         (129, 4, 4), (200, 4, 1), (257, 2, 2),
         # 2, 8 or 16 query heads per K/V head: the dK/dV work of a key tile
         # is cut into chunks whose partial sums are reduced afterwards (also
         # a one-row and a 33-row key tile; at G = 2 only the two longest
         # causal key tiles are cut)
         (65, 16, 1), (130, 8, 1), (257, 16, 2), (1, 8, 1), (33, 16, 2), (1024, 4, 2)]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32],
                         ids=["f16", "bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_sweep_small(ea, oracle_lib, dtype, d, causal):
    """Every gradient element; N across tile edges and ragged tails, with
    multi-head, grouped-query and multi-query head counts."""
    for n, H, H_kv in SWEEP:
        seed = 9000 + 3 * n + H + H_kv + d
        q, k, v = make_qkv(2, H, n, d, dtype, seed=seed, H_kv=H_kv)
        dout = make_dout(2, H, n, d, dtype, seed=seed)
        _bwd_and_check(ea, oracle_lib, q, k, v, dout, causal, ea.default_scale(d),
                       f"N={n} H={H} H_kv={H_kv} d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("kind", ["rising", "wide", "spikes"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32],
                         ids=["f16", "bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_structured_scores(ea, oracle_lib, kind, dtype, causal):
    """The backward on the forward's running-maximum inputs: rows whose
    scores climb across key tiles, rows nearly one-hot (score std ~4), and
    rows with keys ~100, 200 and 300 nats above the rest (p exactly 0 or 1
    for most entries, lse dominated by one key). Every element against the
    oracle, N = 300 (five key tiles, ragged)."""
    q, k, v = make_structured_qkv(kind, 1, 2, 300, 64, dtype, seed=9900)
    dout = make_dout(1, 2, 300, 64, dtype, seed=9900)
    _bwd_and_check(ea, oracle_lib, q, k, v, dout, causal, ea.default_scale(64),
                   f"{kind} N=300 d=64 {dtype} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_mqa_midsize(ea, oracle_lib, d):
    """Multi-query attention (16 query heads, one K/V head) at N = 2048,
    causal: the split dK/dV path with four query-head groups, every element."""
    q, k, v = make_qkv(1, 16, 2048, d, torch.bfloat16, seed=9800 + d, H_kv=1)
    dout = make_dout(1, 16, 2048, d, torch.bfloat16, seed=9800 + d)
    _bwd_and_check(ea, oracle_lib, q, k, v, dout, True, ea.default_scale(d),
                   f"MQA H=16 N=2048 d={d}")


def test_bwd_scale_and_values(ea, oracle_lib):
    """A non-default scale and larger scores (sharper softmax)."""
    q, k, v = make_qkv(1, 2, 150, 64, torch.bfloat16, seed=9501, value_scale=2.0)
    dout = make_dout(1, 2, 150, 64, torch.bfloat16, seed=9501)
    _bwd_and_check(ea, oracle_lib, q, k, v, dout, True, 0.3, "scale 0.3, values x2")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_bwd_one_group_noncausal_mha(ea, oracle_lib, dtype):
    """Non-causal multi-head d = 64 with 640 dK/dV items (B1 H64 N1280):
    enough to fill rounds of the one-group dK/dV kernel, which the launcher
    therefore picks over the three-group one (the choice is pinned on the
    host in tests/test_bwd_plan.py); every element."""
    q, k, v = make_qkv(1, 64, 1280, 64, dtype, seed=9700)
    dout = make_dout(1, 64, 1280, 64, dtype, seed=9700)
    _bwd_and_check(ea, oracle_lib, q, k, v, dout, False, ea.default_scale(64),
                   f"one-group dK/dV B1 H64 N1280 {dtype}")


FULL = ["c3_bf16_causal", "g1_bf16_causal_gqa4", "c4_bf16_d128_causal", "c2_f32_causal"]


@pytest.mark.parametrize("name", FULL)
def test_bwd_workload_full_size(ea, oracle_lib, name):
    """Full-size workloads in the bench's launch configuration: every element
    of the first and last K/V slices (the last only at d = 128; their query
    heads' o and lse replaced by the oracle's), identities on every slice."""
    w = WORKLOADS[name]
    print(f"workload {name}: {w.describe()}", flush=True)
    q, k, v = workload_inputs(w)
    dout = workload_dout(w)
    H_kv = w.kv_heads
    G = w.H // H_kv
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    o, lse = ea.fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    # The oracle needs ~15 s for one d = 128, N = 8192 slice: one slice there.
    picks = [(w.B - 1, H_kv - 1)] if w.d == 128 else [(0, 0), (w.B - 1, H_kv - 1)]
    subs = {}
    for b, hk in picks:
        hs = slice(hk * G, (hk + 1) * G)
        sub = (q[b:b + 1, hs], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1],
               dout[b:b + 1, hs])
        sub = tuple(t.contiguous() for t in sub)
        o_s, lse_s = _fwd_stats(oracle_lib, sub[0], sub[1], sub[2], w.causal, w.scale)
        o[b, hs] = o_s[0].cuda()
        lse[b, hs] = lse_s[0].cuda()
        subs[(b, hk)] = sub
    dq, dk, dv = ea.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    n_acc = G * w.N / 16 + 32
    for (b, hk), sub in subs.items():
        rq, rk, rv, eq, ek, ev, zq, zk, zv = oracle_lib.attn_bwd_ref(*sub, w.causal, w.scale,
                                                                     error_scales=True)
        hs = slice(hk * G, (hk + 1) * G)
        tag = f"{name} slice b={b} h_kv={hk}"
        u_s = _score_term(sub[0], sub[1], w.scale)
        fq, fk, fv = _flush_terms(*sub, w.scale)
        _check(dq[b:b + 1, hs], rq, eq, zq, w.dtype, n_acc, tag + " dq", u_s, fq)
        _check(dk[b:b + 1, hk:hk + 1], rk, ek, zk, w.dtype, n_acc, tag + " dk", u_s, fk)
        _check(dv[b:b + 1, hk:hk + 1], rv, ev, zv, w.dtype, n_acc, tag + " dv", u_s, fv)
    # Identities on every slice: the keys' gradients sum to zero over keys;
    # the values' gradients sum to the group's summed dout.
    dk64 = dk.to(torch.float64)
    dv64 = dv.to(torch.float64)
    dsum = dod.to(torch.float64).reshape(w.B, H_kv, G, w.N, w.d).sum(dim=(2, 3))
    tol_v = 4 * U[w.dtype] * dout.to(torch.float64).abs().reshape(
        w.B, H_kv, G, w.N, w.d).sum(dim=(2, 3)).cuda() + 1e-3
    assert torch.all((dv64.sum(dim=2) - dsum).abs() <= tol_v)
    tol_k = 4 * U[w.dtype] * dk64.abs().sum(dim=2) + 1e-3
    assert torch.all(dk64.sum(dim=2).abs() <= tol_k)


@pytest.mark.parametrize("dtype,n,H,H_kv", [
    (torch.bfloat16, 32768, 2, 1),
    (torch.float32, 16384, 1, 1),
], ids=["bf16-32k-gqa2", "f32-16k"])
def test_bwd_long_sequence(ea, dtype, n, H, H_kv):
    """Sequence lengths far past the workloads, causal, d = 64: the oracle's
    backward is too slow there, so the identities that hold at any size are
    checked on every element sum: dK sums to zero over keys, dV sums to the
    group's summed dO; and the gradients are finite."""
    G = H // H_kv
    q, k, v = (t.cuda() for t in make_qkv(1, H, n, 64, dtype, seed=9900 + n, H_kv=H_kv))
    dout = make_dout(1, H, n, 64, dtype, seed=9900 + n).cuda()
    o, lse = ea.fwd(q, k, v, causal=True)
    dq, dk, dv = ea.bwd(q, k, v, o, lse, dout, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.all(torch.isfinite(t.float()))
    dk64, dv64, do64 = (t.to(torch.float64) for t in (dk, dv, dout))
    dsum = do64.reshape(1, H_kv, G, n, 64).sum(dim=(2, 3))
    tol_v = 4 * U[dtype] * do64.abs().reshape(1, H_kv, G, n, 64).sum(dim=(2, 3)) + 1e-3
    err_v = float(((dv64.sum(dim=2) - dsum).abs() / tol_v).max())
    tol_k = 4 * U[dtype] * dk64.abs().sum(dim=2) + 1e-3
    err_k = float((dk64.sum(dim=2).abs() / tol_k).max())
    print(f"N={n} {dtype}: identity errors / bounds: dv {err_v:.3f}, dk {err_k:.3f}", flush=True)
    assert err_v <= 1 and err_k <= 1


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_bwd_offsets_past_2_31_elements(ea, oracle_lib, dtype):
    """Q, K, V, O, dO and the gradients at more than 2^31 elements each
    (B = 1, H = 32800, N = 1024, d = 64, causal): the gradient kernels
    address every slice with 64-bit offsets. Inputs are drawn on the device;
    the slices on both sides of the 32-bit wrap points (2^31 and 2^32 bytes,
    2^31 elements) and the first and last get the oracle's o and lse and are
    checked on every element against the oracle's gradients."""
    N, d, H = 1024, 64, 32800
    q, k, v = make_qkv_device(1, H, N, d, dtype, seed=32)
    dout = make_dout_device(1, H, N, d, dtype, seed=32)
    scale = ea.default_scale(d)
    o, lse = ea.fwd(q, k, v, causal=True, scale=scale)
    picks = set()
    for lim in (2 ** 31 // q.element_size(), 2 ** 32 // q.element_size(), 2 ** 31):
        first = -(-lim // (N * d))
        picks |= {t for t in (first - 1, first) if 0 <= t < H}
    picks = sorted(picks | {0, H - 1})
    print(f"{dtype}: slices {picks}", flush=True)
    subs = {}
    for h in picks:
        sub = tuple(t[:, h:h + 1].cpu() for t in (q, k, v, dout))
        o_s, lse_s = _fwd_stats(oracle_lib, sub[0], sub[1], sub[2], True, scale)
        o[:, h:h + 1] = o_s.cuda()
        lse[:, h:h + 1] = lse_s.cuda()
        subs[h] = sub
    dq, dk, dv = ea.bwd(q, k, v, o, lse, dout, causal=True, scale=scale)
    torch.cuda.synchronize()
    n_acc = N / 16 + 32
    for h, sub in subs.items():
        rq, rk, rv, eq, ek, ev, zq, zk, zv = oracle_lib.attn_bwd_ref(*sub, True, scale,
                                                                     error_scales=True)
        u_s = _score_term(sub[0], sub[1], scale)
        fq, fk, fv = _flush_terms(*sub, scale)
        tag = f"slice {h} (offset {h * N * d} elements)"
        _check(dq[:, h:h + 1], rq, eq, zq, dtype, n_acc, tag + " dq", u_s, fq)
        _check(dk[:, h:h + 1], rk, ek, zk, dtype, n_acc, tag + " dk", u_s, fk)
        _check(dv[:, h:h + 1], rv, ev, zv, dtype, n_acc, tag + " dv", u_s, fv)
    del q, k, v, dout, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_bwd_deterministic(ea, dtype):
    """No atomics, partial sums added in a fixed order: repeated runs are
    bitwise identical."""
    q, k, v = (t.cuda() for t in make_qkv(1, 4, 700, 64, dtype, seed=5, H_kv=2))
    dout = make_dout(1, 4, 700, 64, dtype, seed=5).cuda()
    o, lse = ea.fwd(q, k, v, causal=True)
    a = ea.bwd(q, k, v, o, lse, dout, causal=True)
    b = ea.bwd(q, k, v, o, lse, dout, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_composes_with_forward(ea, oracle_lib):
    """The GPU forward's own o and lse as inputs: the gradients stay within
    the bound widened by the forward's o error (up to the forward tolerance
    2e-2 per element, which enters through D_i = dout_i . o_i)."""
    dtype = torch.bfloat16
    q, k, v = make_qkv(2, 4, 300, 64, dtype, seed=9601, H_kv=2)
    dout = make_dout(2, 4, 300, 64, dtype, seed=9601)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    o, lse = ea.fwd(qd, kd, vd, causal=True)
    dq, dk, dv = ea.bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_lib.attn_bwd_ref(q, k, v, dout, True, ea.default_scale(64))
    o_ref, _ = oracle_lib.attn_fwd_ref(q, k, v, True, ea.default_scale(64))
    o_err = np.abs(o.cpu().double().numpy() - o_ref).max()
    assert o_err <= 2e-2
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        rel = np.abs(got.cpu().double().numpy() - ref).max() / np.abs(ref).max()
        print(f"composed: rel max-abs {rel:.3e} (o err {o_err:.2e})", flush=True)
        assert rel <= 4e-2
