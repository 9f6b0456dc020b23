"""GPU parity of the unfused three-kernel forward (the comparison path)
against the CPU fp64 oracle, through the C ABI.

Bars as for the fused forward: O max-abs <= 2e-2 (fp16/bf16), 1e-4 (fp32);
lse max-abs <= 1e-4 + (N/64) 2^-24 (the unfused softmax sums unrounded fp32
probabilities: no rounding of P enters lse).
"""
import numpy as np
import pytest
import torch

from exact_attention_15_amd.inputs import WORKLOADS, make_qkv, workload_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.load_library()
    return ea


def _check(o, lse, o_ref, lse_ref, n, what, o_tol):
    eo = float(np.abs(o - o_ref).max())
    el = float(np.abs(lse - lse_ref).max())
    print(f"{what}: O max-abs {eo:.3e}, lse max-abs {el:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= o_tol, (what, eo)
    assert el <= 1e-4 + (n / 64) * 2.0 ** -24, (what, el)


def _o_tol(dtype):
    return 1e-4 if dtype == torch.float32 else 2e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_unfused_small(ea, oracle_lib, dtype, d, causal):
    for n in [1, 2, 63, 64, 65, 127, 130, 257]:
        q, k, v = make_qkv(2, 2, n, d, dtype, seed=9700 + n + d)
        scale = ea.default_scale(d)
        o, lse = ea.fwd_unfused(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle_lib.attn_fwd_ref(q, k, v, causal, scale)
        _check(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, n,
               f"unfused N={n} d={d} {dtype} causal={causal}", _o_tol(dtype))


@pytest.mark.parametrize("name", ["c3_bf16_causal", "c5_f16_ragged", "c2_f32_causal"])
def test_unfused_full_size(ea, oracle_lib, name):
    """The bench's comparison workloads, sampled rows."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    o, lse = ea.fwd_unfused(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([np.arange(40), np.arange(w.N - 40, w.N),
                                     rng.integers(0, w.B * w.H * w.N, 200)]))
    o_ref, lse_ref = oracle_lib.attn_fwd_ref_rows(q, k, v, w.causal, w.scale, rows)
    _check(o.cpu().double().numpy().reshape(-1, w.d)[rows], lse.cpu().double().numpy().reshape(-1)[rows],
           o_ref, lse_ref, w.N, f"unfused {name} ({len(rows)} rows)", _o_tol(w.dtype))
