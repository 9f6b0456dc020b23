"""Pins for the CPU fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: the pages' printed
worked values (tests/golden/worked_values.json), closed forms, invariants the
pages state, exhaustive checks of the input decoders against the formats'
library conversion, and brute force on tiny inputs against a library softmax.
They are chosen so that a plausible slip in the oracle (a dropped max
subtraction, a wrong causal bound, a transposed operand, a missing or doubled
scale, a wrong decoder bit) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from exact_attention_15_amd.inputs import make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_values.json")

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


def _f64(t):
    return t.to(torch.float64).numpy()


def _library_attention(q, k, v, causal, scale):
    """torch CPU fp64: softmax(scale * Q K^T [+ causal -inf]) V, plus logsumexp."""
    q64, k64, v64 = (t.to(torch.float64) for t in (q, k, v))
    s = float(scale) * torch.matmul(q64, k64.transpose(-1, -2).contiguous())
    if causal:
        n = s.shape[-1]
        mask = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        s = s.masked_fill(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v64).numpy(), torch.logsumexp(s, dim=-1).numpy(), p.numpy()


# ---------------------------------------------------------------- decoding

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_decode_exhaustive_16bit(orc, dtype):
    """Every 16-bit pattern decodes to the value the format defines."""
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16)
    x = bits.view(dtype)
    got = orc.decode(x)
    want = x.to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_f32_roundtrip(orc):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(10000, generator=g) * 1e3
    x[:4] = torch.tensor([0.0, -0.0, 1e-40, -3.5e38])
    assert np.array_equal(orc.decode(x), x.to(torch.float64).numpy())


# ---------------------------------------------------------- page values

def test_golden_dot_product(orc):
    """N = 1: lse = scale * q.k; with the page's vectors q.k = 6.25."""
    g = json.load(open(GOLDEN))["dot_product"]
    q = torch.tensor(g["q"], dtype=torch.float32).view(1, 1, 1, 2)
    k = torch.tensor(g["k"], dtype=torch.float32).view(1, 1, 1, 2)
    v = torch.tensor([[-0.5, 3.0]], dtype=torch.float32).view(1, 1, 1, 2)
    o, lse = orc.attn_fwd_ref(q, k, v, causal=False, scale=1.0)
    assert lse[0, 0, 0] == g["value"]
    assert np.array_equal(o[0, 0, 0], [-0.5, 3.0])


def test_golden_row_max_example(orc):
    """A score row equal to the page's reduction example.

    q = e_0 and k_j = a_j e_0 give s_ij = a_j; V = identity makes o_i = the
    whole softmax row, which must peak at the page's argmax, and
    lse = max + ln sum_j exp(a_j - max).
    """
    g = json.load(open(GOLDEN))["row_max_example"]
    a = g["row"]
    n = len(a)
    q = torch.zeros(1, 1, n, n, dtype=torch.float32)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, n, n, dtype=torch.float32)
    k[0, 0, :, 0] = torch.tensor(a, dtype=torch.float32)
    v = torch.eye(n, dtype=torch.float32).view(1, 1, n, n)
    o, lse = orc.attn_fwd_ref(q, k, v, causal=False, scale=1.0)
    m = g["max"]
    z = math.fsum(math.exp(x - m) for x in a)
    want_p = np.array([math.exp(x - m) / z for x in a])
    for i in range(n):
        assert int(np.argmax(o[0, 0, i])) == g["argmax"]
        np.testing.assert_allclose(o[0, 0, i], want_p, rtol=1e-15, atol=1e-17)
        assert abs(lse[0, 0, i] - (m + math.log(z))) < 1e-14


# ------------------------------------------------------ brute force tiny

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("d", [1, 2, 3, 8])
def test_brute_force_small_integers(orc, causal, n, d):
    """Small-integer Q, K make every score exact; compare with torch fp64."""
    g = torch.Generator().manual_seed(100 * n + d + causal)
    q = torch.randint(-3, 4, (2, 1, n, d), generator=g).to(torch.float32)
    k = torch.randint(-3, 4, (2, 1, n, d), generator=g).to(torch.float32)
    v = torch.randn((2, 1, n, d), generator=g)
    o, lse = orc.attn_fwd_ref(q, k, v, causal, 1.0)
    o2, lse2, _ = _library_attention(q, k, v, causal, 1.0)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("causal", [False, True])
def test_random_small_vs_library(orc, dtype, causal):
    """Random N(0,1) inputs in every dtype, non-trivial fp32 scale."""
    q, k, v = make_qkv(2, 3, 37, 16, dtype, seed=11 + causal)
    scale = float(torch.tensor(0.3, dtype=torch.float32))
    o, lse = orc.attn_fwd_ref(q, k, v, causal, scale)
    o2, lse2, _ = _library_attention(q, k, v, causal, scale)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(orc, causal):
    """sum_j exp(s_ij - lse_i) = 1 for every row (rows of P sum to 1)."""
    q, k, v = make_qkv(1, 2, 50, 8, torch.float32, seed=3)
    scale = float(np.float32(0.7))  # the oracle widens the fp32 scale
    _, lse = orc.attn_fwd_ref(q, k, v, causal, scale)
    s = scale * np.einsum("bhid,bhjd->bhij", _f64(q), _f64(k))
    if causal:
        s = np.where(np.tril(np.ones((50, 50), bool)), s, -np.inf)
    tot = np.exp(s - lse[..., None]).sum(-1)
    np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(orc, dtype, causal):
    """Constant V (every entry c) gives O = c: the weights sum to one."""
    q, k, _ = make_qkv(1, 2, 33, 16, dtype, seed=5)
    c = 0.375
    v = torch.full_like(q, c)
    o, _ = orc.attn_fwd_ref(q, k, v, causal, 0.25)
    np.testing.assert_allclose(o, c, rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("zero", ["q", "scale"])
def test_zero_scores_give_mean(orc, causal, zero):
    """All scores equal: O_i = mean of visible v_j (prefix mean if causal);
    lse_i = ln |J_i|."""
    q, k, v = make_qkv(2, 1, 20, 4, torch.float32, seed=9)
    scale = 0.5
    if zero == "q":
        q = torch.zeros_like(q)
    else:
        scale = 0.0
    o, lse = orc.attn_fwd_ref(q, k, v, causal, scale)
    vv = _f64(v)
    n = 20
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[:, :, i], vv[:, :, :cnt].mean(axis=2), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], math.log(cnt), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_unit_basis_probe_reconstructs_p(orc, causal):
    """V[k][0] = 1, all else 0 makes O[:,0] equal column k of P.

    Sweeping k rebuilds P: rows sum to 1, masked entries are exactly 0, and
    ratios follow exp(s_ik - s_ik')."""
    n, d = 12, 6
    q, k, _ = make_qkv(1, 1, n, d, torch.bfloat16, seed=21)
    scale = 0.375
    cols = []
    for kk in range(n):
        v = torch.zeros(1, 1, n, d, dtype=torch.bfloat16)
        v[0, 0, kk, 0] = 1.0
        o, _ = orc.attn_fwd_ref(q, k, v, causal, scale)
        assert np.all(o[..., 1:] == 0.0)
        cols.append(o[0, 0, :, 0])
    p = np.stack(cols, axis=1)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    s = scale * (_f64(q)[0, 0] @ _f64(k)[0, 0].T)
    if causal:
        assert np.all(p[np.triu_indices(n, 1)] == 0.0)
    for i in range(n):
        hi = i + 1 if causal else n
        ratio = p[i, :hi] / p[i, 0]
        np.testing.assert_allclose(ratio, np.exp(s[i, :hi] - s[i, 0]), rtol=1e-12)
    _, _, p_lib = _library_attention(q, k, torch.zeros_like(q), causal, scale)
    np.testing.assert_allclose(p, p_lib[0, 0], rtol=1e-12, atol=1e-15)


def test_causal_row0(orc):
    """Causal row 0 sees only key 0: O_0 = v_0 and lse_0 = s_00."""
    q, k, v = make_qkv(2, 2, 9, 8, torch.float32, seed=4)
    scale = 0.125
    o, lse = orc.attn_fwd_ref(q, k, v, True, scale)
    np.testing.assert_array_equal(o[:, :, 0], _f64(v)[:, :, 0])
    s00 = scale * (_f64(q)[:, :, 0] * _f64(k)[:, :, 0]).sum(-1)
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=1e-15, atol=1e-15)


def test_n1(orc):
    """N = 1: O = V, lse = scale * q.k."""
    q, k, v = make_qkv(3, 2, 1, 16, torch.float16, seed=8)
    o, lse = orc.attn_fwd_ref(q, k, v, False, 0.25)
    np.testing.assert_array_equal(o, _f64(v))
    np.testing.assert_allclose(lse, 0.25 * (_f64(q) * _f64(k)).sum(-1), rtol=1e-15)


def test_n2_closed_form(orc):
    """N = 2 non-causal: p_i0 = 1 / (1 + e^(s_i1 - s_i0))."""
    q, k, v = make_qkv(1, 1, 2, 4, torch.float32, seed=12)
    scale = 0.875
    o, _ = orc.attn_fwd_ref(q, k, v, False, scale)
    qq, kk, vv = _f64(q)[0, 0], _f64(k)[0, 0], _f64(v)[0, 0]
    for i in range(2):
        s0 = scale * qq[i] @ kk[0]
        s1 = scale * qq[i] @ kk[1]
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(o[0, 0, i], p0 * vv[0] + (1 - p0) * vv[1], rtol=1e-14, atol=1e-15)


def test_prefix_invariance_causal(orc):
    """Causal rows <= r do not depend on K, V rows > r."""
    q, k, v = make_qkv(1, 2, 30, 8, torch.bfloat16, seed=13)
    o1, l1 = orc.attn_fwd_ref(q, k, v, True, 0.35)
    r = 17
    k2, v2 = k.clone(), v.clone()
    k2[:, :, r + 1:] = torch.randn(k2[:, :, r + 1:].shape).to(k.dtype) * 5
    v2[:, :, r + 1:] = torch.randn(v2[:, :, r + 1:].shape).to(v.dtype) * 5
    o2, l2 = orc.attn_fwd_ref(q, k2, v2, True, 0.35)
    np.testing.assert_array_equal(o1[:, :, :r + 1], o2[:, :, :r + 1])
    np.testing.assert_array_equal(l1[:, :, :r + 1], l2[:, :, :r + 1])
    assert not np.array_equal(o1[:, :, r + 1:], o2[:, :, r + 1:])


def test_future_key_trap(orc):
    """k_t = alpha * q_i for a future t: causal row i must ignore it, while the
    non-causal row i collapses onto v_t."""
    n, d, i, t = 16, 8, 5, 11
    q, k, v = make_qkv(1, 1, n, d, torch.float32, seed=14)
    k = k.clone()
    k[0, 0, t] = q[0, 0, i] * 50.0
    oc, _ = orc.attn_fwd_ref(q, k, v, True, 1.0)
    onc, _ = orc.attn_fwd_ref(q, k, v, False, 1.0)
    np.testing.assert_allclose(onc[0, 0, i], _f64(v)[0, 0, t], atol=1e-10)
    o_ref, _, _ = _library_attention(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], False, 1.0)
    np.testing.assert_allclose(oc[0, 0, i], o_ref[0, 0, i], rtol=1e-12, atol=1e-13)


def test_large_scores_stay_finite(orc):
    """Scores of order 1e3 overflow exp without the max subtraction."""
    q, k, v = make_qkv(1, 1, 10, 4, torch.float32, seed=15)
    o, lse = orc.attn_fwd_ref(q * 400, k, v, False, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s = 400 * (_f64(q)[0, 0] @ _f64(k)[0, 0].T)
    j = np.argmax(s, axis=1)
    np.testing.assert_allclose(o[0, 0], _f64(v)[0, 0][j], atol=1e-6)


def test_key_permutation_invariance(orc):
    """Non-causal: permuting K and V rows jointly leaves O and lse unchanged;
    permuting Q rows permutes O rows."""
    q, k, v = make_qkv(1, 2, 25, 8, torch.float16, seed=16)
    o1, l1 = orc.attn_fwd_ref(q, k, v, False, 0.3)
    perm = torch.randperm(25, generator=torch.Generator().manual_seed(1))
    o2, l2 = orc.attn_fwd_ref(q, k[:, :, perm], v[:, :, perm], False, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    o3, l3 = orc.attn_fwd_ref(q[:, :, perm], k, v, False, 0.3)
    np.testing.assert_array_equal(o3, o1[:, :, perm.numpy()])
    np.testing.assert_array_equal(l3, l1[:, :, perm.numpy()])


def test_shift_invariance(orc):
    """K' = K + w for every key shifts row i's scores by scale q_i.w:
    O is unchanged and lse moves by exactly that amount (integers: exact)."""
    g = torch.Generator().manual_seed(17)
    q = torch.randint(-2, 3, (1, 1, 9, 4), generator=g).to(torch.float32)
    k = torch.randint(-2, 3, (1, 1, 9, 4), generator=g).to(torch.float32)
    v = torch.randn((1, 1, 9, 4), generator=g)
    w = torch.tensor([1.0, -2.0, 0.0, 3.0])
    for causal in (False, True):
        o1, l1 = orc.attn_fwd_ref(q, k, v, causal, 1.0)
        o2, l2 = orc.attn_fwd_ref(q, k + w, v, causal, 1.0)
        np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(l2 - l1, (_f64(q) @ w.double().numpy()), atol=1e-13)


def test_slices_independent(orc):
    """Each (b,h) slice equals a separate call with B = H = 1."""
    q, k, v = make_qkv(2, 3, 14, 8, torch.bfloat16, seed=18)
    o, lse = orc.attn_fwd_ref(q, k, v, True, 0.3)
    for b in range(2):
        for h in range(3):
            sl = (slice(b, b + 1), slice(h, h + 1))
            o1, l1 = orc.attn_fwd_ref(q[sl], k[sl], v[sl], True, 0.3)
            np.testing.assert_array_equal(o1[0, 0], o[b, h])
            np.testing.assert_array_equal(l1[0, 0], lse[b, h])


@pytest.mark.parametrize("causal", [False, True])
def test_same_values_any_dtype(orc, causal):
    """Values exactly representable in all three formats give identical output."""
    g = torch.Generator().manual_seed(19)
    base = [torch.randint(-8, 9, (1, 2, 11, 8), generator=g).to(torch.float32) / 4 for _ in range(3)]
    outs = [orc.attn_fwd_ref(*(t.to(dt) for t in base), causal, 0.5) for dt in DTYPES]
    for o, lse in outs[1:]:
        np.testing.assert_array_equal(o, outs[0][0])
        np.testing.assert_array_equal(lse, outs[0][1])


def test_rows_api_matches_full(orc):
    q, k, v = make_qkv(2, 2, 40, 16, torch.float16, seed=20)
    o, lse = orc.attn_fwd_ref(q, k, v, True, 0.25)
    rows = np.array([0, 39, 40, 77, 159, 5, 5, 120])
    o_r, l_r = orc.attn_fwd_ref_rows(q, k, v, True, 0.25, rows)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(l_r, lse.reshape(-1)[rows])


def test_thread_count_does_not_change_result(orc):
    q, k, v = make_qkv(1, 2, 64, 8, torch.float32, seed=22)
    a = orc.attn_fwd_ref(q, k, v, True, 0.3, num_threads=1)
    b = orc.attn_fwd_ref(q, k, v, True, 0.3, num_threads=7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ------------------------------------------ the fused method is exact

def _online_model(q, k, v, causal, scale, bn):
    """fp64 model of the tiled online-softmax recurrence: running max m,
    running sum l, unnormalised accumulator rescaled by exp(m_old - m_new),
    one division at the end ('Flash Attention（二）v2版本朴素实现 cuda core',
    sections 1.2-1.3 and 3.3; 'Flash Attention v2 的核心优化原理与工程实现',
    section 2)."""
    qq, kk, vv = _f64(q), _f64(k), _f64(v)
    B, H, N, d = qq.shape
    o = np.zeros_like(qq)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                hi = i + 1 if causal else N
                for j0 in range(0, hi, bn):
                    j1 = min(j0 + bn, hi)
                    s = scale * (kk[b, h, j0:j1] @ qq[b, h, i])
                    m_new = max(m, s.max())
                    alpha = math.exp(m - m_new) if m != -np.inf else 0.0
                    p = np.exp(s - m_new)
                    l = alpha * l + p.sum()
                    acc = alpha * acc + p @ vv[b, h, j0:j1]
                    m = m_new
                o[b, h, i] = acc / l
                lse[b, h, i] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("bn", [1, 3, 16, 100])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_matches_definition(orc, bn, causal):
    q, k, v = make_qkv(1, 2, 45, 8, torch.bfloat16, seed=23)
    o, lse = orc.attn_fwd_ref(q, k, v, causal, 0.375)
    o2, lse2 = _online_model(q, k, v, causal, 0.375, bn)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


# ------------------------------------------------ grouped-query attention
# ('Flash Attention v2 的核心优化原理与工程实现', References item 5: Flash
# Attention with GQA; query head h reads K/V head h // (H // H_kv)).

@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 3), (4, 1), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_library_on_expanded_kv(orc, H, H_kv, causal):
    """GQA = MHA with each K/V head repeated for its group of query heads
    (library fp64 softmax on repeat_interleave'd K/V). A grouping by h % H_kv
    instead of h // G gives different heads and fails here."""
    g = torch.Generator().manual_seed(31 + H * 10 + H_kv)
    q = torch.randn(2, H, 13, 8, generator=g).to(torch.bfloat16)
    k = torch.randn(2, H_kv, 13, 8, generator=g).to(torch.bfloat16)
    v = torch.randn(2, H_kv, 13, 8, generator=g).to(torch.bfloat16)
    G = H // H_kv
    ke, ve = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    o, lse = orc.attn_fwd_ref(q, k, v, causal, 0.375)
    o2, lse2, _ = _library_attention(q, ke, ve, causal, 0.375)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)
    # and the expanded inputs through the oracle's MHA path give the same bits
    o3, lse3 = orc.attn_fwd_ref(q, ke.contiguous(), ve.contiguous(), causal, 0.375)
    np.testing.assert_array_equal(o, o3)
    np.testing.assert_array_equal(lse, lse3)


def test_mqa_heads_share_one_kv(orc):
    """H_kv = 1: every query head of a batch reads the single K/V head, so a
    query head equal to another's gives identical rows."""
    g = torch.Generator().manual_seed(41)
    q = torch.randn(2, 3, 9, 8, generator=g)
    q[:, 2] = q[:, 0]
    k = torch.randn(2, 1, 9, 8, generator=g)
    v = torch.randn(2, 1, 9, 8, generator=g)
    o, lse = orc.attn_fwd_ref(q, k, v, True, 0.5)
    np.testing.assert_array_equal(o[:, 2], o[:, 0])
    assert not np.array_equal(o[0], o[1])   # batches use their own K/V
    for b in range(2):
        for h in range(3):
            o1, l1 = orc.attn_fwd_ref(q[b:b + 1, h:h + 1], k[b:b + 1], v[b:b + 1], True, 0.5)
            np.testing.assert_array_equal(o1[0, 0], o[b, h])
            np.testing.assert_array_equal(l1[0, 0], lse[b, h])


def test_gqa_rows_api_matches_full(orc):
    q, _, _ = make_qkv(2, 4, 30, 16, torch.float16, seed=42)
    _, k, v = make_qkv(2, 2, 30, 16, torch.float16, seed=43)
    o, lse = orc.attn_fwd_ref(q, k, v, False, 0.25)
    rows = np.array([0, 29, 30, 61, 119, 200, 239])
    o_r, l_r = orc.attn_fwd_ref_rows(q, k, v, False, 0.25, rows)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(l_r, lse.reshape(-1)[rows])


def test_gqa_rejects_bad_head_counts(orc):
    import ctypes
    lib = orc._load()
    q, k, v = make_qkv(1, 4, 4, 4, torch.float32, seed=1)
    o = np.zeros((1, 4, 4, 4))
    dp = o.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    for H_kv, want in [(4, 0), (2, 0), (1, 0), (3, -1), (0, -1), (-2, -1), (8, -1)]:
        rc = lib.attn_fwd_ref_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), dp, None,
                                  1, 4, H_kv, 4, 4, 0, 1.0, 0, 1)
        assert rc == want, (H_kv, rc)
    with pytest.raises(RuntimeError):
        orc.attn_fwd_ref(q, k[:, :3], v[:, :3], False, 1.0)   # 3 does not divide 4
    with pytest.raises(ValueError):
        orc.attn_fwd_ref(q, k[:, :2], v[:, :1], False, 1.0)   # k, v shapes differ


# ---------------------------------------------------------- backward
# The pages name the backward pass without formulas ('Flash Attention v2 的核心
# 优化原理与工程实现', comparison section); the oracle's gradient is the chain
# rule of the forward definition. Pinned to torch's fp64 autograd (a library
# routine), to central differences of the oracle's own forward, and to
# identities every correct gradient satisfies.

def _autograd_grads(q, k, v, dout, causal, scale):
    qq, kk, vv = (t.to(torch.float64).requires_grad_() for t in (q, k, v))
    G = q.shape[1] // k.shape[1]
    ke, ve = kk.repeat_interleave(G, dim=1), vv.repeat_interleave(G, dim=1)
    s = float(scale) * torch.matmul(qq, ke.transpose(-1, -2).contiguous())
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), ve)
    o.backward(dout.to(torch.float64))
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


def _grads_inputs(B, H, H_kv, N, d, dtype, seed):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=seed, H_kv=H_kv)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(B, H, N, d, generator=g).to(dtype)
    return q, k, v, dout


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2), (3, 1)])
def test_bwd_matches_autograd(orc, dtype, causal, H, H_kv):
    q, k, v, dout = _grads_inputs(2, H, H_kv, 11, 8, dtype, seed=50 + H + H_kv)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, dout, causal, 0.375)
    rq, rk, rv = _autograd_grads(q, k, v, dout, causal, 0.375)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_bwd_central_differences_of_forward(orc):
    """dL/dx for L = sum(O * dout), by central differences of the oracle's own
    forward with exactly representable fp32 steps."""
    g = torch.Generator().manual_seed(61)
    B, H, N, d = 1, 1, 6, 4
    q, k, v = (torch.randint(-8, 9, (B, H, N, d), generator=g).to(torch.float32) / 8
               for _ in range(3))
    dout = torch.randint(-4, 5, (B, H, N, d), generator=g).to(torch.float32) / 4
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd_ref(q, k, v, dout, causal, 0.5)
        h = 2.0 ** -12

        def loss(qx, kx, vx):
            o, _ = orc.attn_fwd_ref(qx, kx, vx, causal, 0.5)
            return float((o * dout.double().numpy()).sum())
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            for idx in [(0, 0, 0, 0), (0, 0, 2, 1), (0, 0, 5, 3), (0, 0, 3, 2)]:
                xs = [q.clone(), k.clone(), v.clone()]
                xs[which][idx] += h
                lp = loss(*xs)
                xs[which][idx] -= 2 * h
                lm = loss(*xs)
                fd = (lp - lm) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(grad[idx])), (which, idx, fd, grad[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_identities(orc, causal):
    """Softmax rows are shift invariant, so sum_j ds_ij = 0 and the keys'
    gradients sum to zero; rows of P sum to one, so the values' gradients sum
    to the group's summed dout; the error scales dominate the gradients."""
    q, k, v, dout = _grads_inputs(2, 4, 2, 37, 16, torch.bfloat16, seed=70)
    dq, dk, dv, eq, ek, ev, zq, zk, zv = orc.attn_bwd_ref(q, k, v, dout, causal, 0.25,
                                                          error_scales=True)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    g = _f64(dout).reshape(2, 2, 2, 37, 16).sum(axis=(2, 3))   # [B, H_kv, d]
    np.testing.assert_allclose(dv.sum(axis=2), g, rtol=1e-12, atol=1e-12)
    for grad, e in ((dq, eq), (dk, ek), (dv, ev)):
        assert np.all(e >= np.abs(grad) * (1 - 1e-12))
    # the absolute-rounding scales of dv count each visible row's |dout| once
    da = np.abs(_f64(dout)).reshape(2, 2, 2, 37, 16)
    if causal:
        cnt = np.flip(np.cumsum(np.flip(da, axis=3), axis=3), axis=3).sum(axis=2)
    else:
        cnt = np.broadcast_to(da.sum(axis=(2, 3))[:, :, None, :], zv.shape)
    np.testing.assert_allclose(zv, cnt, rtol=1e-12)
    assert np.all(zk >= 0) and np.all(zq >= 0)


def _bwd_model(q, k, v, dout, causal, scale):
    """The backward pass written out from the chain rule in numpy fp64, with
    K/V heads expanded to one per query head: P, O, dP = dO V^T, D and dS."""
    G = q.shape[1] // k.shape[1]
    Q, K, V, dO = (_f64(t) for t in (q, k, v, dout))
    K, V = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    s = float(scale) * Q @ np.swapaxes(K, -1, -2)
    vis = np.ones(s.shape[-2:], dtype=bool)
    if causal:
        vis = np.tril(vis)
    s = np.where(vis, s, -np.inf)
    P = np.exp(s - s.max(axis=-1, keepdims=True))
    P /= P.sum(axis=-1, keepdims=True)
    O = P @ V
    dP = dO @ np.swapaxes(V, -1, -2)
    D = (dO * O).sum(axis=-1)
    return Q, K, dO, P, O, dP, D, vis, G


def _bwd_grads(Q, K, dO, P, dS, scale, G):
    """dq, dk, dv from P and dS; dk, dv summed over each K/V head's query heads."""
    B, H, N, d = Q.shape
    dq = float(scale) * dS @ K
    dk = float(scale) * np.swapaxes(dS, -1, -2) @ Q
    dv = np.swapaxes(P, -1, -2) @ dO
    fold = lambda x: x.reshape(B, H // G, G, N, d).sum(axis=2)   # noqa: E731
    return dq, fold(dk), fold(dv)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_error_scales_are_attained(orc, causal):
    """The error scales are the exact worst case of their rounding model, not
    just an upper bound. The model: p, dS and O are each rounded once, with a
    relative error of at most u (the e scales) or an absolute one of at most
    s/2 (the z scales), and the rounded O enters dS through D. With Q, K and
    dO non-negative every gradient element is moved furthest by one and the
    same perturbation (dS and p pushed up, O pushed against the sign of
    dO * O), so the perturbed chain rule, recomputed from scratch, must move
    dq, dk, dv by exactly u e (and s/2 z): an inflated, deflated or
    mis-assembled scale fails, where the bound e >= |grad| alone would let an
    inflated scale pass."""
    B, H, H_kv, N, d = 1, 4, 2, 13, 8
    q, k, v, dout = _grads_inputs(B, H, H_kv, N, d, torch.float32, seed=120)
    q, k, dout = q.abs(), k.abs(), dout.abs()
    scale = 0.375
    dq, dk, dv, eq, ek, ev, zq, zk, zv = orc.attn_bwd_ref(q, k, v, dout, causal, scale,
                                                          error_scales=True)
    Q, K, dO, P, O, dP, D, vis, G = _bwd_model(q, k, v, dout, causal, scale)
    g0 = _bwd_grads(Q, K, dO, P, P * (dP - D[..., None]), scale, G)
    for got, ref in zip((dq, dk, dv), g0):
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)

    u = 2.0 ** -20
    dS = P * (dP - D[..., None])
    o_t = O * (1 - u * np.sign(dO * O))                      # D moves by -u sum |dO o|
    dS_t = P * (dP - (dO * o_t).sum(axis=-1)[..., None]) * (1 + u * np.sign(dS))
    g_rel = _bwd_grads(Q, K, dO, P * (1 + u), dS_t, scale, G)
    for moved, base, e in zip(g_rel, g0, (eq, ek, ev)):
        np.testing.assert_allclose((moved - base) / u, e, rtol=2e-5, atol=1e-12)

    h = 2.0 ** -20                                           # s / 2
    o_a = O - h * np.sign(dO)                                # D moves by -h sum |dO|
    dS_a = P * (dP - (dO * o_a).sum(axis=-1)[..., None]) + h * vis
    g_abs = _bwd_grads(Q, K, dO, P + h * vis, dS_a, scale, G)
    for moved, base, z in zip(g_abs, g0, (zq, zk, zv)):
        np.testing.assert_allclose((moved - base) / h, z, rtol=2e-5, atol=1e-12)
    # dO >= 0: the value gradient's relative scale is the gradient itself
    np.testing.assert_allclose(ev, dv, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_error_scales_bound_signed_worst_case(orc, causal):
    """With signed inputs the scales still bound the worst case of the model,
    found here element by element: for each column c of dq (and of dk) the
    perturbation of dS takes the sign of dS_ij k_jc (q_ic), and O's moves D
    in the direction that adds to it; the perturbed chain rule is recomputed
    per column. The relative part of that worst case, sum_j |dS_ij k_jc|, is
    attained exactly, so a scale that dropped an absolute value (or a term)
    falls below it."""
    B, H, H_kv, N, d = 1, 2, 1, 11, 6
    q, k, v, dout = _grads_inputs(B, H, H_kv, N, d, torch.float32, seed=121)
    scale = 0.5
    _, _, _, eq, ek, _, _, _, _ = orc.attn_bwd_ref(q, k, v, dout, causal, scale,
                                                   error_scales=True)
    Q, K, dO, P, O, dP, D, vis, G = _bwd_model(q, k, v, dout, causal, scale)
    dS = P * (dP - D[..., None])
    u = 2.0 ** -20
    base = _bwd_grads(Q, K, dO, P, dS, scale, G)
    for c in range(d):
        # dq column c: sign of dS_ij k_jc; D's move adds sign(sum_j p_ij k_jc)
        kc = K[..., c]                                        # [B, H, N] (expanded heads)
        dSk = dS * kc[..., None, :]
        turn = np.sign((P * kc[..., None, :]).sum(axis=-1))   # [B, H, N] per query row
        o_t = O * (1 - u * turn[..., None] * np.sign(dO * O))
        Dt = (dO * o_t).sum(axis=-1)
        dS_t = P * (dP - Dt[..., None]) * (1 + u * np.sign(dSk))
        worst = np.abs(_bwd_grads(Q, K, dO, P, dS_t, scale, G)[0][..., c] - base[0][..., c]) / u
        ds_part = float(scale) * np.abs(dSk).sum(axis=-1)
        assert np.all(worst <= eq[..., c] * (1 + 1e-5) + 1e-12)
        assert np.all(worst >= ds_part * (1 - 1e-5) - 1e-12)
        assert np.all(eq[..., c] >= ds_part * (1 - 1e-9))
        # dk column c: sign of dS_ij q_ic, summed over the group's query heads
        qc = Q[..., c]                                        # [B, H, N]
        dSq = dS * qc[..., :, None]
        dS_t = dS * (1 + u * np.sign(dSq))
        worst_k = np.abs(_bwd_grads(Q, K, dO, P, dS_t, scale, G)[1][..., c] - base[1][..., c]) / u
        assert np.all(ek[..., c] >= worst_k * (1 - 1e-5) - 1e-12)


def test_bwd_special_cases(orc):
    # N = 1: o = v, so dv = dout and dq = dk = 0
    q, k, v, dout = _grads_inputs(1, 2, 2, 1, 8, torch.float32, seed=80)
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, dout, True, 0.5)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dv, _f64(dout), rtol=0, atol=0)
    # constant V: o does not depend on q or k
    q, k, v, dout = _grads_inputs(1, 2, 1, 20, 8, torch.bfloat16, seed=81)
    v = torch.full_like(v, 0.75)
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd_ref(q, k, v, dout, causal, 0.5)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_bwd_linear_in_dout(orc):
    q, k, v, d1 = _grads_inputs(1, 2, 1, 19, 8, torch.float32, seed=90)
    g = torch.Generator().manual_seed(91)
    d2 = torch.randint(-4, 5, d1.shape, generator=g).to(torch.float32) / 4
    d1 = torch.randint(-4, 5, d1.shape, generator=g).to(torch.float32) / 4
    a = orc.attn_bwd_ref(q, k, v, d1, True, 0.5)
    b = orc.attn_bwd_ref(q, k, v, d2, True, 0.5)
    c = orc.attn_bwd_ref(q, k, v, d1 + d2, True, 0.5)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(x + y, z, rtol=1e-12, atol=1e-13)


def test_bwd_causal_key_sees_only_later_rows(orc):
    """Under the causal mask key j only receives gradient from rows i >= j:
    changing dout rows < r leaves dk, dv of keys >= r unchanged."""
    q, k, v, dout = _grads_inputs(1, 2, 2, 30, 8, torch.float32, seed=95)
    r = 17
    d2 = dout.clone()
    d2[:, :, :r] = torch.randn(1, 2, r, 8)
    a = orc.attn_bwd_ref(q, k, v, dout, True, 0.5)
    b = orc.attn_bwd_ref(q, k, v, d2, True, 0.5)
    np.testing.assert_array_equal(a[1][:, :, r:], b[1][:, :, r:])
    np.testing.assert_array_equal(a[2][:, :, r:], b[2][:, :, r:])
    np.testing.assert_array_equal(a[0][:, :, r:], b[0][:, :, r:])   # dq rows >= r too
    assert not np.array_equal(a[1][:, :, :r], b[1][:, :, :r])


def test_bwd_gqa_sums_expanded_heads(orc):
    q, k, v, dout = _grads_inputs(2, 6, 2, 15, 8, torch.float16, seed=99)
    G = 3
    ke = k.repeat_interleave(G, dim=1).contiguous()
    ve = v.repeat_interleave(G, dim=1).contiguous()
    dq, dk, dv = orc.attn_bwd_ref(q, k, v, dout, True, 0.5)
    eq_, ek_, ev_ = orc.attn_bwd_ref(q, ke, ve, dout, True, 0.5)
    np.testing.assert_array_equal(dq, eq_)
    np.testing.assert_allclose(dk, ek_.reshape(2, 2, 3, 15, 8).sum(axis=2), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, ev_.reshape(2, 2, 3, 15, 8).sum(axis=2), rtol=1e-13, atol=1e-14)


def test_bwd_thread_count_does_not_change_result(orc):
    q, k, v, dout = _grads_inputs(1, 2, 1, 40, 8, torch.bfloat16, seed=97)
    a = orc.attn_bwd_ref(q, k, v, dout, False, 0.5, num_threads=1)
    b = orc.attn_bwd_ref(q, k, v, dout, False, 0.5, num_threads=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a[2], b[2], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------ errors

def test_oracle_rejects_bad_arguments(orc):
    import ctypes
    lib = orc._load()
    q, k, v = make_qkv(1, 1, 4, 4, torch.float32, seed=1)
    o = np.zeros((1, 1, 4, 4))
    dp = o.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), dp, None, 1, 1, 4, 4, 0, 1.0, 0, 1]
    assert lib.attn_fwd_ref(*args) == 0
    for idx, bad in [(0, None), (5, 0), (7, -1), (8, 0), (9, 2), (10, float("nan")), (11, 7)]:
        a = list(args)
        a[idx] = bad
        assert lib.attn_fwd_ref(*a) == -1, (idx, bad)
    with pytest.raises(RuntimeError):
        orc.attn_fwd_ref_rows(q, k, v, False, 1.0, [4])
