"""The allocation-free backward entry point, attn_bwd_noalloc, through the
C ABI: on two calls in a row (the second with a smaller input, so that it
runs over the first call's leftovers in the shared static array) its
gradients are bit-identical to attn_bwd's on the same inputs, which keeps
its row statistic in a caller-allocated buffer; and sizes past the static
array are refused before any launch."""
import pytest
import torch

from exact_attention_15_amd.inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.load_library()
    return ea


def _grads(ea, q, k, v, o, lse, dout, causal, noalloc):
    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    tail = (B, H, k.shape[1], N, d, int(causal), ea.default_scale(d), ea.dtype_code(q.dtype),
            stream)
    if noalloc:
        rc = ea.attn_bwd_noalloc(*args, *tail)
    else:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        rc = ea.attn_bwd(*args, delta.data_ptr(), *tail)
    assert rc == 0, ea.strerror(rc)
    return dq, dk, dv


@pytest.mark.parametrize("dtype,d,causal,H_kv", [
    (torch.bfloat16, 64, True, 2),
    (torch.float16, 128, False, 4),
    (torch.float32, 64, True, 1),
], ids=["bf16-d64-causal-gqa", "f16-d128-mha", "f32-d64-causal-mqa"])
def test_noalloc_matches_attn_bwd_twice(ea, dtype, d, causal, H_kv):
    for B, H, N, seed in ((2, 4, 1000, 11), (1, 4, 300, 12)):
        q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, dtype, seed=seed, H_kv=min(H_kv, H)))
        dout = make_dout(B, H, N, d, dtype, seed=seed).cuda()
        o, lse = ea.fwd(q, k, v, causal=causal)
        want = _grads(ea, q, k, v, o, lse, dout, causal, noalloc=False)
        got = _grads(ea, q, k, v, o, lse, dout, causal, noalloc=True)
        torch.cuda.synchronize()
        for x, y, name in zip(got, want, ("dq", "dk", "dv")):
            assert torch.equal(x, y), (name, B, H, N)


def test_noalloc_refuses_sizes_past_its_array(ea):
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    p = q.data_ptr()
    # B*H*N = 2^22 + 64 rows: one row block past the limit; nothing is launched
    rc = ea.attn_bwd_noalloc(p, p, p, p, lse.data_ptr(), p, p, p, p, 1, 65537, 65537, 64, 64,
                             0, 0.125, ea.ATTN_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == ea.ATTN_ETOOBIG
    assert "ATTN_BWD_NOALLOC_MAX_ROWS" in ea.strerror(rc)
