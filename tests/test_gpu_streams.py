"""Calls on several streams at once: the library keeps no state between
calls and allocates nothing, so independent calls launched on two streams,
interleaved and running concurrently, give exactly the results of the same
calls run one after another on one stream."""
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


def _problems():
    """Two forward + backward problems of different kinds (bf16 causal MHA at
    d = 64; fp16 grouped-query d = 128 with chunked dK/dV partial sums)."""
    out = []
    for (B, H, H_kv, n, d, dt, causal, seed) in [
            (2, 8, 8, 1500, 64, torch.bfloat16, True, 8100),
            (1, 8, 1, 777, 128, torch.float16, False, 8101)]:
        q, k, v = (t.cuda() for t in make_qkv(B, H, n, d, dt, seed=seed, H_kv=H_kv))
        dout = make_dout(B, H, n, d, dt, seed=seed).cuda()
        out.append((q, k, v, dout, causal))
    return out


def _run(ea, prob):
    q, k, v, dout, causal = prob
    o, lse = ea.fwd(q, k, v, causal=causal)
    dq, dk, dv = ea.bwd(q, k, v, o, lse, dout, causal=causal)
    return [o, lse, dq, dk, dv]


def test_two_streams_match_one_stream(ea):
    probs = _problems()
    serial = [_run(ea, p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = [[], []]
    for rep in range(3):
        for i, (s, p) in enumerate(zip(streams, probs)):
            with torch.cuda.stream(s):
                results[i].append(_run(ea, p))
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(2):
        for rep, got in enumerate(results[i]):
            for g, w in zip(got, serial[i]):
                assert torch.equal(g, w), (i, rep)
