"""The C-ABI calls captured in a HIP graph (torch.cuda.CUDAGraph over the
capture stream): the library launches on the caller's stream and allocates
nothing, so attn_fwd / attn_bwd record as plain kernel nodes. Each replay
runs on new inputs copied into the captured buffers, with eager work and
synchronisations in between, and must equal the eager result bit for bit."""
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


def test_forward_and_backward_in_a_graph(ea):
    B, H, H_kv, N, d = 1, 4, 2, 300, 64
    dtype = torch.bfloat16
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, dtype, seed=61, H_kv=H_kv))
    dout = make_dout(B, H, N, d, dtype, seed=61).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((B, H, N), dtype=torch.float32, device="cuda"))

    def step():
        ea.fwd(q, k, v, causal=True, out=(o, lse))
        ea.bwd(q, k, v, o, lse, dout, causal=True, out=grads)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # warm-up outside capture
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        nq, nk, nv = make_qkv(B, H, N, d, dtype, seed=70 + rep, H_kv=H_kv)
        nd = make_dout(B, H, N, d, dtype, seed=70 + rep)
        for dst, src in ((q, nq), (k, nk), (v, nv), (dout, nd)):
            dst.copy_(src.cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse) + grads[:3]]
        # eager work between replays, then the eager result on the same inputs
        _ = (q.float() * 2).sum().item()
        o_e, lse_e = ea.fwd(q, k, v, causal=True)
        dq_e, dk_e, dv_e = ea.bwd(q, k, v, o_e, lse_e, dout, causal=True)
        torch.cuda.synchronize()
        for g_, e_ in zip(got, (o_e, lse_e, dq_e, dk_e, dv_e)):
            assert torch.equal(g_, e_), rep
