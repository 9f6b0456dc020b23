"""The C-ABI calls captured in a HIP graph (torch.cuda.CUDAGraph over the
capture stream): the library launches on the caller's stream and allocates
nothing, so attn_fwd / attn_bwd / attn_fwd_unfused record as plain kernel
nodes. Each replay runs on new inputs copied into the captured buffers,
with eager work and synchronisations in between, and must equal the eager
result bit for bit."""
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


def _replay_and_compare(graph, inputs, fresh, eager, got_fn):
    for rep in range(4):
        for dst, src in zip(inputs, fresh(rep)):
            dst.copy_(src.cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in got_fn()]
        # eager work between replays, then the eager result on the same inputs
        _ = (inputs[0].float() * 2).sum().item()
        want = eager()
        torch.cuda.synchronize()
        for g_, e_ in zip(got, want):
            assert torch.equal(g_, e_), rep


def _capture(step):
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
    return graph


@pytest.mark.parametrize("dtype,d,H,H_kv", [
    (torch.bfloat16, 64, 4, 2),
    (torch.float32, 64, 4, 2),
    # eight query heads per K/V head: chunked dK/dV partial sums and their
    # reduction kernel inside the graph
    (torch.float16, 128, 8, 1),
], ids=["bf16-d64-gqa", "f32-d64-gqa", "f16-d128-split"])
def test_forward_and_backward_in_a_graph(ea, dtype, d, H, H_kv):
    B, N = 1, 300
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, dtype, seed=61, H_kv=H_kv))
    dout = make_dout(B, H, N, d, dtype, seed=61).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((B, H, N), dtype=torch.float32, device="cuda"))

    def step():
        ea.fwd(q, k, v, causal=True, out=(o, lse))
        ea.bwd(q, k, v, o, lse, dout, causal=True, out=grads)

    graph = _capture(step)

    def fresh(rep):
        nq, nk, nv = make_qkv(B, H, N, d, dtype, seed=70 + rep, H_kv=H_kv)
        return nq, nk, nv, make_dout(B, H, N, d, dtype, seed=70 + rep)

    def eager():
        o_e, lse_e = ea.fwd(q, k, v, causal=True)
        return (o_e, lse_e) + tuple(ea.bwd(q, k, v, o_e, lse_e, dout, causal=True))

    _replay_and_compare(graph, (q, k, v, dout), fresh, eager, lambda: (o, lse) + grads[:3])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_unfused_in_a_graph(ea, dtype):
    B, H, N, d = 1, 2, 200, 64
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, dtype, seed=81))
    ws = torch.empty(ea.unfused_workspace_bytes(B, H, N, ea.dtype_code(dtype)),
                     dtype=torch.uint8, device="cuda")
    res = {}

    def step():
        res["o"], res["lse"] = ea.fwd_unfused(q, k, v, causal=True, workspace=ws)

    graph = _capture(step)

    def fresh(rep):
        return make_qkv(B, H, N, d, dtype, seed=90 + rep)

    def eager():
        return ea.fwd_unfused(q, k, v, causal=True)

    _replay_and_compare(graph, (q, k, v), fresh, eager, lambda: (res["o"], res["lse"]))
