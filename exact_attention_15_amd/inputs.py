"""Seeded synthetic inputs for exact attention forward.

This module only draws random numbers and names workloads; it holds none of
the attention arithmetic. Both the GPU path's tests/bench and the CPU oracle
are fed from here, so they see identical bits.

Recipe: Q, K, V drawn i.i.d. N(0,1) in float32 from ``torch.Generator('cpu')``
seeded with ``seed``, in the order Q, K, V; Q is ``[B, H, N, d]`` and K, V are
``[B, H_kv, N, d]`` (H_kv = H unless the workload is grouped-query), contiguous;
optionally multiplied by ``value_scale`` in float32; then rounded to the
target dtype with round-to-nearest-even (``Tensor.to``). The unit-variance
inputs are the setting in which the cishoon.github.io "flashattention" post,
section 1.1.2 item 2, derives that q.k/sqrt(d) has variance 1.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    N: int
    d: int
    causal: bool
    value_scale: float = 1.0
    seed: int = 0
    H_kv: int | None = None   # K/V heads (grouped-query attention); None: H

    @property
    def kv_heads(self) -> int:
        return self.H if self.H_kv is None else self.H_kv

    @property
    def scale(self) -> float:
        """Default softmax scale 1/sqrt(d), as the fp32 value both sides use."""
        return float(torch.tensor(1.0 / (self.d ** 0.5), dtype=torch.float32).item())

    def describe(self) -> str:
        dt = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}[self.dtype]
        c = "causal" if self.causal else "non-causal"
        kv = "" if self.H_kv is None else f" H_kv={self.H_kv}"
        return f"{dt} {c} attention fwd B={self.B} H={self.H}{kv} N={self.N} d={self.d}"


def _wl(cfg: int, variant: int, **kw) -> Workload:
    return Workload(seed=1000 * cfg + variant, **kw)


# The five workloads: a small fp32 case, an fp32 causal case, the bf16 causal
# headline case, a long-context d=128 case (causal and not), and an fp16 case
# with a ragged-tail variant.
WORKLOADS = {
    "c1_f32_small": _wl(1, 0, name="c1_f32_small", dtype=torch.float32,
                        B=1, H=1, N=128, d=64, causal=False),
    "c2_f32_causal": _wl(2, 0, name="c2_f32_causal", dtype=torch.float32,
                         B=1, H=32, N=1024, d=64, causal=True),
    "c3_bf16_causal": _wl(3, 0, name="c3_bf16_causal", dtype=torch.bfloat16,
                          B=4, H=16, N=4096, d=64, causal=True),
    "c4_bf16_d128_causal": _wl(4, 0, name="c4_bf16_d128_causal", dtype=torch.bfloat16,
                               B=1, H=32, N=8192, d=128, causal=True),
    "c4_bf16_d128": _wl(4, 1, name="c4_bf16_d128", dtype=torch.bfloat16,
                        B=1, H=32, N=8192, d=128, causal=False),
    "c5_f16": _wl(5, 0, name="c5_f16", dtype=torch.float16,
                  B=1, H=8, N=16384, d=64, causal=False, value_scale=0.5),
    "c5_f16_ragged": _wl(5, 1, name="c5_f16_ragged", dtype=torch.float16,
                         B=1, H=8, N=16383, d=64, causal=False, value_scale=0.5),
    # Grouped-query forms of the headline case (4 query heads per K/V head)
    # and of the long d=128 case with a single K/V head (multi-query).
    "g1_bf16_causal_gqa4": _wl(6, 0, name="g1_bf16_causal_gqa4", dtype=torch.bfloat16,
                               B=4, H=16, H_kv=4, N=4096, d=64, causal=True),
    "g2_bf16_d128_mqa": _wl(6, 1, name="g2_bf16_d128_mqa", dtype=torch.bfloat16,
                            B=1, H=32, H_kv=1, N=8192, d=128, causal=True),
}

HEADLINE = "c3_bf16_causal"


def make_qkv(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
             value_scale: float = 1.0, H_kv: int | None = None):
    """Draw Q [B,H,N,d], then K and V [B,H_kv,N,d] (H_kv defaults to H) on the
    CPU; return dtype tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for heads in (H, H if H_kv is None else H_kv, H if H_kv is None else H_kv):
        x = torch.randn((B, heads, N, d), dtype=torch.float32, generator=g)
        if value_scale != 1.0:
            x = x * torch.tensor(value_scale, dtype=torch.float32)
        out.append(x.to(dtype).contiguous())
    return tuple(out)


def make_qkv_device(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
                    H_kv: int | None = None, device: str = "cuda"):
    """Like ``make_qkv`` (i.i.d. N(0,1) float32, rounded to the dtype; Q, then
    K and V) but drawn by the device's generator seeded with ``seed``, for
    tensors too large to draw on the host. Other bits than ``make_qkv``'s;
    a test copies the slices it checks to the host for the oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    kv = H if H_kv is None else H_kv
    return tuple(torch.randn((B, heads, N, d), dtype=torch.float32, device=device,
                             generator=g).to(dtype)
                 for heads in (H, kv, kv))


def make_dout_device(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
                     device: str = "cuda"):
    """The incoming gradient drawn on the device (seed + 10**6)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 10 ** 6)
    return torch.randn((B, H, N, d), dtype=torch.float32, device=device,
                       generator=g).to(dtype)


def make_dout(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int):
    """The incoming gradient of O for the backward pass: i.i.d. N(0,1) fp32
    from its own generator (seed + 10**6), rounded to the dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 10 ** 6)
    return torch.randn((B, H, N, d), dtype=torch.float32, generator=g).to(dtype).contiguous()


def workload_dout(w: Workload):
    return make_dout(w.B, w.H, w.N, w.d, w.dtype, w.seed)


def workload_inputs(w: Workload):
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.value_scale, w.H_kv)


def make_structured_qkv(kind: str, B: int, H: int, N: int, d: int, dtype: torch.dtype,
                        seed: int, peak: float = 40.0):
    """Inputs whose score rows have a chosen shape, to drive the online
    softmax's running maximum (drawn in float32, then rounded to the dtype):

    * ``"rising"``:  q_i = u + 0.25 n, k_j = (peak j / N) u / sqrt(d) + 0.25 n
      with u a random +-1 vector and n fresh N(0,1) noise, so that (at the
      default scale 1/sqrt(d)) the score of key j grows by about peak / N per
      key: the row maximum moves on every key tile.
    * ``"falling"``: the same with j replaced by N - 1 - j: the maximum sits
      in the first tile and never moves afterwards.
    * ``"wide"``:    Q, K i.i.d. N(0, 4), scores with standard deviation ~4:
      rows are nearly one-hot and their maxima jump irregularly.
    * ``"spikes"``:  q_i = u + 0.25 n, k_j = 0.25 n except three keys
      j_s = (s + 1) N / 4 + 3 (s = 0, 1, 2), where k_j += 2.5 (s + 1) peak u
      / sqrt(d): at the default scale their scores are about 2.5 (s + 1)
      peak (100, 200, 300 at peak = 40), so a row's maximum jumps by more
      than 128 log2 units inside one key tile, past what exp2 against the
      old maximum can represent in fp32.

    V is i.i.d. N(0,1) in every case.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    if kind == "wide":
        q = torch.randn((B, H, N, d), dtype=torch.float32, generator=g) * 2.0
        k = torch.randn((B, H, N, d), dtype=torch.float32, generator=g) * 2.0
    elif kind in ("rising", "falling"):
        u = torch.randint(0, 2, (B, H, 1, d), generator=g).to(torch.float32) * 2.0 - 1.0
        q = u + 0.25 * torch.randn((B, H, N, d), dtype=torch.float32, generator=g)
        j = torch.arange(N, dtype=torch.float32)
        if kind == "falling":
            j = (N - 1) - j
        ramp = (peak / N) * j / (d ** 0.5)
        k = ramp.view(1, 1, N, 1) * u + 0.25 * torch.randn((B, H, N, d), dtype=torch.float32,
                                                            generator=g)
    elif kind == "spikes":
        u = torch.randint(0, 2, (B, H, 1, d), generator=g).to(torch.float32) * 2.0 - 1.0
        q = u + 0.25 * torch.randn((B, H, N, d), dtype=torch.float32, generator=g)
        k = 0.25 * torch.randn((B, H, N, d), dtype=torch.float32, generator=g)
        for s_ in range(3):
            j = (s_ + 1) * N // 4 + 3
            if j < N:
                k[:, :, j, :] += (2.5 * (s_ + 1) * peak / d ** 0.5) * u[:, :, 0, :]
    else:
        raise ValueError(f"unknown kind {kind!r}")
    v = torch.randn((B, H, N, d), dtype=torch.float32, generator=g)
    return tuple(x.to(dtype).contiguous() for x in (q, k, v))
