"""Exact attention (forward, backward, unfused comparison) for MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (``include/attn.h``):
it checks tensors, allocates the outputs with torch on the inputs' device
and passes raw pointers plus torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no fallback path,
and a missing library raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EALIGN, ATTN_EHIP, ATTN_ETOOBIG = 0, -1, -2, -3, -4, -5
BWD_NOALLOC_MAX_ROWS = 4 * 1024 * 1024   # ATTN_BWD_NOALLOC_MAX_ROWS

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str, entry: str = "attn_fwd"):
        super().__init__(f"{entry} failed ({code}): {msg}")
        self.code = code
        self.entry = entry


def load_library():
    """Load libattn.so (built by ``exact_attention_15_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_15_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


def load_probe_library():
    """The race-check build (timing probes compiled in, same entry points),
    for the tests that compare it with the library bit for bit."""
    path = os.path.join(_PKG, "libattn_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_attention_15_amd.build`")
    return _configure(ctypes.CDLL(path))


def _configure(lib):
    """Declare the C signatures of include/attn.h on a loaded library."""
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                             ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                 ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd_gqa.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                             ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_fwd_unfused.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd_unfused.restype = ctypes.c_int
    lib.attn_unfused_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.attn_unfused_workspace_bytes.restype = i64
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_debug_set_fwd_variant.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.attn_debug_set_fwd_variant.restype = ctypes.c_int
    lib.attn_debug_set_fwd_first_pass.argtypes = [ctypes.c_int]
    lib.attn_debug_set_fwd_first_pass.restype = ctypes.c_int
    return lib


def strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def debug_set_fwd_variant(query_blocks: int = 0, order: int = 0) -> None:
    """Debugging and testing only: force the 16-bit forward's query blocks
    per wave (0 automatic, 1, 2) and work order (0 automatic, 1 tile-major,
    2 XCD-major) for every later call in the process; outputs are
    bit-identical across variants. `debug_set_fwd_variant()` restores the
    automatic choice."""
    rc = load_library().attn_debug_set_fwd_variant(int(query_blocks), int(order))
    if rc != ATTN_OK:
        raise AttnError(rc, strerror(rc), "attn_debug_set_fwd_variant")


def debug_set_fwd_first_pass(mode: int = 0) -> None:
    """Debugging and testing only: at d = 64 force the 16-bit forward's
    first pass without the per-tile overflow test (0 automatic, 1 the exact
    pass only, 2 the first pass at any sequence length) for every later call
    in the process; outputs are bit-identical across modes.
    `debug_set_fwd_first_pass()` restores the automatic choice."""
    rc = load_library().attn_debug_set_fwd_first_pass(int(mode))
    if rc != ATTN_OK:
        raise AttnError(rc, strerror(rc), "attn_debug_set_fwd_first_pass")


def dtype_code(dtype) -> int:
    import torch
    m = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
    if dtype not in m:
        raise TypeError(f"unsupported dtype {dtype}; need float32, float16 or bfloat16")
    return m[dtype]


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32 (the value the library multiplies in)."""
    import struct
    return struct.unpack("f", struct.pack("f", 1.0 / math.sqrt(d)))[0]


def attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream) -> int:
    """Raw C-ABI call with integer pointers; returns the library's code."""
    return load_library().attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal),
                                   float(scale), int(dtype), stream)


def attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, dtype, stream) -> int:
    """Raw C-ABI call (grouped-query form) with integer pointers."""
    return load_library().attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, int(causal),
                                       float(scale), int(dtype), stream)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None):
    """O, lse = attention forward of q [B,H,N,d] and k, v [B,H_kv,N,d].

    H_kv = H is multi-head attention; a smaller H_kv dividing H is
    grouped-query attention (query head h reads K/V head h // (H // H_kv)),
    H_kv = 1 multi-query attention.

    Returns ``o`` (same dtype/shape as q) and ``lse`` (float32 [B,H,N],
    natural-log log-sum-exp of the scaled scores). ``out`` may pass
    preallocated ``(o, lse)`` tensors.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or \
            (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]):
        raise ValueError("need q [B, H, N, d] and k, v [B, H_kv, N, d]")
    if k.shape[1] < 1 or q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"K/V heads ({k.shape[1]}) must divide query heads ({q.shape[1]})")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.device.type != "cuda" or k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one GPU device")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = default_scale(d)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
            raise ValueError("out[0] must match q")
        if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
                or lse.device != q.device:
            raise ValueError("out[1] must be float32 [B, H, N] on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          lse.data_ptr(), B, H, H_kv, N, d, causal, scale,
                          dtype_code(q.dtype), stream)
    if rc != ATTN_OK:
        raise AttnError(rc, strerror(rc), "attn_fwd_gqa")
    return o, lse


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, causal, scale,
             dtype, stream) -> int:
    """Raw C-ABI call of the backward pass with integer pointers."""
    return load_library().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d,
                                   int(causal), float(scale), int(dtype), stream)


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, out=None):
    """dq, dk, dv = gradients of the forward pass for the incoming gradient
    ``dout`` of ``o``, from the forward's ``o`` and ``lse``.

    q, o, dout: [B,H,N,d]; k, v: [B,H_kv,N,d]; lse: float32 [B,H,N]; all on
    one GPU, contiguous, q/k/v/o/dout of one dtype. ``out`` may pass
    preallocated ``(dq, dk, dv, delta)`` (delta: float32 [B,H,N], written
    with the row statistic D_i = dout_i . o_i).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or \
            (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]):
        raise ValueError("need q [B, H, N, d] and k, v [B, H_kv, N, d]")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must match q")
    if k.shape[1] < 1 or q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"K/V heads ({k.shape[1]}) must divide query heads ({q.shape[1]})")
    if len({t.dtype for t in (q, k, v, o, dout)}) != 1:
        raise TypeError("q, k, v, o, dout must share one dtype")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    for t in (q, k, v, o, lse, dout):
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError("all tensors must be on one GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if scale is None:
        scale = default_scale(d)
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, delta = out
        for t, ref in ((dq, q), (dk, k), (dv, v)):
            if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() \
                    or t.device != q.device:
                raise ValueError("out gradients must match q, k, v")
        if delta.shape != (B, H, N) or delta.dtype != torch.float32 or \
                not delta.is_contiguous() or delta.device != q.device:
            raise ValueError("out[3] must be float32 [B, H, N] on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      delta.data_ptr(), B, H, H_kv, N, d, causal, scale,
                      dtype_code(q.dtype), stream)
    if rc != ATTN_OK:
        raise AttnError(rc, strerror(rc), "attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, causal, scale, dtype,
                     stream) -> int:
    """Raw C-ABI call of the allocation-free backward (no delta argument)."""
    return load_library().attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d,
                                           int(causal), float(scale), int(dtype), stream)


def attn_fwd_unfused(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, causal, scale,
                     dtype, stream) -> int:
    """Raw C-ABI call of the unfused three-kernel forward."""
    return load_library().attn_fwd_unfused(q, k, v, o, lse, workspace, workspace_bytes, B, H, N,
                                           d, int(causal), float(scale), int(dtype), stream)


def unfused_workspace_bytes(B: int, H: int, N: int, dtype: int) -> int:
    """Workspace bytes of ``attn_fwd_unfused`` for the dtype code ``dtype``."""
    return int(load_library().attn_unfused_workspace_bytes(B, H, N, int(dtype)))


def fwd_unfused(q, k, v, causal: bool = False, scale: float | None = None, workspace=None):
    """The unfused forward (S, softmax, P V as three kernels with N x N
    buffers): the comparison path. Returns (o, lse) like ``fwd``.
    ``workspace`` may pass a preallocated uint8 device tensor of at least
    ``unfused_workspace_bytes(B, H, N, dtype_code(q.dtype))`` bytes."""
    import torch
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    for t in (q, k, v):
        if t.device.type != "cuda" or t.device != q.device or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous tensors on one GPU device")
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    need = unfused_workspace_bytes(B, H, N, dtype_code(q.dtype))
    if need < 0:
        raise ValueError("sizes out of range")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = attn_fwd_unfused(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H, N,
                              d, causal, scale, dtype_code(q.dtype), stream)
    if rc != ATTN_OK:
        raise AttnError(rc, strerror(rc), "attn_fwd_unfused")
    return o, lse


__all__ = ["fwd", "bwd", "debug_set_fwd_variant", "debug_set_fwd_first_pass", "fwd_unfused", "attn_fwd_unfused", "unfused_workspace_bytes", "attn_bwd", "attn_bwd_noalloc", "attn_fwd", "attn_fwd_gqa", "load_library", "strerror", "AttnError", "default_scale",
           "dtype_code", "LIB_PATH", "ATTN_F32", "ATTN_F16", "ATTN_BF16"]
