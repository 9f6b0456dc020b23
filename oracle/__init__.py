"""CPU fp64 oracle for exact attention forward — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports, links or
calls it, and the two share no code.

This module is a thin ctypes loader for ``liboracle_attn.so`` (built from
``attn_ref.c`` by :func:`build`). The arithmetic lives entirely in the C file,
which follows the attention definition of the cishoon.github.io
"flashattention" post, section 1.1.2, with the causal convention of
"Flash Attention（二）v2版本朴素实现 cuda core", section 3.4. Grouped-query
attention (the FlashAttention-2 principles page, References item 5) is taken
from k/v having fewer heads than q: query head h reads K/V head h // (H // H_kv).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_attn.so")
SRC_PATH = os.path.join(_HERE, "attn_ref.c")

F32, F16, BF16 = 0, 1, 2

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain C, IEEE fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off",
           SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # ATTN_ORACLE_LIB: a library built from a deliberately altered copy of
    # attn_ref.c, loaded only by the mutation test that checks the pins catch it.
    path = os.environ.get("ATTN_ORACLE_LIB", LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(f"oracle library missing: {path}; run oracle.build()")
    lib = ctypes.CDLL(path)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
    lib.attn_fwd_ref.argtypes = [vp, vp, vp, dp, dp, i64, i64, i64, i64,
                                 ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.attn_fwd_ref.restype = ctypes.c_int
    lib.attn_fwd_ref_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64,
                                      ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_int64), i64, dp, dp,
                                      ctypes.c_int]
    lib.attn_fwd_ref_rows.restype = ctypes.c_int
    lib.attn_fwd_ref_gqa.argtypes = [vp, vp, vp, dp, dp, i64, i64, i64, i64, i64,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                     ctypes.c_int]
    lib.attn_fwd_ref_gqa.restype = ctypes.c_int
    lib.attn_fwd_ref_rows_gqa.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64,
                                          ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int64), i64, dp, dp,
                                          ctypes.c_int]
    lib.attn_fwd_ref_rows_gqa.restype = ctypes.c_int
    lib.attn_bwd_ref.argtypes = [vp, vp, vp, vp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                 i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_int]
    lib.attn_bwd_ref.restype = ctypes.c_int
    lib.attn_ref_decode.argtypes = [vp, dp, i64, ctypes.c_int]
    lib.attn_ref_decode.restype = ctypes.c_int
    _lib = lib
    return lib


def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in m:
        raise TypeError(f"oracle: unsupported dtype {t.dtype}")
    return m[t.dtype]


def _as_host(t):
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be host (CPU) tensors")
    return t.contiguous()


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _kv_heads(q, k, v) -> int:
    B, H, N, d = q.shape
    if k.dim() != 4 or tuple(k.shape) != tuple(v.shape) or \
            (k.shape[0], k.shape[2], k.shape[3]) != (B, N, d):
        raise ValueError(f"oracle: k/v shapes {tuple(k.shape)}, {tuple(v.shape)} "
                         f"do not fit q {tuple(q.shape)}")
    return int(k.shape[1])


def attn_fwd_ref(q, k, v, causal: bool, scale: float, num_threads: int = 0):
    """Full oracle. q: CPU tensor [B,H,N,d]; k, v: [B,H_kv,N,d], one dtype.

    H_kv = H is multi-head attention; H_kv < H (dividing H) is grouped-query.
    Returns (o, lse) as float64 numpy arrays of shapes [B,H,N,d] and [B,H,N].
    """
    lib = _load()
    q, k, v = _as_host(q), _as_host(k), _as_host(v)
    B, H, N, d = q.shape
    H_kv = _kv_heads(q, k, v)
    o = np.empty((B, H, N, d), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = lib.attn_fwd_ref_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dptr(o),
                              _dptr(lse), B, H, H_kv, N, d, int(bool(causal)),
                              float(scale), _dtype_code(q), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"attn_fwd_ref failed with code {rc}")
    return o, lse


def attn_fwd_ref_rows(q, k, v, causal: bool, scale: float, rows, num_threads: int = 0):
    """Oracle on selected flat row ids r = (b*H + h)*N + i.

    Returns (o_rows [n, d], lse_rows [n]) as float64 numpy arrays.
    """
    lib = _load()
    q, k, v = _as_host(q), _as_host(k), _as_host(v)
    B, H, N, d = q.shape
    H_kv = _kv_heads(q, k, v)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.attn_fwd_ref_rows_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, H_kv,
                                   N, d, int(bool(causal)), float(scale), _dtype_code(q),
                                   rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n,
                                   _dptr(o), _dptr(lse), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"attn_fwd_ref_rows failed with code {rc}")
    return o, lse


def attn_bwd_ref(q, k, v, dout, causal: bool, scale: float, error_scales: bool = False,
                 num_threads: int = 0):
    """Gradients (dq, dk, dv) of the forward definition for the incoming
    gradient dout, by the chain rule in fp64. q, dout: CPU [B,H,N,d];
    k, v: CPU [B,H_kv,N,d]; one dtype.

    With ``error_scales`` also returns (eq, ek, ev, zq, zk, zv): rounding p,
    ds and o to a type with rounding error u|x| + s/2 moves each gradient
    element by at most u e + (s/2) z to first order (see include/attn_ref.h).
    """
    lib = _load()
    q, k, v, dout = _as_host(q), _as_host(k), _as_host(v), _as_host(dout)
    B, H, N, d = q.shape
    H_kv = _kv_heads(q, k, v)
    if tuple(dout.shape) != tuple(q.shape) or dout.dtype != q.dtype:
        raise ValueError("oracle: dout must match q")
    outs = [np.empty((B, H, N, d)), np.empty((B, H_kv, N, d)), np.empty((B, H_kv, N, d))]
    errs = [np.empty_like(a) for a in outs + outs] if error_scales else [None] * 6
    ptr = lambda a: None if a is None else _dptr(a)   # noqa: E731
    rc = lib.attn_bwd_ref(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                          *(ptr(a) for a in outs), *(ptr(a) for a in errs),
                          B, H, H_kv, N, d, int(bool(causal)), float(scale),
                          _dtype_code(q), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"attn_bwd_ref failed with code {rc}")
    return tuple(outs) + (tuple(errs) if error_scales else ())


def decode(t) -> np.ndarray:
    """Widen a CPU tensor of f32/f16/bf16 to float64 via the oracle's decoder."""
    lib = _load()
    t = _as_host(t)
    out = np.empty(t.numel(), dtype=np.float64)
    rc = lib.attn_ref_decode(t.data_ptr(), _dptr(out), t.numel(), _dtype_code(t))
    if rc != 0:
        raise RuntimeError(f"attn_ref_decode failed with code {rc}")
    return out.reshape(tuple(t.shape))
