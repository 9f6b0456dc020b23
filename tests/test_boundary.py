"""C-ABI boundary checks that need no GPU.

* Both shared libraries load and export every function their header in
  include/ declares.
* attn_fwd rejects bad arguments with the documented codes. Validation runs
  before any HIP call, so these calls never touch a device.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared_functions(header):
    text = open(os.path.join(INCLUDE, header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def _exported(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], check=True,
                         capture_output=True, text=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


@pytest.fixture(scope="module")
def attn_lib_path():
    import exact_attention_15_amd as ea
    if not os.path.exists(ea.LIB_PATH):
        from exact_attention_15_amd.build import build_library
        build_library()
    return ea.LIB_PATH


def test_every_header_is_covered():
    headers = sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h"))
    assert headers == ["attn.h", "attn_ref.h"]


def test_attn_library_exports_header(attn_lib_path):
    decl = _declared_functions("attn.h")
    assert decl == ["attn_bwd", "attn_bwd_noalloc", "attn_debug_set_fwd_first_pass",
                    "attn_debug_set_fwd_variant", "attn_fwd", "attn_fwd_gqa", "attn_fwd_unfused",
                    "attn_strerror", "attn_unfused_workspace_bytes"]
    missing = set(decl) - _exported(attn_lib_path)
    assert not missing, missing
    ctypes.CDLL(attn_lib_path)   # loads without a GPU


def test_probe_build_exports_the_same_entry_points(attn_lib_path):
    """The race-check build (timing probes compiled in) is the same library:
    the same exported functions, loadable without a GPU."""
    from exact_attention_15_amd.build import PROBE_LIB_PATH, build_library
    if not os.path.exists(PROBE_LIB_PATH):
        build_library()
    assert _exported(PROBE_LIB_PATH) == _exported(attn_lib_path)
    ctypes.CDLL(PROBE_LIB_PATH)


def test_oracle_library_exports_header(oracle_lib):
    decl = _declared_functions("attn_ref.h")
    assert decl == ["attn_bwd_ref", "attn_fwd_ref", "attn_fwd_ref_gqa", "attn_fwd_ref_rows",
                    "attn_fwd_ref_rows_gqa", "attn_ref_decode"]
    missing = set(decl) - _exported(oracle_lib.LIB_PATH)
    assert not missing, missing


def test_libraries_share_no_symbols(attn_lib_path, oracle_lib):
    """The GPU library neither contains nor imports the oracle."""
    gpu = _exported(attn_lib_path)
    assert not any(s.startswith("attn_fwd_ref") or s.startswith("attn_ref") for s in gpu)
    undef = subprocess.run(["nm", "-D", "--undefined-only", attn_lib_path], check=True,
                           capture_output=True, text=True).stdout
    assert "attn_fwd_ref" not in undef
    needed = subprocess.run(["readelf", "-d", attn_lib_path], check=True,
                            capture_output=True, text=True).stdout
    assert "oracle" not in needed


def test_debug_variant_switch(attn_lib_path):
    """attn_debug_set_fwd_variant takes 0..2 for each argument (no HIP
    call), rejects anything else without changing the setting, and the
    automatic choice can always be restored."""
    import exact_attention_15_amd as ea
    lib = ea.load_library()
    for qb, order in ((0, 0), (1, 2), (2, 1), (0, 0)):
        assert lib.attn_debug_set_fwd_variant(qb, order) == ea.ATTN_OK
    for qb, order in ((3, 0), (-1, 0), (0, 3), (0, -1)):
        assert lib.attn_debug_set_fwd_variant(qb, order) == ea.ATTN_EINVAL
    with pytest.raises(ea.AttnError):
        ea.debug_set_fwd_variant(5, 0)
    ea.debug_set_fwd_variant()


def test_debug_first_pass_switch(attn_lib_path):
    """attn_debug_set_fwd_first_pass takes 0..2 (no HIP call) and returns
    ATTN_EINVAL for anything else; the wrapper raises on it."""
    import exact_attention_15_amd as ea
    lib = ea.load_library()
    for mode in (0, 1, 2, 0):
        assert lib.attn_debug_set_fwd_first_pass(mode) == ea.ATTN_OK
    for mode in (3, -1):
        assert lib.attn_debug_set_fwd_first_pass(mode) == ea.ATTN_EINVAL
    with pytest.raises(ea.AttnError):
        ea.debug_set_fwd_first_pass(7)
    ea.debug_set_fwd_first_pass()


def test_strerror(attn_lib_path):
    import exact_attention_15_amd as ea
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(ea.strerror(code), str) and ea.strerror(code)


def test_argument_validation(attn_lib_path):
    """Every rejected argument returns its code before any HIP call."""
    import exact_attention_15_amd as ea
    # Fake, aligned "device" addresses: they are never dereferenced because
    # each call below fails validation first.
    P = 0x7f0000000000
    good = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, lse=P + 0x4000,
                B=1, H=2, N=128, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16, stream=None)
    cases = [
        (dict(q=None), ea.ATTN_EINVAL),
        (dict(k=None), ea.ATTN_EINVAL),
        (dict(v=None), ea.ATTN_EINVAL),
        (dict(o=None), ea.ATTN_EINVAL),
        (dict(lse=None), ea.ATTN_EINVAL),
        (dict(B=0), ea.ATTN_EINVAL),
        (dict(H=-1), ea.ATTN_EINVAL),
        (dict(N=0), ea.ATTN_EINVAL),
        (dict(N=2 ** 40), ea.ATTN_EINVAL),
        (dict(causal=2), ea.ATTN_EINVAL),
        (dict(scale=0.0), ea.ATTN_EINVAL),
        (dict(scale=-1.0), ea.ATTN_EINVAL),
        (dict(scale=float("inf")), ea.ATTN_EINVAL),
        (dict(scale=float("nan")), ea.ATTN_EINVAL),
        (dict(dtype=3), ea.ATTN_EINVAL),
        (dict(d=32), ea.ATTN_EUNSUPPORTED),
        (dict(d=96), ea.ATTN_EUNSUPPORTED),
        (dict(q=P + 8), ea.ATTN_EALIGN),
        (dict(o=P + 0x3002), ea.ATTN_EALIGN),
        (dict(lse=P + 0x4002), ea.ATTN_EALIGN),
    ]
    for change, want in cases:
        a = dict(good, **change)
        rc = ea.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                         a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])
        assert rc == want, (change, rc)
        # The grouped-query entry point with H_kv = H validates identically.
        rc = ea.attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                             a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"],
                             a["stream"])
        assert rc == want, ("gqa", change, rc)
    # K/V head counts that do not divide H (or are not positive) are refused.
    for H, H_kv in [(2, 0), (2, -2), (6, 4), (4, 3), (1, 2), (8, 16)]:
        a = dict(good, H=H)
        rc = ea.attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], H, H_kv,
                             a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])
        assert rc == ea.ATTN_EINVAL, (H, H_kv, rc)


def test_bwd_argument_validation(attn_lib_path):
    """attn_bwd: the forward's checks plus its own pointers, dtype and
    alignment, all before any HIP call."""
    import exact_attention_15_amd as ea
    P = 0x7f0000000000
    good = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, lse=P + 0x4000, dout=P + 0x5000,
                dq=P + 0x6000, dk=P + 0x7000, dv=P + 0x8000, delta=P + 0x9000,
                B=1, H=4, H_kv=2, N=128, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16,
                stream=None)
    cases = [
        (dict(q=None), ea.ATTN_EINVAL),
        (dict(o=None), ea.ATTN_EINVAL),
        (dict(lse=None), ea.ATTN_EINVAL),
        (dict(dout=None), ea.ATTN_EINVAL),
        (dict(dq=None), ea.ATTN_EINVAL),
        (dict(dk=None), ea.ATTN_EINVAL),
        (dict(dv=None), ea.ATTN_EINVAL),
        (dict(delta=None), ea.ATTN_EINVAL),
        (dict(H_kv=3), ea.ATTN_EINVAL),
        (dict(H_kv=0), ea.ATTN_EINVAL),
        (dict(N=0), ea.ATTN_EINVAL),
        (dict(causal=-1), ea.ATTN_EINVAL),
        (dict(scale=float("nan")), ea.ATTN_EINVAL),
        (dict(dtype=5), ea.ATTN_EINVAL),
        (dict(d=96), ea.ATTN_EUNSUPPORTED),
        (dict(dout=P + 0x5008), ea.ATTN_EALIGN),
        (dict(dq=P + 0x6004), ea.ATTN_EALIGN),
        (dict(dk=P + 0x7002), ea.ATTN_EALIGN),
        (dict(dv=P + 0x8008), ea.ATTN_EALIGN),
        (dict(delta=P + 0x9002), ea.ATTN_EALIGN),
    ]
    names = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta", "B", "H", "H_kv",
             "N", "d", "causal", "scale", "dtype", "stream"]
    for change, want in cases:
        a = dict(good, **change)
        rc = ea.attn_bwd(*(a[n] for n in names))
        assert rc == want, (change, rc)


def test_bwd_noalloc_argument_validation(attn_lib_path):
    """attn_bwd_noalloc: attn_bwd's checks (no delta argument) and the size
    limit of its static row-statistic array, all before any HIP call (the
    pointers here are never dereferenced)."""
    import exact_attention_15_amd as ea
    P = 0x7f0000000000
    good = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, lse=P + 0x4000, dout=P + 0x5000,
                dq=P + 0x6000, dk=P + 0x7000, dv=P + 0x8000,
                B=1, H=4, H_kv=2, N=128, d=64, causal=1, scale=0.125, dtype=ea.ATTN_BF16,
                stream=None)
    limit = ea.BWD_NOALLOC_MAX_ROWS
    cases = [
        (dict(q=None), ea.ATTN_EINVAL),
        (dict(lse=None), ea.ATTN_EINVAL),
        (dict(dout=None), ea.ATTN_EINVAL),
        (dict(dv=None), ea.ATTN_EINVAL),
        (dict(H_kv=3), ea.ATTN_EINVAL),
        (dict(N=0), ea.ATTN_EINVAL),
        (dict(dtype=5), ea.ATTN_EINVAL),
        (dict(d=96), ea.ATTN_EUNSUPPORTED),
        (dict(dq=P + 0x6004), ea.ATTN_EALIGN),
        (dict(B=1, H=1, H_kv=1, N=limit + 1), ea.ATTN_ETOOBIG),
        (dict(B=2, H=2, H_kv=2, N=limit // 4 + 1), ea.ATTN_ETOOBIG),
        (dict(B=65, H=65536, H_kv=65536, N=1), ea.ATTN_ETOOBIG),
        # an invalid argument is reported before the size limit
        (dict(B=1, H=1, H_kv=1, N=limit + 1, dtype=7), ea.ATTN_EINVAL),
    ]
    names = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "B", "H", "H_kv",
             "N", "d", "causal", "scale", "dtype", "stream"]
    for change, want in cases:
        a = dict(good, **change)
        rc = ea.attn_bwd_noalloc(*(a[n] for n in names))
        assert rc == want, (change, rc)
    assert "ATTN_BWD_NOALLOC_MAX_ROWS" in ea.strerror(ea.ATTN_ETOOBIG)


def test_unfused_workspace_and_validation(attn_lib_path):
    import exact_attention_15_amd as ea
    BF, F16, F32 = ea.ATTN_BF16, ea.ATTN_F16, ea.ATTN_F32
    assert ea.unfused_workspace_bytes(1, 1, 1, BF) == 64 * 6
    assert ea.unfused_workspace_bytes(2, 3, 100, F16) == 2 * 3 * 100 * 128 * 6
    assert ea.unfused_workspace_bytes(4, 16, 4096, BF) == 4 * 16 * 4096 * 4096 * 6
    # fp32 keeps the probabilities in fp32: 4 + 4 bytes per score.
    assert ea.unfused_workspace_bytes(1, 1, 1, F32) == 64 * 8
    assert ea.unfused_workspace_bytes(2, 3, 100, F32) == 2 * 3 * 100 * 128 * 8
    for bad in [(0, 1, 1, BF), (1, -1, 4, BF), (1, 1, 0, F32), (1, 1, 4, 7)]:
        assert ea.unfused_workspace_bytes(*bad) == -1
    P = 0x7f0000000000
    need = ea.unfused_workspace_bytes(1, 2, 128, BF)
    good = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, lse=P + 0x4000,
                ws=P + 0x10000, wsb=need, B=1, H=2, N=128, d=64, causal=1, scale=0.125,
                dtype=ea.ATTN_BF16, stream=None)
    cases = [
        (dict(ws=None), ea.ATTN_EINVAL),
        (dict(wsb=need - 1), ea.ATTN_EINVAL),
        (dict(q=None), ea.ATTN_EINVAL),
        (dict(N=0), ea.ATTN_EINVAL),
        (dict(causal=3), ea.ATTN_EINVAL),
        (dict(dtype=ea.ATTN_F32), ea.ATTN_EINVAL),   # fp32 needs 8 bytes per score
        (dict(dtype=ea.ATTN_F32, wsb=ea.unfused_workspace_bytes(1, 2, 128, F32),
              d=96), ea.ATTN_EUNSUPPORTED),
        (dict(dtype=9), ea.ATTN_EINVAL),
        (dict(d=32), ea.ATTN_EUNSUPPORTED),
        (dict(ws=P + 0x10080), ea.ATTN_EALIGN),
        (dict(o=P + 0x3008), ea.ATTN_EALIGN),
    ]
    names = ["q", "k", "v", "o", "lse", "ws", "wsb", "B", "H", "N", "d", "causal", "scale",
             "dtype", "stream"]
    for change, want in cases:
        a = dict(good, **change)
        rc = ea.attn_fwd_unfused(*(a[n] for n in names))
        assert rc == want, (change, rc)


def test_python_wrapper_checks(attn_lib_path):
    import torch
    import exact_attention_15_amd as ea
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        ea.fwd(q, q, q)   # host tensors are refused before any call
    q4 = torch.zeros(1, 4, 8, 64)
    with pytest.raises(ValueError):
        ea.fwd(q4, q4[:, :3], q4[:, :3])   # 3 K/V heads do not divide 4
    with pytest.raises(ValueError):
        ea.fwd(q4, q4[:, :2], q4[:, :1])   # k and v differ
    with pytest.raises(TypeError):
        ea.dtype_code(torch.float64)
    assert ea.default_scale(64) == 0.125
    assert abs(ea.default_scale(128) - 128 ** -0.5) < 1e-8
