"""Checks on the gfx950 code of every kernel, compiled on the CPU with the
library's own flags (hipcc cross-compiles without a GPU):
* no packed fp32 VALU form (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32):
  hipcc emits them from ordinary float code unless the packed-fp32-ops
  target feature is turned off, as the build does;
* no register spills (scratch memory per lane) in any kernel, except the
  stack frame of the d = 64 16-bit forward's call into its exact pass, whose
  scratch instructions must all sit in the one block that makes the call;
* no forward kernel asks for the dispatch pointer or the y and z work-item
  ids (what the exact-pass call pulls in when its arguments stop fitting
  in registers)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_15_amd import build

PACKED_F32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")


# Kernels allowed to use scratch (bytes per lane), by mangled-name fragment:
# none.
SCRATCH_ALLOWED = {}


def _compile(src):
    """(assembly, {kernel: scratch bytes per lane}) of one source."""
    flags = [f for f in build.FLAGS if f != "-shared"]
    cmd = [build.HIPCC, *flags, "--cuda-device-only", "-S",
           "-Rpass-analysis=kernel-resource-usage", "-I",
           os.path.join(build.ROOT, "include"), "-I", build.CSRC,
           os.path.join(build.CSRC, src), "-o", "-"]
    r = subprocess.run(cmd, check=True, capture_output=True, text=True)
    scratch, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            scratch[name] = int(m.group(1))
        m = re.search(r"\b([VA])GPRs: (\d+)", line)
        if m and name:
            REGS.setdefault(name, {})[m.group(1)] = int(m.group(2))
    return r.stdout, scratch


REGS = {}   # kernel -> {"V": VGPRs, "A": AGPRs}, filled by _compile


@pytest.fixture(scope="module")
def compiled():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not installed")
    with ThreadPoolExecutor(max_workers=len(build.SOURCES)) as pool:
        return dict(zip(build.SOURCES, pool.map(_compile, build.SOURCES)))


def test_packed_fp32_feature_is_off_in_the_build_flags():
    joined = " ".join(build.FLAGS)
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in joined


def test_no_packed_fp32_instruction_in_any_kernel(compiled):
    found = {src: len(PACKED_F32.findall(asm)) for src, (asm, _) in compiled.items()}
    assert all("amdgcn" in asm for asm, _ in compiled.values())
    assert not any(found.values()), found


# The d = 64 16-bit forward kernels with the first pass (last template
# argument true) call their exact pass (a function of its own) in the rare
# case: the call's frame is scratch, but nothing outside the calling block
# may touch it.
CALLS_EXACT_PASS = re.compile(r"fwd16_kernelILb[01]ELi64ELb[01]ELi[12]ELb1E")


def _function_asm(asm, name):
    start = asm.index(f"\n{name}:")
    return asm[start:asm.index(".Lfunc_end", start)]


def _blocks(fn_asm):
    """Basic blocks of one function's assembly, split at labels."""
    return re.split(r"\n(?=\.LBB\d+_\d+:)", fn_asm)


def test_no_register_spills(compiled):
    kernels = {k: v for _, (_, sc) in compiled.items() for k, v in sc.items()}
    assert len(kernels) >= 30, sorted(kernels)   # every instantiation was seen
    over = {}
    for k, v in kernels.items():
        allowed = next((a for frag, a in SCRATCH_ALLOWED.items() if frag in k), 0)
        if v > allowed and not CALLS_EXACT_PASS.search(k):
            over[k] = v
    assert not over, over


def test_scratch_only_around_the_exact_pass_call(compiled):
    """In the kernels that call the exact pass, every scratch access is in
    the block that makes the call (saves and reloads around it): the main
    path, the tile loop included, spills nothing."""
    asm = compiled["fwd_mfma16.hip"][0]
    names = [k for k in compiled["fwd_mfma16.hip"][1] if CALLS_EXACT_PASS.search(k)]
    assert len(names) == 8, names
    for name in names:
        blocks = _blocks(_function_asm(asm, name))
        calls = [b for b in blocks if "s_swappc_b64" in b]
        assert len(calls) == 1, name
        stray = [b.split("\n", 1)[0] for b in blocks
                 if re.search(r"\bscratch_(load|store)", b) and "s_swappc_b64" not in b]
        assert not stray, (name, stray)


def test_exact_pass_call_takes_no_implicit_inputs(compiled):
    """The call into the exact pass gets its parameters in registers: no
    kernel asks for the dispatch pointer or the y and z work-item ids. A
    kernel parameter struct one word longer made the compiler pass those to
    the callee and hold a per-lane value through the tile loop, 6.7 %
    slower at B4 H16 N4096 d64 causal."""
    asm = compiled["fwd_mfma16.hip"][0]
    descriptors = re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S)
    assert len(descriptors) >= 20
    wide = {name: (re.search(r"dispatch_ptr (\d)", body).group(1),
                   re.search(r"workitem_id (\d)", body).group(1))
            for name, body in descriptors}
    wide = {k: v for k, v in wide.items() if v != ("0", "0")}
    assert not wide, wide


def _waves_per_simd(regs):
    """Waves of one kernel a SIMD holds: 512 registers per lane, VGPRs and
    AGPRs together, allocated in granules of 8."""
    used = regs.get("V", 0) + regs.get("A", 0)
    return 512 // (-(-used // 8) * 8)


def test_dkdv_residency_matches_the_plan(compiled):
    """The backward's work plan (bwd_chunks.h, one_group_per_cu) counts
    three one-group dK/dV workgroups per compute unit at d = 64 and two at
    d = 128; the compiler's register counts must give exactly that."""
    seen = {64: [], 128: []}
    for k, regs in REGS.items():
        m = re.search(r"bwd_dkdv_kernelILb[01]ELi(64|128)ELb[01]ELi1E", k)
        if m:
            seen[int(m.group(1))].append(_waves_per_simd(regs))
    assert len(seen[64]) == 4 and len(seen[128]) == 4, seen
    assert set(seen[64]) == {3} and set(seen[128]) == {2}, seen
