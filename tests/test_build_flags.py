"""The build keeps packed fp32 VALU forms (v_pk_fma_f32, v_pk_mul_f32,
v_pk_add_f32) out of every kernel: each HIP source is compiled to gfx950
assembly with the library's own flags, and none of those instructions may
appear. (hipcc emits them from ordinary float code unless the
packed-fp32-ops target feature is turned off, as the build does.) CPU only:
hipcc cross-compiles without a GPU."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_15_amd import build

PACKED_F32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")


def _asm(src):
    flags = [f for f in build.FLAGS if f != "-shared"]
    cmd = [build.HIPCC, *flags, "--cuda-device-only", "-S", "-I",
           os.path.join(build.ROOT, "include"), "-I", build.CSRC,
           os.path.join(build.CSRC, src), "-o", "-"]
    return subprocess.run(cmd, check=True, capture_output=True, text=True).stdout


def test_packed_fp32_feature_is_off_in_the_build_flags():
    joined = " ".join(build.FLAGS)
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in joined


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_no_packed_fp32_instruction_in_any_kernel():
    with ThreadPoolExecutor(max_workers=len(build.SOURCES)) as pool:
        asm = dict(zip(build.SOURCES, pool.map(_asm, build.SOURCES)))
    found = {src: len(PACKED_F32.findall(text)) for src, text in asm.items()}
    assert all(".amdgcn_target" in text or "amdgcn" in text for text in asm.values())
    assert not any(found.values()), found
