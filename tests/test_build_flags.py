"""The device code is built without packed-fp32 instructions (v_pk_fma_f32, v_pk_mul_f32,
v_pk_add_f32): the build passes the target feature "-packed-fp32-ops" to the device compiler.
(hipcc's host pass warns that it does not know the feature; the device pass honours it.)

A probe kernel whose float2 FMA the compiler turns into v_pk_fma_f32 by default shows that the
check can see such instructions; then every library source is compiled to device assembly with
the build's own flags and must contain none.  CPU only (hipcc cross-compiles for gfx950)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from gated_linear_recurrence_amd import build

PK_F32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")
PROBE = r"""
#include <hip/hip_runtime.h>
__global__ void probe(float2* a, const float2* b, const float2* c, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        float2 x = a[i], y = b[i], z = c[i];
        x.x = x.x * y.x + z.x;
        x.y = x.y * y.y + z.y;
        a[i] = x;
    }
}
"""

pytestmark = pytest.mark.skipif(not os.path.exists(build.hipcc()), reason="hipcc not found")


def _device_flags(with_guard: bool):
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    if not with_guard:
        out, skip = [], 0
        for i, f in enumerate(flags):
            if skip:
                skip -= 1
                continue
            if f == "-Xclang" and i + 1 < len(flags) and flags[i + 1] == "-target-feature":
                skip = 3  # -Xclang -target-feature -Xclang -packed-fp32-ops
                continue
            out.append(f)
        flags = out
    return flags


def _asm(src: str, flags, tmp_path, tag: str) -> str:
    out = os.path.join(str(tmp_path), tag + ".s")
    cmd = [build.hipcc()] + flags + ["--cuda-device-only", "-S", "-I",
                                      os.path.join(build.ROOT, "include"), src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


def test_guard_flag_is_in_the_build():
    assert "-packed-fp32-ops" in build.HIPCC_FLAGS


def test_probe_shows_the_guard_works(tmp_path):
    src = os.path.join(str(tmp_path), "probe.hip")
    with open(src, "w") as f:
        f.write(PROBE)
    assert PK_F32.search(_asm(src, _device_flags(False), tmp_path, "probe_default")), \
        "the probe no longer produces a packed fp32 instruction: it cannot test the guard"
    assert not PK_F32.search(_asm(src, _device_flags(True), tmp_path, "probe_guarded"))


def test_library_device_code_has_no_packed_fp32(tmp_path):
    flags = _device_flags(True)
    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 4)) as ex:
        asms = list(ex.map(lambda s: (s, _asm(s, flags, tmp_path, os.path.basename(s))), srcs))
    bad = [(os.path.basename(s), m.group(0)) for s, a in asms for m in [PK_F32.search(a)] if m]
    assert not bad, bad
