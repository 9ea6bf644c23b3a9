"""Host sanitizer builds (CPU only, no GPU).

- The oracle's C source, built by gcc with AddressSanitizer and UndefinedBehaviorSanitizer, runs
  small cases of every oracle entry point (prefill, one unit, decode, conv-state update, the
  dense projections, the block, RMSNorm, MLP, the local attention block, the backward pass).
- The C-ABI library, built by hipcc with both sanitizers on the host pass only (device code is
  built as usual), runs the argument-validation paths of every entry point: the checks in
  tests/test_abi_cpu.py, all of which return before any HIP call.

Each runs in a subprocess with the sanitizer runtime preloaded (Python itself is not
instrumented); any sanitizer report fails the test.
"""
from __future__ import annotations

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from gated_linear_recurrence_amd import build as hipbuild  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(script: str, preload: str, timeout: int = 600):
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=ROOT + os.pathsep + os.path.join(ROOT, "tests"),
               **SAN_ENV)
    res = subprocess.run([sys.executable, "-c", textwrap.dedent(script)], capture_output=True,
                         text=True, env=env, timeout=timeout, cwd=ROOT)
    report = res.stdout[-3000:] + res.stderr[-6000:]
    assert res.returncode == 0, report
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in res.stderr, report
    return res.stdout


def _gcc_runtime(name: str) -> str:
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc %s not found" % name)
    return p


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    import oracle
    lib = str(tmp_path / "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-D_DEFAULT_SOURCE", oracle._SRC, "-o", lib, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = _run("""
        import numpy as np
        import oracle
        from gated_linear_recurrence_amd import synth
        oracle._lib = oracle.load(%r)
        for name, B, T in ((synth.TINY, 2, 70), (synth.PREFILL_2B, 1, 9)):
            w = synth.small(synth.WORKLOADS[name], B=B, T=T)
            p = synth.make_params(w, biases=True)
            x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
            P = oracle.Params(p["conv_w"], p["conv_b"], p["wa"], p["ba"], p["wx"], p["bx"],
                              p["lambda"], w.H)
            h0 = np.full((B, w.D), 0.25, np.float32)
            c0 = synth.make_conv0(w, B)
            out, hl, cl = oracle.prefill(P, x, y, h0=h0, conv0=c0)
            oracle.prefill_unit(P, x, y, B - 1, w.H - 1, T, h0, c0)
            win = oracle.widen_bf16(c0).astype(np.float64) if c0.dtype == np.uint16 else c0.astype(np.float64)
            hh = h0.astype(np.float64).copy()
            oracle.decode_step(P, x[:, 0], y[:, 0], hh, win)
            oracle.conv1d_state_update(p["conv_w"], p["conv_b"], x, win.copy())
        w = synth.Workload("san", 1, 5, 512, 2, synth.BF16, 0.9, 0.999, 0.0, 3)
        p = synth.make_params(w, biases=True)
        q = synth.make_proj(w, Dm=256, biases=True)
        P = oracle.Params(p["conv_w"], p["conv_b"], p["wa"], p["ba"], p["wx"], p["bx"], p["lambda"], w.H)
        Q = oracle.ProjParams(q["lx_w"], q["lx_b"], q["ly_w"], q["ly_b"], q["lo_w"], q["lo_b"])
        xin = synth.make_block_input(w, Dm=256)
        oracle.block_prefill(P, Q, xin)
        oracle.linear(xin[0], q["lx_w"], q["lx_b"])
        L = synth.make_layer(w, Dm=256, F=384, biases=True)
        oracle.rmsnorm(xin, L["norm_t"])
        M = oracle.MlpParams(L["gate_w"], L["gate_b"], L["up_w"], L["up_b"], L["down_w"], L["down_b"])
        oracle.mlp(M, xin)
        a = synth.make_attn(w, Dm=256, n_heads=2, bias=True)
        oracle.local_attention_block(xin, a["q_w"], a["k_w"], a["v_w"], a["o_w"], a["o_b"], 2, 4)
        wb = synth.Workload("sanb", 2, 64, 512, 2, synth.BF16, 0.9, 0.999, 0.0, 4)
        pb = synth.make_params(wb, biases=True)
        Pb = oracle.Params(pb["conv_w"], pb["conv_b"], pb["wa"], pb["ba"], pb["wx"], pb["bx"], pb["lambda"], wb.H)
        xb, yb = synth.make_act(wb, "x"), synth.make_act(wb, "y")
        dout = synth.make_act(wb, "y", seed=9)
        oracle.prefill_backward(Pb, xb, yb, dout)
        print("oracle ok")
    """ % lib, _gcc_runtime("libasan.so"))
    assert "oracle ok" in out


def test_library_host_code_under_address_and_ub_sanitizers(tmp_path):
    rt = "/opt/rocm/llvm/lib/clang"
    cands = []
    for root, _, files in os.walk(rt):
        cands += [os.path.join(root, f) for f in files if f == "libclang_rt.asan-x86_64.so"]
    if not cands or not os.path.exists(hipbuild.hipcc()):
        pytest.skip("hipcc or clang's AddressSanitizer runtime not found")
    lib = str(tmp_path / "librglru_san.so")
    flags = [f for f in hipbuild.HIPCC_FLAGS if f != "-O3"] + [
        "-O1", "-g", "-fno-omit-frame-pointer",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan"]
    cmd = [hipbuild.hipcc()] + flags + ["-I", os.path.join(ROOT, "include")] + \
        [os.path.join(hipbuild.CSRC, s) for s in hipbuild.SOURCES] + ["-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    out = _run("""
        import inspect
        from gated_linear_recurrence_amd import binding
        lib = binding.load_library(%r)
        import test_abi_cpu as t
        n = 0
        for name, fn in sorted(vars(t).items()):
            if name.startswith("test_") and list(inspect.signature(fn).parameters) == ["lib"]:
                fn(lib)
                n += 1
        print("abi checks", n)
    """ % lib, sorted(cands)[-1])
    assert "abi checks" in out and int(out.split("abi checks")[1].split()[0]) >= 10
