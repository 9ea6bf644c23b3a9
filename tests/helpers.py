"""Shared helpers for the GPU tests: moving storage-form numpy arrays to and from the device,
building library parameters, and comparing with the oracle (no arithmetic of the method)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gated_linear_recurrence_amd import synth  # noqa: E402

TOL = {synth.F32: 1e-5, synth.BF16: 2e-2}   # rel-L2 bars for fp32 and bf16 storage


def torch_dtype(storage: str):
    import torch
    return torch.bfloat16 if storage == synth.BF16 else torch.float32


def to_dev(a: np.ndarray | None, device="cuda"):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t) -> np.ndarray:
    """Device tensor -> storage-form numpy array (bf16 as uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def wide(a: np.ndarray) -> np.ndarray:
    return oracle.widen_bf16(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def dev_params(p: dict, H: int, device="cuda"):
    from gated_linear_recurrence_amd import binding
    t = {k: to_dev(v, device) for k, v in p.items()}
    return binding.Params(t["conv_w"], t["conv_b"], t["wa"], t["ba"], t["wx"], t["bx"], t["lambda"])


def oracle_params(p: dict, H: int):
    return oracle.Params(p["conv_w"], p["conv_b"], p["wa"], p["ba"], p["wx"], p["bx"], p["lambda"], H)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    return num / den if den > 0 else num


def oracle_units(P, x, y, units, t_use, h0=None, conv0=None, threads=16):
    """Run oracle.prefill_unit for several (b, head) units in parallel threads."""
    lib = oracle.load()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {u: ex.submit(oracle.prefill_unit, P, x, y, u[0], u[1], t_use, h0, conv0, lib)
                for u in units}
        return {u: f.result() for u, f in futs.items()}
