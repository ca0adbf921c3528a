"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
HIP library through its binding, compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

# max |gpu - oracle| / max |oracle| over an output tensor must not exceed this
# (the bar for bf16 q/k/v with an fp32 state).
TOL = 2e-3
# the kernels carry fp32 state products as bf16 hi + lo terms (about 2^-16
# relative); this tighter bound catches a lost lo term or a dropped factor,
# which would still pass TOL.
DESIGN_TOL = 2e-4


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t if dtype is None else t.to(dtype)


def qkv_torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_device(x: dict, qkv: str) -> dict:
    """Inputs from workloads.make_inputs (numpy) to device tensors."""
    dt = qkv_torch_dtype(qkv)
    d = {}
    for key in ("q", "k", "v"):
        d[key] = dev(x[key], dt)
    for key in ("a", "beta", "S0"):
        d[key] = dev(x[key])
    d["parent"] = dev(x["parent"])
    if "accepted" in x:
        d["accepted"] = dev(x["accepted"])
    if "pool" in x:
        d["pool"] = dev(x["pool"])
        d["slot"] = dev(x["slot"])
        d["queries"] = dev(x["queries"], dt)
    return d


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0)) if ref.size else 0.0


def check(name, gpu, ref, tol=TOL, design_tol=DESIGN_TOL, slices=None):
    """Assert the relative error of a whole output tensor is within tol and
    the design bound; with slices (a tuple of axes), also that of every slice
    those axes index (e.g. (0, 1) for [B, H, ...] states: every (sequence,
    head)), so that a small slice cannot hide behind a large one.  Returns the
    whole-tensor error."""
    g = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), name + ": non-finite values"
    e = rel_err(g, ref)
    print("%-28s rel err %.3e" % (name, e), flush=True)
    assert e <= tol, "%s: %.3e > %.1e" % (name, e, tol)
    assert e <= design_tol, "%s: %.3e above the design bound %.1e" % (name, e, design_tol)
    if slices:
        rest = [ax for ax in range(g.ndim) if ax not in slices]
        n = int(np.prod([g.shape[ax] for ax in slices]))
        gs = np.transpose(g, list(slices) + rest).reshape(n, -1)
        rs = np.transpose(ref, list(slices) + rest).reshape(n, -1)
        worst = max(rel_err(a, b) for a, b in zip(gs, rs))
        assert worst <= design_tol, "%s: a slice at %.3e above the design bound %.1e" % (name, worst, design_tol)
    return e


def check_logp(name, gpu, ref):
    """log P from the library against the oracle's fp64 log of the gate
    products.  The library clamps each log a at -126 ln 2 = -87.34 (so a
    zero gate stays finite); where the oracle's value is -inf (a zero gate on
    the path) the library's must be at or below -87, elsewhere they must agree
    to the design bound."""
    g = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.all(g[~fin] <= -87.0), name + ": a zero gate above the clamp"
    if np.any(fin):
        e = rel_err(g[fin], ref[fin])
        print("%-28s rel err %.3e" % (name, e), flush=True)
        assert e <= 1e-5, "%s: %.3e" % (name, e)
