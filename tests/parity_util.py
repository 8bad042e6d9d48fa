"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
per-unit oracle references, and the error metric.

Error metric (per output tensor): max |gpu - oracle| / RMS(oracle), over the
elements compared. Gates: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from chunked_gated_linear_simple_amd import inputs as I

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(x, dtype=None):
    """numpy storage array -> cuda tensor (bf16 from uint16 bits)."""
    if x is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(gpu))) if gpu.size else 0.0
    return float(np.max(np.abs(gpu - ref))) / rms


def assert_close(gpu, ref, tol, what):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    e = rel_err(gpu, ref)
    print(f"    {what}: err {e:.3e} (gate {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: max err / RMS = {e:.3e} > {tol:.1e}"
    return e


def schedule32(H, t_min, t_max):
    """fp32 decays from the oracle's schedule (fed to both sides)."""
    return oracle.decay_schedule(H, t_min, t_max).astype(np.float32)


def unit_view(inp, name, n, h, cu=None):
    """float64 slice of one (sequence, head) unit of a token-major input."""
    x = inp[name]
    if cu is None:
        sl = x[n, h]
    else:
        sl = x[0, h, int(cu[n]):int(cu[n + 1])]
    return I.widen(sl, inp["dtype"])


def oracle_fwd_units(inp, lam, units, cu=None):
    out = {}
    for (n, h) in units:
        q = unit_view(inp, "q", n, h, cu)
        k = unit_view(inp, "k", n, h, cu)
        v = unit_view(inp, "v", n, h, cu)
        S0 = None if inp["S0"] is None else inp["S0"][n, h].astype(np.float64)
        out[(n, h)] = oracle.fwd_unit(q, k, v, float(lam[h]), inp["a"][h].astype(np.float64), S0)
    return out


def oracle_bwd_units(inp, lam, units, cu=None):
    out = {}
    for (n, h) in units:
        q = unit_view(inp, "q", n, h, cu)
        k = unit_view(inp, "k", n, h, cu)
        v = unit_view(inp, "v", n, h, cu)
        dO = unit_view(inp, "dO", n, h, cu)
        S0 = None if inp["S0"] is None else inp["S0"][n, h].astype(np.float64)
        dSf = None if inp.get("dSf") is None else inp["dSf"][n, h].astype(np.float64)
        out[(n, h)] = oracle.bwd_unit(q, k, v, dO, float(lam[h]), inp["a"][h].astype(np.float64),
                                      S0, dSf)
    return out


def gpu_unit(t_host, n, h, cu=None):
    """Slice one unit out of a host copy of a token-major GPU output."""
    if cu is None:
        return t_host[n, h]
    return t_host[0, h, int(cu[n]):int(cu[n + 1])]


def device_inputs(inp, cu=None):
    dt = inp["dtype"]
    d = {
        "q": to_dev(inp["q"], dt), "k": to_dev(inp["k"], dt), "v": to_dev(inp["v"], dt),
        "a": to_dev(inp["a"]), "S0": to_dev(inp["S0"]),
        "cu": None if cu is None else to_dev(np.asarray(cu, dtype=np.int32)),
    }
    if "dO" in inp:
        d["dO"] = to_dev(inp["dO"], dt)
        d["dSf"] = to_dev(inp.get("dSf"))
    return d
