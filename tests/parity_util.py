"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
per-unit oracle references, and the error metric.

Error metric (per output tensor, over the elements compared):

    err = max_i max(|gpu_i - ref_i| - half_ulp(gpu_i), 0) / RMS(ref)

where half_ulp is half a unit in the last place of the format the output is
stored in (bf16: 8 significant bits, fp32: 24). Subtracting it removes the
rounding of the result to its own storage format, which no kernel can avoid:
a bf16 copy of the exact result already scores up to 2^-8 max|ref|/RMS(ref)
on the raw metric max|gpu - ref|/RMS(ref) (about 2.3e-2 on these workloads;
see test_metric.py). The raw figure is printed beside the gated one.
Gates: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
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


SIG_BITS = {"bf16": 8, "f32": 24}


def half_ulp(x, store):
    """Half a unit in the last place of |x| in the given storage format."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)  # ax = m * 2^e, m in [0.5, 1)
    h = np.ldexp(1.0, e - SIG_BITS[store] - 1)
    return np.where(ax == 0.0, 0.0, h)


def rel_err(gpu, ref, store="f32", ref_store=None):
    """(gated error, raw error), both normalised by RMS(ref)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    diff = np.abs(gpu - ref)
    slack = half_ulp(gpu, store)
    if ref_store is not None:
        slack = slack + half_ulp(ref, ref_store)
    adj = np.maximum(diff - slack, 0.0)
    if rms == 0.0:
        return (float(np.max(adj)) if adj.size else 0.0), (float(np.max(diff)) if diff.size else 0.0)
    return float(np.max(adj)) / rms, float(np.max(diff)) / rms


def assert_close(gpu, ref, tol, what, store="f32", ref_store=None):
    """Gate the error of GPU values stored in ``store`` against reference values
    (``ref_store`` when the reference is itself a rounded GPU output)."""
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    e, raw = rel_err(gpu, ref, store, ref_store)
    print(f"    {what}: err {e:.3e} (raw {raw:.3e}, gate {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: err / RMS = {e:.3e} > {tol:.1e} (raw {raw:.3e})"
    return e


def per_head_report(what, gpu_units, ref_units, store="f32"):
    """Print the error metric per head (diagnostic, no gate): the long-memory
    heads' outputs are many times larger than the short-memory heads', so the
    whole tensor's RMS hides how well the small heads are matched."""
    heads = sorted(set(h for (_, h) in gpu_units))
    parts = []
    for h in heads:
        us = [u for u in gpu_units if u[1] == h]
        g = np.concatenate([np.ravel(gpu_units[u]) for u in us])
        r = np.concatenate([np.ravel(ref_units[u]) for u in us])
        e, _ = rel_err(g, r, store)
        parts.append(f"h{h} {e:.2e}")
    print(f"    {what} per head (err / that head's RMS): " + ", ".join(parts), flush=True)


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
