"""GPU parity with a = NULL, the default of every mixer entry point.

aug_balance is learned and starts at zero ("GLA mixer"), so a NULL `a` is the
first thing a real caller passes. The library then takes z = 0 and the
kernels run their NULL branches (no gate table is loaded). These tests call
sgla_chunk_fwd, sgla_chunk_bwd (with da), their segmented variants and
sgla_decode_step with a = None, and compare every output against the oracle
given a = None (whose NULL path is pinned to finite differences at a = 0).
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, device_inputs, schedule32, to_dev, to_host64, unit_view

pytestmark = pytest.mark.gpu


def _ref_fwd(inp, lam, n, h):
    S0 = None if inp["S0"] is None else inp["S0"][n, h].astype(np.float64)
    return oracle.fwd_unit(unit_view(inp, "q", n, h), unit_view(inp, "k", n, h), unit_view(inp, "v", n, h),
                           float(lam[h]), None, S0)


def _ref_bwd(inp, lam, n, h):
    S0 = None if inp["S0"] is None else inp["S0"][n, h].astype(np.float64)
    dSf = None if inp.get("dSf") is None else inp["dSf"][n, h].astype(np.float64)
    return oracle.bwd_unit(unit_view(inp, "q", n, h), unit_view(inp, "k", n, h), unit_view(inp, "v", n, h),
                           unit_view(inp, "dO", n, h), float(lam[h]), None, S0, dSf)


def _check_fwd(inp, lam, o, Sf):
    units = [(n, h) for n in range(inp["N"]) for h in range(inp["H"])]
    ref = {u: _ref_fwd(inp, lam, *u) for u in units}
    oh, Sh = to_host64(o), to_host64(Sf)
    tol = TOL[inp["dtype"]]
    assert_close(np.concatenate([oh[u].ravel() for u in units]),
                 np.concatenate([ref[u][0].ravel() for u in units]), tol, "o (a=NULL)", store=inp["dtype"])
    assert_close(np.concatenate([Sh[u].ravel() for u in units]),
                 np.concatenate([ref[u][1].ravel() for u in units]), tol, "final_state (a=NULL)")


def _check_bwd(inp, lam, grads):
    dq, dk, dv, da, dS0 = grads
    units = [(n, h) for n in range(inp["N"]) for h in range(inp["H"])]
    ref = {u: _ref_bwd(inp, lam, *u) for u in units}
    tol = TOL[inp["dtype"]]
    for idx, (nm, t) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        th = to_host64(t)
        assert_close(np.concatenate([th[u].ravel() for u in units]),
                     np.concatenate([ref[u][idx].ravel() for u in units]), tol, f"{nm} (a=NULL)",
                     store=inp["dtype"])
    da_ref = np.zeros((inp["H"], inp["d_k"]))
    for (n, h) in units:
        da_ref[h] += ref[(n, h)][3]
    # sigmoid'(0) = 1/4: the gradient at a = 0 is not zero
    assert np.max(np.abs(da_ref)) > 1e-2
    assert_close(to_host64(da), da_ref, tol, "da (a=NULL)")
    dsh = to_host64(dS0)
    assert_close(np.concatenate([dsh[u].ravel() for u in units]),
                 np.concatenate([ref[u][4].ravel() for u in units]), tol, "d_init_state (a=NULL)")


@pytest.mark.parametrize("dtype,H,T,dk,dv", [("bf16", 16, 300, 96, 192), ("f32", 2, 150, 16, 32)])
def test_fwd_bwd_a_null(dtype, H, T, dk, dv):
    inp = I.chunk_inputs(2, H, T, dk, dv, dtype, seed=150, a_std=None, s0_std=0.02, with_grad=True,
                         dsf_std=0.02)
    lam = schedule32(H, 1.0, 2048.0)
    d = device_inputs(inp)
    lam_d = to_dev(lam)
    chunk = 128 if dtype == "bf16" else 64
    o, Sf = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam_d, None, init_state=d["S0"], chunk=chunk,
                              want_final=True)
    grads = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam_d, None, init_state=d["S0"],
                              d_final_state=d["dSf"], chunk=chunk, want_d_init=True)
    torch.cuda.synchronize()
    _check_fwd(inp, lam, o, Sf)
    _check_bwd(inp, lam, grads)
    # an explicit zero a gives the same result bit for bit
    o0, S0f = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam_d, torch.zeros_like(d["a"]),
                                init_state=d["S0"], chunk=chunk, want_final=True)
    g0 = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam_d, torch.zeros_like(d["a"]),
                           init_state=d["S0"], d_final_state=d["dSf"], chunk=chunk, want_d_init=True)
    for x, y in [(o, o0), (Sf, S0f)] + list(zip(grads, g0)):
        assert torch.equal(x, y)


def test_varlen_a_null():
    L = [130, 0, 1, 257]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 4, int(cu[-1]), 96, 192, "bf16", seed=151, a_std=None, s0_std=0.02,
                         n_seq=len(L), with_grad=True, dsf_std=0.02)
    lam = schedule32(4, 1.0, 2048.0)
    d = device_inputs(inp, cu)
    lam_d = to_dev(lam)
    o, Sf = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam_d, None, init_state=d["S0"],
                              cu_seqlens=d["cu"], want_final=True)
    grads = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam_d, None, init_state=d["S0"],
                              d_final_state=d["dSf"], cu_seqlens=d["cu"], want_d_init=True)
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    host = {"o": to_host64(o), "final_state": to_host64(Sf), "dq": to_host64(grads[0]),
            "dk": to_host64(grads[1]), "dv": to_host64(grads[2]), "d_init_state": to_host64(grads[4])}
    got = {nm: [] for nm in host}
    want = {nm: [] for nm in host}
    da_ref = np.zeros((4, 96))
    for n in range(len(L)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        for h in range(4):
            q, k, v, dO = (I.widen(inp[x][0, h, sl], "bf16") for x in ("q", "k", "v", "dO"))
            S0 = inp["S0"][n, h].astype(np.float64)
            dSf = inp["dSf"][n, h].astype(np.float64)
            of, sf = oracle.fwd_unit(q, k, v, float(lam[h]), None, S0)
            r = oracle.bwd_unit(q, k, v, dO, float(lam[h]), None, S0, dSf)
            for nm, ref in (("o", of), ("dq", r[0]), ("dk", r[1]), ("dv", r[2])):
                got[nm].append(host[nm][0, h, sl].ravel())
                want[nm].append(ref.ravel())
            got["final_state"].append(host["final_state"][n, h].ravel())
            want["final_state"].append(sf.ravel())
            got["d_init_state"].append(host["d_init_state"][n, h].ravel())
            want["d_init_state"].append(r[4].ravel())
            da_ref[h] += r[3]
    # the metric is per output tensor (every unit of it at once)
    for nm in host:
        store = "bf16" if nm in ("o", "dq", "dk", "dv") else "f32"
        assert_close(np.concatenate(got[nm]), np.concatenate(want[nm]), tol, f"{nm} (a=NULL, packed)",
                     store=store)
    assert_close(to_host64(grads[3]), da_ref, tol, "da (a=NULL, packed)")


def test_segmented_a_null():
    inp = I.chunk_inputs(1, 16, 640, 96, 192, "bf16", seed=152, a_std=None, s0_std=0.02, with_grad=True,
                         dsf_std=0.02)
    lam = schedule32(16, 1.0, 2048.0)
    d = device_inputs(inp)
    lam_d = to_dev(lam)
    o, Sf = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, None, init_state=d["S0"],
                                        n_segments=3, want_final=True)
    grads = Bd.sgla_chunk_bwd_segmented(d["q"], d["k"], d["v"], d["dO"], lam_d, None, init_state=d["S0"],
                                        d_final_state=d["dSf"], n_segments=3, want_d_init=True)
    torch.cuda.synchronize()
    _check_fwd(inp, lam, o, Sf)
    _check_bwd(inp, lam, grads)


def test_decode_a_null():
    N, H, dk, dv, steps = 96, 16, 96, 192, 8
    lam = schedule32(H, 1.0, 2048.0)
    S0 = I.gaussian(153, I.STREAM_S0, (N, H, dk, dv), 0.02)
    state = to_dev(S0)
    Sref = S0.astype(np.float64)
    lam_d = to_dev(lam)
    for s in range(steps):
        q, k, v = I.decode_token_inputs(153, s, N, H, dk, dv, "bf16")
        o = Bd.sgla_decode_step(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), lam_d, None, state)
        oh = to_host64(o)
        want = np.zeros((N, H, dv))
        for n in range(N):
            for h in range(H):
                want[n, h] = oracle.decode_step_unit(I.widen(q[n, h], "bf16"), I.widen(k[n, h], "bf16"),
                                                     I.widen(v[n, h], "bf16"), float(lam[h]), None,
                                                     Sref[n, h])
        assert_close(oh, want, TOL["bf16"], f"decode o step {s} (a=NULL)", store="bf16")
    assert_close(to_host64(state), Sref, TOL["bf16"], "decode state (a=NULL)")
