"""sgla_chunk_bwd_noalloc (no workspace, no allocation: the library's fixed
device scratch holds the partial sums of da) against sgla_chunk_bwd with a
caller workspace, on two calls in a row, the second with a smaller input, so
the second call reuses the scratch the first one left behind. Both calls are
also checked against the oracle on sampled units."""
import numpy as np
import pytest
import torch

from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import (TOL, assert_close, device_inputs, gpu_unit, oracle_bwd_units, schedule32,
                               to_dev, to_host64)

pytestmark = pytest.mark.gpu


def _call_both(inp, lam, cu=None):
    d = device_inputs(inp, cu)
    lam_d = to_dev(lam)
    ref = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam_d, d["a"], init_state=d["S0"],
                            d_final_state=d["dSf"], cu_seqlens=d["cu"], chunk=128, want_d_init=True)
    outs = (torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
            torch.empty_like(d["a"]), torch.empty_like(ref[4]))
    # poison the outputs so that a skipped write shows
    for t in outs:
        t.fill_(float("nan"))
    got = Bd.sgla_chunk_bwd_noalloc(d["q"], d["k"], d["v"], d["dO"], lam_d, d["a"], init_state=d["S0"],
                                    d_final_state=d["dSf"], cu_seqlens=d["cu"], chunk=128, dq=outs[0],
                                    dk=outs[1], dv=outs[2], da=outs[3], d_init_state=outs[4])
    torch.cuda.synchronize()
    return ref, got


def _check(inp, lam, ref, got, units, cu=None):
    names = ("dq", "dk", "dv", "da", "d_init_state")
    for nm, r, g in zip(names, ref, got):
        store = "bf16" if nm in ("dq", "dk", "dv") else "f32"
        assert_close(to_host64(g), to_host64(r), TOL["bf16"], f"{nm}: no-alloc vs workspace entry point",
                     store=store, ref_store=store)
        assert torch.equal(g, r), f"{nm}: the two entry points run the same kernels"
    oref = oracle_bwd_units(inp, lam, units, cu)
    for idx, nm in enumerate(("dq", "dk", "dv")):
        th = to_host64(got[idx])
        assert_close(np.concatenate([gpu_unit(th, n, h, cu).ravel() for n, h in units]),
                     np.concatenate([oref[u][idx].ravel() for u in units]), TOL["bf16"], f"{nm} vs oracle",
                     store="bf16")


def test_no_alloc_matches_workspace_entry_point_twice():
    lam = schedule32(16, 1.0, 2048.0)
    # first call: 6 sequences of 400 tokens
    inp1 = I.chunk_inputs(6, 16, 400, 96, 192, "bf16", seed=170, a_std=0.1, s0_std=0.02, with_grad=True,
                          dsf_std=0.02)
    ref1, got1 = _call_both(inp1, lam)
    _check(inp1, lam, ref1, got1, [(0, 0), (3, 9), (5, 15)])
    # second call right after, smaller: 2 sequences of 150 tokens
    inp2 = I.chunk_inputs(2, 16, 150, 96, 192, "bf16", seed=171, a_std=0.1, s0_std=0.02, with_grad=True,
                          dsf_std=0.02)
    ref2, got2 = _call_both(inp2, lam)
    _check(inp2, lam, ref2, got2, [(n, h) for n in range(2) for h in range(16)])
    # da of the second call summed only its own sequences
    units = [(n, h) for n in range(2) for h in range(16)]
    oref = oracle_bwd_units(inp2, lam, units)
    da_ref = np.zeros((16, 96))
    for (n, h) in units:
        da_ref[h] += oref[(n, h)][3]
    assert_close(to_host64(got2[3]), da_ref, TOL["bf16"], "da (second call) vs oracle")


def test_no_alloc_packed_then_dense():
    L = [300, 0, 65]
    cu = I.cu_from_lengths(L)
    lam = schedule32(4, 1.0, 2048.0)
    inp1 = I.chunk_inputs(1, 4, int(cu[-1]), 96, 192, "bf16", seed=172, a_std=0.1, s0_std=0.02,
                          n_seq=len(L), with_grad=True, dsf_std=0.02)
    ref1, got1 = _call_both(inp1, lam, cu)
    _check(inp1, lam, ref1, got1, [(0, 0), (2, 3)], cu)
    inp2 = I.chunk_inputs(1, 4, 70, 96, 192, "bf16", seed=173, a_std=0.1, s0_std=0.02, with_grad=True,
                          dsf_std=0.02)
    ref2, got2 = _call_both(inp2, lam)
    _check(inp2, lam, ref2, got2, [(0, h) for h in range(4)])
