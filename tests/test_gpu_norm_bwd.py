"""GPU parity of the mixer epilogue's gradients (sgla_head_norm_gate_bwd)
against the fp64 oracle, which differentiates the epilogue token by token:
ragged token counts, partial and full 64-channel chunks, one tier per head
and one tier for all, no scales, dg written over dout, the full
Laplace-layer size, and a bitwise repeat of the tier-scale gradient."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, to_dev, to_host64

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _case(inp, in_place=False, flat=False):
    dt = inp["dtype"]
    o, g, dout = (to_dev(inp[x], dt) for x in ("o", "g", "dout"))
    gm = to_dev(inp["gamma"])
    B, H, T, d_v = inp["o"].shape
    print(f"  norm bwd {dt} B={B} H={H} T={T} d_v={d_v} tiers={inp['n_tiers']} "
          f"gamma={'yes' if gm is not None else 'no'} in_place={in_place}", flush=True)
    if flat:
        g, dout = g.reshape(B, T, H * d_v), dout.reshape(B, T, H * d_v)
    d_o, dg, dgamma = Bd.sgla_head_norm_gate_bwd(o, g, dout, gm, inp["n_tiers"], EPS,
                                                 dg=dout if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert dg.data_ptr() == dout.data_ptr()
    r_do, r_dg, r_dgm = oracle.head_norm_gate_bwd(I.widen(inp["o"], dt), I.widen(inp["g"], dt),
                                                  inp["gamma"], I.widen(inp["dout"], dt),
                                                  inp["n_tiers"], EPS)
    tol = TOL[dt]
    assert_close(to_host64(d_o).ravel(), r_do.ravel(), tol, "d_o", store=dt)
    assert_close(to_host64(dg).ravel(), r_dg.ravel(), tol, "dg", store=dt)
    assert_close(to_host64(dgamma).ravel(), r_dgm.ravel(), tol, "dgamma")
    return dgamma


@pytest.mark.parametrize("dtype,B,H,T,d_v,n_tiers", [
    ("bf16", 2, 16, 37, 192, 4),   # Laplace widths, ragged token count (partial token block)
    ("f32", 2, 4, 33, 32, 2),      # half a chunk per row
    ("bf16", 1, 8, 130, 256, 8),   # four full chunks, one tier per head, three token blocks
    ("bf16", 3, 6, 7, 100, 3),     # a partial second chunk
    ("f32", 1, 2, 65, 128, 1),     # one tier for all heads
    ("f32", 2, 16, 11, 192, 4),
])
def test_norm_gate_bwd(dtype, B, H, T, d_v, n_tiers):
    inp = I.norm_inputs(700 + T + d_v, B, H, T, d_v, n_tiers, dtype, with_dout=True)
    _case(inp)


def test_norm_gate_bwd_no_gamma_in_place_flat():
    """gamma = NULL (the gradient at scale one), g and dout as [B, T, H * d_v],
    dg written over dout."""
    inp = I.norm_inputs(741, 2, 16, 19, 192, 4, "bf16", gamma=False, with_dout=True)
    _case(inp, in_place=True, flat=True)


def test_norm_gate_bwd_laplace_size_and_repeat():
    """B=8, T=2048, H=16, d_v=192, 4 tiers (the Laplace layer), every output
    against the oracle; a second call gives the same dgamma bit for bit."""
    inp = I.norm_inputs(743, 8, 16, 2048, 192, 4, "bf16", with_dout=True)
    dgamma = _case(inp)
    o, g, dout = (to_dev(inp[x], "bf16") for x in ("o", "g", "dout"))
    _, _, dgamma2 = Bd.sgla_head_norm_gate_bwd(o, g, dout, to_dev(inp["gamma"]), 4, EPS)
    torch.cuda.synchronize()
    assert torch.equal(dgamma, dgamma2)


def test_norm_gate_bwd_without_dgamma():
    """dgamma = NULL skips the scale gradient (no workspace needed); d_o and dg
    are the same as with it."""
    inp = I.norm_inputs(747, 1, 4, 40, 64, 2, "bf16", with_dout=True)
    o, g, dout = (to_dev(inp[x], "bf16") for x in ("o", "g", "dout"))
    gm = to_dev(inp["gamma"])
    a = Bd.sgla_head_norm_gate_bwd(o, g, dout, gm, 2, EPS, want_dgamma=False)
    b = Bd.sgla_head_norm_gate_bwd(o, g, dout, gm, 2, EPS)
    torch.cuda.synchronize()
    assert a[2] is None
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
