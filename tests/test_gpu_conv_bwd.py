"""GPU parity of the conv prologue's gradients (sgla_conv_bwd) against the
fp64 oracle, which differentiates the conv sequence by sequence and channel
by channel: dense rows whose 64-row runs straddle sequence boundaries, packed
sequences of 0 to 70 tokens (shorter than the history included), no bias or
initial state, fp32, the full Laplace width, and a bitwise repeat."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _run(inp, cu=None, with_dsf=True, want_d_init=True):
    dt = inp["dtype"]
    u, dy = to_dev(inp["u"], dt), to_dev(inp["dy"], dt)
    w, b, s0 = to_dev(inp["w"]), to_dev(inp["b"]), to_dev(inp["S0"])
    dsf = to_dev(inp["dSf"]) if with_dsf else None
    cu_d = None if cu is None else to_dev(np.asarray(cu, np.int32))
    print(f"  conv bwd {dt} shape={tuple(inp['u'].shape)} packed={cu is not None} "
          f"state={s0 is not None} bias={b is not None} dSf={with_dsf}", flush=True)
    du, dw, db, dinit = Bd.sgla_conv_bwd(u, w, dy, b=b, init_state=s0, d_final_state=dsf,
                                         cu_seqlens=cu_d, want_d_init=want_d_init)
    torch.cuda.synchronize()
    return du, dw, db, dinit


def _ref(inp, cu=None, with_dsf=True):
    dt = inp["dtype"]
    u, dy = I.widen(inp["u"], dt), I.widen(inp["dy"], dt)
    D = inp["D"]
    if cu is None:
        segs = [(u[n], dy[n]) for n in range(u.shape[0])]
    else:
        segs = [(u[cu[n]:cu[n + 1]], dy[cu[n]:cu[n + 1]]) for n in range(len(cu) - 1)]
    du, dinit = [], []
    dw, db = np.zeros((D, 4)), np.zeros(D)
    for n, (un, dyn) in enumerate(segs):
        st = None if inp["S0"] is None else inp["S0"][n]
        dso = inp["dSf"][n] if with_dsf else None
        a, d_st, w_, b_ = oracle.conv_bwd_unit(un, inp["w"], inp["b"], st, dyn, dso)
        du.append(a)
        dinit.append(d_st)
        dw += w_
        db += b_
    du = np.stack(du) if cu is None else np.concatenate(du, axis=0)
    return du, dw, db, np.stack(dinit)


def _check(inp, got, ref):
    dt = inp["dtype"]
    tol = TOL[dt]
    du, dw, db, dinit = got
    assert_close(to_host64(du).ravel(), ref[0].ravel(), tol, "du", store=dt)
    assert_close(to_host64(dw).ravel(), ref[1].ravel(), tol, "dw")
    if db is not None:
        assert_close(to_host64(db).ravel(), ref[2].ravel(), tol, "db")
    if dinit is not None:
        assert_close(to_host64(dinit).ravel(), ref[3].ravel(), tol, "d_init_state")


def test_conv_bwd_dense_runs_straddle_sequences():
    """B=2, T=100: the 64-row runs over the 200 rows cross the boundary at 100."""
    inp = I.conv_inputs(801, (2, 100, 64), 64, "bf16", 2, with_grad=True)
    _check(inp, _run(inp), _ref(inp))


def test_conv_bwd_packed_short_sequences():
    """Packed lengths 0, 1, 2, 3, 5, 40, 70 (and an empty one last)."""
    lens = [0, 1, 2, 3, 5, 40, 70, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = int(cu[-1])
    inp = I.conv_inputs(803, (S, 32), 32, "bf16", len(lens), with_grad=True)
    _check(inp, _run(inp, cu=cu), _ref(inp, cu=cu))


def test_conv_bwd_f32_no_bias_no_state():
    """fp32 (1e-4 gate), no bias, no initial state, no final-state gradient."""
    inp = I.conv_inputs(805, (3, 37, 16), 16, "f32", 3, bias=False, state=False, with_grad=True)
    _check(inp, _run(inp, with_dsf=False), _ref(inp, with_dsf=False))


def test_conv_bwd_laplace_width_and_repeat():
    """B=8, T=2048, D=3072 (the Laplace layer's conv), every output against the
    oracle; a second call gives the same dw and db bit for bit."""
    inp = I.conv_inputs(807, (8, 2048, 3072), 3072, "bf16", 8, with_grad=True)
    got = _run(inp)
    _check(inp, got, _ref(inp))
    again = _run(inp)
    assert torch.equal(got[1], again[1]) and torch.equal(got[2], again[2])
