"""GPU parity of the conv prologue (sgla_conv_fwd, sgla_conv_decode_step)
against the fp64 oracle: depthwise causal width-4 Conv1d + SiLU over dense
and packed sequences (empty, one- and two-token ones included), conv states
in and out, and decode steps on a state pool with slot indirection."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _dev_inputs(inp):
    dt = inp["dtype"]
    return (to_dev(inp["u"], dt), to_dev(inp["w"]), to_dev(inp["b"]), to_dev(inp["S0"]))


def _ref(inp, cu=None):
    u = I.widen(inp["u"], inp["dtype"])
    return oracle.conv_fwd(u, inp["w"], inp["b"], inp["S0"], cu)


def _check(y, fin, ref, inp, what=""):
    tol = TOL[inp["dtype"]]
    assert_close(to_host64(y).ravel(), ref[0].ravel(), tol, "y" + what, store=inp["dtype"])
    if fin is not None:
        # the state holds copies of past inputs: exact
        assert np.array_equal(to_host64(fin), ref[1]), "final conv state" + what


@pytest.mark.parametrize("dtype,B,T,D", [("bf16", 2, 97, 3072), ("f32", 2, 65, 64),
                                         ("bf16", 3, 1, 256), ("bf16", 1, 2, 64)])
def test_conv_dense(dtype, B, T, D):
    inp = I.conv_inputs(200 + T, (B, T, D), D, dtype, B)
    u, w, b, s0 = _dev_inputs(inp)
    y, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, want_final=True)
    torch.cuda.synchronize()
    _check(y, fin, _ref(inp), inp)


def test_conv_no_bias_no_state():
    inp = I.conv_inputs(210, (2, 70, 128), 128, "bf16", 2, bias=False, state=False)
    u, w, _, _ = _dev_inputs(inp)
    y, fin = Bd.sgla_conv_fwd(u, w, want_final=True)
    torch.cuda.synchronize()
    _check(y, fin, _ref(inp), inp)


def test_conv_varlen():
    L = [1, 0, 70, 33, 2, 0, 40, 3]
    cu = I.cu_from_lengths(L)
    inp = I.conv_inputs(220, (int(cu[-1]), 256), 256, "bf16", len(L))
    u, w, b, s0 = _dev_inputs(inp)
    y, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, cu_seqlens=to_dev(cu), want_final=True)
    torch.cuda.synchronize()
    _check(y, fin, _ref(inp, cu), inp)


def test_conv_varlen_long():
    """Sequences longer than a 64-token run: runs that lie inside one sequence
    (pipelined blocks of 8 rows) and runs that cross one or more boundaries."""
    L = [130, 64, 0, 200, 5, 128, 1, 67]
    cu = I.cu_from_lengths(L)
    for dtype, D in (("bf16", 512), ("f32", 128)):
        inp = I.conv_inputs(225, (int(cu[-1]), D), D, dtype, len(L))
        u, w, b, s0 = _dev_inputs(inp)
        y, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, cu_seqlens=to_dev(cu), want_final=True)
        torch.cuda.synchronize()
        _check(y, fin, _ref(inp, cu), inp, f" {dtype}")


def test_conv_rows_outside_sequences_untouched():
    """Packed rows before cu_seqlens[0] and after cu_seqlens[-1] belong to no
    sequence: y keeps what it held there, the sequences match the oracle."""
    S, D = 300, 256
    cu = np.array([70, 71, 150, 290], np.int32)
    inp = I.conv_inputs(227, (S, D), D, "bf16", len(cu) - 1)
    u, w, b, s0 = _dev_inputs(inp)
    y = torch.full((S, D), 7.0, dtype=torch.bfloat16, device="cuda")
    Bd.sgla_conv_fwd(u, w, b, init_state=s0, y=y, cu_seqlens=to_dev(cu))
    torch.cuda.synchronize()
    ref = _ref(inp, cu)[0]
    yh = to_host64(y)
    assert (yh[:70] == 7.0).all() and (yh[290:] == 7.0).all(), "rows outside every sequence written"
    assert_close(yh[70:290].ravel(), ref[70:290].ravel(), TOL["bf16"], "y", store="bf16")


def test_conv_state_carry_in_place():
    """[0, T) at once == [0, t0) then [t0, T) with the state carried in place."""
    T, t0, D = 90, 37, 512
    inp = I.conv_inputs(230, (2, T, D), D, "bf16", 2)
    u, w, b, s0 = _dev_inputs(inp)
    y, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, want_final=True)
    st = s0.clone()
    y1, _ = Bd.sgla_conv_fwd(u[:, :t0].contiguous(), w, b, init_state=st, final_state=st)
    y2, _ = Bd.sgla_conv_fwd(u[:, t0:].contiguous(), w, b, init_state=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], dim=1), y)
    assert torch.equal(st, fin)


def test_conv_full_size():
    """The prologue at the Laplace layer's size: B=8, T=2048, D=3072, bf16."""
    B, T, D = 8, 2048, 3072
    inp = I.conv_inputs(240, (B, T, D), D, "bf16", B)
    u, w, b, s0 = _dev_inputs(inp)
    y, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, want_final=True)
    torch.cuda.synchronize()
    _check(y, fin, _ref(inp), inp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_decode_pool(dtype):
    """Five decode steps of 6 sequences on an 8-page pool through a permuted
    slot table (one invalid entry: NaN output, pages untouched), against the
    oracle's decode steps and the sequence forward."""
    N, P, D, steps = 6, 8, 384, 5
    inp = I.conv_inputs(250, (N, steps, D), D, dtype, P)
    slot = np.array([3, 0, 7, 5, -1, 2], np.int32)
    u, w, b, pool = _dev_inputs(inp)
    pool0 = pool.clone()
    slot_d = to_dev(slot)
    ys = []
    for s in range(steps):
        ys.append(Bd.sgla_conv_decode_step(u[:, s].contiguous(), w, b, pool, slot=slot_d))
    torch.cuda.synchronize()
    uh = I.widen(inp["u"], dtype)
    tol = TOL[dtype]
    for n in range(N):
        if slot[n] < 0:
            assert all(torch.isnan(y[n]).all().item() for y in ys)
            continue
        st = inp["S0"][slot[n]].astype(np.float64).copy()
        for s in range(steps):
            r = oracle.conv_decode_step_unit(uh[n, s], inp["w"], inp["b"], st)
            assert_close(to_host64(ys[s][n]), r, tol, f"decode y n={n} s={s}", store=dtype)
        assert np.array_equal(to_host64(pool[slot[n]]), st), f"decode state n={n}"
    used = set(int(x) for x in slot if x >= 0)
    for p in range(P):
        if p not in used:
            assert torch.equal(pool[p], pool0[p]), f"page {p} touched"


def test_conv_decode_full_size():
    """Decode at serving size (1280 sequences, D=3072, bf16, pages = sequence
    index): three steps equal the sequence forward over the same three tokens
    from the same states bit for bit (same fp32 multiply-adds in the same
    order), and sampled sequences match the oracle's decode steps."""
    N, D, steps = 1280, 3072, 3
    inp = I.conv_inputs(260, (N, steps, D), D, "bf16", N)
    u, w, b, s0 = _dev_inputs(inp)
    pool = s0.clone()
    ys = [Bd.sgla_conv_decode_step(u[:, s].contiguous(), w, b, pool) for s in range(steps)]
    yf, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, want_final=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, dim=1), yf), "decode steps != forward"
    assert torch.equal(pool, fin), "decode state != forward final state"
    uh = I.widen(inp["u"], "bf16")
    for n in (0, 1, 2, 3, 511, 1277, 1278, 1279):
        st = inp["S0"][n].astype(np.float64).copy()
        for s in range(steps):
            r = oracle.conv_decode_step_unit(uh[n, s], inp["w"], inp["b"], st)
            assert_close(to_host64(ys[s][n]), r, TOL["bf16"], f"decode y n={n} s={s}", store="bf16")
        assert np.array_equal(to_host64(pool[n]), st), f"decode state n={n}"
