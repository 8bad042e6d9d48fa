"""GPU parity of the mixer epilogue (sgla_head_norm_gate: Head RMSNorm per
decay tier, concatenation, SiLU(g) gate) against the fp64 oracle: ragged
token counts, widths that fill one to four 64-channel chunks or part of one,
one tier per head and one tier for all, no scales, the gate in place, the
decode layout, the full Laplace-layer size (sampled tokens), and the chunk
forward's output fed straight in."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import (TOL, assert_close, device_inputs, oracle_fwd_units, schedule32,
                               to_dev, to_host64)

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _dev(inp):
    dt = inp["dtype"]
    return to_dev(inp["o"], dt), to_dev(inp["g"], dt), to_dev(inp["gamma"])


def _ref(inp, eps=EPS):
    dt = inp["dtype"]
    return oracle.head_norm_gate(I.widen(inp["o"], dt), I.widen(inp["g"], dt), inp["gamma"],
                                 inp["n_tiers"], eps)


@pytest.mark.parametrize("dtype,B,H,T,d_v,n_tiers", [
    ("bf16", 2, 16, 37, 192, 4),   # Laplace widths, ragged token count
    ("f32", 2, 4, 33, 32, 2),      # half a chunk per row
    ("bf16", 1, 8, 5, 256, 8),     # four full chunks, one tier per head
    ("bf16", 3, 6, 7, 100, 3),     # a partial second chunk
    ("f32", 1, 2, 9, 128, 1),      # one tier for all heads
    ("f32", 2, 16, 11, 192, 4),
])
def test_norm_gate(dtype, B, H, T, d_v, n_tiers):
    inp = I.norm_inputs(300 + T + d_v, B, H, T, d_v, n_tiers, dtype)
    o, g, gm = _dev(inp)
    out = Bd.sgla_head_norm_gate(o, g, gm, n_tiers, EPS)
    torch.cuda.synchronize()
    assert_close(to_host64(out).ravel(), _ref(inp).ravel(), TOL[dtype], "out", store=dtype)


def test_norm_gate_no_gamma_in_place_flat_g():
    """gamma = NULL (scale one), g given as [B, T, H * d_v], out written over g."""
    inp = I.norm_inputs(331, 2, 16, 19, 192, 4, "bf16", gamma=False)
    o, g, _ = _dev(inp)
    g = g.reshape(2, 19, 16 * 192)
    out = Bd.sgla_head_norm_gate(o, g, None, 4, EPS, out=g)
    torch.cuda.synchronize()
    assert out.data_ptr() == g.data_ptr()
    assert_close(to_host64(out).ravel(), _ref(inp).ravel(), TOL["bf16"], "out in place", store="bf16")


def test_norm_gate_zero_head_and_large_gate():
    """An all-zero head gives zeros (eps > 0 keeps the root finite); gates far
    into both SiLU tails give g and -0."""
    inp = I.norm_inputs(333, 1, 4, 6, 192, 2, "f32")
    inp["o"][0, 2] = 0.0
    inp["g"][0, :, 1, :96] = 60.0
    inp["g"][0, :, 1, 96:] = -60.0
    o, g, gm = _dev(inp)
    out = Bd.sgla_head_norm_gate(o, g, gm, 2, 1e-5)
    torch.cuda.synchronize()
    oh = to_host64(out)
    assert (oh[0, :, 2] == 0.0).all()
    assert_close(oh.ravel(), _ref(inp, 1e-5).ravel(), TOL["f32"], "out", store="f32")


def test_norm_gate_full_size_sampled():
    """The Laplace layer's size (B=8, T=2048, H=16, d_v=192, bf16, 4 tiers):
    every output finite and within the bound |o_c| / RMS(o) <= sqrt(d_v), and
    256 sampled tokens (all 16 heads each) against the oracle."""
    B, H, T, d_v, n_tiers = 8, 16, 2048, 192, 4
    inp = I.norm_inputs(340, B, H, T, d_v, n_tiers, "bf16")
    o, g, gm = _dev(inp)
    out = Bd.sgla_head_norm_gate(o, g, gm, n_tiers, EPS)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    gd = g.float()
    bound = (gd * torch.sigmoid(gd)).abs() * gm.abs().repeat_interleave(H // n_tiers, 0) * d_v ** 0.5
    assert (out.float().abs() <= bound * 1.01 + 1e-30).all()
    oh = to_host64(out)
    r = np.random.default_rng(7)
    toks = [(0, 0), (0, 1), (7, 2047), (3, 1024)] + [
        (int(b), int(t)) for b, t in zip(r.integers(0, B, 252), r.integers(0, T, 252))]
    got, ref = [], []
    for b, t in toks:
        got.append(oh[b, t].ravel())
        ref.append(oracle.head_norm_gate_token(I.widen(inp["o"][b, :, t, :], "bf16"),
                                               I.widen(inp["g"][b, t], "bf16"), inp["gamma"],
                                               n_tiers, EPS).ravel())
    assert_close(np.concatenate(got), np.concatenate(ref), TOL["bf16"], "sampled", store="bf16")


def test_norm_gate_on_chunk_forward_output():
    """sgla_chunk_fwd then the epilogue (the path the layer runs), each link
    against the oracle on that link's own inputs: the forward's o against the
    oracle's forward, and the epilogue's output against the oracle's epilogue
    of that same bf16 o. (Gating the composition against the oracle's fp64 o
    would charge the epilogue for the storage rounding of o, which the norm
    and the gate scale by |silu(g) gamma o_c| / RMS(o), up to ~16x the
    output's RMS here.)"""
    B, H, T, dk, dv, n_tiers = 2, 16, 150, 96, 192, 4
    inp = I.chunk_inputs(B, H, T, dk, dv, "bf16", seed=350, a_std=0.1)
    lam = schedule32(H, 1.0, 2048.0)
    d = device_inputs(inp)
    o, _ = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], to_dev(lam), d["a"], chunk=128)
    assert o.shape == (B, H, T, dv)
    nin = I.norm_inputs(351, B, H, T, dv, n_tiers, "bf16")
    g, gm = to_dev(nin["g"], "bf16"), to_dev(nin["gamma"])
    out = Bd.sgla_head_norm_gate(o, g, gm, n_tiers, EPS)
    torch.cuda.synchronize()
    ref_o = oracle_fwd_units(inp, lam, [(n, h) for n in range(B) for h in range(H)])
    o64 = np.stack([np.stack([ref_o[(n, h)][0] for h in range(H)]) for n in range(B)])
    oh = to_host64(o)
    assert_close(oh.ravel(), o64.ravel(), TOL["bf16"], "forward o", store="bf16")
    ref = oracle.head_norm_gate(oh, I.widen(nin["g"], "bf16"), nin["gamma"], n_tiers, EPS)
    assert_close(to_host64(out).ravel(), ref.ravel(), TOL["bf16"], "epilogue of that o", store="bf16")


def test_norm_gate_decode_layout():
    """A decode step's o [N, H, d_v] is the epilogue's [B = N, H, T = 1, d_v]."""
    N, H, dv = 40, 16, 192
    inp = I.norm_inputs(360, N, H, 1, dv, 4, "bf16")
    o, g, gm = _dev(inp)
    out = Bd.sgla_head_norm_gate(o.reshape(N, H, 1, dv), g, gm, 4, EPS)
    torch.cuda.synchronize()
    assert_close(to_host64(out).ravel(), _ref(inp).ravel(), TOL["bf16"], "decode layout", store="bf16")
