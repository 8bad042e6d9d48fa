"""GPU parity of sgla_chunk_fwd / sgla_chunk_bwd against the fp64 oracle, at
sizes the oracle finishes in seconds that still span several chunks and a
ragged tail, plus the edge cases of the method."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import (DEV, TOL, assert_close, device_inputs, gpu_unit, oracle_bwd_units,
                               oracle_fwd_units, schedule32, to_dev, to_host64)

pytestmark = pytest.mark.gpu


def _units(N, H):
    return [(n, h) for n in range(N) for h in range(H)]


def run_fwd_case(inp, lam, chunk, cu=None, units=None):
    d = device_inputs(inp, cu)
    lam_d = to_dev(lam)
    o, Sf = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam_d, d["a"], init_state=d["S0"],
                              cu_seqlens=d["cu"], chunk=chunk, want_final=True)
    torch.cuda.synchronize()
    oh, Sh = to_host64(o), to_host64(Sf)
    units = units or _units(inp["N"], inp["H"])
    ref = oracle_fwd_units(inp, lam, units, cu)
    og = np.concatenate([gpu_unit(oh, n, h, cu).ravel() for n, h in units])
    orf = np.concatenate([ref[u][0].ravel() for u in units])
    sg = np.concatenate([Sh[n, h].ravel() for n, h in units])
    sr = np.concatenate([ref[u][1].ravel() for u in units])
    tol = TOL[inp["dtype"]]
    assert_close(og, orf, tol, "o", store=inp["dtype"])
    assert_close(sg, sr, tol, "final_state")
    return o, Sf


def run_bwd_case(inp, lam, chunk, cu=None, units=None):
    d = device_inputs(inp, cu)
    lam_d = to_dev(lam)
    dq, dk, dv, da, dS0 = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam_d, d["a"],
                                            init_state=d["S0"], d_final_state=d["dSf"],
                                            cu_seqlens=d["cu"], chunk=chunk, want_d_init=True)
    torch.cuda.synchronize()
    units = units or _units(inp["N"], inp["H"])
    ref = oracle_bwd_units(inp, lam, units, cu)
    tol = TOL[inp["dtype"]]
    for idx, (name, t) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        th = to_host64(t)
        g = np.concatenate([gpu_unit(th, n, h, cu).ravel() for n, h in units])
        r = np.concatenate([ref[u][idx].ravel() for u in units])
        assert_close(g, r, tol, name, store=inp["dtype"])
    if len(units) == inp["N"] * inp["H"]:
        da_ref = np.zeros_like(inp["a"], dtype=np.float64)
        for (n, h) in units:
            da_ref[h] += ref[(n, h)][3]
        assert_close(to_host64(da), da_ref, tol, "da")
    dsh = to_host64(dS0)
    assert_close(np.concatenate([dsh[n, h].ravel() for n, h in units]),
                 np.concatenate([ref[u][4].ravel() for u in units]), tol, "d_init_state")
    return dq, dk, dv, da, dS0


# ------------------------------------------------------------------ fp32 (1e-4 gate)


def test_fwd_f32_tiny_config():
    """B=1 H=2 T=256 d_k=16 d_v=32 chunk 64, fp32, schedule 1..256, zero init."""
    inp = I.chunk_inputs(1, 2, 256, 16, 32, "f32", seed=1, a_std=0.1)
    run_fwd_case(inp, schedule32(2, 1.0, 256.0), 64)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_fwd_f32_ragged_with_state(T):
    inp = I.chunk_inputs(2, 4, T, 16, 32, "f32", seed=10 + T, a_std=0.3, s0_std=0.2)
    lam = np.array([0.0, 0.5, 0.99, 1.0], np.float32)  # lam = 0 and 1 included
    run_fwd_case(inp, lam, 64)


def test_fwd_f32_other_widths():
    inp = I.chunk_inputs(1, 3, 130, 8, 24, "f32", seed=30, a_std=0.3, s0_std=0.1)
    run_fwd_case(inp, np.array([0.3, 0.8, 0.999], np.float32), 64)


@pytest.mark.parametrize("T", [1, 64, 150])
def test_bwd_f32(T):
    inp = I.chunk_inputs(2, 3, T, 16, 32, "f32", seed=40 + T, a_std=0.5, s0_std=0.2,
                         with_grad=True, dsf_std=0.3)
    run_bwd_case(inp, np.array([0.0, 0.9, 1.0], np.float32), 64)


def test_bwd_f32_no_aug_no_state():
    inp = I.chunk_inputs(1, 2, 100, 16, 32, "f32", seed=50, a_std=None, with_grad=True)
    run_bwd_case(inp, np.array([0.6, 0.97], np.float32), 64)


def test_varlen_f32_fwd_bwd():
    L = [1, 0, 130, 64, 65, 7]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 2, int(cu[-1]), 16, 32, "f32", seed=60, a_std=0.4, s0_std=0.2,
                         n_seq=len(L), with_grad=True, dsf_std=0.2)
    lam = np.array([0.7, 0.995], np.float32)
    run_fwd_case(inp, lam, 64, cu=cu)
    run_bwd_case(inp, lam, 64, cu=cu)


@pytest.mark.parametrize("dk,dv,T,chunk", [(64, 64, 150, 64), (96, 192, 130, 128), (48, 72, 97, 32),
                                           (96, 96, 70, 64), (8, 132, 65, 64), (36, 20, 33, 128)])
def test_f32_wide_heads(dk, dv, T, chunk):
    """fp32 heads wider than 32 x 32 (32-token tiles, widths padded to the
    next of 32, 64, 96 or 192), forward and backward at the fp32 bound, with
    decays 0 and 1 among the heads."""
    inp = I.chunk_inputs(2, 3, T, dk, dv, "f32", seed=700 + dk + dv, a_std=0.4, s0_std=0.1,
                         with_grad=True, dsf_std=0.1)
    lam = np.array([0.0, 0.93, 1.0], np.float32)
    run_fwd_case(inp, lam, chunk)
    run_bwd_case(inp, lam, chunk)


def test_f32_wide_heads_packed():
    L = [70, 0, 1, 33]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 2, int(cu[-1]), 96, 160, "f32", seed=710, a_std=0.3, s0_std=0.1,
                         n_seq=len(L), with_grad=True, dsf_std=0.1)
    lam = np.array([0.8, 0.999], np.float32)
    run_fwd_case(inp, lam, 64, cu=cu)
    run_bwd_case(inp, lam, 64, cu=cu)


# ------------------------------------------------------------------ bf16 (2e-2 gate)


# chunk 32 and 64 run different tilings (32- and 64-token tiles of the
# forward and dv scans); chunk 128 runs the 64-token tiles of chunk 64
@pytest.mark.parametrize("chunk", [32, 64])
def test_fwd_bf16_several_chunks(chunk):
    inp = I.chunk_inputs(2, 16, 320, 96, 192, "bf16", seed=70, a_std=0.1, s0_std=0.02)
    run_fwd_case(inp, schedule32(16, 1.0, 2048.0), chunk)


@pytest.mark.parametrize("chunk", [32, 64])
def test_bwd_bf16_several_chunks(chunk):
    inp = I.chunk_inputs(1, 16, 300, 96, 192, "bf16", seed=80, a_std=0.1, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    run_bwd_case(inp, schedule32(16, 1.0, 2048.0), chunk)


def test_bf16_special_decays_and_short():
    inp = I.chunk_inputs(1, 4, 37, 96, 192, "bf16", seed=90, a_std=0.2, s0_std=0.05,
                         with_grad=True, dsf_std=0.05)
    lam = np.array([0.0, 0.5, 0.9997, 1.0], np.float32)
    run_fwd_case(inp, lam, 128)
    run_bwd_case(inp, lam, 128)


@pytest.mark.parametrize("dk,chunk", [(8, 128), (96, 64), (8, 32)])
def test_bf16_single_short_memory_head(dk, chunk):
    """One head of half-life 1 (lambda = 0.5) with a = 0: its output is led by
    the diagonal term (q_t . k_t + sigmoid(0)) v_t, and with no long-memory
    head in the tensor the metric's RMS does not hide that term's rounding. A
    bf16 diagonal in the intra-tile scores scored 3.0e-2 on o and 3.2e-2 on dv
    here; the kernels carry the diagonal in fp32."""
    inp = I.chunk_inputs(1, 1, 438, dk, 192, "bf16", seed=6008, a_std=None, with_grad=True, dsf_std=0.05)
    lam = np.array([0.5], np.float32)
    run_fwd_case(inp, lam, chunk)
    run_bwd_case(inp, lam, chunk)


@pytest.mark.parametrize("a_std", [None, 2.0])
def test_bf16_zero_decay_is_the_diagonal_alone(a_std):
    """With lambda = 0 every token sees only itself: o_t = (q_t . k_t +
    sigmoid(z_t)) v_t, carried in fp32 with no bf16 score on the way, and z_t
    is formed in fp32 from a in fp32 and the exact products of the bf16
    inputs. So o matches the oracle to fp32 rounding, with a = 0 and with a
    large a alike (bf16 operands in the gate gave 1.1e-3 here)."""
    inp = I.chunk_inputs(1, 2, 300, 8, 192, "bf16", seed=6013, a_std=a_std, with_grad=True, dsf_std=0.05)
    lam = np.array([0.0, 0.0], np.float32)
    d = device_inputs(inp)
    o, _ = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], to_dev(lam), d["a"], chunk=128)
    torch.cuda.synchronize()
    units = _units(1, 2)
    ref = oracle_fwd_units(inp, lam, units)
    oh = to_host64(o)
    assert_close(np.concatenate([gpu_unit(oh, n, h).ravel() for n, h in units]),
                 np.concatenate([ref[u][0].ravel() for u in units]), 1e-5, "o (lambda = 0)", store="bf16")
    run_bwd_case(inp, lam, 128)


@pytest.mark.parametrize("B,T,d_k,d_v,lengths,s0_std,dsf_std,seed", [
    (2, 311, 96, 56, None, 1.0, 0.05, 5506),
    (1, 419, 72, 136, [129, 257, 0, 33], 5.0, 0.05, 6334),
    (2, 240, 96, 136, None, 0.05, None, 5722),
])
def test_bf16_short_memory_head_large_a(B, T, d_k, d_v, lengths, s0_std, dsf_std, seed):
    """One head of half-life 1 (lambda = 0.5) with a ~ N(0, 2^2): z_t spreads
    over several units and the gate terms sigmoid'(z_t) (dO_t . v_t) of dq, dk
    and da carry much of their RMS. With the gate argument formed from bf16(a)
    and bf16(a (.) q) these configurations scored 2.5e-2 (dq), 2.8e-2 (dq)
    and 2.4e-2 (dk); the kernels form it in fp32."""
    cu = None if lengths is None else I.cu_from_lengths(lengths)
    inp = I.chunk_inputs(B, 1, T, d_k, d_v, "bf16", seed=seed, a_std=2.0, s0_std=s0_std,
                         n_seq=None if lengths is None else len(lengths), with_grad=True, dsf_std=dsf_std)
    lam = np.array([0.5], np.float32)
    run_fwd_case(inp, lam, 64, cu=cu)
    run_bwd_case(inp, lam, 64, cu=cu)


def test_bf16_narrow_dims():
    inp = I.chunk_inputs(1, 2, 140, 32, 64, "bf16", seed=95, a_std=0.2, s0_std=0.05,
                         with_grad=True, dsf_std=0.05)
    lam = np.array([0.8, 0.99], np.float32)
    run_fwd_case(inp, lam, 64)
    run_bwd_case(inp, lam, 64)


@pytest.mark.parametrize("dk,dv,T", [(8, 8, 70), (40, 136, 97), (64, 96, 130), (96, 152, 33)])
def test_bf16_padded_and_partial_widths(dk, dv, T):
    """Widths that are not multiples of the kernels' 32-row blocks or 96-column
    slices (zero-padded operand columns, a partial second value slice) and
    lengths with a ragged last tile, forward and backward."""
    inp = I.chunk_inputs(2, 3, T, dk, dv, "bf16", seed=97 + dk + dv, a_std=0.2, s0_std=0.05,
                         with_grad=True, dsf_std=0.05)
    lam = np.array([0.7, 0.98, 0.9995], np.float32)
    run_fwd_case(inp, lam, 64)
    run_bwd_case(inp, lam, 64)


def test_varlen_bf16_fwd_bwd():
    L = [1, 0, 257, 128, 5, 300]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 16, int(cu[-1]), 96, 192, "bf16", seed=100, a_std=0.1, s0_std=0.02,
                         n_seq=len(L), with_grad=True, dsf_std=0.02)
    lam = schedule32(16, 1.0, 2048.0)
    run_fwd_case(inp, lam, 128, cu=cu)
    run_bwd_case(inp, lam, 128, cu=cu)


def test_varlen_bf16_equal_lengths_and_repeat():
    """Packed sequences run longest first, equal lengths in packed order: with
    ties, an empty sequence and a one-token one, every output still matches
    the oracle, and a second call is bitwise identical."""
    L = [64, 200, 64, 0, 64, 1, 200]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 4, int(cu[-1]), 96, 192, "bf16", seed=104, a_std=0.1, s0_std=0.02,
                         n_seq=len(L), with_grad=True, dsf_std=0.02)
    lam = schedule32(4, 1.0, 2048.0)
    o1, S1 = run_fwd_case(inp, lam, 128, cu=cu)
    g1 = run_bwd_case(inp, lam, 128, cu=cu)
    o2, S2 = run_fwd_case(inp, lam, 128, cu=cu)
    g2 = run_bwd_case(inp, lam, 128, cu=cu)
    for x, y in [(o1, o2), (S1, S2)] + list(zip(g1, g2)):
        assert torch.equal(x, y)


def test_varlen_bf16_longest_first_at_its_limit():
    """256 packed sequences, the most that run longest first (the length table
    fills the workgroup's LDS slot): lengths 0 to 40 with many ties, forward
    and backward against the oracle on a sample of units."""
    L = [(37 * i) % 41 for i in range(256)]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 2, int(cu[-1]), 32, 64, "bf16", seed=106, a_std=0.1, s0_std=0.02,
                         n_seq=len(L), with_grad=True, dsf_std=0.02)
    lam = schedule32(2, 1.0, 2048.0)
    longest = int(np.argmax(L))
    units = [(n, h) for n in (0, 1, 2, 127, 254, 255, longest) for h in (0, 1)]
    run_fwd_case(inp, lam, 64, cu=cu, units=units)
    run_bwd_case(inp, lam, 64, cu=cu, units=units)


def test_varlen_bf16_many_sequences_keep_packed_order():
    """Above 256 packed sequences the longest-first order is not used: 300
    short sequences of 0 to 9 tokens, forward and backward, against the oracle
    on a sample of (sequence, head) units."""
    L = [(7 * i) % 10 for i in range(300)]
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, 2, int(cu[-1]), 32, 64, "bf16", seed=105, a_std=0.1, s0_std=0.02,
                         n_seq=len(L), with_grad=True, dsf_std=0.02)
    lam = schedule32(2, 1.0, 2048.0)
    units = [(n, h) for n in (0, 1, 9, 150, 298, 299) for h in (0, 1)]
    run_fwd_case(inp, lam, 64, cu=cu, units=units)
    run_bwd_case(inp, lam, 64, cu=cu, units=units)


# ------------------------------------------------------------------ invariants


def test_chunk_size_invariance_bf16():
    """The chunk form is exact for any chunk length ("Challenge 1"): the
    32-token and 64-token tilings of the forward and of the dv scan both
    match the oracle, and they are different evaluations (not bit-identical),
    so this compares two tilings, not one kernel with itself. chunk 128 runs
    the 64-token tiles and gives chunk 64's result bit for bit."""
    inp = I.chunk_inputs(1, 16, 300, 96, 192, "bf16", seed=110, a_std=0.1, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    lam = schedule32(16, 1.0, 2048.0)
    o32, S32 = run_fwd_case(inp, lam, 32)
    o64, S64 = run_fwd_case(inp, lam, 64)
    assert not torch.equal(o32, o64), "chunk 32 and 64 must run different tilings"
    assert_close(to_host64(o32), to_host64(o64), TOL["bf16"], "chunk 32 vs 64", store="bf16",
                 ref_store="bf16")
    g32 = run_bwd_case(inp, lam, 32)
    g64 = run_bwd_case(inp, lam, 64)
    assert not torch.equal(g32[2], g64[2]), "dv: chunk 32 and 64 must run different tilings"
    d = device_inputs(inp)
    o128, S128 = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], to_dev(lam), d["a"], init_state=d["S0"],
                                   chunk=128, want_final=True)
    assert torch.equal(o128, o64) and torch.equal(S128, S64)


@pytest.mark.parametrize("T", [1, 100, 300])
def test_chunk_size_invariance_f32(T):
    """fp32 tiles by the chunk length itself: chunks of 32, 64 and 128 tokens
    all match the oracle at the fp32 gate, forward and backward, and differ
    from one another only in rounding."""
    inp = I.chunk_inputs(2, 3, T, 16, 32, "f32", seed=111 + T, a_std=0.3, s0_std=0.2,
                         with_grad=True, dsf_std=0.3)
    lam = np.array([0.0, 0.9, 0.999], np.float32)
    outs = {}
    for chunk in (32, 64, 128):
        outs[chunk] = run_fwd_case(inp, lam, chunk)[0]
        run_bwd_case(inp, lam, chunk)
    if T > 64:
        assert not torch.equal(outs[32], outs[128]), "chunk 32 and 128 must run different tilings"


def test_state_carry_bf16():
    """Running [0,T) at once == [0,t0) then [t0,T) from the carried state."""
    T, t0 = 384, 200
    inp = I.chunk_inputs(2, 16, T, 96, 192, "bf16", seed=120, a_std=0.1, s0_std=0.02)
    d = device_inputs(inp)
    lam = to_dev(schedule32(16, 1.0, 2048.0))
    o, Sf = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam, d["a"], init_state=d["S0"],
                              want_final=True)
    part = lambda x, sl: x[:, :, sl].contiguous()
    o1, S1 = Bd.sgla_chunk_fwd(part(d["q"], slice(0, t0)), part(d["k"], slice(0, t0)),
                               part(d["v"], slice(0, t0)), lam, d["a"], init_state=d["S0"],
                               want_final=True)
    o2, S2 = Bd.sgla_chunk_fwd(part(d["q"], slice(t0, T)), part(d["k"], slice(t0, T)),
                               part(d["v"], slice(t0, T)), lam, d["a"], init_state=S1,
                               final_state=S1)  # in-place carry
    assert_close(to_host64(torch.cat([o1, o2], dim=2)), to_host64(o), TOL["bf16"], "split o",
                 store="bf16", ref_store="bf16")
    assert_close(to_host64(S1), to_host64(Sf), TOL["bf16"], "split state")


def test_deterministic_bitwise():
    inp = I.chunk_inputs(2, 16, 300, 96, 192, "bf16", seed=130, a_std=0.1, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    d = device_inputs(inp)
    lam = to_dev(schedule32(16, 1.0, 2048.0))
    r1 = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam, d["a"], d["S0"], want_final=True)
    r2 = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam, d["a"], d["S0"], want_final=True)
    g1 = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam, d["a"], d["S0"], d["dSf"],
                           want_d_init=True)
    g2 = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam, d["a"], d["S0"], d["dSf"],
                           want_d_init=True)
    for x, y in list(zip(r1, r2)) + list(zip(g1, g2)):
        assert torch.equal(x, y)


def test_nan_in_q_stays_in_its_row():
    inp = I.chunk_inputs(1, 2, 200, 96, 192, "bf16", seed=140, a_std=0.1)
    d = device_inputs(inp)
    q = d["q"].clone()
    q[0, 1, 77, 5] = float("nan")
    lam = to_dev(np.array([0.5, 0.99], np.float32))
    o, _ = Bd.sgla_chunk_fwd(q, d["k"], d["v"], lam, d["a"])
    bad = torch.isnan(o.float())
    assert bad[0, 1, 77].all(), "NaN must propagate to its own output row"
    bad[0, 1, 77] = False
    assert not bad.any(), "NaN leaked outside its row"


def test_bf16_large_aug_balance():
    """aug_balance a is learned ("GLA mixer") and may grow: a ~ N(0, 1) with
    entries of +-4 in every head. The bf16 kernels form the gate argument z
    from a and the products a_i x_i rounded to bf16, so its error grows with
    |z|; forward, backward (da included) and decode still meet the gate."""
    inp = I.chunk_inputs(2, 16, 200, 96, 192, "bf16", seed=160, a_std=1.0, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    inp["a"][:, 0] = 4.0
    inp["a"][:, 5] = -4.0
    inp["a"][::2, 17] = 4.0
    lam = schedule32(16, 1.0, 2048.0)
    run_fwd_case(inp, lam, 128)
    run_bwd_case(inp, lam, 128)
    # decode with the same a: 16 steps from the initial state, against the oracle
    d = device_inputs(inp)
    state = d["S0"].clone()
    S = inp["S0"].astype(np.float64)
    lam_d = to_dev(lam)
    for t in range(16):
        qt, kt, vt = (d[x][:, :, t].contiguous() for x in ("q", "k", "v"))
        o = to_host64(Bd.sgla_decode_step(qt, kt, vt, lam_d, d["a"], state))
        want = np.zeros_like(o)
        for n in range(2):
            for h in range(16):
                want[n, h] = oracle.decode_step_unit(
                    I.widen(inp["q"][n, h, t], "bf16"), I.widen(inp["k"][n, h, t], "bf16"),
                    I.widen(inp["v"][n, h, t], "bf16"), float(lam[h]), inp["a"][h].astype(np.float64),
                    S[n, h])
        assert_close(o, want, TOL["bf16"], f"decode o step {t} (large a)", store="bf16")
