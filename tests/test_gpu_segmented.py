"""GPU parity of sgla_chunk_fwd_segmented (long dense sequences cut into
segments that run on separate workgroups, joined by a scan of the states)
against the fp64 oracle, which runs each sequence token by token with no
segments, and against the single-pass sgla_chunk_fwd."""
import numpy as np
import pytest
import torch

from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import (TOL, assert_close, device_inputs, oracle_fwd_units, schedule32,
                               to_dev, to_host64)

pytestmark = pytest.mark.gpu


def run_segmented_case(inp, lam, n_segments, units=None):
    d = device_inputs(inp)
    lam_d = to_dev(lam)
    print(f"  segmented fwd B={inp['B']} H={inp['H']} T={inp['T']} n_segments={n_segments}",
          flush=True)
    o, Sf = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, d["a"],
                                        init_state=d["S0"], n_segments=n_segments,
                                        want_final=True)
    torch.cuda.synchronize()
    oh, Sh = to_host64(o), to_host64(Sf)
    units = units or [(n, h) for n in range(inp["B"]) for h in range(inp["H"])]
    ref = oracle_fwd_units(inp, lam, units)
    tol = TOL[inp["dtype"]]
    assert_close(np.concatenate([oh[n, h].ravel() for n, h in units]),
                 np.concatenate([ref[u][0].ravel() for u in units]), tol, "o", store="bf16")
    assert_close(np.concatenate([Sh[n, h].ravel() for n, h in units]),
                 np.concatenate([ref[u][1].ravel() for u in units]), tol, "final_state")
    return o, Sf, d


@pytest.mark.parametrize("T,n_segments", [(1000, 2), (1000, 3), (1000, 5), (700, 11), (2048, 4)])
def test_segmented_fwd_matches_oracle(T, n_segments):
    """Ragged T (partial last tile and segment), initial state, a != 0, the
    1..2048 half-life schedule; n_segments = 11 at T = 700 leaves 11 tiles in
    11 one-tile segments."""
    inp = I.chunk_inputs(2, 4, T, 96, 192, "bf16", seed=500 + T + n_segments, a_std=0.1,
                         s0_std=0.02)
    run_segmented_case(inp, schedule32(4, 1.0, 2048.0), n_segments)


def test_segmented_fwd_small_dims_and_extreme_decays():
    """d_k = 32, d_v = 64 (padded tiles) with lambda = 0, 0.5, 0.999, 1."""
    inp = I.chunk_inputs(1, 4, 777, 32, 64, "bf16", seed=77, a_std=0.3, s0_std=0.05)
    lam = np.array([0.0, 0.5, 0.999, 1.0], np.float32)
    run_segmented_case(inp, lam, 4)


def test_segmented_fwd_agrees_with_single_pass():
    """The same inputs through sgla_chunk_fwd: the two differ by rounding only;
    n_segments = 1 is the single pass itself, bit for bit."""
    inp = I.chunk_inputs(2, 4, 1500, 96, 192, "bf16", seed=91, a_std=0.1, s0_std=0.02)
    lam = schedule32(4, 1.0, 2048.0)
    o_seg, S_seg, d = run_segmented_case(inp, lam, 3)
    lam_d = to_dev(lam)
    o1, S1 = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam_d, d["a"], init_state=d["S0"],
                               want_final=True)
    o_one, S_one = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, d["a"],
                                               init_state=d["S0"], n_segments=1, want_final=True)
    torch.cuda.synchronize()
    assert torch.equal(o_one, o1) and torch.equal(S_one, S1)
    assert_close(to_host64(o_seg).ravel(), to_host64(o1).ravel(), TOL["bf16"], "o vs single pass",
                 store="bf16", ref_store="bf16")
    assert_close(to_host64(S_seg).ravel(), to_host64(S1).ravel(), TOL["bf16"],
                 "final_state vs single pass")


def test_segmented_fwd_in_place_carry_and_repeat():
    """final_state may be init_state; a repeated call is bitwise identical."""
    inp = I.chunk_inputs(1, 4, 900, 96, 192, "bf16", seed=93, a_std=0.1, s0_std=0.02)
    lam = schedule32(4, 1.0, 2048.0)
    d = device_inputs(inp)
    lam_d = to_dev(lam)
    o_a, S_a = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, d["a"],
                                           init_state=d["S0"], n_segments=4, want_final=True)
    state = d["S0"].clone()
    o_b, _ = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, d["a"], init_state=state,
                                         final_state=state, n_segments=4)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(S_a, state)


def test_segmented_fwd_without_initial_state():
    """No init_state: the scan starts segment 0 from zero (its workspace
    entry is cleared, not read from a caller pointer)."""
    inp = I.chunk_inputs(1, 4, 1300, 96, 192, "bf16", seed=95, a_std=0.1, s0_std=None)
    run_segmented_case(inp, schedule32(4, 1.0, 2048.0), 5)


def test_segmented_fwd_in_place_carry_two_rounds_of_workgroups():
    """final_state == init_state when the full launch has more workgroups than
    the GPU holds at once (B=1, H=16, 16 segments: 512 workgroups of one per
    CU), so segment 0 may start after the last segment has finished: the
    result must still equal the call with a separate final_state, bit for bit."""
    inp = I.chunk_inputs(1, 16, 4096, 96, 192, "bf16", seed=97, a_std=0.1, s0_std=0.02)
    lam_d = to_dev(schedule32(16, 1.0, 2048.0))
    d = device_inputs(inp)
    print("  segmented fwd in place B=1 H=16 T=4096 n_segments=16", flush=True)
    o_a, S_a = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, d["a"],
                                           init_state=d["S0"], n_segments=16, want_final=True)
    state = d["S0"].clone()
    o_b, _ = Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam_d, d["a"], init_state=state,
                                         final_state=state, n_segments=16)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(S_a, state)


def test_segmented_fwd_long_sequence_sampled_heads():
    """The long-context shape the segments are for: B = 1, H = 16, T = 32768
    (the longest sequence of the packed workload), d_k = 96, d_v = 192, eight
    segments; the oracle checks the shortest- and the longest-memory heads."""
    T = 32768
    inp = I.chunk_inputs(1, 16, T, 96, 192, "bf16", seed=95, a_std=0.1, s0_std=0.02)
    run_segmented_case(inp, schedule32(16, 1.0, 2048.0), 8, units=[(0, 0), (0, 15)])


# ---------------------------------------------------------------- backward

def run_segmented_bwd_case(inp, lam, n_segments, units=None):
    from tests.parity_util import oracle_bwd_units
    d = device_inputs(inp)
    lam_d = to_dev(lam)
    print(f"  segmented bwd B={inp['B']} H={inp['H']} T={inp['T']} n_segments={n_segments}",
          flush=True)
    dq, dk, dv, da, dS0 = Bd.sgla_chunk_bwd_segmented(d["q"], d["k"], d["v"], d["dO"], lam_d, d["a"],
                                                      init_state=d["S0"], d_final_state=d["dSf"],
                                                      n_segments=n_segments, want_d_init=True)
    torch.cuda.synchronize()
    units = units or [(n, h) for n in range(inp["B"]) for h in range(inp["H"])]
    ref = oracle_bwd_units(inp, lam, units)
    tol = TOL[inp["dtype"]]
    for idx, (name, t) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        th = to_host64(t)
        assert_close(np.concatenate([th[n, h].ravel() for n, h in units]),
                     np.concatenate([ref[u][idx].ravel() for u in units]), tol, name, store="bf16")
    if len(units) == inp["B"] * inp["H"]:
        da_ref = np.zeros_like(inp["a"], dtype=np.float64)
        for u in units:
            da_ref[u[1]] += ref[u][3]
        assert_close(to_host64(da), da_ref, tol, "da")
    dsh = to_host64(dS0)
    assert_close(np.concatenate([dsh[n, h].ravel() for n, h in units]),
                 np.concatenate([ref[u][4].ravel() for u in units]), tol, "d_init_state")
    return (dq, dk, dv, da, dS0), d


@pytest.mark.parametrize("T,n_segments", [(1000, 2), (1000, 3), (700, 5), (2048, 4)])
def test_segmented_bwd_matches_oracle(T, n_segments):
    """Ragged T, initial state, final-state gradient, a != 0, the 1..2048
    schedule; every gradient against the oracle's token-by-token backward."""
    inp = I.chunk_inputs(2, 4, T, 96, 192, "bf16", seed=600 + T + n_segments, a_std=0.1,
                         s0_std=0.02, with_grad=True, dsf_std=0.02)
    run_segmented_bwd_case(inp, schedule32(4, 1.0, 2048.0), n_segments)


def test_segmented_bwd_agrees_with_single_pass():
    """Against sgla_chunk_bwd on the same inputs (rounding apart); one segment
    is the single pass, bit for bit."""
    inp = I.chunk_inputs(1, 4, 1500, 96, 192, "bf16", seed=97, a_std=0.1, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    lam = schedule32(4, 1.0, 2048.0)
    seg, d = run_segmented_bwd_case(inp, lam, 3)
    lam_d = to_dev(lam)
    one = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam_d, d["a"], init_state=d["S0"],
                            d_final_state=d["dSf"], want_d_init=True)
    one_s = Bd.sgla_chunk_bwd_segmented(d["q"], d["k"], d["v"], d["dO"], lam_d, d["a"],
                                        init_state=d["S0"], d_final_state=d["dSf"], n_segments=1,
                                        want_d_init=True)
    torch.cuda.synchronize()
    for x, y in zip(one, one_s):
        assert torch.equal(x, y)
    for name, x, y, st in zip(("dq", "dk", "dv", "da", "d_init_state"), seg, one,
                              ("bf16", "bf16", "bf16", "f32", "f32")):
        assert_close(to_host64(x).ravel(), to_host64(y).ravel(), TOL["bf16"], name + " vs single pass",
                     store=st, ref_store=st)


def test_segmented_bwd_long_sequence_sampled_heads():
    """B = 1, H = 16, T = 16384 with eight segments; the oracle checks the
    shortest- and the longest-memory heads."""
    inp = I.chunk_inputs(1, 16, 16384, 96, 192, "bf16", seed=99, a_std=0.1, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    run_segmented_bwd_case(inp, schedule32(16, 1.0, 2048.0), 8, units=[(0, 0), (0, 15)])


def test_segmented_bwd_bench_shape_sampled_heads():
    """The backward as the long-sequence benchmark runs it: B = 1, H = 16,
    T = 32768, four segments; the oracle checks the shortest- and the
    longest-memory heads."""
    inp = I.chunk_inputs(1, 16, 32768, 96, 192, "bf16", seed=101, a_std=0.1, s0_std=0.02,
                         with_grad=True, dsf_std=0.02)
    run_segmented_bwd_case(inp, schedule32(16, 1.0, 2048.0), 4, units=[(0, 0), (0, 15)])
