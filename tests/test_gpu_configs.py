"""The benchmark workloads at their full sizes, in the launch configuration the
bench times, checked against the oracle on every (sequence, head) unit (the
oracle runs one thread per unit on the host's cores), except decode, which
samples 256 of its 20,480 sequence-heads over all 64 steps.

Workloads (H=16, d_k=96, d_v=192, bf16, decays from the 1..2048 schedule):
  Laplace layer fwd:      B=8,  T=2048, chunk 128, a = 0 and a ~ N(0, 0.1)
  Laplace layer fwd+bwd:  B=4,  T=2048, dO ~ N(0, 1); T=64 slice vs finite
                          differences of the oracle
  Decode:                 1280 sequences, state ~ N(0, 0.02), 64 steps
  Packed varlen fwd:      32 sequences, lengths log-uniform in [128, 32768]
                          (one of 32768), init states ~ N(0, 0.02)
  Fused fwd + epilogue:   the Laplace layer fwd with g ~ N(0, 1), 4 tiers of
                          gamma = 1 + N(0, 0.1), out against the oracle's
                          forward followed by its epilogue
"""
import os

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, device_inputs, per_head_report, schedule32, to_dev, to_host64

pytestmark = pytest.mark.gpu

H, DK, DV = 16, 96, 192
LAM = schedule32(H, 1.0, 2048.0)
# host threads for the oracle (the GPU machine's CPU share is 16)
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _wide(inp, names):
    return [None if inp.get(n) is None else I.widen(inp[n], inp["dtype"]) for n in names]


def _finite(t, what):
    assert torch.isfinite(t.float()).all().item(), f"{what}: non-finite values"


@pytest.mark.parametrize("a_std", [None, 0.1], ids=["a_zero", "a_normal"])
def test_laplace_fwd_full(a_std):
    inp = I.chunk_inputs(8, H, 2048, DK, DV, "bf16", seed=2, a_std=a_std)
    d = device_inputs(inp)
    o, Sf = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], to_dev(LAM), d["a"], chunk=128,
                              want_final=True)
    torch.cuda.synchronize()
    _finite(o, "o")
    _finite(Sf, "final_state")
    q, k, v = _wide(inp, ("q", "k", "v"))
    o_ref, S_ref = oracle.fwd(q, k, v, LAM.astype(np.float64), inp["a"].astype(np.float64), threads=THREADS)
    oh, Sh = to_host64(o), to_host64(Sf)
    units = [(n, h) for n in range(8) for h in range(H)]
    per_head_report("o", {u: oh[u] for u in units}, {u: o_ref[u] for u in units}, "bf16")
    assert_close(oh, o_ref, TOL["bf16"], "o (all 128 units)", store="bf16")
    assert_close(Sh, S_ref, TOL["bf16"], "final_state (all 128 units)")


@pytest.mark.parametrize("a_std", [None, 0.1], ids=["a_zero", "a_normal"])
def test_laplace_fwd_bwd_full(a_std):
    inp = I.chunk_inputs(4, H, 2048, DK, DV, "bf16", seed=3, a_std=a_std, with_grad=True)
    d = device_inputs(inp)
    lam = to_dev(LAM)
    o, _ = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam, d["a"], chunk=128)
    dq, dk, dv, da, _ = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam, d["a"], chunk=128)
    torch.cuda.synchronize()
    for t, nm in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv"), (da, "da")):
        _finite(t, nm)
    q, k, v, dO = _wide(inp, ("q", "k", "v", "dO"))
    lam64, a64 = LAM.astype(np.float64), inp["a"].astype(np.float64)
    ref = oracle.bwd(q, k, v, dO, lam64, a64, threads=THREADS)
    units = [(b, h) for b in range(4) for h in range(H)]
    for idx, (nm, t) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        th = to_host64(t)
        per_head_report(nm, {u: th[u] for u in units}, {u: ref[idx][u] for u in units}, "bf16")
        assert_close(th, ref[idx], TOL["bf16"], nm + " (all 64 units)", store="bf16")
    assert_close(to_host64(da), ref[3], TOL["bf16"], "da (all 16 heads)")
    o_ref, _ = oracle.fwd(q, k, v, lam64, a64, threads=THREADS)
    assert_close(to_host64(o), o_ref, TOL["bf16"], "o (all 64 units)", store="bf16")


def test_laplace_bwd_slice_finite_differences():
    """GPU gradients on the T=64 slice (batch row 0, all 16 heads, zero initial
    state) against central finite differences of the fp64 oracle loss
    L = sum dO . o: 512 sampled coordinates of each of q, k, v and a, plus 8
    random directions through all four at once (the directional derivative
    against sum grad . direction)."""
    from concurrent.futures import ThreadPoolExecutor
    full = I.chunk_inputs(4, H, 2048, DK, DV, "bf16", seed=3, a_std=0.1, with_grad=True)
    sl = {k: (v[0:1, :, :64].copy() if isinstance(v, np.ndarray) and v.ndim == 4 else v)
          for k, v in full.items()}
    d = device_inputs(sl)
    dq, dk, dv, da, _ = Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], to_dev(LAM), d["a"],
                                          chunk=128)
    torch.cuda.synchronize()
    g = {"q": to_host64(dq)[0], "k": to_host64(dk)[0], "v": to_host64(dv)[0], "a": to_host64(da)}
    X = {nm: I.widen(sl[nm][0], "bf16") for nm in ("q", "k", "v")}
    X["a"] = sl["a"].astype(np.float64)
    dO = I.widen(sl["dO"][0], "bf16")

    def loss_head(P, h):
        """L restricted to head h (the other heads do not depend on its inputs)."""
        o, _ = oracle.fwd_unit(P["q"][h], P["k"][h], P["v"][h], float(LAM[h]), P["a"][h], None)
        return float(np.sum(dO[h] * o))

    def fd_coord(nm, idx):
        h = idx[0]
        keep = X[nm][idx]
        step = 1e-4 * max(1.0, abs(keep))
        P = {k: v.copy() if k == nm else v for k, v in X.items()}
        P[nm][idx] = keep + step
        lp = loss_head(P, h)
        P[nm][idx] = keep - step
        lm = loss_head(P, h)
        return (lp - lm) / (2 * step)

    rng = np.random.default_rng(64)
    with ThreadPoolExecutor(8) as ex:
        for nm in ("q", "k", "v", "a"):
            arr = X[nm]
            idxs = [tuple(int(rng.integers(0, s)) for s in arr.shape) for _ in range(512)]
            fd = np.array(list(ex.map(lambda i: fd_coord(nm, i), idxs)))
            an = np.array([g[nm][i] for i in idxs])
            assert_close(an, fd, TOL["bf16"], f"d{nm} vs finite differences (512 coordinates)",
                         store="f32" if nm == "a" else "bf16")
        # 8 random directions through q, k, v and a at once
        for r in range(8):
            D = {nm: rng.standard_normal(X[nm].shape) for nm in X}
            want = sum(float(np.sum(g[nm] * D[nm])) for nm in X)
            eps = 1e-4

            def shifted(sign):
                P = {nm: X[nm] + sign * eps * D[nm] for nm in X}
                return sum(ex.map(lambda h: loss_head(P, h), range(H)))

            fd = (shifted(1.0) - shifted(-1.0)) / (2 * eps)
            err = abs(want - fd) / max(abs(fd), 1e-12)
            print(f"    direction {r}: analytic {want:.6e} fd {fd:.6e} rel err {err:.2e}", flush=True)
            assert err <= TOL["bf16"], f"direction {r}: relative error {err:.3e}"


def test_decode_full_64_steps():
    N, steps = 1280, 64
    S0 = I.gaussian(4, I.STREAM_S0, (N, H, DK, DV), 0.02)
    a = I.gaussian(4, I.STREAM_A, (H, DK), 0.1)
    state = to_dev(S0)
    units = sorted(set([(0, 0), (0, 15), (1279, 0), (1279, 15)] +
                       [(int(n), int(h)) for n, h in zip(np.linspace(0, N - 1, 252).round(), np.arange(252) % H)]))
    Sref = {u: S0[u].astype(np.float64).copy() for u in units}
    del S0
    lam_d, a_d = to_dev(LAM), to_dev(a)
    for s in range(steps):
        q, k, v = I.decode_token_inputs(4, s, N, H, DK, DV, "bf16")
        o = Bd.sgla_decode_step(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), lam_d,
                                a_d, state)
        oh = to_host64(o)
        assert np.isfinite(oh).all()
        want = []
        for (n, h) in units:
            want.append(oracle.decode_step_unit(I.widen(q[n, h], "bf16"), I.widen(k[n, h], "bf16"),
                                                I.widen(v[n, h], "bf16"), float(LAM[h]),
                                                a[h].astype(np.float64), Sref[(n, h)]))
        got = np.stack([oh[u] for u in units])
        assert_close(got, np.stack(want), TOL["bf16"], f"o step {s}", store="bf16")
    _finite(state, "state")
    sh = torch.stack([state[n, h] for n, h in units]).double().cpu().numpy()
    assert_close(sh, np.stack([Sref[u] for u in units]), TOL["bf16"], "final state")


def test_varlen_full():
    L = I.varlen_lengths(5)
    cu = I.cu_from_lengths(L)
    inp = I.chunk_inputs(1, H, int(cu[-1]), DK, DV, "bf16", seed=5, a_std=0.1, s0_std=0.02,
                         n_seq=len(L))
    d = device_inputs(inp, cu)
    o, Sf = Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], to_dev(LAM), d["a"], init_state=d["S0"],
                              cu_seqlens=d["cu"], chunk=128, want_final=True)
    torch.cuda.synchronize()
    _finite(o, "o")
    _finite(Sf, "final_states")
    q, k, v = _wide(inp, ("q", "k", "v"))
    o_ref, S_ref = oracle.fwd(q, k, v, LAM.astype(np.float64), inp["a"].astype(np.float64),
                              inp["S0"].astype(np.float64), cu_seqlens=cu, threads=THREADS)
    assert_close(to_host64(o), o_ref, TOL["bf16"], "o (all 512 units)", store="bf16")
    assert_close(to_host64(Sf), S_ref, TOL["bf16"], "final_states (all 512 units)")


def test_laplace_fwd_norm_gate_full():
    """sgla_chunk_fwd_norm_gate at B=8, T=2048 (one launch of 256 workgroups),
    the launch the bench times: every unit's out rows and final state against
    the oracle."""
    tiers, eps = 4, 1e-6
    inp = I.chunk_inputs(8, H, 2048, DK, DV, "bf16", seed=6, a_std=0.1)
    gi = I.norm_inputs(6, 8, H, 2048, DV, tiers, "bf16")
    d = device_inputs(inp)
    x = torch.zeros(Bd.FWD_NORM_GATE_EXCHANGE_BYTES, dtype=torch.uint8, device="cuda")
    out, _, Sf = Bd.sgla_chunk_fwd_norm_gate(d["q"], d["k"], d["v"], to_dev(LAM), to_dev(gi["g"], "bf16"),
                                             a=d["a"], gamma=to_dev(gi["gamma"]), n_tiers=tiers, eps=eps,
                                             chunk=128, want_final=True, exchange=x)
    torch.cuda.synchronize()
    _finite(out, "out")
    assert int(torch.count_nonzero(x).item()) == 0, "exchange buffer not zero-filled after the call"
    q, k, v = _wide(inp, ("q", "k", "v"))
    o_ref, S_ref = oracle.fwd(q, k, v, LAM.astype(np.float64), inp["a"].astype(np.float64), threads=THREADS)
    out_ref = oracle.head_norm_gate(o_ref, I.widen(gi["g"], "bf16"), gi["gamma"].astype(np.float64), tiers, eps)
    assert_close(to_host64(out), out_ref, TOL["bf16"], "out (all 128 units)", store="bf16")
    assert_close(to_host64(Sf), S_ref, TOL["bf16"], "final_state (all 128 units)")
