"""GPU parity of sgla_decode_step against the fp64 oracle (the two tuned
head shapes and a spread of others), its page indirection, batch invariance
and its agreement with the chunked forward."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, schedule32, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _oracle_steps(qs, ks, vs, lam, a, S, units, dtype):
    """Run the oracle decode over steps for the given (n, h) units; S[(n,h)] updated."""
    outs = []
    for q, k, v in zip(qs, ks, vs):
        qw, kw, vw = I.widen(q, dtype), I.widen(k, dtype), I.widen(v, dtype)
        o = {}
        for (n, h) in units:
            o[(n, h)] = oracle.decode_step_unit(qw[n, h], kw[n, h], vw[n, h], float(lam[h]),
                                                a[h].astype(np.float64), S[(n, h)])
        outs.append(o)
    return outs


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 96, 192), ("f32", 16, 32),
                                         ("bf16", 16, 32),
                                         # other head widths: the next larger thread layout, masked
                                         ("bf16", 64, 128), ("f32", 32, 64), ("bf16", 72, 136), ("bf16", 8, 8),
                                         ("f32", 96, 96), ("bf16", 48, 192), ("f32", 4, 4), ("bf16", 40, 20),
                                         ("f32", 92, 188)])
def test_decode_steps_vs_oracle(dtype, dk, dv):
    N, H, steps = 19, 16 if dk == 96 else 2, 6
    lam = schedule32(H, 1.0, 2048.0)
    a = I.gaussian(7, I.STREAM_A, (H, dk), 0.1)
    S0 = I.gaussian(7, I.STREAM_S0, (N, H, dk, dv), 0.02)
    state = to_dev(S0.copy())
    units = [(n, h) for n in range(N) for h in range(H)]
    Sref = {u: S0[u].astype(np.float64).copy() for u in units}
    toks = [I.decode_token_inputs(7, s, N, H, dk, dv, dtype) for s in range(steps)]
    ref = _oracle_steps([t[0] for t in toks], [t[1] for t in toks], [t[2] for t in toks], lam, a,
                        Sref, units, dtype)
    lam_d, a_d = to_dev(lam), to_dev(a)
    for s, (q, k, v) in enumerate(toks):
        o = Bd.sgla_decode_step(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), lam_d, a_d,
                                state)
        oh = to_host64(o)
        assert_close(oh.reshape(-1), np.stack([ref[s][u] for u in units]).reshape(-1),
                     TOL[dtype], f"o step {s}", store=dtype)
    sh = to_host64(state)
    assert_close(sh.reshape(-1), np.stack([Sref[u] for u in units]).reshape(-1), TOL[dtype],
                 "state")


def test_decode_slots_and_invalid_slot():
    N, P, H, dk, dv = 5, 9, 16, 96, 192
    lam = to_dev(schedule32(H, 1.0, 2048.0))
    a = I.gaussian(8, I.STREAM_A, (H, dk), 0.1)
    pool = I.gaussian(8, I.STREAM_S0, (P, H, dk, dv), 0.02)
    q, k, v = I.decode_token_inputs(8, 0, N, H, dk, dv, "bf16")
    slot = np.array([7, 2, -1, 4, 9], np.int32)  # -1 and 9 are outside [0, P)
    state = to_dev(pool.copy())
    o = Bd.sgla_decode_step(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), lam,
                            to_dev(a), state, slot=to_dev(slot))
    oh, sh = to_host64(o), to_host64(state)
    lamh = schedule32(H, 1.0, 2048.0)
    touched = set()
    for n in range(N):
        p = int(slot[n])
        if p < 0 or p >= P:
            assert np.isnan(oh[n]).all()
            continue
        touched.add(p)
        for h in range(H):
            S = pool[p, h].astype(np.float64).copy()
            ro = oracle.decode_step_unit(I.widen(q[n, h], "bf16"), I.widen(k[n, h], "bf16"),
                                         I.widen(v[n, h], "bf16"), float(lamh[h]),
                                         a[h].astype(np.float64), S)
            assert_close(oh[n, h], ro, TOL["bf16"], f"o n={n} h={h}", store="bf16")
            assert_close(sh[p, h], S, TOL["bf16"], f"state page {p} h={h}")
    for p in range(P):
        if p not in touched:
            assert np.array_equal(sh[p], pool[p].astype(np.float64)), f"page {p} modified"


def test_decode_batch_invariance_bitwise():
    """A sequence's output does not depend on N or on its position in the batch."""
    H, dk, dv = 16, 96, 192
    lam = to_dev(schedule32(H, 1.0, 2048.0))
    a = to_dev(I.gaussian(9, I.STREAM_A, (H, dk), 0.1))
    pool = I.gaussian(9, I.STREAM_S0, (40, H, dk, dv), 0.02)
    q, k, v = I.decode_token_inputs(9, 0, 40, H, dk, dv, "bf16")
    full_state = to_dev(pool.copy())
    o_full = Bd.sgla_decode_step(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), lam, a,
                                 full_state)
    # sequence 33 alone, as batch position 0 with N = 1
    one_state = to_dev(pool[33:34].copy())
    o_one = Bd.sgla_decode_step(to_dev(q[33:34], "bf16"), to_dev(k[33:34], "bf16"),
                                to_dev(v[33:34], "bf16"), lam, a, one_state)
    assert torch.equal(o_one[0], o_full[33])
    assert torch.equal(one_state[0], full_state[33])
    # sequence 33 at position 2 of a permuted batch with page indirection
    perm = np.array([5, 11, 33, 0], np.int32)
    st = to_dev(pool.copy())
    o_perm = Bd.sgla_decode_step(to_dev(q[perm], "bf16"), to_dev(k[perm], "bf16"),
                                 to_dev(v[perm], "bf16"), lam, a, st, slot=to_dev(perm))
    assert torch.equal(o_perm[2], o_full[33])
    assert torch.equal(st[33], full_state[33])


def test_decode_matches_chunk_fwd():
    """T decode steps from S0 == one chunked forward over the same T tokens."""
    N, H, dk, dv, T = 3, 16, 96, 192, 70
    lam = to_dev(schedule32(H, 1.0, 2048.0))
    inp = I.chunk_inputs(N, H, T, dk, dv, "bf16", seed=11, a_std=0.1, s0_std=0.02)
    q, k, v = (to_dev(inp[x], "bf16") for x in ("q", "k", "v"))
    a, S0 = to_dev(inp["a"]), to_dev(inp["S0"])
    o_chunk, S_chunk = Bd.sgla_chunk_fwd(q, k, v, lam, a, init_state=S0, want_final=True)
    state = S0.clone()
    outs = []
    for t in range(T):
        outs.append(Bd.sgla_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                        v[:, :, t].contiguous(), lam, a, state))
    o_dec = torch.stack(outs, dim=2)
    assert_close(to_host64(o_dec), to_host64(o_chunk), TOL["bf16"], "decode vs chunk o",
                 store="bf16", ref_store="bf16")
    assert_close(to_host64(state), to_host64(S_chunk), TOL["bf16"], "decode vs chunk state")
