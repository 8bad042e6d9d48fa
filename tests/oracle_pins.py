"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (values printed on the page, closed forms, brute force, finite
differences, invariants).

Each ``check_*`` raises AssertionError on failure. They are collected by
test_oracle_pins.py and re-run against deliberately broken copies of the
oracle by test_oracle_mutations.py, to show that each plausible mistake is
caught by at least one pin.

Page citations name sections of "Beyond the KV cache: Training and serving
i14's Laplace 3B linear attention model on AWS Trainium2 with native PyTorch"
(the Laplace 3B post).
"""
from __future__ import annotations

import os

import numpy as np
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_unit(seed, T, dk, dv, s0=True, a_std=0.3):
    r = _rng(seed)
    q = r.standard_normal((T, dk)) * dk ** -0.5
    k = r.standard_normal((T, dk))
    v = r.standard_normal((T, dv))
    a = r.standard_normal(dk) * a_std
    S0 = r.standard_normal((dk, dv)) * 0.1 if s0 else None
    return q, k, v, a, S0


def brute_force(q, k, v, lam, a, S0):
    """O(T^2) explicit sum: o_t = sum_{s<=t} lam^(t-s) (q_t.k_s) v_s
    + lam^(t+1) S0^T q_t + sigmoid(sum_i a_i q_ti k_ti) v_t, and
    S_final = lam^T S0 + sum_s lam^(T-1-s) k_s v_s^T."""
    T, dk = q.shape
    dv = v.shape[1]
    o = np.zeros((T, dv))
    for t in range(T):
        acc = np.zeros(dv)
        if S0 is not None:
            acc += lam ** (t + 1) * (S0.T @ q[t])
        for s in range(t + 1):
            acc += lam ** (t - s) * float(q[t] @ k[s]) * v[s]
        acc += expit(float(np.sum(a * q[t] * k[t]))) * v[t]
        o[t] = acc
    Sf = np.zeros((dk, dv)) if S0 is None else lam ** T * S0
    for s in range(T):
        Sf = Sf + lam ** (T - 1 - s) * np.outer(k[s], v[s])
    return o, Sf


def _close(x, y, rtol, what):
    x = np.asarray(x)
    y = np.asarray(y)
    scale = max(1.0, float(np.max(np.abs(y)))) if y.size else 1.0
    err = float(np.max(np.abs(x - y))) if y.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


# ---------------------------------------------------------------- schedule


def check_schedule_printed_values():
    """"Decay schedule's reach": lambda_0 = 0.5, lambda_15 ~= 0.9997 at T_min=1, T_max=2048."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "decay_schedule_reach.txt"))
            if ln.strip() and not ln.startswith("#")]
    for H, tmin, tmax, h, lam, tol, hl in rows:
        got = oracle.decay_schedule(int(H), float(tmin), float(tmax))[int(h)]
        assert abs(got - float(lam)) <= float(tol), (h, got, lam)
        # half-life of hl tokens: lam^hl = 1/2
        assert abs(got ** float(hl) - 0.5) < 1e-12, (h, got ** float(hl))


def check_schedule_geometric():
    """"Decay schedule": half-lives spread geometrically from T_min to T_max."""
    for H, tmin, tmax in ((16, 1.0, 2048.0), (2, 1.0, 256.0), (5, 3.0, 7.0)):
        lam = oracle.decay_schedule(H, tmin, tmax)
        half = -1.0 / np.log2(lam)  # half-life in tokens
        assert abs(half[0] - tmin) < 1e-9 * tmax and abs(half[-1] - tmax) < 1e-9 * tmax
        ratios = half[1:] / half[:-1]
        assert np.allclose(ratios, (tmax / tmin) ** (1.0 / (H - 1)), rtol=1e-11, atol=0)
        assert np.all(np.diff(lam) > 0)
    lam1 = oracle.decay_schedule(1, 4.0, 100.0)
    assert abs(lam1[0] - 2.0 ** -0.25) < 1e-15


# ---------------------------------------------------------------- forward


def check_fwd_brute_force():
    """Recurrence == O(T^2) explicit sum (the brute-force evaluation)."""
    for seed, (T, dk, dv), lam in ((1, (9, 3, 5), 0.83), (2, (17, 4, 6), 0.37),
                                   (3, (32, 5, 4), 0.999), (4, (5, 2, 3), 0.5)):
        q, k, v, a, S0 = _rand_unit(seed, T, dk, dv)
        o, Sf = oracle.fwd_unit(q, k, v, lam, a, S0)
        ob, Sb = brute_force(q, k, v, lam, a, S0)
        _close(o, ob, 1e-12, "o vs brute force")
        _close(Sf, Sb, 1e-12, "S_final vs brute force")
        # no initial state
        o, Sf = oracle.fwd_unit(q, k, v, lam, a, None)
        ob, Sb = brute_force(q, k, v, lam, a, None)
        _close(o, ob, 1e-12, "o vs brute force (S0=0)")
        _close(Sf, Sb, 1e-12, "S_final vs brute force (S0=0)")


def check_fwd_lambda_zero():
    """lam = 0: o_t = (q_t.k_t) v_t + sigmoid(z_t) v_t and S_final = k_{T-1} v_{T-1}^T."""
    q, k, v, a, S0 = _rand_unit(11, 7, 4, 6)
    o, Sf = oracle.fwd_unit(q, k, v, 0.0, a, S0)
    z = np.sum(a * q * k, axis=1)
    want = (np.sum(q * k, axis=1) + expit(z))[:, None] * v
    _close(o, want, 1e-14, "lam=0 closed form")
    _close(Sf, np.outer(k[-1], v[-1]), 1e-15, "lam=0 final state")


def check_fwd_lambda_one():
    """lam = 1: plain causal linear attention, a running sum of k_s v_s^T."""
    q, k, v, a, S0 = _rand_unit(12, 13, 3, 5)
    o, Sf = oracle.fwd_unit(q, k, v, 1.0, a, S0)
    outer = np.einsum("ti,tj->tij", k, v)
    S = S0[None] + np.cumsum(outer, axis=0)
    want = np.einsum("tij,ti->tj", S, q) + expit(np.sum(a * q * k, axis=1))[:, None] * v
    _close(o, want, 1e-12, "lam=1 prefix sum")
    _close(Sf, S[-1], 1e-12, "lam=1 final state")


def check_fwd_T1():
    """T = 1: o_0 = lam S0^T q_0 + (q_0.k_0) v_0 + sigmoid(z_0) v_0."""
    q, k, v, a, S0 = _rand_unit(13, 1, 6, 4)
    lam = 0.71
    o, Sf = oracle.fwd_unit(q, k, v, lam, a, S0)
    want = lam * S0.T @ q[0] + float(q[0] @ k[0]) * v[0] + expit(float(np.sum(a * q[0] * k[0]))) * v[0]
    _close(o[0], want, 1e-14, "T=1 closed form")
    _close(Sf, lam * S0 + np.outer(k[0], v[0]), 1e-15, "T=1 final state")


def check_aug_half_skip():
    """"GLA mixer": a = 0 gives a half-strength value skip (sigmoid(0) = 1/2)."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "aug_half_skip.txt"))
            if ln.strip() and not ln.startswith("#")]
    gate = float(rows[0][1])
    q, k, v, a, S0 = _rand_unit(14, 10, 4, 6)
    # q = 0: the readout vanishes and z = 0 for any a -> o = gate * v exactly
    o, _ = oracle.fwd_unit(np.zeros_like(q), k, v, 0.9, a, S0)
    assert np.array_equal(o, gate * v), "q=0 must give exactly half of v"
    # a = 0: o minus the aug-free readout (brute force with the gate removed) = gate * v
    o, _ = oracle.fwd_unit(q, k, v, 0.9, np.zeros_like(a), S0)
    ob, _ = brute_force(q, k, v, 0.9, np.full_like(a, 0.0), S0)
    _close(o, ob, 1e-12, "a=0 brute force")
    ob_noaug = ob - gate * v
    _close(o - ob_noaug, gate * v, 1e-12, "a=0 half skip")


def check_state_carry():
    """Running [0,T) at once == running [0,t0) then [t0,T) from its final state."""
    q, k, v, a, S0 = _rand_unit(15, 23, 4, 5)
    lam = 0.93
    o, Sf = oracle.fwd_unit(q, k, v, lam, a, S0)
    for t0 in (1, 9, 22):
        o1, S1 = oracle.fwd_unit(q[:t0], k[:t0], v[:t0], lam, a, S0)
        o2, S2 = oracle.fwd_unit(q[t0:], k[t0:], v[t0:], lam, a, S1)
        _close(np.concatenate([o1, o2]), o, 1e-13, "split output")
        _close(S2, Sf, 1e-13, "split final state")


def check_varlen_wrapper():
    """Packed batch with cu_seqlens == independent runs per sequence."""
    r = _rng(16)
    L = [3, 8, 1, 6]
    cu = np.concatenate([[0], np.cumsum(L)])
    H, dk, dv = 2, 3, 4
    q = r.standard_normal((1, H, cu[-1], dk))
    k = r.standard_normal((1, H, cu[-1], dk))
    v = r.standard_normal((1, H, cu[-1], dv))
    a = r.standard_normal((H, dk)) * 0.2
    S0 = r.standard_normal((len(L), H, dk, dv)) * 0.1
    lam = np.array([0.5, 0.95])
    o, Sf = oracle.fwd(q, k, v, lam, a, S0, cu_seqlens=cu)
    for n in range(len(L)):
        for h in range(H):
            sl = slice(cu[n], cu[n + 1])
            ob, Sb = brute_force(q[0, h, sl], k[0, h, sl], v[0, h, sl], lam[h], a[h], S0[n, h])
            _close(o[0, h, sl], ob, 1e-12, "varlen o")
            _close(Sf[n, h], Sb, 1e-12, "varlen S_final")


def check_decode_brute_force():
    """A run of decode steps == the brute-force sum over the tokens seen so far."""
    q, k, v, a, S0 = _rand_unit(17, 6, 4, 5)
    lam = 0.8
    S = S0.copy()
    ob, Sb = brute_force(q, k, v, lam, a, S0)
    for t in range(len(q)):
        o = oracle.decode_step_unit(q[t], k[t], v[t], lam, a, S)
        _close(o, ob[t], 1e-12, "decode o")
    _close(S, Sb, 1e-12, "decode state")


# ---------------------------------------------------------------- backward


def _loss(q, k, v, lam, a, S0, dO, dSf):
    o, Sf = oracle.fwd_unit(q, k, v, lam, a, S0)
    return float(np.sum(dO * o) + np.sum(dSf * Sf))


def check_bwd_finite_differences():
    """Analytic gradients == central finite differences of
    L = sum_t dO_t.o_t + sum(dS_final * S_final), every coordinate."""
    for seed, lam in ((21, 0.87), (22, 0.5)):
        T, dk, dv = 16, 4, 8
        q, k, v, a, S0 = _rand_unit(seed, T, dk, dv, a_std=0.8)
        r = _rng(seed + 100)
        dO = r.standard_normal((T, dv))
        dSf = r.standard_normal((dk, dv)) * 0.3
        dq, dk_, dv_, da, dS0 = oracle.bwd_unit(q, k, v, dO, lam, a, S0, dSf)
        params = {"q": q, "k": k, "v": v, "a": a, "S0": S0}
        grads = {"q": dq, "k": dk_, "v": dv_, "a": da, "S0": dS0}
        for name, x in params.items():
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                h = 1e-5 * max(1.0, abs(x[idx]))
                keep = x[idx]
                x[idx] = keep + h
                lp = _loss(**params, lam=lam, dO=dO, dSf=dSf)
                x[idx] = keep - h
                lm = _loss(**params, lam=lam, dO=dO, dSf=dSf)
                x[idx] = keep
                fd[idx] = (lp - lm) / (2 * h)
            scale = max(1e-3, float(np.max(np.abs(fd))))
            err = float(np.max(np.abs(fd - grads[name])))
            assert err <= 1e-6 * scale, f"d{name}: FD err {err:.3e} (scale {scale:.3e})"


def check_bwd_lambda_zero():
    """lam = 0, dS_final = 0: dq_t = (dO_t.v_t) k_t + aug, dk_t = (dO_t.v_t) q_t + aug,
    dv_t = (q_t.k_t) dO_t + sigmoid(z_t) dO_t."""
    T, dk, dv = 9, 3, 5
    q, k, v, a, S0 = _rand_unit(23, T, dk, dv, a_std=0.5)
    dO = _rng(123).standard_normal((T, dv))
    dq, dk_, dv_, da, dS0 = oracle.bwd_unit(q, k, v, dO, 0.0, a, S0, None)
    u = np.sum(dO * v, axis=1)
    s = expit(np.sum(a * q * k, axis=1))
    c = s * (1 - s) * u
    _close(dq, u[:, None] * k + c[:, None] * a[None] * k, 1e-14, "lam=0 dq")
    _close(dk_, u[:, None] * q + c[:, None] * a[None] * q, 1e-14, "lam=0 dk")
    _close(dv_, (np.sum(q * k, axis=1) + s)[:, None] * dO, 1e-14, "lam=0 dv")
    _close(da, np.sum(c[:, None] * q * k, axis=0), 1e-14, "lam=0 da")
    _close(dS0, np.zeros((dk, dv)), 0, "lam=0 dS0")


def check_bwd_at_a_null():
    """a = NULL is the gradient at a = 0 (the initial value of aug_balance,
    "GLA mixer"): dq, dk, dv, da and dS0 from bwd_unit(a=None) equal central
    finite differences of L computed with an explicit zero a, in every
    coordinate. da is not zero there: sigmoid'(0) = 1/4."""
    T, dk, dv, lam = 12, 3, 5, 0.83
    q, k, v, _, S0 = _rand_unit(24, T, dk, dv)
    r = _rng(124)
    dO = r.standard_normal((T, dv))
    dSf = r.standard_normal((dk, dv)) * 0.3
    a0 = np.zeros(dk)
    # the NULL forward branch is the a = 0 brute force
    o, Sf = oracle.fwd_unit(q, k, v, lam, None, S0)
    ob, Sb = brute_force(q, k, v, lam, a0, S0)
    _close(o, ob, 1e-12, "fwd a=NULL vs brute force at a=0")
    _close(Sf, Sb, 1e-12, "fwd a=NULL final state")
    dq, dk_, dv_, da, dS0 = oracle.bwd_unit(q, k, v, dO, lam, None, S0, dSf)
    params = {"q": q, "k": k, "v": v, "a": a0, "S0": S0}
    grads = {"q": dq, "k": dk_, "v": dv_, "a": da, "S0": dS0}
    for name, x in params.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-5 * max(1.0, abs(x[idx]))
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(**params, lam=lam, dO=dO, dSf=dSf)
            x[idx] = keep - h
            lm = _loss(**params, lam=lam, dO=dO, dSf=dSf)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1e-3, float(np.max(np.abs(fd))))
        err = float(np.max(np.abs(fd - grads[name])))
        assert err <= 1e-6 * scale, f"d{name} at a=NULL: FD err {err:.3e} (scale {scale:.3e})"
    assert float(np.max(np.abs(da))) > 1e-3, "da at a = 0 must not vanish"


def check_bwd_varlen_wrapper():
    """The packed batch backward (oracle.bwd with cu_seqlens) against central
    finite differences of the packed batch loss L = sum dO.o + sum dS_final.S_final
    computed through the packed forward (itself pinned to brute force), in
    every coordinate of q, k, v, a and the initial states: distinct initial
    states and final-state gradients per sequence, an empty and a one-token
    sequence, and da summed over sequences."""
    r = _rng(26)
    L = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(L)])
    H, dk, dv = 2, 2, 3
    Tt = int(cu[-1])
    q = r.standard_normal((1, H, Tt, dk)) * 0.7
    k = r.standard_normal((1, H, Tt, dk))
    v = r.standard_normal((1, H, Tt, dv))
    a = r.standard_normal((H, dk)) * 0.5
    S0 = r.standard_normal((len(L), H, dk, dv)) * 0.3
    dO = r.standard_normal((1, H, Tt, dv))
    dSf = r.standard_normal((len(L), H, dk, dv)) * 0.3
    lam = np.array([0.6, 0.9])

    def loss():
        o, Sf = oracle.fwd(q, k, v, lam, a, S0, cu_seqlens=cu)
        return float(np.sum(dO * o) + np.sum(dSf * Sf))

    dq, dk_, dv_, da, dS0 = oracle.bwd(q, k, v, dO, lam, a, S0, dSf, cu_seqlens=cu)
    for name, x, gr in (("q", q, dq), ("k", k, dk_), ("v", v, dv_), ("a", a, da), ("S0", S0, dS0)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-5 * max(1.0, abs(x[idx]))
            keep = x[idx]
            x[idx] = keep + h
            lp = loss()
            x[idx] = keep - h
            lm = loss()
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1e-3, float(np.max(np.abs(fd))))
        err = float(np.max(np.abs(fd - gr)))
        assert err <= 1e-6 * scale, f"packed d{name}: FD err {err:.3e} (scale {scale:.3e})"


# ---------------------------------------------------------- conv prologue


def _silu(x):
    return x * expit(x)


def _conv_case(seed, L, D, st=True, bias=True):
    r = _rng(seed)
    u = r.standard_normal((L, D))
    w = r.standard_normal((D, 4)) * 0.5
    b = r.standard_normal(D) * 0.3 if bias else None
    s0 = r.standard_normal((3, D)) if st else None
    return u, w, b, s0


def check_conv_correlate():
    """Against numpy's cross-correlation, channel by channel: with the history
    p = [u_-3, u_-2, u_-1, u_0, ...], y_t = silu(b + sum_j w_j p_{t+j})."""
    for st in (True, False):
        u, w, b, s0 = _conv_case(31 + st, 11, 5, st=st)
        y, _ = oracle.conv_fwd_unit(u, w, b, s0)
        hist = s0 if s0 is not None else np.zeros((3, 5))
        p = np.concatenate([hist, u], axis=0)
        ref = np.stack([np.correlate(p[:, c], w[c], mode="valid") for c in range(5)], axis=1) + b
        _close(y, _silu(ref), 1e-13, "conv vs correlate")


def check_conv_single_taps():
    """w = e_3 (current token only): y = silu(u + b). w = e_0: y_t = silu(u_{t-3}),
    the first three from the conv state."""
    u, _, b, s0 = _conv_case(33, 9, 4)
    w = np.zeros((4, 4))
    w[:, 3] = 1.0
    y, _ = oracle.conv_fwd_unit(u, w, b, s0)
    _close(y, _silu(u + b), 1e-14, "current tap")
    w = np.zeros((4, 4))
    w[:, 0] = 1.0
    y, _ = oracle.conv_fwd_unit(u, w, None, s0)
    _close(y, _silu(np.concatenate([s0, u[:-3]], axis=0)), 1e-14, "oldest tap")


def check_conv_state_carry():
    """Running [0, L) at once == [0, t0) then [t0, L) from the carried state,
    also for pieces shorter than the three-token state."""
    u, w, b, s0 = _conv_case(35, 10, 6)
    y, sf = oracle.conv_fwd_unit(u, w, b, s0)
    for cuts in ([4], [1, 2], [2, 3, 9]):
        st = s0
        ys = []
        edges = [0] + cuts + [10]
        for a0, a1 in zip(edges, edges[1:]):
            yp, st = oracle.conv_fwd_unit(u[a0:a1], w, b, st)
            ys.append(yp)
        _close(np.concatenate(ys, axis=0), y, 1e-14, f"carry y {cuts}")
        _close(st, sf, 0, f"carry state {cuts}")
    _close(sf, u[-3:], 0, "final state = last three inputs")


def check_conv_decode_steps():
    """Decode steps from the conv state reproduce the sequence forward."""
    u, w, b, s0 = _conv_case(37, 6, 5)
    y, sf = oracle.conv_fwd_unit(u, w, b, s0)
    st = s0.copy()
    yd = np.stack([oracle.conv_decode_step_unit(u[t], w, b, st) for t in range(6)])
    _close(yd, y, 1e-14, "conv decode y")
    _close(st, sf, 0, "conv decode state")


def check_conv_varlen_wrapper():
    """The packed conv (oracle.conv_fwd with cu_seqlens) against numpy's
    cross-correlation per sequence, each sequence with its own initial conv
    state (empty and one-token sequences included), and the final states
    against the last three entries of each sequence's history."""
    r = _rng(39)
    L = [5, 1, 0, 7, 2]
    cu = np.concatenate([[0], np.cumsum(L)])
    D = 3
    u = r.standard_normal((int(cu[-1]), D))
    w = r.standard_normal((D, 4)) * 0.5
    b = r.standard_normal(D) * 0.3
    st = r.standard_normal((len(L), 3, D))
    y, fin = oracle.conv_fwd(u, w, b, st, cu_seqlens=cu)
    for n in range(len(L)):
        p = np.concatenate([st[n], u[cu[n]:cu[n + 1]]], axis=0)
        ref = np.stack([np.correlate(p[:, c], w[c], mode="valid") for c in range(D)], axis=1) + b
        _close(y[cu[n]:cu[n + 1]], _silu(ref[:L[n]]) if L[n] else np.zeros((0, D)), 1e-13,
               f"packed conv y, sequence {n}")
        _close(fin[n], p[-3:], 0, f"packed conv final state, sequence {n}")
    # dense batch rows: the same, one initial state per row
    ud = r.standard_normal((3, 4, D))
    std = r.standard_normal((3, 3, D))
    yd, fd = oracle.conv_fwd(ud, w, None, std)
    for n in range(3):
        p = np.concatenate([std[n], ud[n]], axis=0)
        ref = np.stack([np.correlate(p[:, c], w[c], mode="valid") for c in range(D)], axis=1)
        _close(yd[n], _silu(ref), 1e-13, f"dense conv y, row {n}")
        _close(fd[n], p[-3:], 0, f"dense conv final state, row {n}")


# ------------------------------------------------- mixer epilogue (Head RMSNorm + gate)

def _hng_case(seed, H, d_v, n_tiers, B=1, T=3):
    r = _rng(seed)
    o = r.standard_normal((B, H, T, d_v)) * 0.7
    g = r.standard_normal((B, T, H, d_v)) * 2.0
    gamma = 1.0 + 0.3 * r.standard_normal((n_tiers, d_v))
    return o, g, gamma


def check_hng_unit_rms():
    """With gamma = 1 and eps = 0, dividing out the gate (SiLU from scipy's
    logistic function) leaves every head of every token with mean square
    exactly 1 over its d_v channels, pointing along that head's own o."""
    o, g, _ = _hng_case(41, 4, 24, 2)
    out = oracle.head_norm_gate(o, g, None, 2, 0.0)
    pre = out / _silu(g)
    ms = np.mean(pre ** 2, axis=-1)
    _close(ms, np.ones_like(ms), 1e-12, "unit mean square")
    ratio = pre / np.transpose(o, (0, 2, 1, 3))
    _close(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), 1e-12, "multiple of o")
    assert (ratio > 0).all(), "pre-gate output is not a positive multiple of o"


def check_hng_scale_sign():
    """eps = 0: invariant to a positive scale of the outputs, odd in their
    sign, and invariant to scaling ONE head alone (the statistic is per head,
    not per tier)."""
    o, g, gamma = _hng_case(43, 6, 16, 3, B=2, T=2)
    out = oracle.head_norm_gate(o, g, gamma, 3, 0.0)
    _close(oracle.head_norm_gate(3.7 * o, g, gamma, 3, 0.0), out, 1e-13, "scale")
    _close(oracle.head_norm_gate(-o, g, gamma, 3, 0.0), -out, 1e-13, "sign")
    o2 = o.copy()
    o2[:, 1] *= 5.0
    _close(oracle.head_norm_gate(o2, g, gamma, 3, 0.0), out, 1e-13, "one head scaled")


def check_hng_tiers_and_channels():
    """A constant head vector normalises to +-1 in every channel, so
    out[h][c] = +-silu(g[h][c]) gamma[tier(h)][c]: with distinct gamma entries
    this fixes which tier each head uses (contiguous groups of H / n_tiers)
    and that gamma is indexed by channel."""
    H, d_v, n_tiers = 8, 6, 4
    r = _rng(45)
    vals = r.uniform(0.5, 2.0, H) * np.where(np.arange(H) % 3 == 1, -1.0, 1.0)
    o = np.broadcast_to(vals[None, :, None, None], (1, H, 1, d_v)).copy()
    g = r.standard_normal((1, 1, H, d_v))
    gamma = np.arange(1.0, n_tiers * d_v + 1.0).reshape(n_tiers, d_v)
    out = oracle.head_norm_gate(o, g, gamma, n_tiers, 0.0)
    for h in range(H):
        ref = np.sign(vals[h]) * _silu(g[0, 0, h]) * gamma[h // (H // n_tiers)]
        _close(out[0, 0, h], ref, 1e-14, f"head {h}")


def check_hng_eps():
    """eps sits inside the square root: a constant head of value sqrt(eps)
    normalises to 1/sqrt(2); an all-zero head gives zeros, not NaN."""
    H, d_v, eps = 2, 8, 0.25
    o = np.full((1, H, 1, d_v), 0.5)
    o[0, 1] = 0.0
    g = np.full((1, 1, H, d_v), 3.0)
    out = oracle.head_norm_gate(o, g, None, 1, eps)
    _close(out[0, 0, 0], np.full(d_v, _silu(3.0) / np.sqrt(2.0)), 1e-14, "eps inside sqrt")
    _close(out[0, 0, 1], np.zeros(d_v), 0, "zero head")


def check_hng_gate_silu():
    """The gate is SiLU, channel by channel, also far into both tails: with
    a normalised constant head and gamma = 1, out = g * logistic(g) (scipy)."""
    g = np.array([-30.0, -5.0, -1.0, -1e-3, 0.0, 1e-3, 1.0, 5.0, 30.0])
    d_v = g.size
    out = oracle.head_norm_gate(np.ones((1, 1, 1, d_v)), g.reshape(1, 1, 1, d_v), None, 1, 0.0)
    _close(out[0, 0, 0], g * expit(g), 1e-15, "silu")


def _conv_loss(u, w, b, st, dy, dso):
    y, so = oracle.conv_fwd_unit(u, w, b, st)
    return float(np.sum(dy * y) + np.sum(dso * so))


def check_conv_bwd_finite_differences():
    """Gradients of the conv against central finite differences of
    L = sum(dy * y) + sum(d_final * final_state) in every coordinate of u, the
    initial state, the taps and the bias, for a sequence longer than the
    history (L = 6) and one shorter (L = 2, whose final state reaches into
    the initial state)."""
    for seed, L in ((61, 6), (62, 2)):
        u, w, b, st = _conv_case(seed, L, 3)
        r = _rng(seed + 100)
        dy = r.standard_normal(u.shape)
        dso = r.standard_normal((3, 3))
        du, d_st, dw, db = oracle.conv_bwd_unit(u, w, b, st, dy, dso)
        for name, grad in (("u", du), ("st", d_st), ("w", dw), ("b", db)):
            args = {"u": u, "w": w, "b": b, "st": st}
            x = args[name]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                h = 1e-6 * max(1.0, abs(x[idx]))
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args[name] = xp
                lp = _conv_loss(args["u"], args["w"], args["b"], args["st"], dy, dso)
                args[name] = xm
                lm = _conv_loss(args["u"], args["w"], args["b"], args["st"], dy, dso)
                fd[idx] = (lp - lm) / (2 * h)
            args[name] = x
            err = np.max(np.abs(fd - grad)) / max(np.max(np.abs(fd)), 1e-300)
            assert err < 1e-7, f"conv d{name} (L={L}): FD mismatch {err:.2e}"


def check_conv_bwd_single_tap():
    """w = e_3 (the current token only): y_t = silu(b + u_t), so du_t =
    dy_t silu'(b + u_t) with silu' from scipy's logistic, the initial state
    gets nothing, and the final state's gradient passes straight to the last
    three inputs."""
    L, D = 5, 4
    u, _, b, st = _conv_case(63, L, D)
    w = np.zeros((D, 4))
    w[:, 3] = 1.0
    dy = _rng(64).standard_normal((L, D))
    dso = _rng(65).standard_normal((3, D))
    du, d_st, dw, db = oracle.conv_bwd_unit(u, w, b, st, dy, dso)
    pre = u + b
    sg = expit(pre)
    ref = dy * sg * (1.0 + pre * (1.0 - sg))
    _close(db, ref.sum(axis=0), 1e-13, "db")
    ref = ref.copy()
    ref[L - 3:] += dso
    _close(du, ref, 1e-13, "du")
    _close(d_st, np.zeros((3, D)), 0, "d_st")


def _hng_loss(o, g, gamma, dout, n_tiers, eps):
    return float(np.sum(dout * oracle.head_norm_gate(o, g, gamma, n_tiers, eps)))


def check_hng_bwd_finite_differences():
    """Gradients of the epilogue against central finite differences of
    L = sum(dout * out) in every coordinate of o, g and gamma (eps > 0, two
    tiers, two tokens)."""
    n_tiers, eps = 2, 1e-3
    o, g, gamma = _hng_case(51, 4, 6, n_tiers, B=1, T=2)
    dout = _rng(52).standard_normal(g.shape)
    d_o, dg, dgamma = oracle.head_norm_gate_bwd(o, g, gamma, dout, n_tiers, eps)
    for name, x, grad in (("o", o, d_o), ("g", g, dg), ("gamma", gamma, dgamma)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[idx]))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"o": o, "g": g, "gamma": gamma}
            args[name] = xp
            lp = _hng_loss(args["o"], args["g"], args["gamma"], dout, n_tiers, eps)
            args[name] = xm
            lm = _hng_loss(args["o"], args["g"], args["gamma"], dout, n_tiers, eps)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - grad)) / max(np.max(np.abs(fd)), 1e-300)
        assert err < 1e-7, f"epilogue d{name}: FD mismatch {err:.2e}"


def check_hng_bwd_scale_invariance():
    """eps = 0: the output does not change when a head's o is scaled, so the
    gradient in o is orthogonal to o, head by head; gamma = None matches
    gamma = 1 in every gradient."""
    o, g, gamma = _hng_case(53, 4, 10, 2, B=2, T=3)
    dout = _rng(54).standard_normal(g.shape)
    d_o, _, _ = oracle.head_norm_gate_bwd(o, g, gamma, dout, 2, 0.0)
    dots = np.sum(d_o * o, axis=-1)
    scale = np.sum(np.abs(d_o) * np.abs(o), axis=-1)
    assert np.max(np.abs(dots) / scale) < 1e-13, "d_o not orthogonal to o"
    a = oracle.head_norm_gate_bwd(o, g, None, dout, 2, 1e-4)
    b = oracle.head_norm_gate_bwd(o, g, np.ones_like(gamma), dout, 2, 1e-4)
    for x, y, nm in zip(a, b, ("d_o", "dg", "dgamma")):
        _close(x, y, 0, nm + " (gamma None vs ones)")


ALL_CHECKS = [
    check_schedule_printed_values,
    check_schedule_geometric,
    check_fwd_brute_force,
    check_fwd_lambda_zero,
    check_fwd_lambda_one,
    check_fwd_T1,
    check_aug_half_skip,
    check_state_carry,
    check_varlen_wrapper,
    check_decode_brute_force,
    check_bwd_finite_differences,
    check_bwd_lambda_zero,
    check_bwd_at_a_null,
    check_bwd_varlen_wrapper,
    check_conv_correlate,
    check_conv_single_taps,
    check_conv_state_carry,
    check_conv_decode_steps,
    check_conv_varlen_wrapper,
    check_hng_unit_rms,
    check_hng_scale_sign,
    check_hng_tiers_and_channels,
    check_hng_eps,
    check_hng_gate_silu,
    check_hng_bwd_finite_differences,
    check_hng_bwd_scale_invariance,
    check_conv_bwd_finite_differences,
    check_conv_bwd_single_tap,
]
