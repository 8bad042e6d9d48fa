"""Python access to the fp64 Simple GLA oracle (oracle.c).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this package; the library under
``chunked_gated_linear_simple_amd`` never does. It shares no code with the HIP
path: it compiles ``oracle.c`` with the host C compiler and calls it through
ctypes on float64 numpy arrays.

Layouts follow the library's: q, k are [B, H, T, d_k]; v, o, dO are
[B, H, T, d_v]; states are [N, H, d_k, d_v]. With ``cu_seqlens`` (int array of
N+1 offsets) the token axis is packed ([1, H, sum T, d]) and sequence n is the
token range [cu[n], cu[n+1]).

Pins (tests/oracle_pins.py) tie every function here to something other than
itself: the unit functions to brute force, closed forms and finite
differences (also with a = None, the gradient at a = 0), and the batch
wrappers fwd, bwd and conv_fwd to per-sequence brute force, finite
differences of the packed loss and numpy's cross-correlation, with distinct
states per sequence. tests/test_oracle_mutations.py plants mistakes in
oracle.c and in this file and shows that a pin catches each. What no pin can
fix is a reading, not code: the decay schedule's intermediate heads follow
the reading that half-lives are geometric in the head index (the page prints
only the two end values), and the Head RMSNorm's tier grouping follows the
reading of contiguous tiers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, no HIP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.orc_decay_schedule.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, _dp]
        lib.orc_fwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.orc_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.orc_decode_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                        _dp, _dp, _dp, _dp, _dp, _dp]
        lib.orc_conv_fwd.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.orc_conv_decode_step.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, _dp]
        lib.orc_head_norm_gate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, _dp, _dp, _dp, _dp]
        lib.orc_head_norm_gate_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_double, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.orc_conv_bwd.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                     _dp, _dp, _dp]
        for f in (lib.orc_decay_schedule, lib.orc_fwd, lib.orc_bwd, lib.orc_decode_step,
                  lib.orc_conv_fwd, lib.orc_conv_decode_step, lib.orc_head_norm_gate,
                  lib.orc_head_norm_gate_bwd, lib.orc_conv_bwd):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    assert x.dtype == np.float64 and x.flags["C_CONTIGUOUS"]
    return x.ctypes.data_as(_dp)


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def decay_schedule(H: int, t_min: float, t_max: float) -> np.ndarray:
    lam = np.zeros(H, dtype=np.float64)
    _load().orc_decay_schedule(H, t_min, t_max, _ptr(lam))
    return lam


def fwd_unit(q, k, v, lam, a=None, S0=None):
    """One (sequence, head): q,k [T,dk], v [T,dv] -> (o [T,dv], S_final [dk,dv])."""
    q, k, v, a, S0 = map(_f64, (q, k, v, a, S0))
    T, dk = q.shape
    dv = v.shape[1]
    o = np.zeros((T, dv))
    Sf = np.zeros((dk, dv))
    _load().orc_fwd(T, dk, dv, float(lam), _ptr(a), _ptr(q), _ptr(k), _ptr(v), _ptr(S0),
                    _ptr(o), _ptr(Sf))
    return o, Sf


def bwd_unit(q, k, v, dO, lam, a=None, S0=None, dSf=None):
    """One (sequence, head) -> (dq, dk, dv, da [dk], dS0 [dk,dv])."""
    q, k, v, dO, a, S0, dSf = map(_f64, (q, k, v, dO, a, S0, dSf))
    T, dk = q.shape
    dv = v.shape[1]
    dq = np.zeros((T, dk))
    dkk = np.zeros((T, dk))
    dvv = np.zeros((T, dv))
    da = np.zeros(dk)
    dS0 = np.zeros((dk, dv))
    _load().orc_bwd(T, dk, dv, float(lam), _ptr(a), _ptr(q), _ptr(k), _ptr(v), _ptr(S0),
                    _ptr(dO), _ptr(dSf), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(da), _ptr(dS0))
    return dq, dkk, dvv, da, dS0


def decode_step_unit(q, k, v, lam, a, S):
    """One decode step for one (sequence, head); S [dk,dv] is updated in place."""
    q, k, v, a = map(_f64, (q, k, v, a))
    assert S.dtype == np.float64 and S.flags["C_CONTIGUOUS"]
    o = np.zeros(v.shape[0])
    _load().orc_decode_step(q.shape[0], v.shape[0], float(lam), _ptr(a), _ptr(q), _ptr(k),
                            _ptr(v), _ptr(S), _ptr(o))
    return o


def _units(B, H, T, cu_seqlens):
    """(n, h, token slice) for every unit, in (n, h) order."""
    out = []
    if cu_seqlens is None:
        for b in range(B):
            for h in range(H):
                out.append((b, h, b, slice(0, T)))
    else:
        cu = [int(c) for c in cu_seqlens]
        for n in range(len(cu) - 1):
            for h in range(H):
                out.append((n, h, 0, slice(cu[n], cu[n + 1])))
    return out


def fwd(q, k, v, lam, a=None, S0=None, cu_seqlens=None, units=None, threads=1):
    """Batched forward over [B,H,T,d] (or packed with cu_seqlens).

    Returns (o, S_final [N,H,dk,dv]). ``units`` restricts the work to a list of
    (n, h) pairs (the other outputs stay zero)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros(v.shape, dtype=np.float64)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    todo = _units(B, H, T, cu_seqlens)
    if units is not None:
        keep = set((int(n), int(h)) for n, h in units)
        todo = [u for u in todo if (u[0], u[1]) in keep]

    def run(u):
        n, h, b, sl = u
        oo, ss = fwd_unit(q[b, h, sl], k[b, h, sl], v[b, h, sl], lam[h],
                          None if a is None else a[h], None if S0 is None else S0[n, h])
        o[b, h, sl] = oo
        Sf[n, h] = ss

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, todo))
    else:
        for u in todo:
            run(u)
    return o, Sf


def bwd(q, k, v, dO, lam, a=None, S0=None, dSf=None, cu_seqlens=None, units=None, threads=1):
    """Batched backward. Returns (dq, dk, dv, da [H,dk], dS0 [N,H,dk,dv])."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    dq = np.zeros(q.shape)
    dkk = np.zeros(k.shape)
    dvv = np.zeros(v.shape)
    da_parts = {}
    dS0 = np.zeros((N, H, dk, dv))
    todo = _units(B, H, T, cu_seqlens)
    if units is not None:
        keep = set((int(n), int(h)) for n, h in units)
        todo = [u for u in todo if (u[0], u[1]) in keep]

    def run(u):
        n, h, b, sl = u
        r = bwd_unit(q[b, h, sl], k[b, h, sl], v[b, h, sl], dO[b, h, sl], lam[h],
                     None if a is None else a[h], None if S0 is None else S0[n, h],
                     None if dSf is None else dSf[n, h])
        dq[b, h, sl], dkk[b, h, sl], dvv[b, h, sl] = r[0], r[1], r[2]
        da_parts[(n, h)] = r[3]
        dS0[n, h] = r[4]

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, todo))
    else:
        for u in todo:
            run(u)
    da = np.zeros((H, dk))
    for (n, h) in sorted(da_parts):
        da[h] += da_parts[(n, h)]
    return dq, dkk, dvv, da, dS0


# ------------------------------------------------------------ conv prologue


def conv_fwd_unit(u, w, b=None, st=None):
    """One sequence: u [L, D], w [D, 4], b [D] or None, st [3, D] or None ->
    (y [L, D], st_out [3, D])."""
    u, w, b, st = _f64(u), _f64(w), _f64(b), _f64(st)
    L, D = u.shape
    y = np.zeros((L, D))
    st_out = np.zeros((3, D))
    _load().orc_conv_fwd(L, D, _ptr(w), _ptr(b), _ptr(u), _ptr(st), _ptr(y), _ptr(st_out))
    return y, st_out


def conv_fwd(x, w, b=None, st=None, cu_seqlens=None):
    """x [B, T, D] (or packed [S, D] with cu_seqlens); st [N, 3, D] or None.
    Returns (y like x, final state [N, 3, D])."""
    x = np.asarray(x)
    if cu_seqlens is None:
        B, T, D = x.shape
        spans = [(n, None) for n in range(B)]
    else:
        D = x.shape[-1]
        cu = np.asarray(cu_seqlens)
        spans = [(n, (int(cu[n]), int(cu[n + 1]))) for n in range(len(cu) - 1)]
    y = np.zeros(x.shape)
    fin = np.zeros((len(spans), 3, D))
    for n, sp in spans:
        s0 = None if st is None else st[n]
        if sp is None:
            y[n], fin[n] = conv_fwd_unit(x[n], w, b, s0)
        else:
            y[sp[0]:sp[1]], fin[n] = conv_fwd_unit(x[sp[0]:sp[1]], w, b, s0)
    return y, fin


def conv_decode_step_unit(x, w, b, st):
    """x [D]; st [3, D] float64, updated in place. Returns y [D]."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    assert st.dtype == np.float64 and st.flags["C_CONTIGUOUS"]
    y = np.zeros(x.shape[0])
    _load().orc_conv_decode_step(x.shape[0], _ptr(w), _ptr(b), _ptr(x), _ptr(st), _ptr(y))
    return y


def head_norm_gate_token(o, g, gamma, n_tiers, eps):
    """One token: o, g [H, d_v]; gamma [n_tiers, d_v] or None -> out [H, d_v]."""
    o, g, gamma = _f64(o), _f64(g), _f64(gamma)
    H, d_v = o.shape
    out = np.zeros((H, d_v))
    _load().orc_head_norm_gate(H, d_v, int(n_tiers), float(eps), _ptr(o), _ptr(g), _ptr(gamma),
                               _ptr(out))
    return out


def head_norm_gate(o, g, gamma=None, n_tiers=1, eps=1e-6):
    """Mixer epilogue over a batch: o [B, H, T, d_v] (the mixer's layout),
    g [B, T, H, d_v] (token-major gate stream), gamma [n_tiers, d_v] or None.
    Returns out [B, T, H, d_v] (token-major, heads concatenated)."""
    o = np.asarray(o)
    B, H, T, d_v = o.shape
    out = np.zeros((B, T, H, d_v))
    for b in range(B):
        for t in range(T):
            out[b, t] = head_norm_gate_token(o[b, :, t, :], g[b, t], gamma, n_tiers, eps)
    return out


def head_norm_gate_bwd(o, g, gamma, dout, n_tiers=1, eps=1e-6):
    """Gradients of head_norm_gate for L = sum(dout * out): o [B, H, T, d_v],
    g and dout [B, T, H, d_v], gamma [n_tiers, d_v] or None (one). Returns
    (d_o [B, H, T, d_v], dg [B, T, H, d_v], dgamma [n_tiers, d_v]); dgamma is
    the gradient at gamma = 1 when gamma is None."""
    o = np.asarray(o)
    B, H, T, d_v = o.shape
    gam = _f64(gamma)
    d_o = np.zeros((B, H, T, d_v))
    dg = np.zeros((B, T, H, d_v))
    dgamma = np.zeros((n_tiers, d_v))
    lib = _load()
    for b in range(B):
        for t in range(T):
            ot = _f64(o[b, :, t, :])
            do_t = np.zeros((H, d_v))
            dg_t = np.zeros((H, d_v))
            lib.orc_head_norm_gate_bwd(H, d_v, int(n_tiers), float(eps), _ptr(ot), _ptr(_f64(g[b, t])),
                                       _ptr(gam), _ptr(_f64(dout[b, t])), _ptr(do_t), _ptr(dg_t),
                                       _ptr(dgamma))
            d_o[b, :, t, :] = do_t
            dg[b, t] = dg_t
    return d_o, dg, dgamma


def conv_bwd_unit(u, w, b, st, dy, d_st_out=None):
    """Gradients of conv_fwd_unit for one sequence: u, dy [L, D]; w [D, 4];
    b [D] or None; st, d_st_out [3, D] or None. Returns (du [L, D],
    d_st [3, D], dw [D, 4], db [D])."""
    u, w, b, st, dy, dso = _f64(u), _f64(w), _f64(b), _f64(st), _f64(dy), _f64(d_st_out)
    L, D = u.shape
    du = np.zeros((L, D))
    d_st = np.zeros((3, D))
    dw = np.zeros((D, 4))
    db = np.zeros(D)
    _load().orc_conv_bwd(L, D, _ptr(w), _ptr(b), _ptr(u), _ptr(st), _ptr(dy), _ptr(dso), _ptr(du),
                         _ptr(d_st), _ptr(dw), _ptr(db))
    return du, d_st, dw, db
