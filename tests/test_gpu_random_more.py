"""GPU parity against the fp64 oracle over seeded random configurations: fp32
chunk forward and backward with heads up to 96 x 192 (widths, dense or
packed, chunk lengths, decays 0 and 1, a up to N(0, 2^2)); and the entry
points beside the chunk forward and backward: the segmented forward and
backward (segment counts, ragged lengths, widths, decays 0 and 1, a absent,
moderate or large), the decode
step (pool size, slot tables, both head shapes, several steps), the conv
prologue forward and gradients (width, dense or packed with empty and short
sequences, bias and state on or off) with its decode step, and the mixer
epilogue forward and gradients (width, tiers, scales on or off)."""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, schedule32, to_dev, to_host64
from tests.test_gpu_conv import _check as conv_check
from tests.test_gpu_conv import _dev_inputs as conv_dev
from tests.test_gpu_conv import _ref as conv_ref
from tests.test_gpu_conv_bwd import _check as conv_bwd_check
from tests.test_gpu_conv_bwd import _ref as conv_bwd_ref
from tests.test_gpu_conv_bwd import _run as conv_bwd_run
from tests.test_gpu_decode import _oracle_steps
from tests.test_gpu_norm import EPS
from tests.test_gpu_norm import _dev as norm_dev
from tests.test_gpu_norm import _ref as norm_ref
from tests.test_gpu_norm_bwd import _case as norm_bwd_case
from tests.test_gpu_chunk import run_bwd_case, run_fwd_case
from tests.test_gpu_segmented import run_segmented_bwd_case, run_segmented_case

pytestmark = pytest.mark.gpu

RNG_SEED = 4242


def _lam(rng, H):
    lam = schedule32(H, 1.0, 2048.0).copy()
    if rng.integers(0, 3) == 0:
        lam[int(rng.integers(0, H))] = float(rng.choice([0.0, 1.0, 0.5]))
    return lam


def _f32_cases(n=24):
    rng = np.random.default_rng(RNG_SEED + 20)
    out = []
    for i in range(n):
        H = int(rng.integers(1, 4))
        packed = bool(rng.integers(0, 2))
        L = None
        if packed:
            L = [int(x) for x in rng.choice([0, 1, 2, 31, 33, 64, 65, 100], size=int(rng.integers(2, 5)))]
            if sum(L) == 0:
                L[0] = 5
        out.append(dict(id=i, H=H, L=L, B=1 if packed else int(rng.integers(1, 3)),
                        T=sum(L) if packed else int(rng.integers(1, 160)),
                        d_k=4 * int(rng.integers(1, 25)), d_v=4 * int(rng.integers(1, 49)),
                        chunk=int(rng.choice([32, 64, 128])), a_std=[None, 0.3, 2.0][int(rng.integers(0, 3))],
                        lam=_lam(rng, H)))
    return out


F32 = _f32_cases()


@pytest.mark.parametrize("c", F32, ids=[f"{c['id']}-H{c['H']}-" + (f"packed{c['L']}" if c["L"] else f"B{c['B']}T{c['T']}")
                                        + f"-dk{c['d_k']}dv{c['d_v']}-C{c['chunk']}" for c in F32])
def test_random_f32_fwd_bwd(c):
    cu = None if c["L"] is None else I.cu_from_lengths(c["L"])
    inp = I.chunk_inputs(c["B"], c["H"], c["T"], c["d_k"], c["d_v"], "f32", seed=6500 + c["id"], a_std=c["a_std"],
                         s0_std=0.1, n_seq=None if cu is None else len(c["L"]), with_grad=True, dsf_std=0.1)
    run_fwd_case(inp, c["lam"], c["chunk"], cu=cu)
    run_bwd_case(inp, c["lam"], c["chunk"], cu=cu)


def _seg_cases(n=12):
    rng = np.random.default_rng(RNG_SEED)
    out = []
    for i in range(n):
        H = int(rng.integers(1, 5))
        out.append(dict(id=i, B=int(rng.integers(1, 3)), H=H, T=int(rng.integers(1, 1000)),
                        G=int(rng.integers(1, 13)),
                        d_k=int(rng.choice([8, 32, 48, 96])), d_v=int(rng.choice([8, 64, 104, 192])),
                        a_std=[None, 0.3, 2.0][int(rng.integers(0, 3))],
                        s0_std=None if rng.integers(0, 2) == 0 else 0.05,
                        dsf_std=None if rng.integers(0, 2) == 0 else 0.05, lam=_lam(rng, H)))
    return out


SEG = _seg_cases()


@pytest.mark.parametrize("c", SEG, ids=[f"{c['id']}-B{c['B']}H{c['H']}T{c['T']}G{c['G']}-dk{c['d_k']}dv{c['d_v']}"
                                        for c in SEG])
def test_random_segmented_fwd_bwd(c):
    inp = I.chunk_inputs(c["B"], c["H"], c["T"], c["d_k"], c["d_v"], "bf16", seed=6000 + c["id"],
                         a_std=c["a_std"], s0_std=c["s0_std"], with_grad=True, dsf_std=c["dsf_std"])
    run_segmented_case(inp, c["lam"], c["G"])
    run_segmented_bwd_case(inp, c["lam"], c["G"])


def _dec_cases(n=8):
    rng = np.random.default_rng(RNG_SEED + 1)
    out = []
    for i in range(n):
        dk, dv = ((96, 192), (16, 32), (64, 128), (36, 100))[int(rng.integers(0, 4))]
        N = int(rng.integers(1, 41))
        H = int(rng.integers(1, 5))
        P = N + int(rng.integers(0, 9))
        out.append(dict(id=i, dtype=str(rng.choice(["bf16", "f32"])), dk=dk, dv=dv, N=N, H=H, P=P,
                        slot=bool(rng.integers(0, 2)), steps=int(rng.integers(1, 5)), lam=_lam(rng, H),
                        perm=rng.permutation(P)[:N].astype(np.int32)))
    return out


DEC = _dec_cases()


@pytest.mark.parametrize("c", DEC, ids=[f"{c['id']}-{c['dtype']}-{c['dk']}x{c['dv']}-N{c['N']}P{c['P']}H{c['H']}"
                                        f"-slot{int(c['slot'])}-s{c['steps']}" for c in DEC])
def test_random_decode(c):
    N, H, P, dk, dv, dt = c["N"], c["H"], c["P"], c["dk"], c["dv"], c["dtype"]
    a = I.gaussian(7000 + c["id"], I.STREAM_A, (H, dk), 0.3)
    pool0 = I.gaussian(7000 + c["id"], I.STREAM_S0, (P, H, dk, dv), 0.02)
    page = c["perm"] if c["slot"] else np.arange(N, dtype=np.int32)
    state = to_dev(pool0.copy())
    units = [(n, h) for n in range(N) for h in range(H)]
    Sref = {(n, h): pool0[page[n], h].astype(np.float64).copy() for (n, h) in units}
    toks = [I.decode_token_inputs(7000 + c["id"], s, N, H, dk, dv, dt) for s in range(c["steps"])]
    ref = _oracle_steps([t[0] for t in toks], [t[1] for t in toks], [t[2] for t in toks], c["lam"], a,
                        Sref, units, dt)
    lam_d, a_d = to_dev(c["lam"]), to_dev(a)
    slot_d = to_dev(page) if c["slot"] else None
    for s, (q, k, v) in enumerate(toks):
        o = Bd.sgla_decode_step(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), lam_d, a_d, state, slot=slot_d)
        oh = to_host64(o)
        assert_close(oh.reshape(-1), np.stack([ref[s][u] for u in units]).reshape(-1), TOL[dt],
                     f"o step {s}", store=dt)
    sh = to_host64(state)
    assert_close(np.stack([sh[page[n], h] for (n, h) in units]).reshape(-1),
                 np.stack([Sref[u] for u in units]).reshape(-1), TOL[dt], "state")
    untouched = sorted(set(range(P)) - set(int(x) for x in page))
    for p in untouched:
        assert np.array_equal(sh[p], pool0[p].astype(np.float64)), f"page {p} touched"


def _conv_cases(n=12):
    rng = np.random.default_rng(RNG_SEED + 2)
    out = []
    for i in range(n):
        dt = str(rng.choice(["bf16", "f32"]))
        D = int(rng.integers(1, 97)) * (8 if dt == "bf16" else 4)
        packed = bool(rng.integers(0, 2))
        L = [int(x) for x in rng.choice([0, 1, 2, 3, 4, 5, 63, 64, 65, 130], size=int(rng.integers(1, 6)))]
        if sum(L) == 0:
            L[0] = 3
        out.append(dict(id=i, dtype=dt, D=D, L=L if packed else None, B=int(rng.integers(1, 4)),
                        T=int(rng.integers(1, 200)), bias=bool(rng.integers(0, 2)),
                        state=bool(rng.integers(0, 2))))
    return out


CONV = _conv_cases()


def _conv_name(c):
    lay = f"packed{c['L']}" if c["L"] is not None else f"B{c['B']}T{c['T']}"
    return f"{c['id']}-{c['dtype']}-D{c['D']}-{lay}-bias{int(c['bias'])}-state{int(c['state'])}"


@pytest.mark.parametrize("c", CONV, ids=[_conv_name(c) for c in CONV])
def test_random_conv_fwd_bwd(c):
    if c["L"] is not None:
        cu = I.cu_from_lengths(c["L"])
        shape, n_seq = (int(cu[-1]), c["D"]), len(c["L"])
    else:
        cu, shape, n_seq = None, (c["B"], c["T"], c["D"]), c["B"]
    inp = I.conv_inputs(8000 + c["id"], shape, c["D"], c["dtype"], n_seq, bias=c["bias"], state=c["state"],
                        with_grad=True)
    u, w, b, s0 = conv_dev(inp)
    y, fin = Bd.sgla_conv_fwd(u, w, b, init_state=s0, cu_seqlens=None if cu is None else to_dev(cu),
                              want_final=True)
    torch.cuda.synchronize()
    conv_check(y, fin, conv_ref(inp, cu), inp)
    conv_bwd_check(inp, conv_bwd_run(inp, cu), conv_bwd_ref(inp, cu))


@pytest.mark.parametrize("seed", range(4))
def test_random_conv_decode(seed):
    rng = np.random.default_rng(RNG_SEED + 10 + seed)
    dt = str(rng.choice(["bf16", "f32"]))
    D = int(rng.integers(1, 65)) * 8
    N = int(rng.integers(1, 30))
    P = N + int(rng.integers(0, 6))
    steps = int(rng.integers(1, 5))
    inp = I.conv_inputs(8500 + seed, (N, steps, D), D, dt, P, bias=bool(rng.integers(0, 2)))
    page = rng.permutation(P)[:N].astype(np.int32)
    u, w, b, pool = conv_dev(inp)
    ys = [Bd.sgla_conv_decode_step(u[:, s].contiguous(), w, b, pool, slot=to_dev(page)) for s in range(steps)]
    torch.cuda.synchronize()
    uh = I.widen(inp["u"], dt)
    for n in range(N):
        st = inp["S0"][page[n]].astype(np.float64).copy()
        for s in range(steps):
            r = oracle.conv_decode_step_unit(uh[n, s], inp["w"], inp["b"], st)
            assert_close(to_host64(ys[s][n]), r, TOL[dt], f"decode y n={n} s={s}", store=dt)
        assert np.array_equal(to_host64(pool[page[n]]), st), f"decode state n={n}"


def _norm_cases(n=12):
    rng = np.random.default_rng(RNG_SEED + 3)
    out = []
    for i in range(n):
        H = int(rng.integers(1, 9))
        out.append(dict(id=i, dtype=str(rng.choice(["bf16", "f32"])), B=int(rng.integers(1, 4)), H=H,
                        T=int(rng.integers(1, 150)), d_v=int(rng.integers(1, 65)) * 4,
                        tiers=int(rng.choice([t for t in range(1, H + 1) if H % t == 0])),
                        gamma=bool(rng.integers(0, 2))))
    return out


NORM = _norm_cases()


@pytest.mark.parametrize("c", NORM, ids=[f"{c['id']}-{c['dtype']}-B{c['B']}H{c['H']}T{c['T']}-dv{c['d_v']}"
                                         f"-tiers{c['tiers']}-gamma{int(c['gamma'])}" for c in NORM])
def test_random_norm_fwd_bwd(c):
    inp = I.norm_inputs(9000 + c["id"], c["B"], c["H"], c["T"], c["d_v"], c["tiers"], c["dtype"],
                        gamma=c["gamma"], with_dout=True)
    o, g, gm = norm_dev(inp)
    out = Bd.sgla_head_norm_gate(o, g, gm, c["tiers"], EPS)
    torch.cuda.synchronize()
    assert_close(to_host64(out).ravel(), norm_ref(inp).ravel(), TOL[c["dtype"]], "out", store=c["dtype"])
    norm_bwd_case(inp)
