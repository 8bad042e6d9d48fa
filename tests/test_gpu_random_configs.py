"""GPU parity of sgla_chunk_fwd / sgla_chunk_bwd against the fp64 oracle on a
fixed list of pseudo-random configurations: dtype, head widths (including
partial value slices and widths below a tile), sequence lengths (dense, or
packed with empty and one-token sequences), chunk length, decays (including
0 and 1), and whether a, the initial state and the final state's gradient are
given. Each case is small enough for the oracle to check every unit. The bf16
cases also run the forward with the mixer epilogue before the store
(sgla_chunk_fwd_norm_gate) with a random tier count and with or without scales."""
import numpy as np
import pytest
import torch

from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import TOL, assert_close, device_inputs, oracle_fwd_units, schedule32, to_dev, to_host64
from tests.test_gpu_chunk import run_bwd_case, run_fwd_case
from tests.test_gpu_fwd_norm_gate import EPS, _check_exchange, _gate_inputs, _out_unit, _ref_out

pytestmark = pytest.mark.gpu


def _cases(n=64, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        f32 = i % 6 == 5
        if f32:
            d_k = int(rng.choice([4, 8, 16, 24, 32]))
            d_v = int(rng.choice([4, 12, 16, 32]))
        else:
            d_k = int(rng.choice([8, 16, 24, 40, 64, 72, 96]))
            d_v = int(rng.choice([8, 32, 56, 96, 104, 136, 192]))
        H = int(rng.integers(1, 5))
        packed = bool(rng.integers(0, 2))
        if packed:
            L = [int(x) for x in rng.choice([0, 1, 2, 31, 33, 64, 65, 127, 129, 200, 257], size=int(rng.integers(2, 6)))]
            if sum(L) == 0:
                L[0] = 5
            B, T = 1, sum(L)
        else:
            L = None
            B, T = int(rng.integers(1, 4)), int(rng.integers(1, 330))
        lam = schedule32(H, 1.0, 2048.0)
        if rng.integers(0, 3) == 0:  # edge decays on some heads
            lam = lam.copy()
            lam[int(rng.integers(0, H))] = float(rng.choice([0.0, 1.0, 0.5]))
        out.append(dict(
            id=i, dtype="f32" if f32 else "bf16", B=B, H=H, T=T, d_k=d_k, d_v=d_v, L=L,
            chunk=int(rng.choice([32, 64, 128])), lam=lam,
            a_std=None if rng.integers(0, 3) == 0 else float(rng.choice([0.1, 0.5, 1.0])),
            s0_std=None if rng.integers(0, 2) == 0 else 0.05,
            dsf_std=None if rng.integers(0, 2) == 0 else 0.05,
            tiers=int(rng.choice([t for t in (1, 2, 4) if H % t == 0])),
            gamma=bool(rng.integers(0, 2)),
        ))
    return out


CASES = _cases()


def _name(c):
    lay = f"packed{c['L']}" if c["L"] is not None else f"B{c['B']}T{c['T']}"
    return f"{c['id']}-{c['dtype']}-H{c['H']}-{lay}-dk{c['d_k']}-dv{c['d_v']}-C{c['chunk']}"


@pytest.mark.parametrize("case", CASES, ids=[_name(c) for c in CASES])
def test_random_config_fwd_bwd(case):
    c = case
    cu = None if c["L"] is None else I.cu_from_lengths(c["L"])
    n_seq = None if c["L"] is None else len(c["L"])
    inp = I.chunk_inputs(c["B"], c["H"], c["T"], c["d_k"], c["d_v"], c["dtype"], seed=5000 + c["id"],
                         a_std=c["a_std"], s0_std=c["s0_std"], n_seq=n_seq, with_grad=True,
                         dsf_std=c["dsf_std"])
    print("case", _name(c), flush=True)
    run_fwd_case(inp, c["lam"], c["chunk"], cu=cu)
    run_bwd_case(inp, c["lam"], c["chunk"], cu=cu)


BF16 = [c for c in CASES if c["dtype"] == "bf16"]


@pytest.mark.parametrize("case", BF16, ids=[_name(c) for c in BF16])
def test_random_config_fwd_norm_gate(case):
    c = case
    cu = None if c["L"] is None else I.cu_from_lengths(c["L"])
    N = c["B"] if c["L"] is None else len(c["L"])
    inp = I.chunk_inputs(c["B"], c["H"], c["T"], c["d_k"], c["d_v"], "bf16", seed=5000 + c["id"],
                         a_std=c["a_std"], s0_std=c["s0_std"], n_seq=None if cu is None else N)
    gi = _gate_inputs(5000 + c["id"], c["B"], c["H"], c["T"], c["d_v"], c["tiers"], c["gamma"])
    d = device_inputs(inp, cu)
    x = torch.zeros(Bd.FWD_NORM_GATE_EXCHANGE_BYTES, dtype=torch.uint8, device="cuda")
    print("case", _name(c), "tiers", c["tiers"], "gamma", c["gamma"], flush=True)
    out, _, Sf = Bd.sgla_chunk_fwd_norm_gate(d["q"], d["k"], d["v"], to_dev(c["lam"]), to_dev(gi["g"], "bf16"),
                                             a=d["a"], gamma=to_dev(gi["gamma"]), n_tiers=c["tiers"], eps=EPS,
                                             init_state=d["S0"], cu_seqlens=d["cu"], chunk=c["chunk"],
                                             want_final=True, exchange=x)
    _check_exchange(x)
    units = [(n, h) for n in range(N) for h in range(c["H"])]
    ref = _ref_out(inp, c["lam"], gi, c["tiers"], units, cu)
    oh = to_host64(out)
    assert_close(np.concatenate([_out_unit(oh, n, h, cu).ravel() for n, h in units]),
                 np.concatenate([ref[u].ravel() for u in units]), TOL["bf16"], "out", store="bf16")
    fw = oracle_fwd_units(inp, c["lam"], units, cu)
    Sh = to_host64(Sf)
    assert_close(np.concatenate([Sh[u].ravel() for u in units]),
                 np.concatenate([fw[u][1].ravel() for u in units]), TOL["bf16"], "final_state")
