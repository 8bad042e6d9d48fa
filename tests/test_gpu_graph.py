"""HIP graph capture of the entry points. The library allocates nothing,
clears nothing with a memset and never synchronises: every buffer, workspace
and exchange buffer is the caller's, so a call can be recorded into a graph
on the caller's stream. Each test captures one call (outputs, workspaces and
exchange buffer allocated beforehand), replays it several times with eager
work (the outputs poisoned with NaN) and a synchronisation between the
replays, and compares every replay bit for bit with an eager call on the
same inputs; the kernels are deterministic, so any difference is a replay
that read or wrote something other than the eager call did."""
import numpy as np
import pytest
import torch

from chunked_gated_linear_simple_amd import binding as Bd
from chunked_gated_linear_simple_amd import inputs as I
from tests.parity_util import device_inputs, schedule32, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _poison(ts):
    for t in ts:
        t.fill_(float("nan"))


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _check_replays(g, outs, want, before=None):
    for r in range(REPLAYS):
        _poison(outs)
        if before is not None:
            before()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert torch.equal(t, w), f"replay {r}, output {i}"


def _chunk_case(seed, with_grad=False):
    B, H, T, dk, dv = 2, 4, 300, 96, 192
    inp = I.chunk_inputs(B, H, T, dk, dv, "bf16", seed=seed, a_std=0.3, s0_std=0.05, with_grad=with_grad,
                         dsf_std=0.05 if with_grad else None)
    return inp, device_inputs(inp), to_dev(schedule32(H, 1.0, 2048.0))


def test_graph_chunk_fwd():
    inp, d, lam = _chunk_case(9100)
    B, H, T, dk, dv = inp["B"], inp["H"], inp["T"], inp["d_k"], inp["d_v"]

    def call(o, sf):
        Bd.sgla_chunk_fwd(d["q"], d["k"], d["v"], lam, d["a"], init_state=d["S0"], final_state=sf, o=o,
                          chunk=128)

    o_e = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda")
    sf_e = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    call(o_e, sf_e)
    o_g, sf_g = torch.empty_like(o_e), torch.empty_like(sf_e)
    g = _capture(lambda: call(o_g, sf_g))
    _check_replays(g, [o_g, sf_g], [o_e, sf_e])


def test_graph_chunk_bwd():
    inp, d, lam = _chunk_case(9101, with_grad=True)
    B, H, dk = inp["B"], inp["H"], inp["d_k"]
    ws = torch.empty(max(Bd.sgla_chunk_bwd_workspace_bytes(B, H, dk), 16), dtype=torch.uint8, device="cuda")

    def outs():
        return [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
                torch.empty((H, dk), dtype=torch.float32, device="cuda"), torch.empty_like(d["S0"])]

    def call(t):
        Bd.sgla_chunk_bwd(d["q"], d["k"], d["v"], d["dO"], lam, d["a"], init_state=d["S0"],
                          d_final_state=d["dSf"], chunk=128, dq=t[0], dk=t[1], dv=t[2], da=t[3],
                          d_init_state=t[4], workspace=ws)

    e = outs()
    call(e)
    t = outs()
    g = _capture(lambda: call(t))
    _check_replays(g, t, e)


def test_graph_chunk_fwd_norm_gate():
    """The fused forward takes its tickets from counters in the exchange
    buffer, which each call leaves zero-filled, so replays need no reset."""
    inp, d, lam = _chunk_case(9102)
    B, H, T, dv, tiers = inp["B"], inp["H"], inp["T"], inp["d_v"], 2
    gi = I.norm_inputs(9102, B, H, T, dv, tiers, "bf16")
    gt, gm = to_dev(gi["g"], "bf16"), to_dev(gi["gamma"])
    x = torch.zeros(Bd.FWD_NORM_GATE_EXCHANGE_BYTES, dtype=torch.uint8, device="cuda")

    def call(out, sf):
        Bd.sgla_chunk_fwd_norm_gate(d["q"], d["k"], d["v"], lam, gt, a=d["a"], gamma=gm, n_tiers=tiers, eps=1e-6,
                                    init_state=d["S0"], final_state=sf, out=out, chunk=128, exchange=x)

    out_e = torch.empty_like(gt)
    sf_e = torch.empty_like(d["S0"])
    call(out_e, sf_e)
    out_g, sf_g = torch.empty_like(out_e), torch.empty_like(sf_e)
    g = _capture(lambda: call(out_g, sf_g))
    _check_replays(g, [out_g, sf_g], [out_e, sf_e])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(x).item()) == 0, "the exchange buffer is not zero-filled after the replays"


def test_graph_chunk_fwd_segmented():
    inp, d, lam = _chunk_case(9103)
    B, H, dk, dv = inp["B"], inp["H"], inp["d_k"], inp["d_v"]
    nseg = 3
    ws = torch.empty((max(Bd.sgla_chunk_fwd_segmented_workspace_bytes(B, H, dk, dv, nseg), 16) + 3) // 4,
                     dtype=torch.float32, device="cuda")

    def call(o, sf):
        Bd.sgla_chunk_fwd_segmented(d["q"], d["k"], d["v"], lam, d["a"], init_state=d["S0"], final_state=sf,
                                    o=o, n_segments=nseg, chunk=128, workspace=ws)

    o_e = torch.empty_like(d["v"])
    sf_e = torch.empty_like(d["S0"])
    call(o_e, sf_e)
    o_g, sf_g = torch.empty_like(o_e), torch.empty_like(sf_e)
    g = _capture(lambda: call(o_g, sf_g))
    _check_replays(g, [o_g, sf_g], [o_e, sf_e])


def test_graph_decode_step():
    """The decode step updates the state pool in place: before each replay
    the pool is restored (eager copy), and o and the pool must equal one
    eager step's."""
    N, H, dk, dv, P = 40, 4, 96, 192, 44
    a = to_dev(I.gaussian(9104, I.STREAM_A, (H, dk), 0.3))
    pool0 = to_dev(I.gaussian(9104, I.STREAM_S0, (P, H, dk, dv), 0.02))
    q, k, v = (to_dev(x, "bf16") for x in I.decode_token_inputs(9104, 0, N, H, dk, dv, "bf16"))
    lam = to_dev(schedule32(H, 1.0, 2048.0))
    slot = to_dev(np.random.default_rng(9104).permutation(P)[:N].astype(np.int32))
    pool_e = pool0.clone()
    o_e = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    Bd.sgla_decode_step(q, k, v, lam, a, pool_e, o=o_e, slot=slot)
    pool_g = pool0.clone()
    o_g = torch.empty_like(o_e)
    g = _capture(lambda: Bd.sgla_decode_step(q, k, v, lam, a, pool_g, o=o_g, slot=slot))
    _check_replays(g, [o_g], [o_e], before=lambda: pool_g.copy_(pool0))
    assert torch.equal(pool_g, pool_e)


def test_graph_conv_fwd_and_head_norm_gate():
    """The conv prologue and the epilogue on its own, captured in one graph
    one after the other, as a layer would run them."""
    B, T, D = 2, 150, 384
    inp = I.conv_inputs(9105, (B, T, D), D, "bf16", B)
    u = to_dev(inp["u"], "bf16")
    w, b, s0 = to_dev(inp["w"]), to_dev(inp["b"]), to_dev(inp["S0"])
    H, dv, tiers = 4, 96, 2
    ni = I.norm_inputs(9105, B, H, T, dv, tiers, "bf16")
    o, gg, gm = to_dev(ni["o"], "bf16"), to_dev(ni["g"], "bf16"), to_dev(ni["gamma"])

    def call(y, sf, out):
        Bd.sgla_conv_fwd(u, w, b, init_state=s0, final_state=sf, y=y)
        Bd.sgla_head_norm_gate(o, gg, gm, tiers, 1e-6, out=out)

    y_e, sf_e = torch.empty_like(u), torch.empty((B, 3, D), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(gg)
    call(y_e, sf_e, out_e)
    y_g, sf_g, out_g = torch.empty_like(y_e), torch.empty_like(sf_e), torch.empty_like(out_e)
    g = _capture(lambda: call(y_g, sf_g, out_g))
    _check_replays(g, [y_g, sf_g, out_g], [y_e, sf_e, out_e])
