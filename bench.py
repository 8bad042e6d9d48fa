"""Benchmark of the Simple GLA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only fwd|fwdbwd|decode|varlen|long|norm|fused|conv|tiny]
                    [--no-cpu]

Prints ONE JSON line. The headline ("value") is the Laplace-layer forward:
B=8, H=16, T=2048, d_k=96, d_v=192, chunk 128, bf16 q/k/v (q scaled by
d_k^-1/2), fp32 state, decays from the 1..2048 half-life schedule,
a ~ N(0, 0.1), final state written. One step = one sgla_chunk_fwd call over
that batch, inputs resident in HBM, rotating over 3 input sets (their 0.9 GB
exceeds the 256 MB last-level cache, so each call streams from HBM).

Also measured in the same run and reported under "secondary" (same clock):
  fwdbwd: B=4 forward + backward (dO ~ N(0,1)), tokens/s = 8192 / (t_fwd + t_bwd)
  decode: 1280 sequences x 16 heads, fp32 state ~ N(0, 0.02) (1.5 GB), 64
          consecutive in-place steps, tokens/s = 1280 * 64 / t
  varlen: 32 packed sequences, lengths log-uniform in [128, 32768] (one of
          32768), init states ~ N(0, 0.02), tokens/s = sum T / t
  long:   one sequence of T=32768 (B=1, H=16) with initial and final state,
          single pass and segmented (8 segments joined by a state scan), and
          its backward, single pass and segmented (4 segments),
          tokens/s = 32768 / t
  norm:   the mixer epilogue (Head RMSNorm per decay tier, 4 tiers, + SiLU(g)
          gate) on a B=8 T=2048 forward's output: o and g in, out written,
          bf16, tokens/s = 16384 / t; and its gradients (o, g, dout in, d_o,
          dg, dgamma out)
  conv:   the conv prologue (depthwise causal width-4 Conv1d + SiLU) at the
          layer's width D=3072: forward B=8 T=2048 bf16 with conv states in and
          out, and 64 decode steps of 1280 sequences' conv states, and its
          gradients (B=8 T=2048)
  tiny:   the fp32 case B=1 H=2 T=256 d_k=16 d_v=32 chunk 64 (reported only)

"roofline" is for the dominant kernel of the headline step (k_fwd, bf16 forward):
achieved = algorithmic HBM bytes per launch / mean launch time from HIP events
on the launch stream. Algorithmic bytes per head-token: q 192 + k 192 + v 384
+ o 384 = 1152 B (bf16), plus the fp32 final state (73,728 B per sequence-head).
"cpu_baseline" times the fp64 oracle (test infrastructure, untuned) on a
bounded sample of the headline workload on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
H, DK, DV = 16, 96, 192
HT_BYTES = 2 * DK + 2 * DK + 2 * DV + 2 * DV   # q, k, v, o per head-token (bf16)
STATE_BYTES = DK * DV * 4
MIN_WARM_S = 1.5               # untimed warm-up floor per workload, seconds


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_fwd__laplace_fwd_B8_hbm_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "k_fwd_k_bwd__laplace_mfma_counters.txt")
CSRC = os.path.join(ROOT, "chunked_gated_linear_simple_amd", "csrc")
FWD_SOURCES = [os.path.join(CSRC, f) for f in ("sgla_scan.hpp", "sgla_fwd.hip")]
CHUNK_SOURCES = FWD_SOURCES + [os.path.join(CSRC, "sgla_bwd.hip")]
_CONV, _NORM, _DEC = (os.path.join(CSRC, f) for f in ("sgla_conv.hip", "sgla_norm.hip", "sgla_decode.hip"))
# HBM bytes per call (per step for decode) of the secondary workloads from the
# committed counter summaries: file, the sources its hash covers, and the keys
# whose values add up to one call. For the gradient legs it is the row kernel's
# bytes alone (the small fixed-order sums after it are not counted).
COUNTER_BYTES = {
    "fwdbwd_B4": ("k_bwd__fwdbwd_B4_hbm_traffic.txt", CHUNK_SOURCES,
                  ("fwd_b4_traffic_bytes_per_launch", "bwd_b4_traffic_bytes_per_launch")),
    "decode_N1280_64steps": ("k_decode__decode_N1280_hbm_traffic.txt", [_DEC],
                             ("decode_traffic_bytes_per_step",)),
    "head_norm_gate_B8_T2048": ("k_head_norm_gate__laplace_B8_T2048_hbm_traffic.txt", [_NORM],
                                ("traffic_bytes_per_launch",)),
    "head_norm_gate_bwd_B8_T2048": ("k_conv_bwd_k_head_norm_gate_bwd__B8_T2048_hbm_traffic.txt", [_CONV, _NORM],
                                    ("norm_bwd_traffic_bytes_per_launch",)),
    "fwd_norm_gate_B8_T2048": ("k_fwd_ng__laplace_fwd_norm_gate_B8_hbm_traffic.txt", FWD_SOURCES,
                               ("traffic_bytes_per_launch",)),
    "conv_fwd_B8_T2048_D3072": ("k_conv__prologue_B8_T2048_D3072_and_decode_N1280_hbm_traffic.txt", [_CONV],
                                ("conv_fwd_traffic_bytes_per_launch",)),
    "conv_decode_N1280_D3072_64steps": ("k_conv__prologue_B8_T2048_D3072_and_decode_N1280_hbm_traffic.txt", [_CONV],
                                        ("conv_decode_traffic_bytes_per_step",)),
    "conv_bwd_B8_T2048_D3072": ("k_conv_bwd_k_head_norm_gate_bwd__B8_T2048_hbm_traffic.txt", [_CONV, _NORM],
                                ("conv_bwd_traffic_bytes_per_launch",)),
}
# algorithmic matrix-core FLOPs per head-token with the causal mask exploited
# (C = 128): forward C(d_k + d_v) + 4 d_k d_v + 2 d_k + 2 d_v; backward
# C(3 d_k + 2 d_v) + 10 d_k d_v + 8 d_k + 4 d_v
FWD_FLOPS_HT = 128 * (DK + DV) + 4 * DK * DV + 2 * DK + 2 * DV
BWD_FLOPS_HT = 128 * (3 * DK + 2 * DV) + 10 * DK * DV + 8 * DK + 4 * DV


def code_digest(sources):
    """First 16 hex digits of sha256 over the code lines of the sources, in
    order: each line up to any `//`, trailing blanks cut, empty lines dropped.
    Comments can change without invalidating the committed counters; any
    change to the code itself does."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        for line in open(f, encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode("utf-8") + b"\n")
    return h.hexdigest()[:16]


def _profile_values(path, sources):
    """The key: value lines of a committed counter summary, or None when the
    kernel code has changed since its counters were taken."""
    try:
        kv = {}
        for line in open(path):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
        if code_digest(sources) != kv.get("sources_sha256"):
            return None
        return kv
    except OSError:
        return None


def measured_traffic():
    """HBM bytes per launch of the forward kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a copy kernel of known
    size), or None when the kernel sources have changed since it was taken."""
    kv = _profile_values(TRAFFIC_FILE, FWD_SOURCES)
    try:
        return None if kv is None else int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def executed_mfma_flops(key):
    """Executed bf16 matrix-core FLOPs per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16
    x 512) of one chunk kernel on one workload ("fwd_b8", "fwd_b4", "bwd_b4"),
    or None when the sources have changed since the counters were taken."""
    kv = _profile_values(MFMA_FILE, CHUNK_SOURCES)
    try:
        return None if kv is None else int(kv[key + "_executed_flops"])
    except (KeyError, ValueError):
        return None


def counter_bytes(name):
    """Measured HBM bytes per call of secondary workload name, or None when
    there is no summary or its kernel sources have changed since."""
    if name not in COUNTER_BYTES:
        return None
    fname, sources, keys = COUNTER_BYTES[name]
    kv = _profile_values(os.path.join(ROOT, "profiles", fname), sources)
    try:
        return None if kv is None else sum(int(kv[k]) for k in keys)
    except (KeyError, ValueError):
        return None


def call_seconds(r):
    """The time one call (one step for decode) of a secondary leg takes."""
    if "us_per_step" in r:
        return r["us_per_step"] * 1e-6
    if "ms_bwd" in r:
        return (r["ms_fwd"] + r["ms_bwd"]) * 1e-3
    return r["ms"] * 1e-3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["fwd", "fwdbwd", "decode", "varlen", "long", "norm", "fused",
                                       "conv", "tiny"],
                    default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--min-warm-s", type=float, default=1.5,
                    help="untimed warm-up continues past --warmup steps until this many "
                         "seconds have passed (clock ramp)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 1 GiB elementwise copy (read 1 GiB, write 1 GiB) "
                         "so a counter pass can scale FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def gen(shape, seed, std=1.0, scale=1.0, dtype=None):
    import torch
    g = torch.Generator(device="cuda").manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    x.mul_(std * scale)
    return x if dtype is None else x.to(dtype)


def timed(fn, steps, warmup, min_warm_s=None):
    """(mean, wall-clock mean) milliseconds per call of fn(i); see timed_stats."""
    st = timed_stats(fn, steps, warmup, min_warm_s)
    return st["mean"], st["wall"]


def timed_stats(fn, steps, warmup, min_warm_s=None):
    """Mean, median and minimum milliseconds per call of fn(i), from HIP events
    on the current stream, and the wall-clock mean.

    Runs `warmup` untimed calls, then keeps calling (untimed) until at least
    `min_warm_s` seconds of warm-up have passed: the chip's clocks take on the
    order of a second of sustained load to settle, and a handful of calls
    measures the ramp instead of the kernel."""
    import torch
    if min_warm_s is None:
        min_warm_s = MIN_WARM_S
    t_w = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_w < min_warm_s:
        fn(i)
        i += 1
        if i >= warmup and i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup = i
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(warmup + i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    n = len(per)
    median = per[n // 2] if n % 2 else 0.5 * (per[n // 2 - 1] + per[n // 2])
    return {"mean": sum(per) / n, "median": median, "min": per[0], "wall": wall * 1e3 / steps}


def bench_fwd(args, B=8, T=2048, nsets=3):
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    lam = Bd.sgla_decay_schedule(H, 1.0, 2048.0).cuda()
    a = gen((H, DK), 21, 0.1)
    sets = []
    for s in range(nsets):
        q = gen((B, H, T, DK), 100 + 10 * s, scale=DK ** -0.5, dtype=torch.bfloat16)
        k = gen((B, H, T, DK), 101 + 10 * s, dtype=torch.bfloat16)
        v = gen((B, H, T, DV), 102 + 10 * s, dtype=torch.bfloat16)
        o = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device="cuda")
        sf = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda")
        sets.append((q, k, v, o, sf))

    def step(i):
        q, k, v, o, sf = sets[i % nsets]
        Bd.sgla_chunk_fwd(q, k, v, lam, a, final_state=sf, o=o, chunk=128)

    st = timed_stats(step, args.steps, args.warmup)
    ms = st["mean"]
    toks = B * T
    bytes_ = B * H * T * HT_BYTES + B * H * STATE_BYTES
    flops = B * H * T * FWD_FLOPS_HT
    return {"ms": ms, "ms_median": st["median"], "ms_min": st["min"], "wall_ms": st["wall"],
            "tokens": toks, "tok_s": toks / (ms * 1e-3),
            "bytes": bytes_, "gbs": bytes_ / (ms * 1e-3) / 1e9, "flops": flops}


def bench_fwdbwd(args, B=4, T=2048, nsets=3):
    """B=4 forward, then backward, each timed on its own over 3 rotated
    input/output sets (q, k, v, dO in and o, dq, dk, dv out: 0.75 GB in all,
    beyond the 256 MB last-level cache, so every call streams from HBM)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    lam = Bd.sgla_decay_schedule(H, 1.0, 2048.0).cuda()
    a = gen((H, DK), 31, 0.1)
    da = torch.empty((H, DK), dtype=torch.float32, device="cuda")
    ws = torch.empty(Bd.sgla_chunk_bwd_workspace_bytes(B, H, DK), dtype=torch.uint8, device="cuda")
    sets = []
    for s in range(nsets):
        q = gen((B, H, T, DK), 200 + 10 * s, scale=DK ** -0.5, dtype=torch.bfloat16)
        k = gen((B, H, T, DK), 201 + 10 * s, dtype=torch.bfloat16)
        v = gen((B, H, T, DV), 202 + 10 * s, dtype=torch.bfloat16)
        dO = gen((B, H, T, DV), 203 + 10 * s, dtype=torch.bfloat16)
        sets.append((q, k, v, dO, torch.empty_like(v), torch.empty_like(q), torch.empty_like(k),
                     torch.empty_like(v)))

    def fwd(i):
        q, k, v, _, o, _, _, _ = sets[i % nsets]
        Bd.sgla_chunk_fwd(q, k, v, lam, a, o=o, chunk=128)

    def bwd(i):
        q, k, v, dO, _, dq, dk, dv = sets[i % nsets]
        Bd.sgla_chunk_bwd(q, k, v, dO, lam, a, chunk=128, dq=dq, dk=dk, dv=dv, da=da, workspace=ws)

    ms_f, _ = timed(fwd, args.steps, args.warmup)
    ms_b, _ = timed(bwd, args.steps, args.warmup)
    toks = B * T
    # algorithmic bytes, fwd: q,k,v,o (1152/ht); bwd: reads q,k,v,dO 1152 + writes dq,dk,dv 768
    bytes_ = B * H * T * (1152 + 1920)
    t_s = (ms_f + ms_b) * 1e-3
    flops = B * H * T * (FWD_FLOPS_HT + BWD_FLOPS_HT)
    r = {"ms_fwd": ms_f, "ms_bwd": ms_b, "tokens": toks, "tok_s": toks / t_s, "bytes": bytes_,
         "gbs": bytes_ / t_s / 1e9, "flops": flops,
         "mfma_frac_algorithmic": flops / t_s / (BF16_PEAK_TFLOPS * 1e12)}
    ex_f, ex_b = executed_mfma_flops("fwd_b4"), executed_mfma_flops("bwd_b4")
    r["mfma_frac_executed"] = (None if ex_f is None or ex_b is None
                               else (ex_f + ex_b) / t_s / (BF16_PEAK_TFLOPS * 1e12))
    return r


def bench_decode(args, N=1280, steps=64):
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    lam = Bd.sgla_decay_schedule(H, 1.0, 2048.0).cuda()
    a = gen((H, DK), 41, 0.1)
    state = gen((N, H, DK, DV), 400, 0.02)
    qs = gen((steps, N, H, DK), 401, scale=DK ** -0.5, dtype=torch.bfloat16)
    ks = gen((steps, N, H, DK), 402, dtype=torch.bfloat16)
    vs = gen((steps, N, H, DV), 403, dtype=torch.bfloat16)
    o = torch.empty((N, H, DV), dtype=torch.bfloat16, device="cuda")

    def run64(_):
        for s in range(steps):
            Bd.sgla_decode_step(qs[s], ks[s], vs[s], lam, a, state, o=o)

    reps = max(2, args.steps // 4)
    ms, _ = timed(run64, reps, 1)
    toks = N * steps
    bytes_step = N * H * (2 * STATE_BYTES + 2 * DK + 2 * DK + 2 * DV + 2 * DV)
    return {"ms_64_steps": ms, "us_per_step": ms * 1e3 / steps, "tokens": toks,
            "tok_s": toks / (ms * 1e-3), "bytes_per_step": bytes_step,
            "gbs": bytes_step * steps / (ms * 1e-3) / 1e9}


DMODEL = 3072  # residual width of the Laplace layer (the conv prologue's channels)


def bench_conv(args, B=8, T=2048, D=DMODEL, nsets=3):
    """Conv prologue forward: y = silu(depthwise causal width-4 conv(u)), bf16,
    conv states in and out, rotating over input sets (0.6 GB)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    w = gen((D, 4), 60, 0.5)
    b = gen((D,), 61, 0.1)
    sets = []
    for s in range(nsets):
        u = gen((B, T, D), 62 + s, dtype=torch.bfloat16)
        sets.append((u, torch.empty_like(u), gen((B, 3, D), 70 + s), torch.empty((B, 3, D), device="cuda")))

    def step(i):
        u, y, s0, sf = sets[i % nsets]
        Bd.sgla_conv_fwd(u, w, b, init_state=s0, final_state=sf, y=y)

    ms, _ = timed(step, args.steps, args.warmup)
    toks = B * T
    bytes_ = 2 * B * T * D * 2 + 2 * B * 3 * D * 4 + D * 20
    return {"ms": ms, "tokens": toks, "tok_s": toks / (ms * 1e-3), "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9}


def bench_conv_bwd(args, B=8, T=2048, D=DMODEL, nsets=2):
    """Conv prologue gradients at the layer's width: u, dy in (bf16), du out
    (bf16), dw, db and the initial states' gradient (fp32) out, final states'
    gradient in; 2 input sets rotated (0.8 GB)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    w = gen((D, 4), 64, 0.5)
    b = gen((D,), 65, 0.1)
    dw = torch.empty((D, 4), device="cuda")
    db = torch.empty((D,), device="cuda")
    ws = torch.empty(Bd.sgla_conv_bwd_workspace_bytes(B, T, D) // 4, device="cuda")
    sets = []
    for s in range(nsets):
        sets.append((gen((B, T, D), 66 + 4 * s, dtype=torch.bfloat16),
                     gen((B, T, D), 67 + 4 * s, dtype=torch.bfloat16),
                     gen((B, 3, D), 68 + 4 * s), gen((B, 3, D), 69 + 4 * s),
                     torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((B, 3, D), device="cuda")))

    def step(i):
        u, dy, s0, dsf, du, ds0 = sets[i % nsets]
        Bd.sgla_conv_bwd(u, w, dy, b=b, init_state=s0, d_final_state=dsf, du=du, dw=dw, db=db,
                         d_init_state=ds0, workspace=ws)

    ms, _ = timed(step, args.steps, args.warmup)
    toks = B * T
    bytes_ = 3 * B * T * D * 2 + 3 * B * 3 * D * 4 + D * 40
    return {"ms": ms, "tokens": toks, "tok_s": toks / (ms * 1e-3), "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9}


def bench_conv_decode(args, N=1280, D=DMODEL, steps=64, npools=8):
    """Conv decode: 64 consecutive in-place steps of 1280 sequences' conv
    states. Step s uses pool s % 8 (8 x 47 MB, beyond the on-die caches), as a
    whole decode step's other traffic would evict one pool between steps."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    w = gen((D, 4), 80, 0.5)
    b = gen((D,), 81, 0.1)
    pools = [gen((N, 3, D), 82 + i) for i in range(npools)]
    xs = gen((steps, N, D), 83 + npools, dtype=torch.bfloat16)
    y = torch.empty((N, D), dtype=torch.bfloat16, device="cuda")

    def run(_):
        for s in range(steps):
            Bd.sgla_conv_decode_step(xs[s], w, b, pools[s % npools], y=y)

    reps = max(2, args.steps // 4)
    ms, _ = timed(run, reps, 1)
    toks = N * steps
    bytes_step = N * (2 * 3 * D * 4 + 2 * D * 2) + D * 20
    return {"ms_64_steps": ms, "us_per_step": ms * 1e3 / steps, "tokens": toks,
            "tok_s": toks / (ms * 1e-3), "bytes_per_step": bytes_step,
            "gbs": bytes_step * steps / (ms * 1e-3) / 1e9}


def bench_norm(args, B=8, T=2048, n_tiers=4, nsets=3):
    """Mixer epilogue (Head RMSNorm per decay tier + SiLU(g) gate) on the
    Laplace layer's forward output: o [B, H, T, d_v] and g [B, T, H, d_v] bf16
    in, out [B, T, H, d_v] bf16; 3 input sets rotated (0.9 GB)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    gm = (1.0 + gen((n_tiers, DV), 90, 0.1)).contiguous()
    sets = []
    for s in range(nsets):
        o = gen((B, H, T, DV), 91 + 2 * s, dtype=torch.bfloat16)
        g = gen((B, T, H, DV), 92 + 2 * s, dtype=torch.bfloat16)
        sets.append((o, g, torch.empty_like(g)))

    def step(i):
        o, g, out = sets[i % nsets]
        Bd.sgla_head_norm_gate(o, g, gm, n_tiers, 1e-6, out=out)

    ms, _ = timed(step, args.steps, args.warmup)
    toks = B * T
    bytes_ = 3 * B * T * H * DV * 2 + n_tiers * DV * 4
    return {"ms": ms, "tokens": toks, "tok_s": toks / (ms * 1e-3), "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9}


def bench_fused(args, B=8, T=2048, n_tiers=4, nsets=3):
    """The forward with the mixer epilogue applied before the store (one
    launch) against the two-launch pipeline sgla_chunk_fwd then
    sgla_head_norm_gate, on the same
    inputs: the headline workload plus the gate stream g [B, T, H, d_v], out
    [B, T, H, d_v], final state written; 3 input sets rotated (1.5 GB)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    lam = Bd.sgla_decay_schedule(H, 1.0, 2048.0).cuda()
    a = gen((H, DK), 41, 0.1)
    gm = (1.0 + gen((n_tiers, DV), 42, 0.1)).contiguous()
    x = torch.zeros(Bd.FWD_NORM_GATE_EXCHANGE_BYTES, dtype=torch.uint8, device="cuda")
    sets = []
    for s in range(nsets):
        q = gen((B, H, T, DK), 300 + 10 * s, scale=DK ** -0.5, dtype=torch.bfloat16)
        k = gen((B, H, T, DK), 301 + 10 * s, dtype=torch.bfloat16)
        v = gen((B, H, T, DV), 302 + 10 * s, dtype=torch.bfloat16)
        g = gen((B, T, H, DV), 303 + 10 * s, dtype=torch.bfloat16)
        sets.append((q, k, v, g, torch.empty_like(g), torch.empty_like(v),
                     torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda")))

    def fused(i):
        q, k, v, g, out, _, sf = sets[i % nsets]
        Bd.sgla_chunk_fwd_norm_gate(q, k, v, lam, g, a=a, gamma=gm, n_tiers=n_tiers, eps=1e-6,
                                    final_state=sf, out=out, chunk=128, exchange=x)

    def pair(i):
        q, k, v, g, out, o, sf = sets[i % nsets]
        Bd.sgla_chunk_fwd(q, k, v, lam, a, final_state=sf, o=o, chunk=128)
        Bd.sgla_head_norm_gate(o, g, gm, n_tiers, 1e-6, out=out)

    st = timed_stats(fused, args.steps, args.warmup)
    ms_pair, _ = timed(pair, args.steps, args.warmup)
    torch.cuda.synchronize()
    if int(torch.count_nonzero(x).item()) != 0:
        raise RuntimeError("fused forward: the exchange buffer is not zero-filled after the calls")
    toks = B * T
    # q, k, v, g read and out written (bf16), the final state written (fp32)
    bytes_ = B * H * T * (2 * DK + 3 * DV) * 2 + B * H * STATE_BYTES + n_tiers * DV * 4
    return {"ms": st["mean"], "ms_median": st["median"],
            "ms_two_launches": ms_pair, "tokens": toks,
            "tok_s": toks / (st["mean"] * 1e-3), "tok_s_two_launches": toks / (ms_pair * 1e-3),
            "bytes": bytes_, "gbs": bytes_ / (st["mean"] * 1e-3) / 1e9}


def bench_norm_bwd(args, B=8, T=2048, n_tiers=4, nsets=2):
    """Gradients of the mixer epilogue at the Laplace layer's size: o, g,
    dout in (bf16), d_o and dg out (bf16), dgamma [4, 192] fp32 through the
    fixed-order partial sums; 2 input sets rotated (1.0 GB)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    gm = (1.0 + gen((n_tiers, DV), 95, 0.1)).contiguous()
    dgm = torch.empty_like(gm)
    ws = torch.empty(Bd.sgla_head_norm_gate_bwd_workspace_bytes(B, H, T, DV) // 4,
                     dtype=torch.float32, device="cuda")
    sets = []
    for s in range(nsets):
        o = gen((B, H, T, DV), 96 + 3 * s, dtype=torch.bfloat16)
        g = gen((B, T, H, DV), 97 + 3 * s, dtype=torch.bfloat16)
        dout = gen((B, T, H, DV), 98 + 3 * s, dtype=torch.bfloat16)
        sets.append((o, g, dout, torch.empty_like(o), torch.empty_like(g)))

    def step(i):
        o, g, dout, d_o, dg = sets[i % nsets]
        Bd.sgla_head_norm_gate_bwd(o, g, dout, gm, n_tiers, 1e-6, d_o=d_o, dg=dg, dgamma=dgm,
                                   workspace=ws)

    ms, _ = timed(step, args.steps, args.warmup)
    toks = B * T
    bytes_ = 5 * B * T * H * DV * 2 + 2 * n_tiers * DV * 4
    return {"ms": ms, "tokens": toks, "tok_s": toks / (ms * 1e-3), "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9}


def bench_tiny(args, B=1, Ht=2, T=256, dk=16, dv=32):
    """The tiny fp32 case (B=1, H=2, T=256, d_k=16, d_v=32, chunk 64, schedule
    1..256, zero initial state): reported, not a target; it is launch-bound."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    lam = Bd.sgla_decay_schedule(Ht, 1.0, 256.0).cuda()
    a = gen((Ht, dk), 71, 0.1)
    q = gen((B, Ht, T, dk), 700, scale=dk ** -0.5)
    k = gen((B, Ht, T, dk), 701)
    v = gen((B, Ht, T, dv), 702)
    o = torch.empty_like(v)
    sf = torch.empty((B, Ht, dk, dv), dtype=torch.float32, device="cuda")
    ms, _ = timed(lambda i: Bd.sgla_chunk_fwd(q, k, v, lam, a, final_state=sf, o=o, chunk=64),
                  args.steps, args.warmup)
    toks = B * T
    bytes_ = B * Ht * T * 4 * (2 * dk + 2 * dv) + B * Ht * dk * dv * 4
    return {"ms": ms, "tokens": toks, "tok_s": toks / (ms * 1e-3), "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9, "dtype": "f32"}


def bench_varlen(args):
    import numpy as np
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    from chunked_gated_linear_simple_amd import inputs as I
    L = I.varlen_lengths(5)
    cu = torch.from_numpy(I.cu_from_lengths(L)).cuda()
    Ttot = int(cu[-1].item())
    lam = Bd.sgla_decay_schedule(H, 1.0, 2048.0).cuda()
    a = gen((H, DK), 51, 0.1)
    q = gen((1, H, Ttot, DK), 500, scale=DK ** -0.5, dtype=torch.bfloat16)
    k = gen((1, H, Ttot, DK), 501, dtype=torch.bfloat16)
    v = gen((1, H, Ttot, DV), 502, dtype=torch.bfloat16)
    s0 = gen((len(L), H, DK, DV), 503, 0.02)
    sf = torch.empty_like(s0)
    o = torch.empty_like(v)
    ms, _ = timed(lambda i: Bd.sgla_chunk_fwd(q, k, v, lam, a, init_state=s0, final_state=sf,
                                              o=o, cu_seqlens=cu, chunk=128),
                  max(3, args.steps // 2), 2)
    bytes_ = H * Ttot * HT_BYTES + 2 * len(L) * H * STATE_BYTES
    return {"ms": ms, "tokens": Ttot, "tok_s": Ttot / (ms * 1e-3), "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9, "n_seq": int(len(L)), "max_len": int(np.max(L))}


def bench_long(args, T=32768, n_segments=8):
    """One long sequence (B=1, H=16, T=32768: the longest sequence of the
    packed workload as a batch of its own), initial and final state: the
    single-pass forward runs 32 workgroups down a 512-tile chain; the
    segmented forward cuts it into n_segments runs joined by a state scan
    (8: its full forward launch then has 8 x 32 = 256 workgroups, one per
    CU, after a state-only launch over the first 7)."""
    import torch
    from chunked_gated_linear_simple_amd import binding as Bd
    lam = Bd.sgla_decay_schedule(H, 1.0, 2048.0).cuda()
    a = gen((H, DK), 61, 0.1)
    q = gen((1, H, T, DK), 600, scale=DK ** -0.5, dtype=torch.bfloat16)
    k = gen((1, H, T, DK), 601, dtype=torch.bfloat16)
    v = gen((1, H, T, DV), 602, dtype=torch.bfloat16)
    s0 = gen((1, H, DK, DV), 603, 0.02)
    sf = torch.empty_like(s0)
    o = torch.empty_like(v)
    ws = torch.empty(Bd.sgla_chunk_fwd_segmented_workspace_bytes(1, H, DK, DV, n_segments) // 4,
                     dtype=torch.float32, device="cuda")
    steps = max(3, args.steps // 4)
    ms1, _ = timed(lambda i: Bd.sgla_chunk_fwd(q, k, v, lam, a, init_state=s0, final_state=sf,
                                               o=o, chunk=128), steps, 2)
    ms, _ = timed(lambda i: Bd.sgla_chunk_fwd_segmented(q, k, v, lam, a, init_state=s0,
                                                        final_state=sf, o=o, n_segments=n_segments,
                                                        workspace=ws), steps, 2)
    bytes_ = H * T * HT_BYTES + 2 * H * STATE_BYTES
    # the backward of the same sequence: single pass, and 4 segments (its last
    # launch then runs 4 x 64 = 256 workgroups)
    nsb = 4
    dO = gen((1, H, T, DV), 604, dtype=torch.bfloat16)
    dsf = gen((1, H, DK, DV), 605, 0.02)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    da = torch.empty((H, DK), device="cuda")
    ds0 = torch.empty_like(s0)
    wsb = torch.empty(Bd.sgla_chunk_bwd_segmented_workspace_bytes(1, H, DK, DV, nsb) // 4,
                      dtype=torch.float32, device="cuda")
    msb1, _ = timed(lambda i: Bd.sgla_chunk_bwd(q, k, v, dO, lam, a, init_state=s0,
                                                d_final_state=dsf, dq=dq, dk=dk, dv=dv, da=da,
                                                d_init_state=ds0), steps, 2)
    msb, _ = timed(lambda i: Bd.sgla_chunk_bwd_segmented(q, k, v, dO, lam, a, init_state=s0,
                                                         d_final_state=dsf, n_segments=nsb,
                                                         dq=dq, dk=dk, dv=dv, da=da,
                                                         d_init_state=ds0, workspace=wsb),
                   steps, 2)
    return {"ms": ms, "ms_single_pass": ms1, "tokens": T, "tok_s": T / (ms * 1e-3),
            "tok_s_single_pass": T / (ms1 * 1e-3), "n_segments": n_segments, "bytes": bytes_,
            "gbs": bytes_ / (ms * 1e-3) / 1e9,
            "bwd_ms": msb, "bwd_ms_single_pass": msb1, "bwd_n_segments": nsb}


def cpu_baseline(min_seconds=10.0, B=8, T=2048):
    """The fp64 oracle (untuned test infrastructure) on the headline workload:
    all B*H (sequence, head) units of B=8, T=2048, one thread per unit over
    the host's cores, repeated until at least `min_seconds` of wall time."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from chunked_gated_linear_simple_amd import inputs as I
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build(force=True)
    # one thread per core of the host share this process may use; the GPU
    # hosts here give a one-GPU job 16 CPUs whatever the machine reports
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cores = min(avail, 16)
    lam = oracle.decay_schedule(H, 1.0, 2048.0)
    inp = I.chunk_inputs(B, H, T, DK, DV, "bf16", seed=2, a_std=0.1)
    work = [(I.widen(inp["q"][n, h], "bf16"), I.widen(inp["k"][n, h], "bf16"),
             I.widen(inp["v"][n, h], "bf16"), float(lam[h]), inp["a"][h].astype(np.float64))
            for n in range(B) for h in range(H)]
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        while True:
            list(ex.map(lambda x: oracle.fwd_unit(*x), work))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    tokens = passes * B * T
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": model,
            "sample": f"the full headline forward (B={B}, H={H}, T={T}: {B * H} sequence-head "
                      f"units) run {passes} times in {dt:.1f} s; fp64 token recurrence, one "
                      f"thread per unit"}


def main():
    global MIN_WARM_S
    args = parse()
    MIN_WARM_S = args.min_warm_s
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    from chunked_gated_linear_simple_amd import binding as Bd
    Bd.lib()  # fail loudly if the library is not built

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    secondary = {}
    only = args.only
    fwd = bench_fwd(args) if only in (None, "fwd") else None
    if only in (None, "fwdbwd"):
        secondary["fwdbwd_B4"] = bench_fwdbwd(args)
    if only in (None, "decode"):
        secondary["decode_N1280_64steps"] = bench_decode(args)
    if only in (None, "varlen"):
        secondary["varlen_32seq"] = bench_varlen(args)
    if only in (None, "long"):
        secondary["long_B1_T32768_segmented"] = bench_long(args)
    if only in (None, "norm"):
        secondary["head_norm_gate_B8_T2048"] = bench_norm(args)
        secondary["head_norm_gate_bwd_B8_T2048"] = bench_norm_bwd(args)
    if only in (None, "fused"):
        secondary["fwd_norm_gate_B8_T2048"] = bench_fused(args)
    if only in (None, "tiny"):
        secondary["tiny_fp32_B1_H2_T256"] = bench_tiny(args)
    if only in (None, "conv"):
        secondary["conv_fwd_B8_T2048_D3072"] = bench_conv(args)
        secondary["conv_decode_N1280_D3072_64steps"] = bench_conv_decode(args)
        secondary["conv_bwd_B8_T2048_D3072"] = bench_conv_bwd(args)
    for name, r in secondary.items():
        r["hbm_frac_algorithmic"] = r["gbs"] / HBM_PEAK_GBS
        tb = counter_bytes(name)
        if tb is not None:
            r["traffic_bytes"] = tb
            r["hbm_frac_counter"] = tb / call_seconds(r) / 1e9 / HBM_PEAK_GBS

    line = {"metric": "GLA tokens/s (fwd, fwd+bwd, decode) at H=16 dk=96 dv=192; % MFMA/HBM peak",
            "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "warmup": args.warmup, "min_warm_s": args.min_warm_s, "steps": args.steps}
    if fwd is not None:
        line.update({
            "value": fwd["tok_s"], "ms_per_step": fwd["ms"],
            "config": {"workload": "Laplace layer fwd B=8 H=16 T=2048 dk=96 dv=192 chunk=128 "
                                   "bf16, fp32 state, final state written",
                       "batch": 8, "seq_len": 2048, "heads": H, "d_k": DK, "d_v": DV,
                       "chunk": 128, "tile_tokens": 64},
            "ms_median": fwd["ms_median"], "ms_min": fwd["ms_min"],
            "roofline": {"bound": "hbm", "kernel": "k_fwd", "achieved": fwd["gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": fwd["gbs"] / HBM_PEAK_GBS,
                         "traffic": measured_traffic(), "bytes_per_launch": fwd["bytes"],
                         "flops_per_launch": fwd["flops"],
                         "mfma_frac_algorithmic": fwd["flops"] / (fwd["ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                         "mfma_frac_executed": None},
        })
        tr = line["roofline"]["traffic"]
        line["roofline"]["frac_traffic"] = None if tr is None else tr / (fwd["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        ex = executed_mfma_flops("fwd_b8")
        if ex is not None:
            line["roofline"]["mfma_frac_executed"] = ex / (fwd["ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    else:
        first = next(iter(secondary.values()))
        line.update({"value": first["tok_s"], "config": {"workload": next(iter(secondary))}})
    line["secondary"] = secondary
    if not args.no_cpu and fwd is not None:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
