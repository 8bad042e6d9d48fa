"""The C ABI on the CPU: the library loads, exports what include/sgla.h
declares, computes the decay schedule, and rejects bad arguments on the host
before anything reaches the GPU (no kernel is launched by these tests)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
from chunked_gated_linear_simple_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from chunked_gated_linear_simple_amd import build
        build.build()
    return B.lib()


def test_exports_every_declared_symbol(L):
    declared = B.declared_functions()
    assert set(declared) >= {"sgla_decay_schedule", "sgla_chunk_fwd", "sgla_chunk_bwd",
                             "sgla_chunk_bwd_workspace_bytes", "sgla_decode_step",
                             "sgla_conv_fwd", "sgla_conv_decode_step", "sgla_head_norm_gate",
                             "sgla_last_error", "sgla_status_str", "sgla_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(sgla_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for f in declared:
        getattr(L, f)  # resolvable through ctypes


def test_version_and_status_strings(L):
    assert B.sgla_version() >= 100
    for code, name in enumerate(["SGLA_OK", "SGLA_ERR_INVALID_ARG", "SGLA_ERR_UNSUPPORTED",
                                 "SGLA_ERR_WORKSPACE", "SGLA_ERR_HIP"]):
        assert L.sgla_status_str(code).decode() == name
    assert L.sgla_status_str(99).decode() == "unknown sgla_status"


def test_decay_schedule_matches_oracle(L):
    for H, tmin, tmax in ((16, 1.0, 2048.0), (2, 1.0, 256.0), (1, 3.0, 3.0), (7, 0.5, 9.0)):
        got = B.sgla_decay_schedule(H, tmin, tmax).numpy()
        want = oracle.decay_schedule(H, tmin, tmax).astype(np.float32)
        # same fp64 formula rounded once to fp32: equal to within one fp32 ulp
        ulps = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, (H, got, want)
    lam = B.sgla_decay_schedule(16, 1.0, 2048.0).numpy()
    assert lam[0] == 0.5
    assert abs(lam[15] - 0.9997) < 5e-5


@pytest.mark.parametrize("args", [(0, 1.0, 2.0), (4, 0.0, 2.0), (4, 3.0, 2.0),
                                  (4, float("nan"), 2.0), (4, 1.0, float("inf"))])
def test_decay_schedule_rejects(L, args):
    out = (ctypes.c_float * 8)()
    assert L.sgla_decay_schedule(args[0], args[1], args[2], out) == B.SGLA_ERR_INVALID_ARG
    assert L.sgla_last_error().decode()
    assert L.sgla_decay_schedule(4, 1.0, 2.0, None) == B.SGLA_ERR_INVALID_ARG
    assert L.sgla_decay_schedule(4, 1.0, 2.0, out) == B.SGLA_OK
    assert L.sgla_last_error().decode() == ""


# Fake, never-dereferenced device addresses: validation only looks at the values.
BASE = 0x7F0000000000
P = {n: BASE + i * 0x100000000 for i, n in enumerate(
    ["q", "k", "v", "lam", "a", "s0", "sf", "o", "cu", "dO", "dq", "dk", "dv", "da", "ds0", "ws",
     "state", "slot", "u", "w", "b", "y", "no", "ng", "gm", "nout", "ndo", "ndg", "ndout", "ndgm"])}


def fwd_args(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], lam=P["lam"], a=P["a"], s0=P["s0"], sf=P["sf"],
             o=P["o"], cu=None, n_seq=0, B=2, H=16, T=256, d_k=96, d_v=192, chunk=128,
             dt=B.SGLA_BF16)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["lam"], a["a"], a["s0"], a["sf"], a["o"], a["cu"],
            a["n_seq"], a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["chunk"], a["dt"], None]


FWD_BAD = [
    ("q null", dict(q=None), B.SGLA_ERR_INVALID_ARG),
    ("k misaligned", dict(k=P["k"] + 8), B.SGLA_ERR_INVALID_ARG),
    ("o null", dict(o=None), B.SGLA_ERR_INVALID_ARG),
    ("lambda null", dict(lam=None), B.SGLA_ERR_INVALID_ARG),
    ("a misaligned", dict(a=P["a"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("init misaligned", dict(s0=P["s0"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("B zero", dict(B=0), B.SGLA_ERR_INVALID_ARG),
    ("T negative", dict(T=-5), B.SGLA_ERR_INVALID_ARG),
    ("H zero", dict(H=0), B.SGLA_ERR_INVALID_ARG),
    ("bad dtype", dict(dt=7), B.SGLA_ERR_INVALID_ARG),
    ("d_k too big", dict(d_k=128), B.SGLA_ERR_UNSUPPORTED),
    ("d_v too big", dict(d_v=256), B.SGLA_ERR_UNSUPPORTED),
    ("d_k not mult 8", dict(d_k=20), B.SGLA_ERR_UNSUPPORTED),
    ("chunk 16", dict(chunk=16), B.SGLA_ERR_UNSUPPORTED),
    ("chunk 256", dict(chunk=256), B.SGLA_ERR_UNSUPPORTED),
    ("f32 d_k 100", dict(dt=B.SGLA_F32, d_k=100), B.SGLA_ERR_UNSUPPORTED),
    ("f32 d_v 196", dict(dt=B.SGLA_F32, d_v=196), B.SGLA_ERR_UNSUPPORTED),
    ("f32 d_k not mult 4", dict(dt=B.SGLA_F32, d_k=66), B.SGLA_ERR_UNSUPPORTED),
    ("f32 chunk 96", dict(dt=B.SGLA_F32, d_k=16, d_v=32, chunk=96), B.SGLA_ERR_UNSUPPORTED),
    ("o aliases q", dict(o=P["q"]), B.SGLA_ERR_INVALID_ARG),
    ("o overlaps v", dict(o=P["v"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("packed with B=2", dict(cu=P["cu"], n_seq=3), B.SGLA_ERR_INVALID_ARG),
    ("packed n_seq 0", dict(cu=P["cu"], n_seq=0, B=1), B.SGLA_ERR_INVALID_ARG),
    ("cu misaligned", dict(cu=P["cu"] + 4, n_seq=2, B=1), B.SGLA_ERR_INVALID_ARG),
    ("final overlaps init", dict(sf=P["s0"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("init overlaps final", dict(s0=P["sf"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("final overlaps v", dict(sf=P["v"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("final aliases o", dict(sf=P["o"]), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", FWD_BAD, ids=[x[0] for x in FWD_BAD])
def test_chunk_fwd_rejects(L, name, kw, code):
    assert L.sgla_chunk_fwd(*fwd_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def fng_args(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], lam=P["lam"], a=P["a"], s0=P["s0"], sf=P["sf"], g=P["ng"],
             gm=P["gm"], out=P["nout"], o=P["o"], cu=None, n_seq=0, B=2, H=16, T=256, d_k=96, d_v=192,
             chunk=128, tiers=4, eps=1e-6, dt=B.SGLA_BF16, x=P["ws"], xb=B.FWD_NORM_GATE_EXCHANGE_BYTES, fl=0)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["lam"], a["a"], a["s0"], a["sf"], a["g"], a["gm"], a["out"], a["o"],
            a["cu"], a["n_seq"], a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["chunk"], a["tiers"],
            ctypes.c_float(a["eps"]), a["dt"], a["x"], a["xb"], a["fl"], None]


FNG_BAD = [
    ("q null", dict(q=None), B.SGLA_ERR_INVALID_ARG),
    ("g null", dict(g=None), B.SGLA_ERR_INVALID_ARG),
    ("out null", dict(out=None), B.SGLA_ERR_INVALID_ARG),
    ("out misaligned", dict(out=P["nout"] + 8), B.SGLA_ERR_INVALID_ARG),
    ("gamma misaligned", dict(gm=P["gm"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("o misaligned", dict(o=P["o"] + 8), B.SGLA_ERR_INVALID_ARG),
    ("f32", dict(dt=B.SGLA_F32, d_k=16, d_v=32), B.SGLA_ERR_UNSUPPORTED),
    ("d_v too big", dict(d_v=256), B.SGLA_ERR_UNSUPPORTED),
    ("chunk 16", dict(chunk=16), B.SGLA_ERR_UNSUPPORTED),
    ("exchange null", dict(x=None), B.SGLA_ERR_WORKSPACE),
    ("exchange misaligned", dict(x=P["ws"] + 8), B.SGLA_ERR_WORKSPACE),
    ("exchange short", dict(xb=B.FWD_NORM_GATE_EXCHANGE_BYTES - 1), B.SGLA_ERR_WORKSPACE),
    ("exchange overlaps out", dict(x=P["nout"] + 4096), B.SGLA_ERR_WORKSPACE),
    ("tiers zero", dict(tiers=0), B.SGLA_ERR_INVALID_ARG),
    ("tiers not dividing H", dict(tiers=3), B.SGLA_ERR_INVALID_ARG),
    ("eps negative", dict(eps=-1.0), B.SGLA_ERR_INVALID_ARG),
    ("eps nan", dict(eps=float("nan")), B.SGLA_ERR_INVALID_ARG),
    ("out overlaps q", dict(out=P["q"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("out overlaps g", dict(out=P["ng"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("o aliases out", dict(o=P["nout"]), B.SGLA_ERR_INVALID_ARG),
    ("o overlaps v", dict(o=P["v"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("final overlaps init", dict(sf=P["s0"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("final overlaps out", dict(sf=P["nout"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("final overlaps g", dict(sf=P["ng"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("packed with B=2", dict(cu=P["cu"], n_seq=3), B.SGLA_ERR_INVALID_ARG),
    ("H * d_v above 2^24", dict(H=1 << 18, T=1, B=1, tiers=1), B.SGLA_ERR_UNSUPPORTED),
    ("unknown flag", dict(fl=2), B.SGLA_ERR_INVALID_ARG),
    ("no flags are defined", dict(fl=1), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", FNG_BAD, ids=[x[0] for x in FNG_BAD])
def test_chunk_fwd_norm_gate_rejects(L, name, kw, code):
    """The fused forward and epilogue validates on the host, before any GPU call."""
    assert L.sgla_chunk_fwd_norm_gate(*fng_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def test_exchange_bytes_match_header():
    text = open(os.path.join(ROOT, "include", "sgla.h")).read()
    m = re.search(r"#define SGLA_FWD_NORM_GATE_EXCHANGE_BYTES \(\(size_t\)2 \* 1024 \* 1024 \+ 256\)", text)
    assert m is not None
    assert B.FWD_NORM_GATE_EXCHANGE_BYTES == 2 * 1024 * 1024 + 256


def seg_args(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], lam=P["lam"], a=P["a"], s0=P["s0"], sf=P["sf"],
             o=P["o"], B=2, H=16, T=4096, d_k=96, d_v=192, chunk=128, dt=B.SGLA_BF16, nseg=4,
             ws=P["ws"], wsb=2 * 2 * 4 * 16 * 96 * 192 * 4)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["lam"], a["a"], a["s0"], a["sf"], a["o"], a["B"], a["H"],
            a["T"], a["d_k"], a["d_v"], a["chunk"], a["dt"], a["nseg"], a["ws"], a["wsb"], None]


SEG_BAD = [
    ("q null", dict(q=None), B.SGLA_ERR_INVALID_ARG),
    ("o null", dict(o=None), B.SGLA_ERR_INVALID_ARG),
    ("n_segments zero", dict(nseg=0), B.SGLA_ERR_INVALID_ARG),
    ("n_segments negative", dict(nseg=-2), B.SGLA_ERR_INVALID_ARG),
    ("f32", dict(dt=B.SGLA_F32, d_k=16, d_v=32, chunk=64), B.SGLA_ERR_UNSUPPORTED),
    ("d_k too big", dict(d_k=128), B.SGLA_ERR_UNSUPPORTED),
    ("workspace null", dict(ws=None), B.SGLA_ERR_WORKSPACE),
    ("workspace small", dict(wsb=2 * 2 * 4 * 16 * 96 * 192 * 4 - 16), B.SGLA_ERR_WORKSPACE),
    ("workspace misaligned", dict(ws=P["ws"] + 8), B.SGLA_ERR_WORKSPACE),
    ("o aliases k", dict(o=P["k"]), B.SGLA_ERR_INVALID_ARG),
    ("final misaligned", dict(sf=P["sf"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("final overlaps init", dict(sf=P["s0"] + 2048), B.SGLA_ERR_INVALID_ARG),
    ("final aliases q", dict(sf=P["q"]), B.SGLA_ERR_INVALID_ARG),
    ("workspace overlaps o", dict(ws=P["o"] + 4096), B.SGLA_ERR_WORKSPACE),
    ("workspace overlaps init", dict(ws=P["s0"]), B.SGLA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", SEG_BAD, ids=[x[0] for x in SEG_BAD])
def test_chunk_fwd_segmented_rejects(L, name, kw, code):
    assert L.sgla_chunk_fwd_segmented(*seg_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def test_segmented_workspace_bytes(L):
    # two arrays of B * n_segments * H states of d_k * d_v fp32
    assert B.sgla_chunk_fwd_segmented_workspace_bytes(1, 16, 96, 192, 8) == 2 * 8 * 16 * 96 * 192 * 4
    assert B.sgla_chunk_fwd_segmented_workspace_bytes(2, 4, 32, 64, 3) == 2 * 2 * 3 * 4 * 32 * 64 * 4
    assert B.sgla_chunk_fwd_segmented_workspace_bytes(1, 16, 96, 192, 0) == 0


def bwd_args(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], dO=P["dO"], lam=P["lam"], a=P["a"], s0=P["s0"],
             dsf=P["sf"], dq=P["dq"], dk=P["dk"], dv=P["dv"], da=P["da"], ds0=P["ds0"], cu=None,
             n_seq=0, B=2, H=16, T=256, d_k=96, d_v=192, chunk=128, dt=B.SGLA_BF16, ws=P["ws"],
             wsb=2 * 16 * 96 * 4)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["dO"], a["lam"], a["a"], a["s0"], a["dsf"], a["dq"],
            a["dk"], a["dv"], a["da"], a["ds0"], a["cu"], a["n_seq"], a["B"], a["H"], a["T"],
            a["d_k"], a["d_v"], a["chunk"], a["dt"], a["ws"], a["wsb"], None]


BWD_BAD = [
    ("dO null", dict(dO=None), B.SGLA_ERR_INVALID_ARG),
    ("dq null", dict(dq=None), B.SGLA_ERR_INVALID_ARG),
    ("da null", dict(da=None), B.SGLA_ERR_INVALID_ARG),
    ("ds0 misaligned", dict(ds0=P["ds0"] + 2), B.SGLA_ERR_INVALID_ARG),
    ("workspace null", dict(ws=None), B.SGLA_ERR_WORKSPACE),
    ("workspace small", dict(wsb=100), B.SGLA_ERR_WORKSPACE),
    ("workspace misaligned", dict(ws=P["ws"] + 4), B.SGLA_ERR_WORKSPACE),
    ("dq aliases dO", dict(dq=P["dO"]), B.SGLA_ERR_INVALID_ARG),
    ("dv aliases v", dict(dv=P["v"]), B.SGLA_ERR_INVALID_ARG),
    ("d_init aliases d_final", dict(ds0=P["sf"]), B.SGLA_ERR_INVALID_ARG),
    ("d_init overlaps init", dict(ds0=P["s0"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("dk overlaps dq", dict(dk=P["dq"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("da inside dv", dict(da=P["dv"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("da overlaps a", dict(da=P["a"]), B.SGLA_ERR_INVALID_ARG),
    ("d_init overlaps dq", dict(ds0=P["dq"]), B.SGLA_ERR_INVALID_ARG),
    ("workspace overlaps q", dict(ws=P["q"] + 4096), B.SGLA_ERR_WORKSPACE),
    ("workspace overlaps da", dict(ws=P["da"]), B.SGLA_ERR_WORKSPACE),
    ("unsupported dims", dict(d_v=200), B.SGLA_ERR_UNSUPPORTED),
    ("T zero", dict(T=0), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", BWD_BAD, ids=[x[0] for x in BWD_BAD])
def test_chunk_bwd_rejects(L, name, kw, code):
    assert L.sgla_chunk_bwd(*bwd_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


NOALLOC_BAD = [x for x in BWD_BAD if "workspace" not in x[0]] + [
    ("scratch too small for 700 sequences", dict(B=700), B.SGLA_ERR_WORKSPACE),
    ("scratch too small for 683 packed sequences",
     dict(B=1, cu=P["cu"], n_seq=683, T=4096), B.SGLA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", NOALLOC_BAD, ids=[x[0] for x in NOALLOC_BAD])
def test_chunk_bwd_noalloc_rejects(L, name, kw, code):
    """The allocation-free backward reports argument errors before any GPU
    call, and refuses sizes whose da partial sums exceed its fixed scratch."""
    args = bwd_args(**kw)
    del args[22:24]  # no workspace arguments
    assert L.sgla_chunk_bwd_noalloc(*args) == code
    msg = L.sgla_last_error().decode()
    assert msg != ""
    if "scratch" in name:
        assert "scratch" in msg and str(4 * 1024 * 1024) in msg


def test_workspace_bytes(L):
    assert B.sgla_chunk_bwd_workspace_bytes(4, 16, 96) == 4 * 16 * 96 * 4
    assert B.sgla_chunk_bwd_workspace_bytes(0, 16, 96) == 0


def dec_args(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], lam=P["lam"], a=P["a"], state=P["state"], slot=None,
             o=P["o"], N=8, Pg=8, H=16, d_k=96, d_v=192, dt=B.SGLA_BF16)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["lam"], a["a"], a["state"], a["slot"], a["o"], a["N"],
            a["Pg"], a["H"], a["d_k"], a["d_v"], a["dt"], None]


DEC_BAD = [
    ("state null", dict(state=None), B.SGLA_ERR_INVALID_ARG),
    ("o null", dict(o=None), B.SGLA_ERR_INVALID_ARG),
    ("N zero", dict(N=0), B.SGLA_ERR_INVALID_ARG),
    ("pool too small", dict(Pg=4), B.SGLA_ERR_INVALID_ARG),
    ("slot misaligned", dict(slot=P["slot"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("d_k too big", dict(d_k=100), B.SGLA_ERR_UNSUPPORTED),
    ("d_v too big", dict(d_v=196), B.SGLA_ERR_UNSUPPORTED),
    ("d_k not a multiple of 4", dict(d_k=66), B.SGLA_ERR_UNSUPPORTED),
    ("d_v not a multiple of 4", dict(d_v=130), B.SGLA_ERR_UNSUPPORTED),
    ("d_k zero", dict(d_k=0), B.SGLA_ERR_UNSUPPORTED),
    ("dtype", dict(dt=3), B.SGLA_ERR_INVALID_ARG),
    ("o inside state", dict(o=P["state"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("state aliases q", dict(state=P["q"]), B.SGLA_ERR_INVALID_ARG),
    ("o aliases v", dict(o=P["v"]), B.SGLA_ERR_INVALID_ARG),
    ("state overlaps slot", dict(slot=P["state"] + 1024), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", DEC_BAD, ids=[x[0] for x in DEC_BAD])
def test_decode_rejects(L, name, kw, code):
    assert L.sgla_decode_step(*dec_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def test_binding_fails_loudly_without_library(tmp_path):
    code = ("import chunked_gated_linear_simple_amd.binding as b\n"
            "b.LIB_PATH = '/nonexistent/libsgla.so'\n"
            "try:\n    b.lib()\nexcept RuntimeError as e:\n    print('RAISED', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "RAISED" in r.stdout, r.stdout + r.stderr


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "chunked_gated_linear_simple_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text and "orc_" not in text, f


def conv_args(**kw):
    a = dict(u=P["u"], w=P["w"], b=P["b"], s0=P["s0"], sf=P["sf"], y=P["y"], cu=None, n_seq=2,
             B=2, T=64, D=3072, dt=B.SGLA_BF16)
    a.update(kw)
    return [a["u"], a["w"], a["b"], a["s0"], a["sf"], a["y"], a["cu"], a["n_seq"], a["B"], a["T"],
            a["D"], a["dt"], None]


CONV_BAD = [
    ("u null", dict(u=None), B.SGLA_ERR_INVALID_ARG),
    ("w null", dict(w=None), B.SGLA_ERR_INVALID_ARG),
    ("y null", dict(y=None), B.SGLA_ERR_INVALID_ARG),
    ("b misaligned", dict(b=P["b"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("init misaligned", dict(s0=P["s0"] + 8), B.SGLA_ERR_INVALID_ARG),
    ("D zero", dict(D=0), B.SGLA_ERR_INVALID_ARG),
    ("T negative", dict(T=-1), B.SGLA_ERR_INVALID_ARG),
    ("bad dtype", dict(dt=3), B.SGLA_ERR_INVALID_ARG),
    ("bf16 D not mult 8", dict(D=3076), B.SGLA_ERR_UNSUPPORTED),
    ("f32 D not mult 4", dict(D=3074, dt=B.SGLA_F32), B.SGLA_ERR_UNSUPPORTED),
    ("y aliases u", dict(y=P["u"]), B.SGLA_ERR_INVALID_ARG),
    ("y overlaps u", dict(y=P["u"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("dense n_seq != B", dict(n_seq=3), B.SGLA_ERR_INVALID_ARG),
    ("packed with B=2", dict(cu=P["cu"], n_seq=2), B.SGLA_ERR_INVALID_ARG),
    ("cu misaligned", dict(cu=P["cu"] + 4, n_seq=2, B=1), B.SGLA_ERR_INVALID_ARG),
    ("final state overlaps u", dict(sf=P["u"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("final state overlaps y", dict(sf=P["y"]), B.SGLA_ERR_INVALID_ARG),
    ("final state partly overlaps init", dict(sf=P["s0"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("y overlaps init", dict(y=P["s0"]), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", CONV_BAD, ids=[x[0] for x in CONV_BAD])
def test_conv_fwd_rejects(L, name, kw, code):
    assert L.sgla_conv_fwd(*conv_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def conv_dec_args(**kw):
    a = dict(x=P["u"], w=P["w"], b=P["b"], state=P["state"], slot=None, y=P["y"], N=8, Pg=8,
             D=3072, dt=B.SGLA_BF16)
    a.update(kw)
    return [a["x"], a["w"], a["b"], a["state"], a["slot"], a["y"], a["N"], a["Pg"], a["D"],
            a["dt"], None]


CONV_DEC_BAD = [
    ("x null", dict(x=None), B.SGLA_ERR_INVALID_ARG),
    ("state null", dict(state=None), B.SGLA_ERR_INVALID_ARG),
    ("slot misaligned", dict(slot=P["slot"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("N zero", dict(N=0), B.SGLA_ERR_INVALID_ARG),
    ("pool smaller than N without slot", dict(Pg=4), B.SGLA_ERR_INVALID_ARG),
    ("bf16 D not mult 8", dict(D=12), B.SGLA_ERR_UNSUPPORTED),
    ("y overlaps x", dict(y=P["u"] + 2048), B.SGLA_ERR_INVALID_ARG),
    ("state overlaps x", dict(state=P["u"]), B.SGLA_ERR_INVALID_ARG),
    ("state overlaps y", dict(state=P["y"] + 1024), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", CONV_DEC_BAD, ids=[x[0] for x in CONV_DEC_BAD])
def test_conv_decode_rejects(L, name, kw, code):
    assert L.sgla_conv_decode_step(*conv_dec_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def hng_args(**kw):
    a = dict(o=P["no"], g=P["ng"], gamma=P["gm"], out=P["nout"], B=2, H=16, T=64, d_v=192,
             n_tiers=4, eps=1e-6, dt=B.SGLA_BF16)
    a.update(kw)
    return [a["o"], a["g"], a["gamma"], a["out"], a["B"], a["H"], a["T"], a["d_v"], a["n_tiers"],
            a["eps"], a["dt"], None]


HNG_BAD = [
    ("o null", dict(o=None), B.SGLA_ERR_INVALID_ARG),
    ("g null", dict(g=None), B.SGLA_ERR_INVALID_ARG),
    ("out null", dict(out=None), B.SGLA_ERR_INVALID_ARG),
    ("gamma misaligned", dict(gamma=P["gm"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("T zero", dict(T=0), B.SGLA_ERR_INVALID_ARG),
    ("n_tiers zero", dict(n_tiers=0), B.SGLA_ERR_INVALID_ARG),
    ("n_tiers not dividing H", dict(n_tiers=3), B.SGLA_ERR_INVALID_ARG),
    ("eps negative", dict(eps=-1e-6), B.SGLA_ERR_INVALID_ARG),
    ("eps nan", dict(eps=float("nan")), B.SGLA_ERR_INVALID_ARG),
    ("eps inf", dict(eps=float("inf")), B.SGLA_ERR_INVALID_ARG),
    ("bad dtype", dict(dt=7), B.SGLA_ERR_INVALID_ARG),
    ("d_v not mult 4", dict(d_v=190), B.SGLA_ERR_UNSUPPORTED),
    ("d_v above 256", dict(d_v=260), B.SGLA_ERR_UNSUPPORTED),
    ("out overlaps o", dict(out=P["no"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("out partly overlaps g", dict(out=P["ng"] + 64), B.SGLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,code", HNG_BAD, ids=[x[0] for x in HNG_BAD])
def test_head_norm_gate_rejects(L, name, kw, code):
    assert L.sgla_head_norm_gate(*hng_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def hngb_args(**kw):
    a = dict(o=P["no"], g=P["ng"], gamma=P["gm"], dout=P["ndout"], do=P["ndo"], dg=P["ndg"],
             dgm=P["ndgm"], B=2, H=16, T=64, d_v=192, n_tiers=4, eps=1e-6, dt=B.SGLA_BF16,
             ws=P["ws"], wsb=2 * 16 * 1 * 192 * 4)
    a.update(kw)
    return [a["o"], a["g"], a["gamma"], a["dout"], a["do"], a["dg"], a["dgm"], a["B"], a["H"],
            a["T"], a["d_v"], a["n_tiers"], a["eps"], a["dt"], a["ws"], a["wsb"], None]


HNGB_BAD = [
    ("dout null", dict(dout=None), B.SGLA_ERR_INVALID_ARG),
    ("d_o null", dict(do=None), B.SGLA_ERR_INVALID_ARG),
    ("dg null", dict(dg=None), B.SGLA_ERR_INVALID_ARG),
    ("dgamma misaligned", dict(dgm=P["ndgm"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("tiers not dividing H", dict(n_tiers=3), B.SGLA_ERR_INVALID_ARG),
    ("eps negative", dict(eps=-1.0), B.SGLA_ERR_INVALID_ARG),
    ("d_v 260", dict(d_v=260), B.SGLA_ERR_UNSUPPORTED),
    ("workspace null", dict(ws=None), B.SGLA_ERR_WORKSPACE),
    ("workspace small", dict(wsb=64), B.SGLA_ERR_WORKSPACE),
    ("d_o aliases o", dict(do=P["no"]), B.SGLA_ERR_INVALID_ARG),
    ("dg aliases g", dict(dg=P["ng"]), B.SGLA_ERR_INVALID_ARG),
    ("dg overlaps dout", dict(dg=P["ndout"] + 256), B.SGLA_ERR_INVALID_ARG),
    ("d_o overlaps dg", dict(do=P["ndg"] + 512), B.SGLA_ERR_INVALID_ARG),
    ("dgamma aliases gamma", dict(dgm=P["gm"]), B.SGLA_ERR_INVALID_ARG),
    ("dgamma inside d_o", dict(dgm=P["ndo"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("workspace overlaps dg", dict(ws=P["ndg"]), B.SGLA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", HNGB_BAD, ids=[x[0] for x in HNGB_BAD])
def test_head_norm_gate_bwd_rejects(L, name, kw, code):
    assert L.sgla_head_norm_gate_bwd(*hngb_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def test_head_norm_gate_bwd_workspace_bytes(L):
    # one fp32 row of d_v per 64 tokens of each (b, h)
    assert B.sgla_head_norm_gate_bwd_workspace_bytes(8, 16, 2048, 192) == 8 * 16 * 32 * 192 * 4
    assert B.sgla_head_norm_gate_bwd_workspace_bytes(1, 2, 65, 64) == 1 * 2 * 2 * 64 * 4
    assert B.sgla_head_norm_gate_bwd_workspace_bytes(0, 2, 65, 64) == 0


def cbwd_args(**kw):
    a = dict(u=P["u"], w=P["w"], b=P["b"], s0=P["s0"], dy=P["dO"], dsf=P["sf"], du=P["y"],
             dw=P["dq"], db=P["db"] if "db" in P else P["dk"], ds0=P["ds0"], cu=None, n_seq=2, B=2,
             T=256, D=3072, dt=B.SGLA_BF16, ws=P["ws"], wsb=16 * 5 * 3072 * 4)
    a.update(kw)
    return [a["u"], a["w"], a["b"], a["s0"], a["dy"], a["dsf"], a["du"], a["dw"], a["db"], a["ds0"],
            a["cu"], a["n_seq"], a["B"], a["T"], a["D"], a["dt"], a["ws"], a["wsb"], None]


CBWD_BAD = [
    ("u null", dict(u=None), B.SGLA_ERR_INVALID_ARG),
    ("dy null", dict(dy=None), B.SGLA_ERR_INVALID_ARG),
    ("du null", dict(du=None), B.SGLA_ERR_INVALID_ARG),
    ("dw null", dict(dw=None), B.SGLA_ERR_INVALID_ARG),
    ("db misaligned", dict(db=P["dk"] + 4), B.SGLA_ERR_INVALID_ARG),
    ("dense n_seq != B", dict(n_seq=3), B.SGLA_ERR_INVALID_ARG),
    ("packed with B=2", dict(cu=P["cu"]), B.SGLA_ERR_INVALID_ARG),
    ("D not mult 8", dict(D=100), B.SGLA_ERR_UNSUPPORTED),
    ("workspace null", dict(ws=None), B.SGLA_ERR_WORKSPACE),
    ("workspace small", dict(wsb=1024), B.SGLA_ERR_WORKSPACE),
    ("du aliases u", dict(du=P["u"]), B.SGLA_ERR_INVALID_ARG),
    ("du overlaps dy", dict(du=P["dO"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("d_init aliases init", dict(ds0=P["s0"]), B.SGLA_ERR_INVALID_ARG),
    ("dw inside du", dict(dw=P["y"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("db aliases w", dict(db=P["w"]), B.SGLA_ERR_INVALID_ARG),
    ("d_init overlaps dw", dict(ds0=P["dq"]), B.SGLA_ERR_INVALID_ARG),
    ("workspace overlaps du", dict(ws=P["y"]), B.SGLA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", CBWD_BAD, ids=[x[0] for x in CBWD_BAD])
def test_conv_bwd_rejects(L, name, kw, code):
    assert L.sgla_conv_bwd(*cbwd_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def test_conv_bwd_workspace_bytes(L):
    # five fp32 rows of D per 64 token rows
    assert B.sgla_conv_bwd_workspace_bytes(8, 2048, 3072) == 256 * 5 * 3072 * 4
    assert B.sgla_conv_bwd_workspace_bytes(1, 65, 16) == 2 * 5 * 16 * 4
    assert B.sgla_conv_bwd_workspace_bytes(1, 64, 16) == 1 * 5 * 16 * 4
    assert B.sgla_conv_bwd_workspace_bytes(0, 33, 16) == 0


def segb_args(**kw):
    nbytes = (4 * 2 * 4 * 16 * 96 * 192 + 2 * 4 * 16 * 96) * 4
    a = dict(q=P["q"], k=P["k"], v=P["v"], dO=P["dO"], lam=P["lam"], a=P["a"], s0=P["s0"],
             dsf=P["sf"], dq=P["dq"], dk=P["dk"], dv=P["dv"], da=P["da"], ds0=P["ds0"], B=2, H=16,
             T=4096, d_k=96, d_v=192, chunk=128, dt=B.SGLA_BF16, nseg=4, ws=P["ws"], wsb=nbytes)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["dO"], a["lam"], a["a"], a["s0"], a["dsf"], a["dq"], a["dk"],
            a["dv"], a["da"], a["ds0"], a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["chunk"],
            a["dt"], a["nseg"], a["ws"], a["wsb"], None]


SEGB_BAD = [
    ("dO null", dict(dO=None), B.SGLA_ERR_INVALID_ARG),
    ("da null", dict(da=None), B.SGLA_ERR_INVALID_ARG),
    ("n_segments zero", dict(nseg=0), B.SGLA_ERR_INVALID_ARG),
    ("f32", dict(dt=B.SGLA_F32, d_k=16, d_v=32, chunk=64), B.SGLA_ERR_UNSUPPORTED),
    ("workspace null", dict(ws=None), B.SGLA_ERR_WORKSPACE),
    ("workspace small", dict(wsb=1 << 20), B.SGLA_ERR_WORKSPACE),
    ("dq aliases dO", dict(dq=P["dO"]), B.SGLA_ERR_INVALID_ARG),
    ("dv overlaps dk", dict(dv=P["dk"] + 1024), B.SGLA_ERR_INVALID_ARG),
    ("d_init aliases d_final", dict(ds0=P["sf"]), B.SGLA_ERR_INVALID_ARG),
    ("da overlaps d_init", dict(da=P["ds0"] + 4096), B.SGLA_ERR_INVALID_ARG),
    ("workspace overlaps dv", dict(ws=P["dv"]), B.SGLA_ERR_WORKSPACE),
    ("workspace overlaps init", dict(ws=P["s0"] + 4096), B.SGLA_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", SEGB_BAD, ids=[x[0] for x in SEGB_BAD])
def test_chunk_bwd_segmented_rejects(L, name, kw, code):
    assert L.sgla_chunk_bwd_segmented(*segb_args(**kw)) == code
    assert L.sgla_last_error().decode() != ""


def test_segmented_bwd_workspace_bytes(L):
    # four state arrays and the da partial sums, B * n_segments * H units
    u = 1 * 8 * 16
    assert B.sgla_chunk_bwd_segmented_workspace_bytes(1, 16, 96, 192, 8) == (4 * u * 96 * 192 + u * 96) * 4
    assert B.sgla_chunk_bwd_segmented_workspace_bytes(1, 16, 96, 192, 0) == 0
