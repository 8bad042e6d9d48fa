"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no part of the method's arithmetic: it draws Gaussian
tensors, rounds them to the storage dtype and lays them out. Both the HIP path
and the oracle consume what it returns (the oracle after widening to float64),
so the two sides always see bit-identical inputs.

Every tensor comes from its own stream: numpy's PCG64 seeded with
``SeedSequence([seed, stream_id])``, so any tensor (or a slice of it) can be
regenerated on its own. "N(m, s)" in a recipe means mean m, standard deviation s.
"""
from __future__ import annotations

import math

import numpy as np

# stream ids, one per tensor role
STREAM_Q, STREAM_K, STREAM_V, STREAM_A, STREAM_S0, STREAM_DO, STREAM_DSF, STREAM_LEN = range(1, 9)
STREAM_DECODE_BASE = 1000  # decode step s uses streams 1000 + 3*s + {0,1,2}


def gaussian(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u >> 16) & 1) + 0x7FFF
    out = ((u + r) >> 16).astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> storage array: uint16 bf16 bits ('bf16') or float32 ('f32')."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> exact float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def varlen_lengths(seed: int, n: int = 32, lo: int = 128, hi: int = 32768) -> np.ndarray:
    """n lengths log-uniform in [lo, hi], the largest then set to hi."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), STREAM_LEN])))
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    L = np.rint(np.exp(u)).astype(np.int64)
    L = np.clip(L, lo, hi)
    L[int(np.argmax(L))] = hi
    return L


def cu_from_lengths(L) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(L, dtype=np.int64))]).astype(np.int32)


def chunk_inputs(B: int, H: int, T: int, d_k: int, d_v: int, dtype: str, seed: int,
                 a_std: float | None = 0.1, s0_std: float | None = None,
                 n_seq: int | None = None, with_grad: bool = False,
                 dsf_std: float | None = None) -> dict:
    """Inputs of one chunked call.

    q, k ~ N(0,1) [B,H,T,d_k] with q scaled by d_k^-1/2 before rounding;
    v ~ N(0,1) [B,H,T,d_v]; a ~ N(0, a_std) [H,d_k] (zeros if a_std is None);
    S0 ~ N(0, s0_std) [N,H,d_k,d_v] if s0_std is given; dO ~ N(0,1) like v and
    dS_final ~ N(0, dsf_std) if requested. N = n_seq (packed) or B.
    """
    qs = gaussian(seed, STREAM_Q, (B, H, T, d_k)) * np.float32(d_k ** -0.5)
    ks = gaussian(seed, STREAM_K, (B, H, T, d_k))
    vs = gaussian(seed, STREAM_V, (B, H, T, d_v))
    N = B if n_seq is None else n_seq
    out = {
        "B": B, "H": H, "T": T, "d_k": d_k, "d_v": d_v, "dtype": dtype, "N": N,
        "q": store(qs, dtype), "k": store(ks, dtype), "v": store(vs, dtype),
        "a": (np.zeros((H, d_k), np.float32) if a_std is None
              else gaussian(seed, STREAM_A, (H, d_k), a_std)),
        "S0": None if s0_std is None else gaussian(seed, STREAM_S0, (N, H, d_k, d_v), s0_std),
    }
    if with_grad:
        out["dO"] = store(gaussian(seed, STREAM_DO, (B, H, T, d_v)), dtype)
        out["dSf"] = (None if dsf_std is None
                      else gaussian(seed, STREAM_DSF, (N, H, d_k, d_v), dsf_std))
    return out


def decode_token_inputs(seed: int, step: int, N: int, H: int, d_k: int, d_v: int,
                        dtype: str = "bf16") -> tuple:
    """q, k [N,H,d_k] (q scaled by d_k^-1/2) and v [N,H,d_v] for decode step ``step``."""
    base = STREAM_DECODE_BASE + 3 * step
    q = gaussian(seed, base, (N, H, d_k)) * np.float32(d_k ** -0.5)
    k = gaussian(seed, base + 1, (N, H, d_k))
    v = gaussian(seed, base + 2, (N, H, d_v))
    return store(q, dtype), store(k, dtype), store(v, dtype)


STREAM_CONV = 2000  # conv prologue: u, w, b, init state, decode tokens 2004 + step
STREAM_CONV_GRAD = 2500  # conv prologue gradients: dy, final states' gradient


def conv_inputs(seed: int, shape, D: int, dtype: str, n_seq: int, w_std: float = 0.5,
                b_std: float = 0.1, s0_std: float = 1.0, bias: bool = True, state: bool = True,
                with_grad: bool = False):
    """Seeded inputs of the conv prologue: u (shape, last axis D) in the storage
    dtype, taps w [D, 4], bias b [D] and initial conv states [n_seq, 3, D] in fp32
    (the states hold past inputs, so they are drawn like u and rounded to the
    input dtype's values). with_grad adds dy ~ N(0, 1) like u (storage dtype)
    and the final states' gradient dSf ~ N(0, 1) [n_seq, 3, D] fp32."""
    u = store(gaussian(seed, STREAM_CONV, tuple(shape)), dtype)
    w = gaussian(seed, STREAM_CONV + 1, (D, 4), w_std)
    b = gaussian(seed, STREAM_CONV + 2, (D,), b_std) if bias else None
    s0 = None
    if state:
        s0 = gaussian(seed, STREAM_CONV + 3, (n_seq, 3, D), s0_std)
        s0 = widen(store(s0, dtype), dtype).astype(np.float32)
    out = {"u": u, "w": w, "b": b, "S0": s0, "dtype": dtype, "D": D, "N": n_seq}
    if with_grad:
        out["dy"] = store(gaussian(seed, STREAM_CONV_GRAD, tuple(shape)), dtype)
        out["dSf"] = gaussian(seed, STREAM_CONV_GRAD + 1, (n_seq, 3, D))
    return out


STREAM_NORM = 3000  # mixer epilogue: o, g, gamma, dout


def norm_inputs(seed: int, B: int, H: int, T: int, d_v: int, n_tiers: int, dtype: str,
                o_std: float = 1.0, g_std: float = 1.0, gamma_std: float = 0.1, gamma: bool = True,
                with_dout: bool = False):
    """Seeded inputs of the mixer epilogue: o [B, H, T, d_v] (the mixer's
    head-major output) and the gate stream g [B, T, H, d_v] in the storage
    dtype, and the per-tier scales gamma [n_tiers, d_v] = 1 + N(0, gamma_std)
    in fp32 (or None); with_dout adds the upstream gradient dout ~ N(0, 1)
    [B, T, H, d_v] in the storage dtype."""
    o = store(gaussian(seed, STREAM_NORM, (B, H, T, d_v), o_std), dtype)
    g = store(gaussian(seed, STREAM_NORM + 1, (B, T, H, d_v), g_std), dtype)
    gm = None
    if gamma:
        gm = (1.0 + gaussian(seed, STREAM_NORM + 2, (n_tiers, d_v), gamma_std)).astype(np.float32)
    out = {"o": o, "g": g, "gamma": gm, "dtype": dtype, "n_tiers": n_tiers}
    if with_dout:
        out["dout"] = store(gaussian(seed, STREAM_NORM + 3, (B, T, H, d_v)), dtype)
    return out
