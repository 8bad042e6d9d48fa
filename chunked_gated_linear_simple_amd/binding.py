"""Thin ctypes binding over libsgla (include/sgla.h).

Functions keep the C names. They only marshal arguments: read sizes off the
tensor shapes, check devices and dtypes, allocate outputs the caller did not
pass (torch.empty on the inputs' device), and hand raw device pointers plus
torch's current HIP stream to the library. Every step of the computation runs
in the library's kernels; there is no fallback of any kind. If libsgla.so is
not built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgla.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "sgla.h")

SGLA_OK, SGLA_ERR_INVALID_ARG, SGLA_ERR_UNSUPPORTED, SGLA_ERR_WORKSPACE, SGLA_ERR_HIP = range(5)
SGLA_F32, SGLA_BF16 = 0, 1
# SGLA_FWD_NORM_GATE_EXCHANGE_BYTES of include/sgla.h
FWD_NORM_GATE_EXCHANGE_BYTES = 2 * 1024 * 1024 + 256

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


class SglaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


def lib() -> ctypes.CDLL:
    """Open libsgla.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m chunked_gated_linear_simple_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sgla_version.restype = _i
        L.sgla_status_str.restype = ctypes.c_char_p
        L.sgla_status_str.argtypes = [_i]
        L.sgla_last_error.restype = ctypes.c_char_p
        L.sgla_decay_schedule.argtypes = [_i, ctypes.c_double, ctypes.c_double,
                                          ctypes.POINTER(ctypes.c_float)]
        L.sgla_decay_schedule.restype = _i
        L.sgla_chunk_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                     _i, _i, _i, _i, _i, _i, _i, _vp]
        L.sgla_chunk_fwd.restype = _i
        L.sgla_chunk_fwd_norm_gate.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _i, _i, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _vp,
                                               ctypes.c_size_t, ctypes.c_uint, _vp]
        L.sgla_chunk_fwd_norm_gate.restype = _i
        L.sgla_chunk_fwd_segmented_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.sgla_chunk_fwd_segmented_workspace_bytes.restype = ctypes.c_size_t
        L.sgla_chunk_fwd_segmented.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                               _i, _i, _i, _i, _i, _vp, ctypes.c_size_t, _vp]
        L.sgla_chunk_fwd_segmented.restype = _i
        L.sgla_chunk_bwd_segmented_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.sgla_chunk_bwd_segmented_workspace_bytes.restype = ctypes.c_size_t
        L.sgla_chunk_bwd_segmented.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp,
                                               ctypes.c_size_t, _vp]
        L.sgla_chunk_bwd_segmented.restype = _i
        L.sgla_chunk_bwd_workspace_bytes.argtypes = [_i, _i, _i]
        L.sgla_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.sgla_chunk_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp,
                                     ctypes.c_size_t, _vp]
        L.sgla_chunk_bwd.restype = _i
        L.sgla_chunk_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]
        L.sgla_chunk_bwd_noalloc.restype = _i
        L.sgla_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                       _i, _vp]
        L.sgla_decode_step.restype = _i
        L.sgla_conv_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
        L.sgla_conv_fwd.restype = _i
        L.sgla_conv_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
        L.sgla_conv_decode_step.restype = _i
        L.sgla_head_norm_gate.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, _i,
                                          _vp]
        L.sgla_head_norm_gate.restype = _i
        L.sgla_conv_bwd_workspace_bytes.argtypes = [_i, _i, _i]
        L.sgla_conv_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.sgla_conv_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                    _i, _i, _vp, ctypes.c_size_t, _vp]
        L.sgla_conv_bwd.restype = _i
        L.sgla_head_norm_gate_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i]
        L.sgla_head_norm_gate_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.sgla_head_norm_gate_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                              ctypes.c_float, _i, _vp, ctypes.c_size_t, _vp]
        L.sgla_head_norm_gate_bwd.restype = _i
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions include/sgla.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgla_\w+)\s*\(", text)))


def _check(status: int):
    if status != SGLA_OK:
        msg = lib().sgla_last_error().decode()
        raise SglaError(status, msg or lib().sgla_status_str(status).decode())


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SGLA_BF16
    if t.dtype == torch.float32:
        return SGLA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _stream(dev: torch.device):
    return _vp(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype=None, device=None, shape=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def sgla_version() -> int:
    return lib().sgla_version()


def sgla_decay_schedule(H: int, t_min: float, t_max: float) -> torch.Tensor:
    """[H] fp32 decays on the host."""
    out = (ctypes.c_float * H)()
    _check(lib().sgla_decay_schedule(int(H), float(t_min), float(t_max), out))
    return torch.tensor(list(out), dtype=torch.float32)


def _geometry(q, v, cu_seqlens):
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    n_seq = B if cu_seqlens is None else cu_seqlens.shape[0] - 1
    return B, H, T, d_k, d_v, n_seq


def sgla_chunk_fwd(q, k, v, lam, a=None, init_state=None, final_state=None, o=None,
                   cu_seqlens=None, chunk: int = 128, want_final: bool = False):
    """Chunked forward. Returns (o, final_state) (final_state None unless passed
    or want_final)."""
    dev = q.device
    B, H, T, d_k, d_v, n_seq = _geometry(q, v, cu_seqlens)
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, T, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(init_state, "init_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if o is None:
        o = torch.empty((B, H, T, d_v), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev, (B, H, T, d_v))
    if final_state is None and want_final:
        final_state = torch.empty((n_seq, H, d_k, d_v), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _check(lib().sgla_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(a),
                                _ptr(init_state), _ptr(final_state), _ptr(o), _ptr(cu_seqlens),
                                n_seq, B, H, T, d_k, d_v, int(chunk), _dtype_code(q),
                                _stream(dev)))
    return o, final_state


_exchange = {}


def fwd_norm_gate_exchange(device) -> torch.Tensor:
    """The device's zero-filled exchange buffer for sgla_chunk_fwd_norm_gate
    (allocated on first use; every completed call leaves it zero-filled). A
    caller running calls on several streams at once passes its own buffers."""
    device = torch.device(device)
    if device not in _exchange:
        _exchange[device] = torch.zeros(FWD_NORM_GATE_EXCHANGE_BYTES, dtype=torch.uint8, device=device)
    return _exchange[device]


def sgla_chunk_fwd_norm_gate(q, k, v, lam, g, a=None, gamma=None, n_tiers: int = 1, eps: float = 1e-6,
                             init_state=None, final_state=None, out=None, o=None, cu_seqlens=None,
                             chunk: int = 128, want_final: bool = False, want_o: bool = False, exchange=None):
    """Chunked forward with the mixer epilogue before the store. g and out are
    [B, T, H, d_v] (or [B, T, H * d_v]), token-major. Returns (out, o,
    final_state); o and final_state are None unless passed or wanted."""
    dev = q.device
    B, H, T, d_k, d_v, n_seq = _geometry(q, v, cu_seqlens)
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, T, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(gamma, "gamma", torch.float32, dev, (n_tiers, d_v))
    _need(init_state, "init_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    gshape = (B, T, H * d_v) if g.dim() == 3 else (B, T, H, d_v)
    _need(g, "g", q.dtype, dev, gshape)
    if out is None:
        out = torch.empty(gshape, dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, dev, gshape)
    if o is None and want_o:
        o = torch.empty((B, H, T, d_v), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev, (B, H, T, d_v))
    if final_state is None and want_final:
        final_state = torch.empty((n_seq, H, d_k, d_v), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    if exchange is None:
        exchange = fwd_norm_gate_exchange(dev)
    _need(exchange, "exchange", torch.uint8, dev)
    _check(lib().sgla_chunk_fwd_norm_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(a), _ptr(init_state),
                                          _ptr(final_state), _ptr(g), _ptr(gamma), _ptr(out), _ptr(o),
                                          _ptr(cu_seqlens), n_seq, B, H, T, d_k, d_v, int(chunk), int(n_tiers),
                                          float(eps), _dtype_code(q), _ptr(exchange), exchange.numel(), 0,
                                          _stream(dev)))
    return out, o, final_state


def sgla_chunk_fwd_segmented_workspace_bytes(B: int, H: int, d_k: int, d_v: int,
                                              n_segments: int) -> int:
    return int(lib().sgla_chunk_fwd_segmented_workspace_bytes(int(B), int(H), int(d_k), int(d_v),
                                                              int(n_segments)))


def sgla_chunk_fwd_segmented(q, k, v, lam, a=None, init_state=None, final_state=None, o=None,
                             n_segments: int = 2, chunk: int = 128, want_final: bool = False,
                             workspace=None):
    """Segment-parallel forward of dense sequences. Returns (o, final_state)
    (final_state None unless passed or want_final)."""
    dev = q.device
    B, H, T, d_k, d_v, _ = _geometry(q, v, None)
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, T, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(init_state, "init_state", torch.float32, dev, (B, H, d_k, d_v))
    if o is None:
        o = torch.empty((B, H, T, d_v), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev, (B, H, T, d_v))
    if final_state is None and want_final:
        final_state = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev, (B, H, d_k, d_v))
    nbytes = sgla_chunk_fwd_segmented_workspace_bytes(B, H, d_k, d_v, n_segments)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16) + 3) // 4, dtype=torch.float32, device=dev)
    _need(workspace, "workspace", device=dev)
    _check(lib().sgla_chunk_fwd_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(a),
                                          _ptr(init_state), _ptr(final_state), _ptr(o), B, H, T,
                                          d_k, d_v, int(chunk), _dtype_code(q), int(n_segments),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(dev)))
    return o, final_state


def sgla_chunk_bwd_segmented_workspace_bytes(B: int, H: int, d_k: int, d_v: int,
                                              n_segments: int) -> int:
    return int(lib().sgla_chunk_bwd_segmented_workspace_bytes(int(B), int(H), int(d_k), int(d_v),
                                                              int(n_segments)))


def sgla_chunk_bwd_segmented(q, k, v, dO, lam, a=None, init_state=None, d_final_state=None,
                             n_segments: int = 2, chunk: int = 128, want_d_init: bool = False,
                             dq=None, dk=None, dv=None, da=None, d_init_state=None, workspace=None):
    """Segment-parallel backward of dense sequences. Returns (dq, dk, dv, da,
    d_init_state)."""
    dev = q.device
    B, H, T, d_k, d_v, _ = _geometry(q, v, None)
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, T, d_v))
    _need(dO, "dO", q.dtype, dev, (B, H, T, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(init_state, "init_state", torch.float32, dev, (B, H, d_k, d_v))
    _need(d_final_state, "d_final_state", torch.float32, dev, (B, H, d_k, d_v))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    da = torch.empty((H, d_k), dtype=torch.float32, device=dev) if da is None else da
    if d_init_state is None and want_d_init:
        d_init_state = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=dev)
    _need(d_init_state, "d_init_state", torch.float32, dev, (B, H, d_k, d_v))
    nbytes = sgla_chunk_bwd_segmented_workspace_bytes(B, H, d_k, d_v, n_segments)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16) + 3) // 4, dtype=torch.float32, device=dev)
    _need(workspace, "workspace", device=dev)
    _check(lib().sgla_chunk_bwd_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lam), _ptr(a),
                                          _ptr(init_state), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(da), _ptr(d_init_state), B, H, T, d_k, d_v,
                                          int(chunk), _dtype_code(q), int(n_segments),
                                          _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(dev)))
    return dq, dk, dv, da, d_init_state


def sgla_chunk_bwd_workspace_bytes(N: int, H: int, d_k: int) -> int:
    return int(lib().sgla_chunk_bwd_workspace_bytes(int(N), int(H), int(d_k)))


def sgla_chunk_bwd(q, k, v, dO, lam, a=None, init_state=None, d_final_state=None,
                   cu_seqlens=None, chunk: int = 128, want_d_init: bool = False,
                   dq=None, dk=None, dv=None, da=None, d_init_state=None, workspace=None):
    """Chunked backward. Returns (dq, dk, dv, da, d_init_state)."""
    dev = q.device
    B, H, T, d_k, d_v, n_seq = _geometry(q, v, cu_seqlens)
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, T, d_v))
    _need(dO, "dO", q.dtype, dev, (B, H, T, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(init_state, "init_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _need(d_final_state, "d_final_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    da = torch.empty((H, d_k), dtype=torch.float32, device=dev) if da is None else da
    if d_init_state is None and want_d_init:
        d_init_state = torch.empty((n_seq, H, d_k, d_v), dtype=torch.float32, device=dev)
    for t, nm, shp in ((dq, "dq", q.shape), (dk, "dk", q.shape), (dv, "dv", v.shape)):
        _need(t, nm, q.dtype, dev, shp)
    _need(da, "da", torch.float32, dev, (H, d_k))
    _need(d_init_state, "d_init_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    nbytes = sgla_chunk_bwd_workspace_bytes(n_seq, H, d_k)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _check(lib().sgla_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lam), _ptr(a),
                                _ptr(init_state), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(da), _ptr(d_init_state), _ptr(cu_seqlens), n_seq,
                                B, H, T, d_k, d_v, int(chunk), _dtype_code(q), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk, dv, da, d_init_state


def sgla_chunk_bwd_noalloc(q, k, v, dO, lam, a=None, init_state=None, d_final_state=None,
                           cu_seqlens=None, chunk: int = 128, dq=None, dk=None, dv=None, da=None,
                           d_init_state=None):
    """sgla_chunk_bwd without a workspace: the library's fixed device scratch
    holds the partial sums. All outputs must be passed (the entry point is for
    callers that allocate nothing while it runs). Returns (dq, dk, dv, da,
    d_init_state)."""
    dev = q.device
    B, H, T, d_k, d_v, n_seq = _geometry(q, v, cu_seqlens)
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (da, "da")):
        if t is None:
            raise ValueError(f"{nm} must be passed")
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, T, d_v))
    _need(dO, "dO", q.dtype, dev, (B, H, T, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(init_state, "init_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _need(d_final_state, "d_final_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    for t, nm, shp in ((dq, "dq", q.shape), (dk, "dk", q.shape), (dv, "dv", v.shape)):
        _need(t, nm, q.dtype, dev, shp)
    _need(da, "da", torch.float32, dev, (H, d_k))
    _need(d_init_state, "d_init_state", torch.float32, dev, (n_seq, H, d_k, d_v))
    _check(lib().sgla_chunk_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lam), _ptr(a),
                                        _ptr(init_state), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                                        _ptr(dv), _ptr(da), _ptr(d_init_state), _ptr(cu_seqlens),
                                        n_seq, B, H, T, d_k, d_v, int(chunk), _dtype_code(q),
                                        _stream(dev)))
    return dq, dk, dv, da, d_init_state


def sgla_decode_step(q, k, v, lam, a, state, o=None, slot=None):
    """One in-place decode step. q,k [N,H,d_k], v [N,H,d_v], state [P,H,d_k,d_v].
    Returns o [N,H,d_v]."""
    dev = q.device
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    P = state.shape[0]
    _need(q, "q", device=dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (N, H, d_v))
    _need(lam, "lambda", torch.float32, dev, (H,))
    _need(a, "a", torch.float32, dev, (H, d_k))
    _need(state, "state", torch.float32, dev, (P, H, d_k, d_v))
    _need(slot, "slot", torch.int32, dev, (N,))
    if o is None:
        o = torch.empty((N, H, d_v), dtype=q.dtype, device=dev)
    _need(o, "o", q.dtype, dev, (N, H, d_v))
    _check(lib().sgla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(a), _ptr(state),
                                  _ptr(slot), _ptr(o), N, P, H, d_k, d_v, _dtype_code(q),
                                  _stream(dev)))
    return o


def sgla_conv_fwd(u, w, b=None, init_state=None, final_state=None, y=None, cu_seqlens=None,
                  want_final=False):
    """Conv prologue over whole sequences. u [B, T, D] (or [T, D] packed with
    cu_seqlens [N+1] int32), w [D, 4] fp32, b [D] fp32 or None, init_state /
    final_state [N, 3, D] fp32 or None. Returns (y, final_state or None)."""
    dev = u.device
    if cu_seqlens is None:
        Bn, T, D = u.shape
        n_seq = Bn
    else:
        T, D = u.shape
        Bn = 1
        n_seq = cu_seqlens.numel() - 1
    _need(u, "u", device=dev)
    _need(w, "w", torch.float32, dev, (D, 4))
    _need(b, "b", torch.float32, dev, (D,))
    _need(init_state, "init_state", torch.float32, dev, (n_seq, 3, D))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, (n_seq + 1,))
    if final_state is None and want_final:
        final_state = torch.empty((n_seq, 3, D), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, dev, (n_seq, 3, D))
    if y is None:
        y = torch.empty_like(u)
    _need(y, "y", u.dtype, dev, tuple(u.shape))
    _check(lib().sgla_conv_fwd(_ptr(u), _ptr(w), _ptr(b), _ptr(init_state), _ptr(final_state),
                               _ptr(y), _ptr(cu_seqlens), n_seq, Bn, T, D, _dtype_code(u),
                               _stream(dev)))
    return y, final_state


def sgla_conv_bwd_workspace_bytes(B: int, T: int, D: int) -> int:
    return int(lib().sgla_conv_bwd_workspace_bytes(int(B), int(T), int(D)))


def sgla_conv_bwd(u, w, dy, b=None, init_state=None, d_final_state=None, cu_seqlens=None,
                  want_db=True, want_d_init=False, du=None, dw=None, db=None, d_init_state=None,
                  workspace=None):
    """Gradients of sgla_conv_fwd. u, dy [B, T, D] (or [T, D] packed with
    cu_seqlens). Returns (du, dw [D, 4], db [D] or None, d_init_state
    [N, 3, D] or None)."""
    dev = u.device
    if cu_seqlens is None:
        Bn, T, D = u.shape
        n_seq = Bn
    else:
        T, D = u.shape
        Bn = 1
        n_seq = cu_seqlens.numel() - 1
    _need(u, "u", device=dev)
    _need(dy, "dy", u.dtype, dev, tuple(u.shape))
    _need(w, "w", torch.float32, dev, (D, 4))
    _need(b, "b", torch.float32, dev, (D,))
    _need(init_state, "init_state", torch.float32, dev, (n_seq, 3, D))
    _need(d_final_state, "d_final_state", torch.float32, dev, (n_seq, 3, D))
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, (n_seq + 1,))
    if du is None:
        du = torch.empty_like(u)
    _need(du, "du", u.dtype, dev, tuple(u.shape))
    if dw is None:
        dw = torch.empty((D, 4), dtype=torch.float32, device=dev)
    _need(dw, "dw", torch.float32, dev, (D, 4))
    if db is None and want_db:
        db = torch.empty((D,), dtype=torch.float32, device=dev)
    _need(db, "db", torch.float32, dev, (D,))
    if d_init_state is None and want_d_init:
        d_init_state = torch.empty((n_seq, 3, D), dtype=torch.float32, device=dev)
    _need(d_init_state, "d_init_state", torch.float32, dev, (n_seq, 3, D))
    nbytes = sgla_conv_bwd_workspace_bytes(Bn, T, D)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16) + 3) // 4, dtype=torch.float32, device=dev)
    _need(workspace, "workspace", device=dev)
    _check(lib().sgla_conv_bwd(_ptr(u), _ptr(w), _ptr(b), _ptr(init_state), _ptr(dy),
                               _ptr(d_final_state), _ptr(du), _ptr(dw), _ptr(db), _ptr(d_init_state),
                               _ptr(cu_seqlens), n_seq, Bn, T, D, _dtype_code(u), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(dev)))
    return du, dw, db, d_init_state


def sgla_conv_decode_step(x, w, b, state, y=None, slot=None):
    """One in-place conv decode step. x [N, D], state [P, 3, D] fp32. Returns y [N, D]."""
    dev = x.device
    N, D = x.shape
    P = state.shape[0]
    _need(x, "x", device=dev)
    _need(w, "w", torch.float32, dev, (D, 4))
    _need(b, "b", torch.float32, dev, (D,))
    _need(state, "state", torch.float32, dev, (P, 3, D))
    _need(slot, "slot", torch.int32, dev, (N,))
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, dev, (N, D))
    _check(lib().sgla_conv_decode_step(_ptr(x), _ptr(w), _ptr(b), _ptr(state), _ptr(slot),
                                       _ptr(y), N, P, D, _dtype_code(x), _stream(dev)))
    return y


def sgla_head_norm_gate(o, g, gamma=None, n_tiers=1, eps=1e-6, out=None):
    """Head RMSNorm per decay tier + SiLU(g) gate. o [B, H, T, d_v] (the mixer's
    layout), g [B, T, H, d_v] or [B, T, H * d_v], gamma [n_tiers, d_v] fp32 or
    None. Returns out shaped like g (token-major, heads concatenated)."""
    dev = o.device
    B, H, T, d_v = o.shape
    _need(o, "o", device=dev)
    if g.dim() == 3:
        _need(g, "g", o.dtype, dev, (B, T, H * d_v))
    else:
        _need(g, "g", o.dtype, dev, (B, T, H, d_v))
    _need(gamma, "gamma", torch.float32, dev, (n_tiers, d_v))
    if out is None:
        out = torch.empty_like(g)
    _need(out, "out", o.dtype, dev, tuple(g.shape))
    _check(lib().sgla_head_norm_gate(_ptr(o), _ptr(g), _ptr(gamma), _ptr(out), B, H, T, d_v,
                                     int(n_tiers), float(eps), _dtype_code(o), _stream(dev)))
    return out


def sgla_head_norm_gate_bwd_workspace_bytes(B: int, H: int, T: int, d_v: int) -> int:
    return int(lib().sgla_head_norm_gate_bwd_workspace_bytes(int(B), int(H), int(T), int(d_v)))


def sgla_head_norm_gate_bwd(o, g, dout, gamma=None, n_tiers=1, eps=1e-6, want_dgamma=True,
                            d_o=None, dg=None, dgamma=None, workspace=None):
    """Gradients of sgla_head_norm_gate. o [B, H, T, d_v]; g and dout shaped
    like the forward's g ([B, T, H, d_v] or [B, T, H * d_v]). Returns
    (d_o [B, H, T, d_v], dg shaped like g, dgamma [n_tiers, d_v] fp32 or None)."""
    dev = o.device
    B, H, T, d_v = o.shape
    _need(o, "o", device=dev)
    gshape = (B, T, H * d_v) if g.dim() == 3 else (B, T, H, d_v)
    _need(g, "g", o.dtype, dev, gshape)
    _need(dout, "dout", o.dtype, dev, gshape)
    _need(gamma, "gamma", torch.float32, dev, (n_tiers, d_v))
    if d_o is None:
        d_o = torch.empty_like(o)
    _need(d_o, "d_o", o.dtype, dev, (B, H, T, d_v))
    if dg is None:
        dg = torch.empty_like(g)
    _need(dg, "dg", o.dtype, dev, gshape)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty((n_tiers, d_v), dtype=torch.float32, device=dev)
    _need(dgamma, "dgamma", torch.float32, dev, (n_tiers, d_v))
    nbytes = sgla_head_norm_gate_bwd_workspace_bytes(B, H, T, d_v)
    if workspace is None and dgamma is not None:
        workspace = torch.empty((max(nbytes, 16) + 3) // 4, dtype=torch.float32, device=dev)
    _need(workspace, "workspace", device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sgla_head_norm_gate_bwd(_ptr(o), _ptr(g), _ptr(gamma), _ptr(dout), _ptr(d_o),
                                         _ptr(dg), _ptr(dgamma), B, H, T, d_v, int(n_tiers),
                                         float(eps), _dtype_code(o), _ptr(workspace), wsb,
                                         _stream(dev)))
    return d_o, dg, dgamma
