"""Multi-scale retention (RetNet) forward pass on MI355X — Python binding.

A thin ctypes layer over ``librn_retention.so`` (C ABI in include/rn_retention.h).
Functions carry the C names; they only marshal arguments: check tensors, allocate
outputs with torch, pass device pointers and the current HIP stream. Every step of
the computation runs in the library's HIP kernels. There is no CPU fallback: if the
library is missing, importing this package raises.

Build the library with ``python linear_recurrent_sequence_rn_amd/build.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "RN_OK", "RN_ERR_INVALID_ARG", "RN_ERR_UNSUPPORTED", "RN_ERR_HIP", "RN_ERR_WORKSPACE",
    "RN_ERR_EXCHANGE", "RN_ERR_NONFINITE",
    "RN_F32", "RN_BF16", "RN_NORM_D_ROW", "RN_NORM_R_ROW", "RN_EPI_GN", "RN_EPI_GATE",
    "RN_FORCE_GENERIC", "RN_CHUNK_PARALLEL", "RN_CHUNK_SEGMENTED", "RN_TEST_FORCE_TIMEOUT",
    "RnError", "RnDesc", "lib", "LIB_PATH", "EXPORTED_SYMBOLS", "rn_chunkwise_check",
    "rn_retention_parallel", "rn_retention_chunkwise", "rn_retention_recurrent_step",
    "rn_retention_chunkwise_varlen", "rn_retention_recurrent_step_at", "rn_groupnorm_gate",
    "rn_retention_chunkwise_backward", "rn_chunkwise_backward_workspace_bytes", "rn_chunkwise_workspace_bytes", "rn_parallel_workspace_bytes",
    "rn_version", "make_desc", "rn_msr_layer_forward", "rn_msr_layer_workspace_bytes",
    "rn_retention_chunkwise_noalloc",
]

# The in-tree build; RN_LIB_PATH names another build of the same sources (the host-side
# tests use it for a copy built with the sanitizers).
LIB_PATH = Path(os.environ.get("RN_LIB_PATH") or Path(__file__).resolve().parent / "librn_retention.so")

RN_OK, RN_ERR_INVALID_ARG, RN_ERR_UNSUPPORTED, RN_ERR_HIP, RN_ERR_WORKSPACE = 0, -1, -2, -3, -4
RN_ERR_EXCHANGE, RN_ERR_NONFINITE = -5, -6
RN_F32, RN_BF16 = 0, 1
RN_NORM_D_ROW, RN_NORM_R_ROW, RN_EPI_GN, RN_EPI_GATE = 1, 2, 4, 8
RN_FORCE_GENERIC = 1 << 8
RN_CHUNK_PARALLEL = 1 << 9
RN_CHUNK_SEGMENTED = 1 << 10
RN_TEST_FORCE_TIMEOUT = 1 << 12

EXPORTED_SYMBOLS = (
    "rn_parallel_workspace_bytes", "rn_retention_parallel", "rn_chunkwise_workspace_bytes", "rn_retention_chunkwise",
    "rn_retention_recurrent_step", "rn_retention_chunkwise_varlen",
    "rn_retention_recurrent_step_at", "rn_groupnorm_gate", "rn_status_str", "rn_last_error",
    "rn_version", "rn_retention_chunkwise_backward", "rn_chunkwise_backward_workspace_bytes",
    "rn_msr_layer_workspace_bytes", "rn_msr_layer_forward", "rn_chunkwise_check",
    "rn_retention_chunkwise_noalloc",
)


class RnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class RnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("pos0", ctypes.c_int64),
        ("qk_scale", ctypes.c_float), ("gn_eps", ctypes.c_float),
        ("gamma", ctypes.POINTER(ctypes.c_float)), ("theta", ctypes.POINTER(ctypes.c_float)),
        ("gn_weight", ctypes.c_void_p), ("gn_bias", ctypes.c_void_p),
        ("gamma_pair", ctypes.c_void_p),
    ]


def _load():
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python linear_recurrent_sequence_rn_amd/build.py`")
    L = ctypes.CDLL(str(LIB_PATH))
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(RnDesc)
    L.rn_parallel_workspace_bytes.argtypes = [D]
    L.rn_parallel_workspace_bytes.restype = sz
    L.rn_retention_parallel.argtypes = [D, vp, vp, vp, vp, vp, vp, sz, vp]
    L.rn_retention_parallel.restype = i32
    L.rn_chunkwise_workspace_bytes.argtypes = [D, i32]
    L.rn_chunkwise_workspace_bytes.restype = sz
    L.rn_retention_chunkwise.argtypes = [D, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.rn_retention_chunkwise.restype = i32
    L.rn_retention_recurrent_step.argtypes = [D, vp, vp, vp, vp, vp, vp, vp]
    L.rn_retention_recurrent_step.restype = i32
    L.rn_retention_chunkwise_varlen.argtypes = [D, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.rn_retention_chunkwise_varlen.restype = i32
    L.rn_retention_recurrent_step_at.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp]
    L.rn_retention_recurrent_step_at.restype = i32
    L.rn_chunkwise_backward_workspace_bytes.argtypes = [D, i32]
    L.rn_chunkwise_backward_workspace_bytes.restype = sz
    L.rn_retention_chunkwise_backward.argtypes = [D, i32] + [vp] * 14 + [vp, sz, vp]
    L.rn_retention_chunkwise_backward.restype = i32
    L.rn_msr_layer_workspace_bytes.argtypes = [D, i32, i32]
    L.rn_msr_layer_workspace_bytes.restype = sz
    L.rn_msr_layer_forward.argtypes = [D, i32, i32] + [vp] * 9 + [vp, sz, vp]
    L.rn_msr_layer_forward.restype = i32
    L.rn_chunkwise_check.argtypes = [D, i32, vp, sz, vp]
    L.rn_chunkwise_check.restype = i32
    L.rn_retention_chunkwise_noalloc.argtypes = [D, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.rn_retention_chunkwise_noalloc.restype = i32
    L.rn_groupnorm_gate.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                    ctypes.c_float, vp, vp]
    L.rn_groupnorm_gate.restype = i32
    L.rn_status_str.argtypes = [i32]
    L.rn_status_str.restype = ctypes.c_char_p
    L.rn_last_error.argtypes = []
    L.rn_last_error.restype = ctypes.c_char_p
    L.rn_version.argtypes = []
    L.rn_version.restype = ctypes.c_char_p
    return L


lib = _load()


def _status_name(s: int) -> str:
    return lib.rn_status_str(s).decode()


def _check(status: int):
    if status != RN_OK:
        raise RnError(status, lib.rn_last_error().decode())


def rn_version() -> str:
    return lib.rn_version().decode()


_DT = {torch.float32: RN_F32, torch.bfloat16: RN_BF16}


def _dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")
    return _DT[t]


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _out(out, shape, dtype, device, fill=None):
    """A new output tensor, or the caller's after checking it matches the call."""
    if out is None:
        if fill is None:
            return torch.empty(shape, dtype=dtype, device=device)
        return torch.full(shape, fill, dtype=dtype, device=device)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError(f"out must be {dtype} {tuple(shape)}; got {out.dtype} {tuple(out.shape)}")
    return out


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _is_pair_decay(gamma) -> bool:
    return isinstance(gamma, torch.Tensor) and gamma.dim() == 2 or \
        isinstance(gamma, np.ndarray) and gamma.ndim == 2


def make_desc(B: int, H: int, N: int, d_k: int, d_v: int, in_dtype: int, out_dtype: int,
              gamma, theta: Sequence[float], *, flags: int = 0, pos0: int = 0,
              qk_scale: float = 1.0, gn_eps: float = 1e-5, gn_weight=None, gn_bias=None,
              device=None):
    """Builds an rn_desc; returns (desc, keepalive) — keep both alive across the call.

    ``gamma`` is either H per-head decays (host sequence) or one decay per (head,
    coordinate pair): a float32 [H, d_k/2] tensor on the GPU, or a 2-D host array that is
    copied to ``device`` (the descriptor's gamma_pair). With a CPU ``device`` the copy
    stays on the host, which only calls that never read it may take (workspace sizes,
    argument checks)."""
    th = np.ascontiguousarray(np.asarray(theta, dtype=np.float32))
    d = RnDesc()
    d.B, d.H, d.N, d.d_k, d.d_v = B, H, N, d_k, d_v
    d.in_dtype, d.out_dtype, d.flags, d.pos0 = in_dtype, out_dtype, flags, pos0
    d.qk_scale, d.gn_eps = qk_scale, gn_eps
    if _is_pair_decay(gamma):
        gp = gamma
        if not isinstance(gp, torch.Tensor) or not gp.is_cuda:
            host = gamma.detach().cpu().numpy() if isinstance(gamma, torch.Tensor) else gamma
            dev = torch.device(device) if device is not None else torch.device("cpu")
            gp = torch.as_tensor(np.asarray(host, dtype=np.float32), device=dev)
        if gp.dtype != torch.float32 or tuple(gp.shape) != (H, d_k // 2):
            raise ValueError(f"pair decays must be float32 [{H}, {d_k // 2}]")
        gp = gp.contiguous()
        g = None
        d.gamma = None
        d.gamma_pair = gp.data_ptr()
    else:
        gp = None
        g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
        d.gamma = g.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        d.gamma_pair = None
    d.theta = th.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    d.gn_weight = None if gn_weight is None else gn_weight.data_ptr()
    d.gn_bias = None if gn_bias is None else gn_bias.data_ptr()
    return d, (g, gp, th, gn_weight, gn_bias)


def _flags(norm_d, norm_r, gn, gate, force_generic, chunk_parallel=False, segmented=False,
           test_force_timeout=False):
    f = 0
    if test_force_timeout: f |= RN_TEST_FORCE_TIMEOUT
    if chunk_parallel: f |= RN_CHUNK_PARALLEL
    if segmented: f |= RN_CHUNK_SEGMENTED
    if norm_d: f |= RN_NORM_D_ROW
    if norm_r: f |= RN_NORM_R_ROW
    if gn: f |= RN_EPI_GN
    if gate is not None: f |= RN_EPI_GATE
    if force_generic: f |= RN_FORCE_GENERIC
    return f


def _check_affine(gn_weight, gn_bias, n, device):
    """GroupNorm weight and bias: float32 with n elements, on the call's device."""
    for t in (gn_weight, gn_bias):
        if t is not None:
            if t.dtype != torch.float32 or t.numel() != n or t.device != device:
                raise ValueError(f"gn_weight/gn_bias must be float32 with {n} elements on {device}")
            _ptr(t)


def _qkv_desc(q, k, v, gamma, theta, out_dtype, flags, pos0, qk_scale, gn_eps, gn_weight, gn_bias,
              gate=None):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q,k [B,H,N,d_k] and v [B,H,N,d_v]; got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not (k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one device")
    if gate is not None and (gate.shape != v.shape or gate.dtype != q.dtype or gate.device != q.device):
        raise ValueError(f"gate must match v: {q.dtype} {tuple(v.shape)} on {q.device}; got "
                         f"{gate.dtype} {tuple(gate.shape)} on {gate.device}")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if len(gamma) != H or len(theta) != dk // 2:
        raise ValueError(f"need gamma[{H}] (or [{H}, {dk // 2}]) and theta[{dk // 2}]")
    od = q.dtype if out_dtype is None else out_dtype
    _check_affine(gn_weight, gn_bias, H * dv, q.device)
    d, keep = make_desc(B, H, N, dk, dv, _dtype_code(q.dtype), _dtype_code(od), gamma, theta,
                        flags=flags, pos0=pos0, qk_scale=qk_scale, gn_eps=gn_eps,
                        gn_weight=gn_weight, gn_bias=gn_bias, device=q.device)
    return d, keep, od


def rn_retention_parallel(q, k, v, gamma, theta, *, gate=None, out=None, out_dtype=None,
                          workspace=None, pos0=0, qk_scale=1.0, norm_d=False, norm_r=False,
                          gn=False, gn_eps=1e-5, gn_weight=None, gn_bias=None,
                          force_generic=False):
    """Parallel form; returns out [B,H,N,d_v]."""
    flags = _flags(norm_d, norm_r, gn, gate, force_generic)
    d, keep, od = _qkv_desc(q, k, v, gamma, theta, out_dtype, flags, pos0, qk_scale, gn_eps,
                            gn_weight, gn_bias, gate)
    out = _out(out, v.shape, od, v.device)
    need = int(lib.rn_parallel_workspace_bytes(ctypes.byref(d)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nws = 0 if workspace is None else workspace.numel()
    _check(lib.rn_retention_parallel(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                     _ptr(out), _ptr(workspace), nws, _stream(q)))
    return out


def rn_parallel_workspace_bytes(q, v, gamma, theta, *, norm_d=False, norm_r=False, gn=False,
                                gate=None, out_dtype=None, force_generic=False) -> int:
    B, H, N, dk = q.shape
    flags = _flags(norm_d, norm_r, gn, gate, force_generic)
    od = q.dtype if out_dtype is None else out_dtype
    d, keep = make_desc(B, H, N, dk, v.shape[-1], _dtype_code(q.dtype), _dtype_code(od), gamma,
                        theta, flags=flags, device=q.device)
    return int(lib.rn_parallel_workspace_bytes(ctypes.byref(d)))


def rn_chunkwise_workspace_bytes(q, v, gamma, theta, chunk, *, gn=False, gate=None,
                                 out_dtype=None, force_generic=False, chunk_parallel=False,
                                 segmented=False) -> int:
    B, H, N, dk = q.shape
    flags = _flags(False, False, gn, gate, force_generic, chunk_parallel, segmented)
    od = q.dtype if out_dtype is None else out_dtype
    d, keep = make_desc(B, H, N, dk, v.shape[-1], _dtype_code(q.dtype), _dtype_code(od), gamma,
                        theta, flags=flags, device=q.device)
    return int(lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), chunk))


def _seq_array(t, B, dtype, name):
    if t is None:
        return None
    if t.dtype != dtype or tuple(t.shape) != (B,):
        raise ValueError(f"{name} must be a {dtype} tensor of shape [{B}]")
    return _ptr(t)


def rn_retention_chunkwise(q, k, v, gamma, theta, chunk, *, gate=None, state_in=None,
                           state_out=None, out=None, out_dtype=None, workspace=None, pos0=0,
                           qk_scale=1.0, gn=False, gn_eps=1e-5, gn_weight=None, gn_bias=None,
                           force_generic=False, chunk_parallel=False, segmented=False,
                           test_force_timeout=False):
    """Chunkwise form; returns (out, state_out). ``state_out`` may be a tensor (written),
    True (allocated), or None/False (discarded). ``chunk_parallel`` selects the two-kernel
    chunk-parallel pair (RN_CHUNK_PARALLEL), ``segmented`` the segmented schedule
    (RN_CHUNK_SEGMENTED); by default the sequential kernel runs where it applies.
    ``test_force_timeout`` sets RN_TEST_FORCE_TIMEOUT (exercises the error path)."""
    return _chunkwise(q, k, v, gamma, theta, chunk, None, None, gate, state_in, state_out, out,
                      out_dtype, workspace, pos0, qk_scale, gn, gn_eps, gn_weight, gn_bias,
                      force_generic, chunk_parallel, segmented, test_force_timeout)


def rn_retention_chunkwise_varlen(q, k, v, gamma, theta, chunk, *, pos=None, lengths=None,
                                  gate=None, state_in=None, state_out=None, out=None,
                                  out_dtype=None, workspace=None, pos0=0, qk_scale=1.0, gn=False,
                                  gn_eps=1e-5, gn_weight=None, gn_bias=None, force_generic=False,
                                  chunk_parallel=False, segmented=False):
    """Chunkwise form over a padded batch: sequence b holds ``lengths[b]`` tokens
    (device int32 [B]) starting at position ``pos[b]`` (device int64 [B]); either may be
    None (N tokens / ``pos0``). Rows past a sequence's length are not written (a new
    ``out`` is zero-filled there). Returns (out, state_out)."""
    if out is None and lengths is not None:
        od = q.dtype if out_dtype is None else out_dtype
        out = _out(None, v.shape, od, v.device, fill=0)
    return _chunkwise(q, k, v, gamma, theta, chunk, pos, lengths, gate, state_in, state_out, out,
                      out_dtype, workspace, pos0, qk_scale, gn, gn_eps, gn_weight, gn_bias,
                      force_generic, chunk_parallel, segmented)


def _chunkwise(q, k, v, gamma, theta, chunk, pos, lengths, gate, state_in, state_out, out,
               out_dtype, workspace, pos0, qk_scale, gn, gn_eps, gn_weight, gn_bias,
               force_generic, chunk_parallel, segmented=False, test_force_timeout=False):
    flags = _flags(False, False, gn, gate, force_generic, chunk_parallel, segmented,
                   test_force_timeout)
    d, keep, od = _qkv_desc(q, k, v, gamma, theta, out_dtype, flags, pos0, qk_scale, gn_eps,
                            gn_weight, gn_bias, gate)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    out = _out(out, v.shape, od, v.device)
    if state_out is True:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    for s in (state_in, state_out):
        if s is not None and (s.dtype != torch.float32 or tuple(s.shape) != (B, H, dk, dv)):
            raise ValueError("states must be float32 [B,H,d_k,d_v]")
    need = int(lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), chunk))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(state_in), _ptr(state_out), _ptr(out),
            _ptr(workspace), workspace.numel(), _stream(q))
    if pos is None and lengths is None:
        _check(lib.rn_retention_chunkwise(ctypes.byref(d), chunk, *args))
    else:
        _check(lib.rn_retention_chunkwise_varlen(
            ctypes.byref(d), chunk, _seq_array(pos, B, torch.int64, "pos"),
            _seq_array(lengths, B, torch.int32, "lengths"), *args))
    return out, state_out


def rn_retention_chunkwise_noalloc(q, k, v, gamma, theta, chunk, *, gate=None, state_in=None,
                                   state_out=None, out=None, out_dtype=None, pos0=0,
                                   qk_scale=1.0, gn=False, gn_eps=1e-5, gn_weight=None,
                                   gn_bias=None, force_generic=False, chunk_parallel=False,
                                   segmented=False):
    """rn_retention_chunkwise with the library's own device workspace (the C call allocates
    nothing; pass ``out`` and a ``state_out`` tensor to keep this wrapper from allocating
    them). Returns (out, state_out)."""
    flags = _flags(False, False, gn, gate, force_generic, chunk_parallel, segmented)
    d, keep, od = _qkv_desc(q, k, v, gamma, theta, out_dtype, flags, pos0, qk_scale, gn_eps,
                            gn_weight, gn_bias, gate)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    out = _out(out, v.shape, od, v.device)
    if state_out is True:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    for s in (state_in, state_out):
        if s is not None and (s.dtype != torch.float32 or tuple(s.shape) != (B, H, dk, dv)):
            raise ValueError("states must be float32 [B,H,d_k,d_v]")
    _check(lib.rn_retention_chunkwise_noalloc(ctypes.byref(d), chunk, _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(gate), _ptr(state_in), _ptr(state_out),
                                              _ptr(out), _stream(q)))
    return out, state_out


def rn_retention_recurrent_step(q, k, v, gamma, theta, state, pos, *, gate=None, out=None,
                                out_dtype=None, qk_scale=1.0, gn=False, gn_eps=1e-5,
                                gn_weight=None, gn_bias=None):
    """One decode step at position ``pos``; ``state`` [B,H,d_k,d_v] float32 is updated in
    place. q, k: [B,H,1,d_k]; v: [B,H,1,d_v]. Returns out [B,H,1,d_v]."""
    flags = _flags(False, False, gn, gate, False)
    d, keep, od = _qkv_desc(q, k, v, gamma, theta, out_dtype, flags, pos, qk_scale, gn_eps,
                            gn_weight, gn_bias, gate)
    if state.dtype != torch.float32 or tuple(state.shape) != (q.shape[0], q.shape[1], q.shape[3], v.shape[3]):
        raise ValueError("state must be float32 [B,H,d_k,d_v]")
    out = _out(out, v.shape, od, v.device)
    _check(lib.rn_retention_recurrent_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                           _ptr(state), _ptr(out), _stream(q)))
    return out


def rn_retention_recurrent_step_at(q, k, v, gamma, theta, state, pos, *, gate=None, out=None,
                                   out_dtype=None, qk_scale=1.0, gn=False, gn_eps=1e-5,
                                   gn_weight=None, gn_bias=None):
    """One decode step with the token of sequence b at position ``pos[b]`` (device int64
    [B]); otherwise as rn_retention_recurrent_step. Returns out [B,H,1,d_v]."""
    flags = _flags(False, False, gn, gate, False)
    d, keep, od = _qkv_desc(q, k, v, gamma, theta, out_dtype, flags, 0, qk_scale, gn_eps,
                            gn_weight, gn_bias, gate)
    if state.dtype != torch.float32 or tuple(state.shape) != (q.shape[0], q.shape[1], q.shape[3], v.shape[3]):
        raise ValueError("state must be float32 [B,H,d_k,d_v]")
    pp = _seq_array(pos, q.shape[0], torch.int64, "pos")
    if pp is None:
        raise ValueError("pos is required")
    out = _out(out, v.shape, od, v.device)
    _check(lib.rn_retention_recurrent_step_at(ctypes.byref(d), pp, _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(gate), _ptr(state), _ptr(out), _stream(q)))
    return out


def rn_chunkwise_backward_workspace_bytes(q, v, gamma, theta, chunk, *, gn=False, gate=None,
                                          out_dtype=None, force_generic=False) -> int:
    B, H, N, dk = q.shape
    flags = _flags(False, False, gn, gate, force_generic)
    od = q.dtype if out_dtype is None else out_dtype
    d, keep = make_desc(B, H, N, dk, v.shape[-1], _dtype_code(q.dtype), _dtype_code(od), gamma,
                        theta, flags=flags, device=q.device)
    return int(lib.rn_chunkwise_backward_workspace_bytes(ctypes.byref(d), chunk))


def rn_retention_chunkwise_backward(q, k, v, gamma, theta, chunk, dout, *, gate=None,
                                    state_in=None, dstate_out=None, want_dstate_in=False,
                                    pos0=0, qk_scale=1.0, gn=False, gn_eps=1e-5, gn_weight=None,
                                    gn_bias=None, workspace=None, force_generic=False):
    """Gradients of the chunkwise call with respect to q, k, v (and the gate, the initial
    state, the GroupNorm weight and bias). ``dout`` has the forward output's dtype.
    Returns a dict with dq, dk, dv and, when they apply, dgate, dstate_in, dgn_weight,
    dgn_bias. ``force_generic`` takes the kernels that stage operands through registers
    (64-bit addressing) also where the copy-fed matrix-core kernels apply."""
    flags = _flags(False, False, gn, gate, force_generic)
    d, keep, od = _qkv_desc(q, k, v, gamma, theta, dout.dtype, flags, pos0, qk_scale, gn_eps,
                            gn_weight, gn_bias, gate)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if tuple(dout.shape) != tuple(v.shape):
        raise ValueError("dout must have v's shape")
    for s_ in (state_in, dstate_out):
        if s_ is not None and (s_.dtype != torch.float32 or tuple(s_.shape) != (B, H, dk, dv)):
            raise ValueError("states must be float32 [B,H,d_k,d_v]")
    res = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
    if gate is not None:
        res["dgate"] = torch.empty_like(gate)
    if want_dstate_in:
        res["dstate_in"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if gn:
        res["dgn_weight"] = torch.empty(H * dv, dtype=torch.float32, device=q.device)
        res["dgn_bias"] = torch.empty(H * dv, dtype=torch.float32, device=q.device)
    need = int(lib.rn_chunkwise_backward_workspace_bytes(ctypes.byref(d), chunk))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib.rn_retention_chunkwise_backward(
        ctypes.byref(d), chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(state_in),
        _ptr(dout), _ptr(dstate_out), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]),
        _ptr(res.get("dgate")), _ptr(res.get("dstate_in")), _ptr(res.get("dgn_weight")),
        _ptr(res.get("dgn_bias")), _ptr(workspace), workspace.numel(), _stream(q)))
    return res


def _layer_desc(x, H, d_k, d_v, gamma, theta, flags, pos0, qk_scale, gn_eps, gn_weight, gn_bias,
                out_dtype):
    if x.dim() != 3 or x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16 [B, N, d_model]")
    B, N, _ = x.shape
    if len(gamma) != H or len(theta) != d_k // 2:
        raise ValueError(f"need gamma[{H}] (or [{H}, {d_k // 2}]) and theta[{d_k // 2}]")
    od = torch.bfloat16 if out_dtype is None else out_dtype
    for t in (gn_weight, gn_bias):
        if t is not None:
            _ptr(t)
            if t.dtype != torch.float32 or t.numel() != H * d_v:
                raise ValueError("gn_weight/gn_bias must be float32 with H*d_v elements")
    d, keep = make_desc(B, H, N, d_k, d_v, RN_BF16, _dtype_code(od), gamma, theta, flags=flags,
                        pos0=pos0, qk_scale=qk_scale, gn_eps=gn_eps, gn_weight=gn_weight,
                        gn_bias=gn_bias, device=x.device)
    return d, keep, od


def rn_msr_layer_workspace_bytes(x, H, d_k, d_v, gamma, theta, chunk, *, gn=True, gate=True,
                                 out_dtype=None) -> int:
    d, keep, _ = _layer_desc(x, H, d_k, d_v, gamma, theta, _flags(False, False, gn, gate or None, False),
                             0, 1.0, 1e-5, None, None, out_dtype)
    return int(lib.rn_msr_layer_workspace_bytes(ctypes.byref(d), x.shape[-1], chunk))


def rn_msr_layer_forward(x, w_q, w_k, w_v, w_g, w_o, gamma, theta, H, d_k, d_v, chunk, *,
                         state_in=None, state_out=None, out=None, out_dtype=None, workspace=None,
                         pos0=0, qk_scale=1.0, gn=True, gn_eps=1e-5, gn_weight=None,
                         gn_bias=None):
    """Gated multi-scale retention layer: (swish(X W_G) ⊙ GN_h(Retention_h)) W_O with the
    heads' Q, K, V projected from x [B, N, d_model] (bf16). Weights: w_q, w_k
    [d_model, H*d_k], w_v, w_g [d_model, H*d_v], w_o [H*d_v, d_model] (bf16); w_g=None
    leaves the gate out. Returns (out [B, N, d_model], state_out)."""
    B, N, D = x.shape
    gate = w_g is not None
    for name, w, shape in (("w_q", w_q, (D, H * d_k)), ("w_k", w_k, (D, H * d_k)),
                           ("w_v", w_v, (D, H * d_v)), ("w_g", w_g, (D, H * d_v)),
                           ("w_o", w_o, (H * d_v, D))):
        if w is not None and (tuple(w.shape) != shape or w.dtype != torch.bfloat16):
            raise ValueError(f"{name} must be bfloat16 {shape}")
    flags = _flags(False, False, gn, True if gate else None, False)
    d, keep, od = _layer_desc(x, H, d_k, d_v, gamma, theta, flags, pos0, qk_scale, gn_eps,
                              gn_weight, gn_bias, out_dtype)
    out = _out(out, (B, N, D), od, x.device)
    if state_out is True:
        state_out = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=x.device)
    elif state_out is False:
        state_out = None
    for s_ in (state_in, state_out):
        if s_ is not None and (s_.dtype != torch.float32 or tuple(s_.shape) != (B, H, d_k, d_v)):
            raise ValueError("states must be float32 [B,H,d_k,d_v]")
    need = int(lib.rn_msr_layer_workspace_bytes(ctypes.byref(d), D, chunk))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib.rn_msr_layer_forward(ctypes.byref(d), D, chunk, _ptr(x), _ptr(w_q), _ptr(w_k),
                                    _ptr(w_v), _ptr(w_g), _ptr(w_o), _ptr(state_in),
                                    _ptr(state_out), _ptr(out), _ptr(workspace),
                                    workspace.numel(), _stream(x)))
    return out, state_out


def rn_groupnorm_gate(x, gate=None, weight=None, bias=None, eps=1e-5, *, out=None, out_dtype=None):
    """Per-head GroupNorm over the last axis of x [B,H,N,d_v] (+ swish gate)."""
    B, H, N, dv = x.shape
    od = x.dtype if out_dtype is None else out_dtype
    out = _out(out, x.shape, od, x.device)
    if gate is not None and (gate.shape != x.shape or gate.dtype != x.dtype or gate.device != x.device):
        raise ValueError("gate must match x in shape, dtype and device")
    _check_affine(weight, bias, H * dv, x.device)
    _check(lib.rn_groupnorm_gate(B, H, N, dv, _dtype_code(x.dtype), _dtype_code(od), _ptr(x),
                                 _ptr(gate), _ptr(weight), _ptr(bias), eps, _ptr(out), _stream(x)))
    return out


def rn_chunkwise_check(q, v, gamma, theta, chunk, workspace, *, gn=False, gate=None,
                       out_dtype=None, force_generic=False, chunk_parallel=False,
                       segmented=False) -> int:
    """Status of a completed chunkwise call (same arguments as the call) read from its
    ``workspace``: a GPU tensor (the call's stream is synchronised first) or a CPU copy of
    its first bytes. Returns the status code (RN_OK, RN_ERR_EXCHANGE, RN_ERR_NONFINITE);
    argument errors raise."""
    B, H, N, dk = q.shape
    flags = _flags(False, False, gn, gate, force_generic, chunk_parallel, segmented)
    od = q.dtype if out_dtype is None else out_dtype
    d, keep = make_desc(B, H, N, dk, v.shape[-1], _dtype_code(q.dtype), _dtype_code(od), gamma,
                        theta, flags=flags, device=q.device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    stream = _stream(workspace) if workspace.is_cuda else None
    st = int(lib.rn_chunkwise_check(ctypes.byref(d), chunk, ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(), stream))
    if st not in (RN_OK, RN_ERR_EXCHANGE, RN_ERR_NONFINITE):
        _check(st)
    return st
