"""MI355X (gfx950) KDA: chunkwise gated delta rule with a per-channel forget
gate, and its one-token decode step.

Thin ctypes binding over the C ABI of ``libkda.so`` (declared in
``include/kda.h``): tensors in, device pointers and the current HIP stream
out.  PyTorch only allocates device memory and provides the stream; every
step of the computation runs in the library's HIP kernels.  There is no
fallback: without the built library (``python -m gated_delta_rule_61_amd._build``
or ``__graft_entry__.build()``) every call raises.

Layouts (row-major, contiguous):
  q, k, g [B, T, H, d_k]; v, o [B, T, H, d_v]; beta [B, T, H];
  S0, S_T [B, H, d_k, d_v] float32.  q, k, v, g, beta share one dtype
  (torch.bfloat16 or torch.float32); o has that dtype.

Variants (keyword arguments of chunk_fwd and recurrent_step): scalar_gate=True
takes one log-gate per token and head (g [B, T, H]; Gated DeltaNet), and
delta=False drops the delta rule (S_t = Diag(exp g_t) S_{t-1} + k_t v_t^T;
beta unused, may be None).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
ROOT = os.path.dirname(_PKG)
HEADER = os.path.join(ROOT, "include", "kda.h")

KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_SCALAR, KDA_NO_DELTA = 1, 2
KDA_STATES_SAVED = 4
_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}

_lock = threading.Lock()
_lib = None

_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "kda_chunk_fwd": ([_vp] * 8 + [_i] * 6 + [_vp, _sz, _vp], _i),
    "kda_chunk_fwd_staged": ([_vp] * 8 + [_i] * 6 + [_vp, _sz, _vp], _i),
    "kda_chunk_fwd_workspace_size": ([_i] * 6, _sz),
    "kda_chunk_fwd_ex": ([_vp] * 8 + [_i] * 7 + [_vp, _sz, _vp], _i),
    "kda_chunk_fwd_noalloc": ([_vp] * 8 + [_i] * 6 + [_vp], _i),
    "kda_chunk_fwd_ex_workspace_size": ([_i] * 7, _sz),
    "kda_chunk_fwd_save": ([_vp] * 8 + [_i] * 7 + [_vp, _sz, _vp], _i),
    "kda_chunk_fwd_varlen_save": ([_vp] * 10 + [_i] * 7 + [_vp, _sz, _vp], _i),
    "kda_recurrent_step_ex": ([_vp] * 7 + [_i] * 6 + [_vp], _i),
    "kda_chunk_fwd_varlen": ([_vp] * 10 + [_i] * 7 + [_vp], _i),
    "kda_chunk_fwd_varlen_ws": ([_vp] * 10 + [_i] * 7 + [_vp, _sz, _vp], _i),
    "kda_chunk_fwd_varlen_workspace_size": ([_i] * 7, _sz),
    "kda_varlen_schedule": ([_vp, _i, _i, _vp, _vp], _i),
    "kda_chunk_bwd": ([_vp] * 14 + [_i] * 6 + [_vp, _sz, _vp], _i),
    "kda_chunk_bwd_workspace_size": ([_i] * 6, _sz),
    "kda_chunk_bwd_ex": ([_vp] * 14 + [_i] * 7 + [_vp, _sz, _vp], _i),
    "kda_chunk_bwd_ex_workspace_size": ([_i] * 7, _sz),
    "kda_chunk_bwd_varlen": ([_vp] * 15 + [_i] * 7 + [_vp, _sz, _vp], _i),
    "kda_chunk_bwd_varlen_workspace_size": ([_i] * 7, _sz),
    "kda_chunk_fwd_staged_workspace_size": ([_i] * 6, _sz),
    "kda_recurrent_step": ([_vp] * 7 + [_i] * 5 + [_vp], _i),
    "kda_stage_cumsum": ([_vp, _vp] + [_i] * 5 + [_vp], _i),
    "kda_stage_ut": ([_vp] * 6 + [_i] * 6 + [_vp], _i),
    "kda_stage_state": ([_vp] * 8 + [_i] * 6 + [_vp], _i),
    "kda_stage_output": ([_vp] * 6 + [_i] * 6 + [_vp], _i),
    "kda_status_string": ([_i], ctypes.c_char_p),
    "kda_last_hip_error": ([], _i),
    "kda_version": ([], _i),
}


class KDAError(RuntimeError):
    pass


def lib():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise KDAError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gated_delta_rule_61_amd._build` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIGS.items():
                fn = getattr(L, name)
                fn.argtypes = args
                fn.restype = res
            _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().kda_status_string(status).decode()
        raise KDAError(f"KDA call failed with status {status}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise KDAError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")
    return _DT[t.dtype]


def _need(t, shape, dtype, name):
    if t is None:
        raise KDAError(f"{name} is required")
    if not t.is_cuda:
        raise KDAError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise KDAError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise KDAError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise KDAError(f"{name} must be contiguous")


def _flags(scalar_gate: bool, delta: bool) -> int:
    return (KDA_GATE_SCALAR if scalar_gate else 0) | (0 if delta else KDA_NO_DELTA)


def _prefill_shapes(q, k, v, g, beta, scalar_gate=False, delta=True):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, (B, T, H, dk), dt, "q")
    _need(k, (B, T, H, dk), dt, "k")
    _need(g, (B, T, H) if scalar_gate else (B, T, H, dk), dt, "g")
    _need(v, (B, T, H, dv), dt, "v")
    if delta or beta is not None:
        _need(beta, (B, T, H), dt, "beta")
    return B, T, H, dk, dv, dt


def chunk_fwd(q, k, v, g, beta, S0=None, *, o=None, S_T=None, staged=False,
              workspace=None, stream=None, want_state=True, scalar_gate=False, delta=True):
    """Prefill: returns (o, S_T).  With staged=True the four-kernel schedule
    runs instead of the fused kernel (same result up to rounding).  The
    variants (scalar_gate, delta=False) run on the fused kernel only."""
    flags = _flags(scalar_gate, delta)
    if flags and staged:
        raise KDAError("the staged schedule computes the KDA rule only (no variants)")
    B, T, H, dk, dv, dt = _prefill_shapes(q, k, v, g, beta, scalar_gate, delta)
    dev = q.device
    if S0 is not None:
        _need(S0, (B, H, dk, dv), torch.float32, "S0")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    L = lib()
    code = _dtype(q)
    if flags:
        wsz = L.kda_chunk_fwd_ex_workspace_size(B, T, H, dk, dv, code, flags)
    else:
        wsz = (L.kda_chunk_fwd_staged_workspace_size if staged else L.kda_chunk_fwd_workspace_size)(
            B, T, H, dk, dv, code)
    if wsz and (workspace is None or workspace.numel() * workspace.element_size() < wsz):
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
            B, T, H, dk, dv, code)
    tail = (_ptr(workspace) if wsz else None, wsz, _stream(stream))
    if flags:
        _check(L.kda_chunk_fwd_ex(*args, flags, *tail))
    else:
        _check((L.kda_chunk_fwd_staged if staged else L.kda_chunk_fwd)(*args, *tail))
    return o, S_T


def chunk_fwd_save(q, k, v, g, beta, S0=None, *, o=None, S_T=None, workspace=None, stream=None, scalar_gate=False,
                   delta=True):
    """Prefill that also keeps every chunk's entry state for the backward
    (kda_chunk_fwd_save; bf16, d = 128, any variant): returns
    (o, S_T, workspace).  Pass the same workspace to chunk_bwd(...,
    workspace=workspace, states_saved=True) on the same inputs, and the
    backward skips its own pass over the states."""
    flags = _flags(scalar_gate, delta)
    B, T, H, dk, dv, dt = _prefill_shapes(q, k, v, g, beta, scalar_gate, delta)
    dev = q.device
    if S0 is not None:
        _need(S0, (B, H, dk, dv), torch.float32, "S0")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    L = lib()
    code = _dtype(q)
    wsz = L.kda_chunk_bwd_ex_workspace_size(B, T, H, dk, dv, code, flags)
    if wsz and (workspace is None or workspace.numel() * workspace.element_size() < wsz):
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
                                B, T, H, dk, dv, code, flags, _ptr(workspace) if wsz else None, wsz, _stream(stream)))
    return o, S_T, workspace


def chunk_fwd_noalloc(q, k, v, g, beta, S0=None, *, o, S_T=None, stream=None):
    """Prefill through kda_chunk_fwd_noalloc: the library's own device scratch
    holds the workspace, so nothing is allocated (o, and S_T if wanted, must
    be passed in).  Returns (o, S_T)."""
    B, T, H, dk, dv, dt = _prefill_shapes(q, k, v, g, beta)
    _need(o, (B, T, H, dv), dt, "o")
    if S0 is not None:
        _need(S0, (B, H, dk, dv), torch.float32, "S0")
    if S_T is not None:
        _need(S_T, (B, H, dk, dv), torch.float32, "S_T")
    _check(lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                       _ptr(S_T), B, T, H, dk, dv, _dtype(q), _stream(stream)))
    return o, S_T


def varlen_schedule(cu_seqlens, T_total, *, out=None, stream=None):
    """Longest-first processing order of the packed sequences (int32 [N] on
    the device), for chunk_fwd_varlen(seq_order=...)."""
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    if out is None:
        out = torch.empty(max(N, 0), dtype=torch.int32, device=cu_seqlens.device)
    _check(lib().kda_varlen_schedule(_ptr(cu_seqlens), N, int(T_total), _ptr(out), _stream(stream)))
    return out


def chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, S0=None, *, seq_order=None, o=None, S_T=None, stream=None,
                     want_state=True, scalar_gate=False, delta=True, workspace=None, segmented=True):
    """Prefill of N packed sequences: q, k, g [T_total, H, d_k] (g [T_total, H]
    with scalar_gate), v [T_total, H, d_v], beta [T_total, H], cu_seqlens
    int32 [N + 1] on the device (sequence i = tokens cu[i] .. cu[i+1] - 1),
    S0 [N, H, d_k, d_v] fp32 or None; seq_order: int32 [N] start order (see
    varlen_schedule) or None.  segmented: pass (or allocate) the workspace of
    kda_chunk_fwd_varlen_ws, whose segmented schedule splits long sequences.
    Returns (o [T_total, H, d_v], S_T)."""
    flags = _flags(scalar_gate, delta)
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise KDAError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _need(q, (Tt, H, dk), dt, "q")
    _need(k, (Tt, H, dk), dt, "k")
    _need(g, (Tt, H) if scalar_gate else (Tt, H, dk), dt, "g")
    _need(v, (Tt, H, dv), dt, "v")
    if delta or beta is not None:
        _need(beta, (Tt, H), dt, "beta")
    if S0 is not None:
        _need(S0, (N, H, dk, dv), torch.float32, "S0")
    if seq_order is not None:
        _need(seq_order, (N,), torch.int32, "seq_order")
    dev = q.device
    if o is None:
        o = torch.zeros((Tt, H, dv), dtype=dt, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    L = lib()
    wsz = L.kda_chunk_fwd_varlen_workspace_size(N, Tt, H, dk, dv, _dtype(q), flags) if segmented else 0
    if wsz and (workspace is None or workspace.numel() * workspace.element_size() < wsz):
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_fwd_varlen_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                     _ptr(S_T), _ptr(cu_seqlens), _ptr(seq_order), N, Tt, H, dk, dv,
                                     _dtype(q), flags, _ptr(workspace) if wsz else None, wsz, _stream(stream)))
    return o, S_T


def chunk_fwd_varlen_save(q, k, v, g, beta, cu_seqlens, S0=None, *, seq_order=None, o=None, S_T=None,
                          workspace=None, stream=None, scalar_gate=False, delta=True):
    """chunk_fwd_varlen (one pass, any variant) that also keeps every
    chunk's entry state for chunk_bwd_varlen(..., workspace=workspace,
    states_saved=True): returns (o, S_T, workspace)."""
    flags = _flags(scalar_gate, delta)
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise KDAError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _need(q, (Tt, H, dk), dt, "q")
    _need(k, (Tt, H, dk), dt, "k")
    _need(g, (Tt, H) if scalar_gate else (Tt, H, dk), dt, "g")
    _need(v, (Tt, H, dv), dt, "v")
    if delta or beta is not None:
        _need(beta, (Tt, H), dt, "beta")
    if S0 is not None:
        _need(S0, (N, H, dk, dv), torch.float32, "S0")
    if seq_order is not None:
        _need(seq_order, (N,), torch.int32, "seq_order")
    dev = q.device
    if o is None:
        o = torch.zeros((Tt, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    L = lib()
    wsz = L.kda_chunk_bwd_varlen_workspace_size(N, Tt, H, dk, dv, _dtype(q), flags)
    if wsz and (workspace is None or workspace.numel() * workspace.element_size() < wsz):
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_fwd_varlen_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
                                       _ptr(cu_seqlens), _ptr(seq_order), N, Tt, H, dk, dv, _dtype(q), flags,
                                       _ptr(workspace) if wsz else None, wsz, _stream(stream)))
    return o, S_T, workspace


def chunk_bwd(q, k, v, g, beta, S0, dO, dS_T=None, *, want_dS0=True, workspace=None, stream=None,
              scalar_gate=False, delta=True, states_saved=False):
    """Gradient of chunk_fwd: returns dict(dq, dk, dv, dg, dbeta, dS0) for the
    adjoints dO [B,T,H,d_v] (and dS_T [B,H,d_k,d_v] fp32 or None).  bf16 at
    d = 128 (chunked), fp32 at d = 64 / 128 and bf16 at d = 64 (token
    recurrence).  scalar_gate: g and dg are [B,T,H] (Gated DeltaNet);
    delta=False: no delta rule (beta may be None, dbeta is None).
    states_saved: workspace comes from chunk_fwd_save on the same inputs and
    already holds the chunk states (KDA_STATES_SAVED)."""
    flags = _flags(scalar_gate, delta) | (KDA_STATES_SAVED if states_saved else 0)
    if states_saved and workspace is None:
        raise KDAError("states_saved needs the workspace that chunk_fwd_save filled")
    B, T, H, dk, dv, dt = _prefill_shapes(q, k, v, g, beta, scalar_gate=scalar_gate, delta=delta)
    _need(dO, (B, T, H, dv), dt, "dO")
    if S0 is not None:
        _need(S0, (B, H, dk, dv), torch.float32, "S0")
    if dS_T is not None:
        _need(dS_T, (B, H, dk, dv), torch.float32, "dS_T")
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
               dbeta=torch.empty((B, T, H), dtype=dt, device=dev) if delta else None,
               dS0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None)
    L = lib()
    code = _dtype(q)
    wsz = L.kda_chunk_bwd_ex_workspace_size(B, T, H, dk, dv, code, flags)
    if wsz and (workspace is None or workspace.numel() * workspace.element_size() < wsz):
        if states_saved:
            raise KDAError("the saved-state workspace is smaller than the backward needs")
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                              _ptr(out["dbeta"]), _ptr(out["dS0"]), B, T, H, dk, dv, code, flags,
                              _ptr(workspace) if wsz else None, wsz, _stream(stream)))
    return out


def chunk_bwd_varlen(q, k, v, g, beta, cu_seqlens, S0, dO, dS_T=None, *, want_dS0=True, workspace=None,
                     stream=None, scalar_gate=False, delta=True, states_saved=False):
    """Gradient of chunk_fwd_varlen for N packed sequences: q, k, g, v, beta,
    dO packed as there ([T_total, H, ...]), S0 and dS_T [N, H, d_k, d_v] fp32
    or None.  Returns dict(dq, dk, dv, dg, dbeta, dS0) (dbeta None without the
    delta rule, dS0 [N, H, d_k, d_v]).  states_saved: workspace comes from
    chunk_fwd_varlen_save on the same inputs."""
    flags = _flags(scalar_gate, delta) | (KDA_STATES_SAVED if states_saved else 0)
    if states_saved and workspace is None:
        raise KDAError("states_saved needs the workspace that chunk_fwd_varlen_save filled")
    Tt, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise KDAError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, (N + 1,), torch.int32, "cu_seqlens")
    _need(q, (Tt, H, dk), dt, "q")
    _need(k, (Tt, H, dk), dt, "k")
    _need(g, (Tt, H) if scalar_gate else (Tt, H, dk), dt, "g")
    _need(v, (Tt, H, dv), dt, "v")
    _need(dO, (Tt, H, dv), dt, "dO")
    if delta or beta is not None:
        _need(beta, (Tt, H), dt, "beta")
    for name, x in (("S0", S0), ("dS_T", dS_T)):
        if x is not None:
            _need(x, (N, H, dk, dv), torch.float32, name)
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
               dbeta=torch.empty((Tt, H), dtype=dt, device=dev) if delta else None,
               dS0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None)
    L = lib()
    code = _dtype(q)
    wsz = L.kda_chunk_bwd_varlen_workspace_size(N, Tt, H, dk, dv, code, flags)
    if wsz and (workspace is None or workspace.numel() * workspace.element_size() < wsz):
        if states_saved:
            raise KDAError("the saved-state workspace is smaller than the backward needs")
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    _check(L.kda_chunk_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
                                  _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                  _ptr(out["dbeta"]), _ptr(out["dS0"]), _ptr(cu_seqlens), N, Tt, H, dk, dv, code,
                                  flags, _ptr(workspace) if wsz else None, wsz, _stream(stream)))
    return out


def recurrent_step(q, k, v, g, beta, S, *, o=None, stream=None, scalar_gate=False, delta=True):
    """One decode token for N sequences; S [N,H,d_k,d_v] fp32 is updated in
    place.  Returns o [N,H,d_v].  Variants as for chunk_fwd (g [N,H] with
    scalar_gate)."""
    flags = _flags(scalar_gate, delta)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, (N, H, dk), dt, "q")
    _need(k, (N, H, dk), dt, "k")
    _need(g, (N, H) if scalar_gate else (N, H, dk), dt, "g")
    _need(v, (N, H, dv), dt, "v")
    if delta or beta is not None:
        _need(beta, (N, H), dt, "beta")
    _need(S, (N, H, dk, dv), torch.float32, "S")
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o), N, H, dk, dv, _dtype(q))
    if flags:
        _check(lib().kda_recurrent_step_ex(*args, flags, _stream(stream)))
    else:
        _check(lib().kda_recurrent_step(*args, _stream(stream)))
    return o


# ---- the staged schedule's steps, one call each ---------------------------

def stage_cumsum(g, *, stream=None):
    B, T, H, dk = g.shape
    b = torch.empty((B, T, H, dk), dtype=torch.float32, device=g.device)
    _check(lib().kda_stage_cumsum(_ptr(g), _ptr(b), B, T, H, dk, _dtype(g), _stream(stream)))
    return b


def stage_ut(k, v, beta, b, *, stream=None):
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    W = torch.empty((B, T, H, dk), dtype=torch.float32, device=k.device)
    U = torch.empty((B, T, H, dv), dtype=torch.float32, device=k.device)
    _check(lib().kda_stage_ut(_ptr(k), _ptr(v), _ptr(beta), _ptr(b), _ptr(W), _ptr(U),
                              B, T, H, dk, dv, _dtype(k), _stream(stream)))
    return W, U


def stage_state(k, b, W, U, S0=None, *, stream=None):
    B, T, H, dk = k.shape
    dv = U.shape[-1]
    N = (T + 63) // 64
    dev = k.device
    Delta = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    S_chunks = torch.empty((B, H, N, dk, dv), dtype=torch.float32, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check(lib().kda_stage_state(_ptr(k), _ptr(b), _ptr(W), _ptr(U), _ptr(S0), _ptr(Delta),
                                 _ptr(S_chunks), _ptr(S_T), B, T, H, dk, dv, _dtype(k), _stream(stream)))
    return Delta, S_chunks, S_T


def stage_output(q, k, b, Delta, S_chunks, *, stream=None):
    B, T, H, dk = q.shape
    dv = Delta.shape[-1]
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _check(lib().kda_stage_output(_ptr(q), _ptr(k), _ptr(b), _ptr(Delta), _ptr(S_chunks), _ptr(o),
                                  B, T, H, dk, dv, _dtype(q), _stream(stream)))
    return o


__all__ = ["chunk_fwd", "chunk_fwd_varlen", "chunk_bwd", "chunk_bwd_varlen", "recurrent_step", "stage_cumsum", "stage_ut", "stage_state",
           "stage_output", "lib", "KDAError", "LIB_PATH", "HEADER"]
