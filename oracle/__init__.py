"""CPU oracle for the KDA gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product path: the two share no code.

Two independent fp64 implementations live here:

* ``recurrent_fwd`` / ``recurrent_step`` -- the definition, token by token, in
  plain C (``kda_oracle.c``) with OpenMP over independent sequences.  It is the
  update rule of "Hybrid Linear Attention Architecture: Making LLM Training and
  Inference More Efficient" §3.3 (KDA equation) with the read-after-write
  output of "Demystifying Hybrid LLM Architectures: Linear Attention,
  Residuals, and Latent MoE" §2.3.
* ``recurrent_bwd`` -- the derivative of that definition by reverse-mode
  differentiation of its token loop (C, fp64), with the per-chunk state
  adjoints on request.  The pages give no backward formulas: the gradient is
  fixed by the forward definition alone.
* ``oracle.chunked`` -- the chunkwise-parallel form of the same pages' §IV /
  §2.4, in NumPy fp64, which exposes the per-chunk intermediates (cumulative
  log-gates, W, U, the residual U - W S, the chunk-entry states).

Pins (tests that tie them to something other than themselves) are in
``tests/test_oracle_pins.py``, ``tests/test_chunked_model.py`` and
``tests/test_oracle_bwd_pins.py`` (finite differences, torch.autograd of an
independent recurrence, adjoint composition).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the .so path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.kda_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                           i64, i64, i64, i64, i64, ctypes.c_int]
            lib.kda_oracle_fwd.restype = ctypes.c_int
            lib.kda_oracle_step.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                            i64, i64, i64, i64, ctypes.c_int]
            lib.kda_oracle_step.restype = ctypes.c_int
            lib.kda_oracle_fwd_ex.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                              i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
            lib.kda_oracle_fwd_ex.restype = ctypes.c_int
            lib.kda_oracle_step_ex.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                               i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
            lib.kda_oracle_step_ex.restype = ctypes.c_int
            lib.kda_oracle_bwd_ex.argtypes = [dp] * 15 + [i64] * 6 + [ctypes.c_int, ctypes.c_int]
            lib.kda_oracle_bwd_ex.restype = ctypes.c_int
            lib.kda_oracle_max_threads.argtypes = []
            lib.kda_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Upcast to a C-contiguous float64 array (exact for bf16/fp32 values)."""
    if hasattr(x, "detach"):            # a torch tensor: copy to host, upcast
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


SCALAR_GATE = 1   # g holds one log-gate per token and head (Gated DeltaNet)
NO_DELTA = 2      # S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T (no erase; beta unused)


def _flags(scalar_gate: bool, delta: bool) -> int:
    return (SCALAR_GATE if scalar_gate else 0) | (0 if delta else NO_DELTA)


def recurrent_fwd(q, k, v, g, beta, S0=None, nthreads: int = 0, scalar_gate: bool = False,
                  delta: bool = True):
    """Token-by-token fp64 forward.

    q, k: [B, T, H, dk]; g: [B, T, H, dk] ([B, T, H] with scalar_gate);
    v: [B, T, H, dv]; beta: [B, T, H] (may be None without the delta rule);
    S0: [B, H, dk, dv] or None (zeros).  Returns (o [B,T,H,dv], S_T [B,H,dk,dv]).
    """
    q, k, v, g = (_f64(a) for a in (q, k, v, g))
    beta = None if beta is None else _f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and g.shape == ((B, T, H) if scalar_gate else (B, T, H, dk))
    assert v.shape == (B, T, H, dv)
    assert (beta is None and not delta) or beta.shape == (B, T, H)
    S0a = None if S0 is None else _f64(S0)
    if S0a is not None:
        assert S0a.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    ST = np.zeros((B, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(S0a), _ptr(o), _ptr(ST), B, T, H, dk, dv,
                                   _flags(scalar_gate, delta), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed ({rc})")
    return o, ST


def recurrent_step(q, k, v, g, beta, S, nthreads: int = 0, scalar_gate: bool = False, delta: bool = True,
                   inplace: bool = False):
    """One decode token for N sequences (g [N,H,dk], or [N,H] with
    scalar_gate).  S [N,H,dk,dv] fp64 is returned updated (a new array and the
    input untouched; with inplace=True a C-contiguous fp64 S is updated in
    place and returned).  Returns (o, S_new)."""
    q, k, v, g = (_f64(a) for a in (q, k, v, g))
    beta = None if beta is None else _f64(beta)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if inplace:
        assert isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous
        Sn = S
    else:
        Sn = _f64(S).copy()
    assert Sn.shape == (N, H, dk, dv)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().kda_oracle_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(Sn), _ptr(o), N, H, dk, dv, _flags(scalar_gate, delta),
                                    int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_step failed ({rc})")
    return o, Sn


def recurrent_bwd(q, k, v, g, beta, S0, dO, dST=None, nthreads: int = 0, scalar_gate: bool = False,
                  delta: bool = True, chunk: int = 64, chunk_adjoints: bool = False):
    """Reverse-mode derivative of ``recurrent_fwd`` (fp64, token by token).

    dO [B,T,H,dv] is the adjoint of o, dST [B,H,dk,dv] that of S_T (None:
    zero).  Returns a dict with dq, dk, dv [B,T,H,*], dg (same shape as g),
    dbeta [B,T,H] (zeros without the delta rule), dS0 [B,H,dk,dv] and, with
    chunk_adjoints, dS_chunks [B,H,ceil(T/chunk),dk,dv] (adjoint of the state
    at the start of each chunk of ``chunk`` tokens)."""
    q, k, v, g, dO = (_f64(a) for a in (q, k, v, g, dO))
    beta = None if beta is None else _f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and g.shape == ((B, T, H) if scalar_gate else (B, T, H, dk))
    assert v.shape == (B, T, H, dv) and dO.shape == (B, T, H, dv)
    assert (beta is None and not delta) or beta.shape == (B, T, H)
    S0a = None if S0 is None else _f64(S0)
    dSTa = None if dST is None else _f64(dST)
    out = dict(dq=np.zeros((B, T, H, dk)), dk=np.zeros((B, T, H, dk)), dv=np.zeros((B, T, H, dv)),
               dg=np.zeros(g.shape), dbeta=np.zeros((B, T, H)), dS0=np.zeros((B, H, dk, dv)))
    nblk = (T + chunk - 1) // chunk
    dSc = np.zeros((B, H, nblk, dk, dv)) if chunk_adjoints else None
    rc = _load().kda_oracle_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0a), _ptr(dO),
                                   _ptr(dSTa), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                   _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dS0"]), _ptr(dSc),
                                   B, T, H, dk, dv, chunk, _flags(scalar_gate, delta), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed ({rc})")
    if chunk_adjoints:
        out["dS_chunks"] = dSc
    return out
