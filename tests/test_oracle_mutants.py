"""The pins must catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a private copy of the C oracle's source
(dropped term, wrong order, wrong sign, read before write, ...), builds it
into a temporary library, and checks that the pin suite rejects it while the
unmodified source passes.  Nothing here touches the real oracle library.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden", "decay_first_example.json")

# (name, original text, replacement) -- each a single plausible slip.
MUTANTS = [
    ("erase_before_decay",
     "    /* 1. per-channel forget gate",
     "    /* (mutant) decay moved after the update */ if (0) {} /* 1."),
    ("decay_sign",
     "? g[0] : g[c]);",
     "? -g[0] : -g[c]);"),
    ("no_erase",
     "S[c * dv + j] += beta * k[c] * (v[j] - r[j]);",
     "S[c * dv + j] += beta * k[c] * (v[j]);"),
    ("erase_sign",
     "S[c * dv + j] += beta * k[c] * (v[j] - r[j]);",
     "S[c * dv + j] += beta * k[c] * (v[j] + r[j]);"),
    ("no_beta",
     "S[c * dv + j] += beta * k[c] * (v[j] - r[j]);",
     "S[c * dv + j] += k[c] * (v[j] - r[j]);"),
    ("read_with_k",
     "o[j] += q[c] * S[c * dv + j];",
     "o[j] += k[c] * S[c * dv + j];"),
    ("retrieve_with_q",
     "r[j] += k[c] * S[c * dv + j];",
     "r[j] += q[c] * S[c * dv + j];"),
    ("scalar_gate_read_per_channel",
     "(flags & KDA_ORACLE_SCALAR_GATE) ? g[0] : g[c]",
     "g[c]"),
    ("no_delta_keeps_beta",
     "S[c * dv + j] += k[c] * v[j];",
     "S[c * dv + j] += beta * k[c] * v[j];"),
    ("no_delta_still_erases",
     "    if (flags & KDA_ORACLE_NO_DELTA) {",
     "    if (0) {"),
]


def _apply(src, name, old, new):
    if name == "erase_before_decay":
        # move the decay loop after erase/write (and before the read)
        start = src.index("    /* 1. per-channel forget gate")
        end = src.index("    if (flags & KDA_ORACLE_NO_DELTA) {")
        decay = src[start:end]
        src = src[:start] + src[end:]
        pos = src.index("    /* 4. read after write")
        return src[:pos] + decay + src[pos:]
    assert old in src, name
    return src.replace(old, new)


def _build(tmp_path, src, tag):
    c = tmp_path / f"o_{tag}.c"
    so = tmp_path / f"o_{tag}.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", str(c), "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_fwd.argtypes = [dp] * 8 + [ctypes.c_int64] * 5 + [ctypes.c_int]
    lib.kda_oracle_fwd_ex.argtypes = [dp] * 8 + [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_int]
    return lib


def _fwd(lib, q, k, v, g, beta, S0, flags=0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, g, beta)]
    S0a = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    o = np.zeros((B, T, H, dv)); ST = np.zeros((B, H, dk, dv))
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = lib.kda_oracle_fwd_ex(*[p(a) for a in arrs], p(S0a), p(o), p(ST), B, T, H, dk, dv, flags, 1)
    assert rc == 0
    return o, ST


def _pins_fail(lib):
    """Return the names of the pins that the oracle library `lib` fails."""
    rng = np.random.default_rng(7)
    fails = []
    # P5 hand-worked example
    ex = json.load(open(GOLDEN))
    i = ex["inputs"]
    o, ST = _fwd(lib, np.array(i["q"])[None, None, None], np.array(i["k"])[None, None, None],
                 np.array(i["v"])[None, None, None], np.array(i["g"])[None, None, None],
                 np.array([[[i["beta"]]]]), np.array(i["S0"])[None, None])
    if np.max(np.abs(ST[0, 0] - np.array(ex["expected"]["S1"]))) > 1e-12 or abs(o[0, 0, 0, 0] - 0.25) > 1e-12:
        fails.append("worked_example")
    # P1 single-token closed form
    dk, dv = 5, 3
    q = rng.standard_normal((1, 1, 1, dk)); k = rng.standard_normal((1, 1, 1, dk)); k /= np.linalg.norm(k)
    v = rng.standard_normal((1, 1, 1, dv)); g = -np.abs(rng.standard_normal((1, 1, 1, dk)))
    beta = np.array([[[0.6]]]); S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = _fwd(lib, q, k, v, g, beta, S0)
    kk = k[0, 0, 0]
    S1 = (np.eye(dk) - 0.6 * np.outer(kk, kk)) @ np.diag(np.exp(g[0, 0, 0])) @ S0[0, 0] + 0.6 * np.outer(kk, v[0, 0, 0])
    if np.max(np.abs(ST[0, 0] - S1)) > 1e-12 or np.max(np.abs(o[0, 0, 0] - S1.T @ q[0, 0, 0])) > 1e-12:
        fails.append("single_token")
    # P4 orthonormal recall
    T = 4
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :T].T
    V = rng.standard_normal((T, dv))
    o, ST = _fwd(lib, K[None, :, None], K[None, :, None], V[None, :, None],
                 np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), S0)
    if np.max(np.abs(K @ ST[0, 0] - V)) > 1e-12:
        fails.append("recall")
    # scalar gate (flag 1): one gate per token, g laid out [B, T, H]; a
    # single token against the matrix form with alpha I
    # (the gates sit at the start of a longer buffer with defined values after
    # them, so that a per-channel read past the two gates, as a planted
    # mistake may do, reads known values rather than whatever memory follows)
    gbuf = np.concatenate([-np.abs(rng.standard_normal(2)), np.full(2 * dk, -0.7)])
    gs = gbuf[:2].reshape(1, 2, 1)
    q2 = rng.standard_normal((1, 2, 1, dk)); k2 = rng.standard_normal((1, 2, 1, dk))
    v2 = rng.standard_normal((1, 2, 1, dv)); b2 = np.full((1, 2, 1), 0.4)
    o, ST = _fwd(lib, q2, k2, v2, gs, b2, S0, flags=1)
    S = S0[0, 0]
    for t in range(2):
        kt = k2[0, t, 0]
        S = (np.eye(dk) - 0.4 * np.outer(kt, kt)) @ (np.exp(gs[0, t, 0]) * S) + 0.4 * np.outer(kt, v2[0, t, 0])
        if np.max(np.abs(o[0, t, 0] - S.T @ q2[0, t, 0])) > 1e-12:
            fails.append("scalar_gate")
            break
    # no delta (flag 2), ungated: causal linear attention o_t = sum_{s<=t} (q_t.k_s) v_s
    o, ST = _fwd(lib, q2, k2, v2, np.zeros((1, 2, 1, dk)), b2, None, flags=2)
    ref = np.tril(q2[0, :, 0] @ k2[0, :, 0].T) @ v2[0, :, 0]
    if np.max(np.abs(o[0, :, 0] - ref)) > 1e-12:
        fails.append("no_delta")
    return fails


# Slips in the backward (reverse-mode) code, each caught by the
# finite-difference pin below.
BWD_MUTANTS = [
    ("bwd_dr_sign", "dr[j] = -bt * ddelta[j];", "dr[j] = bt * ddelta[j];"),
    ("bwd_no_retrieve_adjoint", "dS[c * dv + j] += kt[c] * dr[j];", "(void)0;"),
    ("bwd_decay_not_propagated", "dS[c * dv + j] *= a;", "dS[c * dv + j] *= 1.0;"),
    ("bwd_dq_from_decayed_state", "acc += S[c * dv + j] * dot[j];", "acc += Sd[c * dv + j] * dot[j];"),
    ("bwd_dg_against_new_state", "acc += dS[c * dv + j] * Sd[c * dv + j];", "acc += dS[c * dv + j] * S[c * dv + j];"),
    ("bwd_dbeta_drops_retrieval", "db += ddelta[j] * (vt[j] - r[j]);", "db += ddelta[j] * vt[j];"),
]


def _bwd_pin_fails(lib):
    """Finite differences of the (same build's) forward against its backward."""
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 1, 7, 1, 4, 3
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_bwd_ex.argtypes = [dp] * 15 + [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int]
    x = dict(q=rng.standard_normal((B, T, H, dk)), k=rng.standard_normal((B, T, H, dk)) * 0.5,
             v=rng.standard_normal((B, T, H, dv)), g=-np.abs(rng.standard_normal((B, T, H, dk))) * 0.4,
             beta=rng.uniform(0.1, 1, (B, T, H)), S0=rng.standard_normal((B, H, dk, dv)))
    dO = rng.standard_normal((B, T, H, dv))
    p = lambda a: None if a is None else a.ctypes.data_as(dp)
    out = {n: np.zeros_like(x[n]) for n in x}
    rc = lib.kda_oracle_bwd_ex(*(p(x[n]) for n in ("q", "k", "v", "g", "beta", "S0")), p(dO), None,
                               p(out["q"]), p(out["k"]), p(out["v"]), p(out["g"]), p(out["beta"]), p(out["S0"]),
                               None, B, T, H, dk, dv, 3, 0, 1)
    assert rc == 0
    f = lambda xx: float((_fwd(lib, *(xx[n] for n in ("q", "k", "v", "g", "beta", "S0")))[0] * dO).sum())
    for n in x:
        u = rng.standard_normal(x[n].shape)
        xp = dict(x); xp[n] = x[n] + 1e-6 * u
        xm = dict(x); xm[n] = x[n] - 1e-6 * u
        fd = (f(xp) - f(xm)) / 2e-6
        if abs(fd - float((out[n] * u).sum())) > 1e-6 * max(1.0, abs(fd)):
            return True
    return False


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_planted_backward_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    lib = _build(tmp_path, src.replace(old, new), name)
    assert _pins_fail(lib) == []          # the forward is untouched
    assert _bwd_pin_fails(lib), f"backward mutant {name} passed the finite-difference pin"


def test_unmodified_backward_passes(tmp_path):
    lib = _build(tmp_path, open(SRC).read(), "ok_bwd")
    assert not _bwd_pin_fails(lib)


def test_unmodified_source_passes(tmp_path):
    lib = _build(tmp_path, open(SRC).read(), "ok")
    assert _pins_fail(lib) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = _apply(open(SRC).read(), name, old, new)
    lib = _build(tmp_path, src, name)
    assert _pins_fail(lib), f"mutant {name} passed every pin"
