"""The C-ABI library loads and exports every symbol include/kda.h declares,
and host-side validation rejects bad arguments before any launch.  CPU only:
no call here reaches a kernel (every one returns from argument checks)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def L():
    import gated_delta_rule_61_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return kda.lib()


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ("kda_chunk_fwd", "kda_recurrent_step", "kda_chunk_fwd_workspace_size", "kda_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared():
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.kda_version() == 10000
    for code in range(0, -9, -1):
        assert L.kda_status_string(code)
    assert L.kda_status_string(0) == b"ok"


NULL = None


def _fwd(L, **kw):
    a = dict(q=16, k=16, v=16, g=16, beta=16, S0=None, o=16, ST=None, B=1, T=64, H=1, dk=128, dv=128, dt=1)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kda_chunk_fwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["S0"]), p(a["o"]),
                           p(a["ST"]), a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], None, 0, None)


def test_sync_debug_leaves_validation_alone(L, monkeypatch):
    """KDA_SYNC_DEBUG only adds a wait after launches: argument errors are
    still reported before anything is launched or waited for."""
    monkeypatch.setenv("KDA_SYNC_DEBUG", "1")
    assert _fwd(L, q=None) == -1
    assert _fwd(L, dk=96, dv=96) == -2
    p = ctypes.c_void_p(16)
    assert L.kda_recurrent_step(p, p, p, p, p, None, p, 4, 2, 128, 128, 1, None) == -1


def test_prefill_validation(L):
    # fake aligned addresses: validation must fail before any launch
    assert _fwd(L, q=None) == -1
    assert _fwd(L, dk=96, dv=96) == -2
    assert _fwd(L, dk=128, dv=64) == -2
    assert _fwd(L, dt=0, dk=128, dv=128) == -5           # fp32 at d=128 needs its workspace
    assert _fwd(L, dt=0, dk=128, dv=64) == -2
    assert _fwd(L, dt=7) == -3
    assert _fwd(L, B=-1) == -2
    assert _fwd(L, q=18) == -4                          # misaligned
    assert _fwd(L, beta=17) == -4                       # beta only needs 2-byte alignment
    assert _fwd(L, B=0) == 0                            # nothing to do: no launch
    assert _fwd(L, H=0) == 0
    assert L.kda_chunk_fwd_workspace_size(8, 8192, 32, 128, 128, 1) == 0
    # fp32 at d=128: one 36992-float block of chunk quantities per chunk and head
    assert L.kda_chunk_fwd_workspace_size(2, 65, 3, 128, 128, 0) == 2 * 3 * 2 * 36992 * 4
    assert L.kda_chunk_fwd_workspace_size(2, 0, 3, 128, 128, 0) == 0
    assert L.kda_chunk_fwd_workspace_size(2, 65, 3, 64, 64, 0) == 0


def test_fp32_d128_workspace_checks(L):
    """The fp32 d=128 prefill refuses a missing, short or misaligned workspace,
    and the staged schedule (which has no fp32 d=128 kernels) refuses the size."""
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    need = L.kda_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 0)
    f = lambda ws, n: L.kda_chunk_fwd(p(16), p(16), p(16), p(16), p(16), None, p(16), None, 1, 64, 1, 128, 128, 0,
                                      p(ws), n, None)
    assert f(None, 0) == -5
    assert f(4096, need - 1) == -5
    assert f(4100, need) == -4
    assert L.kda_chunk_fwd_staged_workspace_size(1, 64, 1, 128, 128, 0) == 0
    assert L.kda_chunk_fwd_staged(p(16), p(16), p(16), p(16), p(16), None, p(16), None, 1, 64, 1, 128, 128, 0,
                                  p(4096), 1 << 30, None) == -2
    assert L.kda_stage_cumsum(p(16), p(16), 1, 64, 1, 128, 0, None) == -2
    # more than the allocation-free entry point's scratch holds: refused before any device call
    T = 64 * 454
    assert L.kda_chunk_fwd_workspace_size(1, T, 1, 128, 128, 0) > (64 << 20)
    assert L.kda_chunk_fwd_noalloc(p(16), p(16), p(16), p(16), p(16), None, p(16), None, 1, T, 1, 128, 128, 0,
                                   None) == -8


def test_noalloc_validation(L):
    """kda_chunk_fwd_noalloc checks its arguments like kda_chunk_fwd before it
    looks up its scratch or launches anything."""
    p = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(q=16, B=1, dk=128, dv=128, dt=1, S0=None):
        return L.kda_chunk_fwd_noalloc(p(q), p(16), p(16), p(16), p(16), p(S0), p(16), None, B, 64, 1, dk, dv, dt,
                                       None)
    assert call(q=None) == -1
    assert call(dk=96, dv=96) == -2
    assert call(dt=7) == -3
    assert call(q=18) == -4
    assert call(S0=20) == -4
    assert call(B=0) == 0
    assert b"scratch" in L.kda_status_string(-8)


def test_staged_workspace(L):
    n = L.kda_chunk_fwd_staged_workspace_size(1, 100, 2, 64, 64, 0)
    tok = 100 * 2
    assert n >= tok * 64 * 4 * 4 + 2 * 2 * 64 * 64 * 4
    p = ctypes.c_void_p(16)
    st = L.kda_chunk_fwd_staged(p, p, p, p, p, None, p, None, 1, 100, 2, 64, 64, 0, None, 0, None)
    assert st == -5
    st = L.kda_chunk_fwd_staged(p, p, p, p, p, None, p, None, 1, 100, 2, 64, 64, 0, p, n - 1, None)
    assert st == -5


def test_decode_validation(L):
    p = ctypes.c_void_p(16)
    assert L.kda_recurrent_step(p, p, p, p, p, None, p, 4, 2, 128, 128, 1, None) == -1
    assert L.kda_recurrent_step(p, p, p, p, p, p, p, 4, 2, 100, 100, 1, None) == -2
    assert L.kda_recurrent_step(p, p, p, p, p, p, p, 4, 2, 128, 128, 5, None) == -3
    assert L.kda_recurrent_step(p, p, p, p, p, ctypes.c_void_p(20), p, 4, 2, 128, 128, 1, None) == -4
    assert L.kda_recurrent_step(p, p, p, p, p, p, p, 0, 2, 128, 128, 1, None) == 0
    # more sequence-heads than one launch holds (KDA_STEP_MAX_HEADS = 2^24 - 1)
    assert L.kda_recurrent_step(p, p, p, p, p, p, p, 1 << 16, 256, 64, 64, 1, None) == -2


def test_binding_rejects_cpu_tensors():
    import torch
    import gated_delta_rule_61_amd as kda
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(kda.KDAError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 4, 1), None)


def _fwd_ex(L, flags, **kw):
    a = dict(q=16, k=16, v=16, g=16, beta=16, S0=None, o=16, ST=None, B=1, T=64, H=1, dk=128, dv=128, dt=1)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kda_chunk_fwd_ex(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["S0"]), p(a["o"]),
                              p(a["ST"]), a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], flags, None, 0, None)


def test_variant_validation(L):
    """kda_chunk_fwd_ex / kda_recurrent_step_ex: unknown flags and sizes the
    variants do not cover are rejected, beta may be NULL only without the
    delta rule, and a scalar gate needs only element alignment."""
    assert _fwd_ex(L, 4) == -7                        # unknown flag bit
    assert _fwd_ex(L, 1, dk=64, dv=64) == -7          # variants: bf16 d = 128 only
    assert _fwd_ex(L, 2, dt=0, dk=64, dv=64) == -7
    assert _fwd_ex(L, 1, beta=None) == -1             # the delta rule needs beta
    assert _fwd_ex(L, 1, g=18, q=None) == -1
    assert _fwd_ex(L, 2, beta=None, q=18) == -4       # beta may be NULL, q still checked
    assert _fwd_ex(L, 3, beta=None, g=18, q=18) == -4
    assert _fwd_ex(L, 0, dk=96, dv=96) == -2          # flags 0: the plain entry point's checks
    assert _fwd_ex(L, 3, B=0) == 0
    assert L.kda_chunk_fwd_ex_workspace_size(1, 4096, 16, 64, 64, 1, 1) == 0
    assert L.kda_chunk_fwd_ex_workspace_size(1, 4096, 16, 128, 128, 1, 8) == 0
    p = ctypes.c_void_p(16)
    assert L.kda_recurrent_step_ex(p, p, p, p, p, p, p, 4, 2, 128, 128, 1, 8, None) == -7
    assert L.kda_recurrent_step_ex(p, p, p, p, None, p, p, 4, 2, 128, 128, 1, 1, None) == -1
    assert L.kda_recurrent_step_ex(p, p, p, ctypes.c_void_p(18), p, p, p, 4, 2, 128, 128, 1, 0, None) == -4
    assert L.kda_recurrent_step_ex(p, p, p, p, p, p, p, 0, 2, 128, 128, 1, 3, None) == 0


def test_varlen_validation(L):
    p = ctypes.c_void_p(16)
    cu = ctypes.c_void_p(64)
    f = lambda *a: L.kda_chunk_fwd_varlen(*a[:9], None, *a[9:])
    assert f(p, p, p, p, p, None, p, None, None, 3, 100, 2, 128, 128, 1, 0, None) == -1   # no cu_seqlens
    assert f(p, p, p, p, p, None, p, None, ctypes.c_void_p(66), 3, 100, 2, 128, 128, 1, 0, None) == -4
    assert L.kda_chunk_fwd_varlen(p, p, p, p, p, None, p, None, cu, ctypes.c_void_p(66), 3, 100, 2, 128, 128,
                                  1, 0, None) == -4                                       # misaligned order
    assert f(p, p, p, p, p, None, p, None, cu, 3, 100, 2, 64, 64, 1, 0, None) == -7        # bf16 d128 only
    assert f(p, p, p, p, p, None, p, None, cu, 3, 100, 2, 128, 128, 1, 8, None) == -7      # unknown flag
    assert f(p, p, p, p, None, None, p, None, cu, 3, 100, 2, 128, 128, 1, 0, None) == -1   # beta needed
    assert f(p, p, p, p, p, None, p, None, cu, -1, 100, 2, 128, 128, 1, 0, None) == -2
    assert f(p, p, p, p, p, None, p, None, None, 0, 100, 2, 128, 128, 1, 0, None) == 0     # nothing to do
    s = L.kda_varlen_schedule
    assert s(cu, 0, 100, None, None) == 0
    assert s(None, 3, 100, p, None) == -1
    assert s(cu, 3, 100, None, None) == -1
    assert s(cu, 3, 100, ctypes.c_void_p(18), None) == -4
    assert s(cu, 16385, 100, p, None) == -2
    assert s(cu, -1, 100, p, None) == -2


def _bwd_ex(L, flags, g=16, dg=16, ws=None, wsz=0, T=64, dk=128, beta=16, dbeta=16):
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kda_chunk_bwd_ex(p(16), p(16), p(16), p(g), p(beta), None, p(16), None, p(16), p(16), p(16), p(dg),
                              p(dbeta), None, 1, T, 1, dk, dk, 1, flags, p(ws), wsz, None)


def test_backward_variant_validation(L):
    """kda_chunk_bwd_ex: the scalar gate (g, dg aligned to the element size)
    and the no-delta variant (beta and dbeta may be NULL) are accepted,
    unknown bits are not; the scalar path needs the broadcast gate and the
    fp32 per-channel dg in its workspace."""
    assert _bwd_ex(L, 2, beta=None, dbeta=None) == -5    # KDA_NO_DELTA: checks pass, workspace missing
    assert _bwd_ex(L, 3, g=18, dg=18, beta=None, dbeta=None) == -5
    assert _bwd_ex(L, 0, dbeta=None) == -1           # KDA needs dbeta
    assert _bwd_ex(L, 0, beta=None) == -1            # ... and beta
    assert _bwd_ex(L, 8) == -7                       # unknown bit
    assert _bwd_ex(L, 4) == -5                       # KDA_STATES_SAVED: checks pass, workspace missing
    assert _bwd_ex(L, 5, g=18, dg=18) == -5          # ... with the scalar gate too
    assert _bwd_ex(L, 4, dk=64) == -7                # ... nor on the token path
    assert _bwd_ex(L, 1, dk=64) == -5                # bf16 d = 64: token path, workspace missing
    assert _bwd_ex(L, 1, g=17) == -4                 # g not 2-byte aligned
    assert _bwd_ex(L, 1, g=18, dg=18) == -5          # scalar g / dg 2-byte aligned: workspace missing
    assert _bwd_ex(L, 0, dg=18) == -4                # per-channel dg must be 16-byte aligned
    base = L.kda_chunk_bwd_workspace_size(1, 64, 1, 128, 128, 1)
    assert L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 0) == base
    assert L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 1) == base + 64 * 128 * 6
    assert L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 2) == base
    assert L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 3) == base + 64 * 128 * 6
    assert L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 4) == base   # KDA_STATES_SAVED: same workspace
    assert L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 8) == 0
    assert _bwd_ex(L, 1, ws=1024, wsz=base) == -5    # too small for the scalar path


def test_backward_varlen_validation(L):
    """kda_chunk_bwd_varlen: argument checks before any launch; the workspace
    holds floor(T_total / 64) + N chunk slots per head (each slot a chunk
    state, a chunk-end adjoint and an operand block: 131840 bytes)."""
    p = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(cu=16, N=2, T=100, flags=0, ws=None, wsz=0, dk=128):
        return L.kda_chunk_bwd_varlen(p(16), p(16), p(16), p(16), p(16), None, p(16), None, p(16), p(16), p(16),
                                      p(16), p(16), None, p(cu), N, T, 1, dk, dk, 1, flags, p(ws), wsz, None)
    assert call(cu=None) == -1                        # cu_seqlens required
    assert call(cu=18) == -4                          # int32-aligned
    assert call(flags=8) == -7
    assert call(flags=4) == -5                       # KDA_STATES_SAVED: checks pass, workspace missing
    assert call(dk=64) == -7
    assert call() == -5                               # workspace missing
    assert call(N=0) == 0                             # nothing to do
    assert L.kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, 1, 0) == 3 * 131840
    assert L.kda_chunk_bwd_varlen_workspace_size(5, 64 * 7, 3, 128, 128, 1, 0) == (7 + 5) * 3 * 131840
    assert L.kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, 1, 1) == 3 * 131840 + 100 * 128 * 6
    assert L.kda_chunk_bwd_varlen_workspace_size(2, 0, 1, 128, 128, 1, 0) == 0


def test_varlen_segmented_workspace(L, monkeypatch):
    """Workspace of kda_chunk_fwd_varlen_ws: 0 without a device and without
    an override; with KDA_SEGMENTS = 6 on 6 sequences, 7597 tokens, H = 2:
    segments of ceil(119 / 6) = 20 chunks, at most 2 segmented sequences
    (> 40 chunks each) and 125 // 20 + 2 = 8 map slots: a plan rounded to
    512 bytes plus 8 slots x 2 heads x 3 maps of 64 KiB."""
    monkeypatch.delenv("KDA_SEGMENTS", raising=False)
    assert L.kda_chunk_fwd_varlen_workspace_size(6, 7597, 2, 128, 128, 1, 0) == 0
    monkeypatch.setenv("KDA_SEGMENTS", "6")
    assert L.kda_chunk_fwd_varlen_workspace_size(6, 7597, 2, 128, 128, 1, 0) == 512 + 8 * 2 * 3 * 65536
    assert L.kda_chunk_fwd_varlen_workspace_size(6, 7597, 2, 64, 64, 1, 0) == 0        # pipelined sizes only
    assert L.kda_chunk_fwd_varlen_workspace_size(1025, 7597, 2, 128, 128, 1, 0) == 0   # plan holds 1024
    p = ctypes.c_void_p(16)
    cu = ctypes.c_void_p(64)
    # argument checks before any launch
    f = L.kda_chunk_fwd_varlen_ws
    assert f(p, p, p, p, p, None, p, None, None, None, 6, 7597, 2, 128, 128, 1, 0, None, 0, None) == -1
    assert f(p, p, p, p, p, None, p, None, cu, None, 6, 7597, 2, 96, 96, 1, 0, None, 0, None) == -2
    assert f(p, p, p, p, p, None, p, None, cu, None, 0, 7597, 2, 128, 128, 1, 0, None, 0, None) == 0


def test_fwd_save_validation(L):
    """kda_chunk_fwd_save: bf16 at d = 128, KDA or no delta rule, and the
    backward's workspace, all checked before any launch."""
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    def f(flags=0, dk=128, dt=1, ws=None, wsz=0, q=16, B=1, T=64):
        return L.kda_chunk_fwd_save(p(q), p(16), p(16), p(16), p(16), None, p(16), None, B, T, 1, dk, dk, dt, flags,
                                    p(ws), wsz, None)
    assert f() == -5                                  # workspace missing
    assert f(flags=2) == -5
    assert f(flags=3) == -5                           # every variant
    assert f(flags=8) == -7
    assert f(dk=64) == -7                             # chunked backward sizes only
    assert f(dt=0) == -7
    assert f(q=None) == -1
    need = L.kda_chunk_bwd_ex_workspace_size(1, 64, 1, 128, 128, 1, 0)
    assert f(ws=32, wsz=need - 1) == -5
    assert f(ws=40, wsz=need) == -4                   # workspace not 16-byte aligned
    assert f(B=0) == 0


def test_fwd_varlen_save_validation(L):
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    def f(flags=0, cu=64, ws=None, wsz=0, dk=128):
        return L.kda_chunk_fwd_varlen_save(p(16), p(16), p(16), p(16), p(16), None, p(16), None, p(cu), None, 2, 100,
                                           1, dk, dk, 1, flags, p(ws), wsz, None)
    assert f() == -5                  # workspace missing
    assert f(flags=8) == -7           # unknown bit
    assert f(dk=64) == -7
    assert f(cu=None) == -1
    assert f(cu=66) == -4             # offsets 4-byte aligned
    need = L.kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, 1, 0)
    assert need > 0 and L.kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, 1, 4) == need
    assert L.kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, 1, 5) == \
        L.kda_chunk_bwd_varlen_workspace_size(2, 100, 1, 128, 128, 1, 1)


def test_bwd_token_path_workspace(L):
    """The token-recurrence backward (fp32 at d = 64 / 128, bf16 at d = 64):
    its workspace size, and the missing-workspace refusal before any launch."""
    for dt, d in ((0, 64), (0, 128), (1, 64)):
        B, T, H = 2, 130, 3
        nch, ns, r = (T + 63) // 64, d // 16, d // 16
        floats = B * H * nch * d * d + B * H * ns * 64 * 256 * r + ns * B * T * H * (3 * d + 1)
        assert L.kda_chunk_bwd_ex_workspace_size(B, T, H, d, d, dt, 0) == floats * 4
        assert L.kda_chunk_bwd_workspace_size(B, T, H, d, d, dt) == floats * 4
    p = ctypes.c_void_p(16)
    assert L.kda_chunk_bwd(p, p, p, p, p, None, p, None, p, p, p, p, p, None, 1, 64, 1, 64, 64, 0, None, 0,
                           None) == -5
    assert L.kda_chunk_bwd(p, p, p, p, p, None, p, None, p, p, p, p, p, None, 1, 64, 1, 96, 96, 0, None, 0,
                           None) == -2
