"""GPU parity of the chunked prefill (fused and staged schedules) against the
fp64 oracle, through the C ABI.  Needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_prefill, oracle_prefill, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _case(cfg, B=None, T=None, H=None, seed=None, s0=True):
    inp = W.prefill_inputs(cfg, device="cuda", seed=seed, B=B, T=T, H=H)
    if not s0:
        inp["S0"] = None
    return inp


def _run(kda, inp, staged=False):
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], staged=staged)
    torch.cuda.synchronize()
    return o, S


SMALL = [
    # (cfg, B, T, H, s0)
    (W.PREFILL_FP32_SMALL, 1, 256, 2, False),          # the fp32 workload as specified
    (W.PREFILL_FP32_SMALL, 2, 65, 3, True),
    (W.PREFILL_FP32_SMALL, 1, 1, 1, True),
    (W.PREFILL_FP32_SMALL, 1, 200, 2, True),
    (W.PREFILL_BF16_H16_T4K, 1, 63, 2, True),
    (W.PREFILL_BF16_H16_T4K, 1, 64, 1, False),
    (W.PREFILL_BF16_H16_T4K, 2, 130, 3, True),
    (W.PREFILL_BF16_H16_T4K, 1, 1, 4, True),
    (W.PREFILL_BF16_H16_T4K, 1, 517, 2, True),
]


@pytest.mark.parametrize("staged", [False, True], ids=["fused", "staged"])
@pytest.mark.parametrize("cfg,B,T,H,s0", SMALL, ids=[f"{c.dtype}-B{b}T{t}H{h}{'-S0' if s else ''}" for c, b, t, h, s in SMALL])
def test_small_shapes(kda, cfg, B, T, H, s0, staged):
    inp = _case(cfg, B, T, H, seed=100 + T + H, s0=s0)
    print(f"case {cfg.name} B{B} T{T} H{H} s0={s0} staged={staged}", flush=True)
    o, S = _run(kda, inp, staged)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, cfg.dtype, f"B{B}T{T}H{H}")


def test_bf16_d64(kda):
    cfg = W.Prefill("bf16_d64", 1, 300, 2, 64, 64, torch.bfloat16, 0.05)
    inp = _case(cfg, seed=5)
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "bf16 d64")


@pytest.mark.parametrize("nsplit", [1, 2, 4, 8])
def test_column_split_variants(kda, nsplit, monkeypatch):
    """Every column split of the state gives the oracle's result."""
    monkeypatch.setenv("KDA_FUSED_NSPLIT", str(nsplit))
    inp = _case(W.PREFILL_BF16_H16_T4K, 1, 200, 2, seed=9)
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"nsplit={nsplit}")


PIPE_SHAPES = [(1, 1, 2), (1, 63, 2), (1, 64, 1), (1, 65, 2), (2, 130, 3), (1, 517, 2), (3, 192, 1)]


@pytest.mark.parametrize("B,T,H", PIPE_SHAPES, ids=[f"B{b}T{t}H{h}" for b, t, h in PIPE_SHAPES])
@pytest.mark.parametrize("pipeline", ["1", "0"], ids=["pipelined", "serial"])
def test_bf16_d128_schedules(kda, B, T, H, pipeline, monkeypatch):
    """Both whole-sequence schedules for bf16, d = 128 without a column split
    (the software-pipelined one and the serial one), on single-chunk, exact,
    ragged and multi-chunk lengths."""
    monkeypatch.setenv("KDA_FUSED_NSPLIT", "1")
    monkeypatch.setenv("KDA_FUSED_PIPELINE", pipeline)
    inp = _case(W.PREFILL_BF16_H16_T4K, B, T, H, seed=300 + T + 7 * H, s0=True)
    print(f"case bf16 d128 B{B} T{T} H{H} pipeline={pipeline}", flush=True)
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"B{B}T{T}H{H} pipeline={pipeline}")


# (segment counts 3 .. 8: the combine chains P - 2 steps, three per loop
# iteration, and P = 6, 7 leave one and two steps after a whole iteration)
SEG_SHAPES = [(1, 64 * 12, 2, 3, True), (1, 64 * 13 + 17, 2, 4, True), (2, 64 * 20, 1, 5, False),
              (1, 64 * 9 + 1, 3, 3, True), (1, 64 * 40, 1, 8, True), (1, 64 * 30 + 5, 2, 6, True),
              (1, 64 * 35, 1, 7, False)]


@pytest.mark.parametrize("B,T,H,nseg,s0", SEG_SHAPES, ids=[f"B{b}T{t}H{h}-seg{n}{'-S0' if z else ''}" for b, t, h, n, z in SEG_SHAPES])
def test_segmented_schedule(kda, B, T, H, nseg, s0, monkeypatch):
    """The segmented schedule (segment state maps S_end = M S_start + N formed
    in parallel, chained, then every segment run again from its entry state)
    against the oracle, on exact and ragged lengths, with and without S0; and
    against the one-pass schedule on the same inputs."""
    monkeypatch.setenv("KDA_SEGMENTS", str(nseg))
    inp = _case(W.PREFILL_BF16_H16_T4K, B, T, H, seed=500 + T + nseg, s0=s0)
    assert kda.lib().kda_chunk_fwd_workspace_size(B, T, H, 128, 128, 1) > 0
    print(f"case segmented B{B} T{T} H{H} nseg={nseg} s0={s0}", flush=True)
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"segmented B{B}T{T}H{H}")
    monkeypatch.setenv("KDA_SEGMENTS", "0")
    assert kda.lib().kda_chunk_fwd_workspace_size(B, T, H, 128, 128, 1) == 0
    o1, S1 = _run(kda, inp)
    rel = (o.float() - o1.float()).norm() / o1.float().norm()
    assert rel < 5e-3, rel
    assert ((S - S1).norm() / S1.norm()) < 1e-3


@pytest.mark.parametrize("pipeline", ["1", "0"], ids=["pipelined", "serial"])
def test_single_token_seeds(kda, pipeline, monkeypatch):
    """Single-token prefill over many seeds: the output is q^T S_1 with S_1 one
    rank-one update of S0, so the current-token term q_t . k_t carries much of
    it and is summed exactly (it is the gate-free diagonal of P)."""
    monkeypatch.setenv("KDA_FUSED_NSPLIT", "1")
    monkeypatch.setenv("KDA_FUSED_PIPELINE", pipeline)
    for seed in range(8):
        inp = _case(W.PREFILL_BF16_H16_T4K, 1, 1, 4, seed=4000 + seed, s0=True)
        o, S = _run(kda, inp)
        o_ref, S_ref = oracle_prefill(inp)
        check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"T1 seed {4000 + seed} pipeline={pipeline}")


FP32_D128 = W.Prefill("kda_fwd_fp32_d128", 1, 256, 2, 128, 128, torch.float32, 0.05)
F32W_SHAPES = [
    # (B, T, H, s0, gate_mu)
    (1, 256, 2, False, -3.0),     # the fp32 workload's shape at d = 128
    (2, 65, 3, True, -3.0),       # one full chunk and a one-token tail
    (1, 1, 1, True, -3.0),
    (1, 64, 1, True, -3.0),
    (1, 200, 2, True, -3.0),
    (3, 517, 2, True, -3.0),
    (1, 320, 2, True, 0.0),       # strong forgetting: about e^-50 per chunk and channel
]


@pytest.mark.parametrize("B,T,H,s0,mu", F32W_SHAPES, ids=[f"B{b}T{t}H{h}{'-S0' if z else ''}-mu{m:g}" for b, t, h, z, m in F32W_SHAPES])
def test_fp32_d128(kda, B, T, H, s0, mu):
    """fp32 at d_k = d_v = 128 (chunk quantities through the workspace, then
    the state pass) against the oracle at the fp32 bound, on single-chunk,
    exact, ragged and multi-chunk lengths, and with strong forgetting."""
    cfg = W.Prefill("kda_fwd_fp32_d128", B, T, H, 128, 128, torch.float32, 0.05 if s0 else None, mu)
    inp = W.prefill_inputs(cfg, device="cuda", seed=700 + T + H)
    assert kda.lib().kda_chunk_fwd_workspace_size(B, T, H, 128, 128, 0) == B * H * ((T + 63) // 64) * 36992 * 4
    print(f"case fp32 d128 B{B} T{T} H{H} s0={s0} mu={mu}", flush=True)
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.float32, f"fp32 d128 B{B}T{T}H{H}")


def test_fp32_d128_streaming(kda):
    """fp32 d = 128 in three calls whose S_T aliases S0 (T = 100, 64, 37)
    equals one call over the whole sequence, and the oracle."""
    cfg = W.Prefill("kda_fwd_fp32_d128", 1, 201, 2, 128, 128, torch.float32, 0.05)
    inp = W.prefill_inputs(cfg, device="cuda", seed=77)
    S = inp["S0"].clone()
    outs = []
    for a_, b_ in ((0, 100), (100, 164), (164, 201)):
        part = [inp[n][:, a_:b_].contiguous() for n in ("q", "k", "v", "g", "beta")]
        o, _ = kda.chunk_fwd(*part, S, S_T=S)
        outs.append(o)
    torch.cuda.synchronize()
    o = torch.cat(outs, 1)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.float32, "fp32 d128 streaming")


def test_fp32_d128_needs_workspace(kda):
    """Without its workspace the fp32 d = 128 prefill refuses (KDA_ERR_WORKSPACE)
    and writes nothing."""
    inp = W.prefill_inputs(FP32_D128, device="cuda", seed=3)
    o = torch.full_like(inp["v"], 7.0)
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    L = kda.lib()
    st = L.kda_chunk_fwd(p(inp["q"]), p(inp["k"]), p(inp["v"]), p(inp["g"]), p(inp["beta"]), p(inp["S0"]), p(o),
                         None, 1, 256, 2, 128, 128, 0, None, 0, None)
    assert st == -5
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


def test_workload_fp32_B1_H2_T256(kda):
    """The fp32 workload at its full size (S0 = 0)."""
    inp = W.prefill_inputs(W.PREFILL_FP32_SMALL, device="cuda")
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.float32, "fp32 B1 H2 T256")
    print(st)


def test_workload_bf16_B1_H16_T4096(kda):
    """The H16 T4096 bf16 workload at full size, every head against the
    oracle; here the literal max-error bound holds as well (the correctly
    rounded result meets it with room on this workload)."""
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda")
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "bf16 B1 H16 T4096", literal=True)
    print(st)


def test_workload_bf16_B8_H32_T8192(kda):
    """Full size (the benchmark's launch), all 256 heads against the oracle."""
    cfg = W.PREFILL_BF16_B8_H32_T8K
    inp = W.prefill_inputs(cfg, device="cuda")
    o, S = _run(kda, inp)
    assert torch.isfinite(o.float()).all()
    o_ref, S_ref = oracle_prefill(inp)
    del inp
    st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "bf16 B8 H32 T8192")
    print(st)


def test_workload_bf16_long_T131072(kda):
    """Long-context slow-gate workload at full size (the segmented schedule),
    all 32 heads against the oracle."""
    cfg = W.PREFILL_BF16_LONG_T128K
    inp = W.prefill_inputs(cfg, device="cuda")
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    del inp
    st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "bf16 T131072")
    print(st)


@pytest.mark.parametrize("pipeline", ["1"], ids=["pipelined"])
def test_short_sequences_seed_sweep(kda, pipeline, monkeypatch):
    """T = 2 .. 8 with bf16 inputs over 32 seeds x 4 heads each: one output
    vector is then carried by few tokens, so a rounding of the gated operands
    is not averaged away."""
    monkeypatch.setenv("KDA_FUSED_NSPLIT", "1")
    monkeypatch.setenv("KDA_FUSED_PIPELINE", pipeline)
    worst = {}
    for T in range(2, 9):
        for seed in range(32):
            inp = _case(W.PREFILL_BF16_H16_T4K, 1, T, 4, seed=6000 + 100 * T + seed, s0=True)
            o, S = _run(kda, inp)
            o_ref, S_ref = oracle_prefill(inp)
            st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"T{T} seed {seed} pipeline={pipeline}")
            worst[T] = max(worst.get(T, 0.0), st["rel_l2_o"])
    print("worst per-head rel L2 of o by T:", {t: f"{v:.2e}" for t, v in worst.items()})


def test_short_sequences_seed_sweep_d64(kda):
    """bf16 at d = 64, T = 1 .. 8 over 32 seeds x 4 heads: with its workspace
    (the binding passes it) the prefill takes fp32 matrix operands, which keep
    these outputs inside the bf16 bounds (the one-launch kernel's bf16
    operands reach 8e-3 per-head rel L2 at T = 2)."""
    L = kda.lib()
    assert L.kda_chunk_fwd_workspace_size(1, 8, 4, 64, 64, 1) == 1 * 4 * 1 * (4 * 64 * 64 + 64 * 64 + 64) * 4
    worst = {}
    for T in range(1, 9):
        for seed in range(32):
            cfg = W.Prefill("bf16_d64", 1, T, 4, 64, 64, torch.bfloat16, 0.05)
            inp = W.prefill_inputs(cfg, device="cuda", seed=6000 + 97 * T + seed)
            o, S = _run(kda, inp)
            o_ref, S_ref = oracle_prefill(inp)
            st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"d64 T{T} seed {seed}")
            worst[T] = max(worst.get(T, 0.0), st["rel_l2_o"])
    print("d64 worst per-head rel L2 of o by T:", {t: f"{v:.2e}" for t, v in worst.items()})


def test_bf16_d64_without_workspace(kda):
    """Without a workspace bf16 d = 64 runs the one-launch kernel (bf16
    operands): same result within the bf16 bounds on an ordinary length."""
    import ctypes
    cfg = W.Prefill("bf16_d64", 2, 300, 3, 64, 64, torch.bfloat16, 0.05)
    inp = W.prefill_inputs(cfg, device="cuda", seed=11)
    o = torch.empty_like(inp["v"])
    S = torch.empty(2, 3, 64, 64, dtype=torch.float32, device="cuda")
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = kda.lib().kda_chunk_fwd(p(inp["q"]), p(inp["k"]), p(inp["v"]), p(inp["g"]), p(inp["beta"]), p(inp["S0"]),
                                 p(o), p(S), 2, 300, 3, 64, 64, 1, None, 0, None)
    assert st == 0
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "bf16 d64 one-launch")


def _strong_decay_inputs(B, T, H, seed, burst=None):
    """The H16 T4K recipe, then a quarter of the channels forget fast (log-gate
    -1.2 .. -0.8 per step, 51 - 77 nats per 64-token chunk), everywhere or in
    the token range `burst` only: such chunks leave the fp16 range of the
    referenced gated operands and keep bf16 operands."""
    inp = _case(W.PREFILL_BF16_H16_T4K, B, T, H, seed=seed, s0=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 17)
    g = inp["g"].float()
    fast = -(0.8 + 0.4 * torch.rand(g.shape, device="cuda", generator=gen))
    sel = torch.zeros(g.shape, dtype=torch.bool, device="cuda")
    t0, t1 = burst if burst is not None else (0, T)
    sel[:, t0:t1, :, ::4] = True
    inp["g"] = torch.where(sel, fast, g).to(torch.bfloat16).contiguous()
    return inp


@pytest.mark.parametrize("burst", [None, (200, 330)], ids=["all", "burst"])
def test_bf16_operand_fallback(kda, burst):
    """Chunks whose gated operands would leave the fp16 range run with bf16
    operands (every chunk, or only those overlapping a burst of fast
    forgetting in the middle of the sequence); both kinds of chunk in one
    sequence hand the state over correctly."""
    inp = _strong_decay_inputs(2, 517, 3, 77, burst)
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"strong decay {burst}")


def test_state_beyond_fp16_range(kda):
    """The fp16 read-out Qg S of a state with entries beyond the fp16 range
    (here 16 key channels carry entries of order 1e5 that no key touches:
    k = 0 and g = 0 there, q small) takes the rescaled path and matches the
    oracle; the other channels are ordinary."""
    inp = _case(W.PREFILL_BF16_H16_T4K, 1, 300, 2, seed=91)
    big = slice(0, 16)
    gen = torch.Generator(device="cuda").manual_seed(92)
    S0 = inp["S0"].clone()
    S0[:, :, big, :] = torch.randn(S0[:, :, big, :].shape, generator=gen, device="cuda") * 2e5
    inp["S0"] = S0
    for n, f in (("k", 0.0), ("g", 0.0), ("q", 1e-3)):
        t = inp[n].float()
        t[..., big] *= f
        inp[n] = t.to(inp[n].dtype).contiguous()
    assert float(S0.abs().max()) > 65504
    o, S = _run(kda, inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "state beyond fp16")


def test_empty_sequence_copies_state(kda):
    inp = _case(W.PREFILL_BF16_H16_T4K, 2, 0, 3, seed=1)
    o, S = _run(kda, inp)
    assert o.shape == (2, 0, 3, 128)
    assert torch.equal(S, inp["S0"])
    inp["S0"] = None
    o, S = _run(kda, inp)
    assert torch.count_nonzero(S) == 0


def test_state_aliasing_and_streaming_split(kda):
    """S_T may alias S0; running [0,T1) then [T1,T) from the hand-off state
    equals one call (chunk boundaries inside the second call differ)."""
    inp = _case(W.PREFILL_BF16_H16_T4K, 1, 300, 2, seed=3)
    o_full, S_full = _run(kda, inp)
    T1 = 100
    part = lambda t, a, b: t[:, a:b].contiguous()
    S = inp["S0"].clone()
    o1, _ = kda.chunk_fwd(*(part(inp[n], 0, T1) for n in ("q", "k", "v", "g", "beta")), S, S_T=S)
    o2, _ = kda.chunk_fwd(*(part(inp[n], T1, 300) for n in ("q", "k", "v", "g", "beta")), S, S_T=S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(to64(torch.cat([o1, o2], 1)), to64(S), o_ref, S_ref, torch.bfloat16, "split")


def test_deterministic(kda):
    inp = _case(W.PREFILL_BF16_H16_T4K, 1, 700, 4, seed=11)
    o1, S1 = _run(kda, inp)
    o2, S2 = _run(kda, inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_pins_on_gpu_fp32(kda):
    """Closed-form cases on the GPU in fp32: beta = 0 is pure decay, and
    orthonormal keys with beta = 1, g = 0 give causal linear attention."""
    dev = "cuda"
    rng = np.random.default_rng(0)
    B, T, H, d = 1, 100, 1, 64
    q = rng.standard_normal((B, T, H, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    g = -np.abs(rng.standard_normal((B, T, H, d))) * 0.05
    S0 = rng.standard_normal((B, H, d, d))
    t = lambda x: torch.tensor(x, dtype=torch.float32, device=dev).contiguous()
    # beta = 0
    o, S = kda.chunk_fwd(t(q), t(k), t(v), t(g), t(np.zeros((B, T, H))), t(S0))
    torch.cuda.synchronize()
    cum = np.cumsum(to64(t(g)), axis=1)
    S0f = to64(t(S0))
    S_exp = np.exp(cum[0, -1, 0])[:, None] * S0f[0, 0]
    o_exp = np.stack([(np.exp(cum[0, i, 0])[:, None] * S0f[0, 0]).T @ to64(t(q))[0, i, 0] for i in range(T)])
    scale = np.sqrt(np.mean(o_exp ** 2))
    assert np.max(np.abs(to64(S)[0, 0] - S_exp)) <= 1e-4 * scale
    assert np.max(np.abs(to64(o)[0, :, 0] - o_exp)) <= 1e-4 * scale
    # orthonormal keys (T <= d), beta = 1, g = 0, S0 = 0
    T2 = 48
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    K = Qm[:, :T2].T
    Qr = rng.standard_normal((T2, d))
    V = rng.standard_normal((T2, d))
    o, S = kda.chunk_fwd(t(Qr[None, :, None]), t(K[None, :, None]), t(V[None, :, None]),
                         t(np.zeros((1, T2, 1, d))), t(np.ones((1, T2, 1))), None)
    torch.cuda.synchronize()
    Kf, Qf, Vf = to64(t(K)), to64(t(Qr)), to64(t(V))
    o_exp = np.tril(Qf @ Kf.T) @ Vf
    scale = np.sqrt(np.mean(o_exp ** 2))
    assert np.max(np.abs(to64(o)[0, :, 0] - o_exp)) <= 1e-4 * scale
    # orthonormality holds only to fp32 rounding; compare with the oracle too
    o_ref, S_ref = oracle.recurrent_fwd(Qf[None, :, None], Kf[None, :, None], Vf[None, :, None],
                                        np.zeros((1, T2, 1, d)), np.ones((1, T2, 1)), None)
    assert np.max(np.abs(to64(S)[0, 0] - S_ref[0, 0])) <= 1e-4 * scale


def _f32(x):
    return torch.tensor(np.asarray(x), dtype=torch.float32, device="cuda").contiguous()


def test_pin_orthonormal_recall_and_flush_fp32(kda):
    """beta = 1, g = 0 and orthonormal keys: the final state recalls every
    written value, S_T^T k_i = v_i, and equals (I - K^T K) S0 + K^T V; after
    d_k such keys S0 is erased completely, S_T = K^T V ("Hybrid Linear
    Attention Architecture: Making LLM Training and Inference More Efficient"
    §3.2: beta -> 1 overwrites, d steps flush)."""
    d = 64
    rng = np.random.default_rng(41)
    S0 = rng.standard_normal((1, 1, d, d))
    for T in (40, d):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        K = Qm[:, :T].T                                  # T orthonormal rows
        V = rng.standard_normal((T, d))
        Qr = rng.standard_normal((T, d))
        k_, v_, q_, s0_ = _f32(K[None, :, None]), _f32(V[None, :, None]), _f32(Qr[None, :, None]), _f32(S0)
        o, S = kda.chunk_fwd(q_, k_, v_, _f32(np.zeros((1, T, 1, d))), _f32(np.ones((1, T, 1))), s0_)
        torch.cuda.synchronize()
        Kf, Vf, S0f = to64(k_)[0, :, 0], to64(v_)[0, :, 0], to64(s0_)[0, 0]
        St = to64(S)[0, 0]
        scale = np.sqrt(np.mean(Vf ** 2))
        # recall of every written value
        assert np.max(np.abs(Kf @ St - Vf)) <= 1e-4 * scale, T
        expect = (np.eye(d) - Kf.T @ Kf) @ S0f + Kf.T @ Vf
        assert np.max(np.abs(St - expect)) <= 1e-4 * scale, T
        if T == d:
            assert np.max(np.abs(St - Kf.T @ Vf)) <= 1e-4 * scale


def test_pin_decay_first_worked_example_fp32(kda):
    """The worked one-token example of tests/golden (2 x 1 state, decay by
    channel before the erase) embedded in d = 64 with zeros: o = 1/4 and
    S_1 = (1/4, -1/4) ("Hybrid Linear Attention Architecture: Making LLM
    Training and Inference More Efficient" §3.3)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "decay_first_example.json")) as f:
        ex = json.load(f)
    d = 64
    pad = lambda x: np.concatenate([np.asarray(x, dtype=np.float64), np.zeros(d - len(x))])
    inp = ex["inputs"]
    S0 = np.zeros((1, 1, d, d))
    S0[0, 0, :2, 0] = np.asarray(inp["S0"])[:, 0]
    args = [_f32(pad(inp[n])[None, None, None]) for n in ("q", "k", "v", "g")]
    o, S = kda.chunk_fwd(*args, _f32(np.full((1, 1, 1), inp["beta"])), _f32(S0))
    torch.cuda.synchronize()
    o_exp = pad(ex["expected"]["o"])
    S_exp = np.zeros((d, d))
    S_exp[:2, 0] = np.asarray(ex["expected"]["S1"])[:, 0]
    S_exp[:, 1:] = 0.0
    assert np.max(np.abs(to64(o)[0, 0, 0] - o_exp)) <= 1e-6
    assert np.max(np.abs(to64(S)[0, 0] - S_exp)) <= 1e-6


def test_pin_full_overwrite_fp32(kda):
    """beta = 1, g = 0 and one unit key written again and again: each write
    replaces the value stored under it, so with q = k every output is the
    token's own value, o_t = S_t^T k = v_t, across chunk boundaries (same
    page, §3.2: beta -> 1 is a complete overwrite)."""
    d, T = 64, 150
    rng = np.random.default_rng(43)
    kv = rng.standard_normal(d)
    kv /= np.linalg.norm(kv)
    K = np.tile(kv, (T, 1))
    V = rng.standard_normal((T, d))
    S0 = rng.standard_normal((1, 1, d, d)) * 0.1
    k_ = _f32(K[None, :, None])
    o, S = kda.chunk_fwd(k_, k_, _f32(V[None, :, None]), _f32(np.zeros((1, T, 1, d))),
                         _f32(np.ones((1, T, 1))), _f32(S0))
    torch.cuda.synchronize()
    Vf = to64(_f32(V))
    scale = np.sqrt(np.mean(Vf ** 2))
    assert np.max(np.abs(to64(o)[0, :, 0] - Vf)) <= 1e-4 * scale
    assert np.max(np.abs(to64(k_)[0, -1, 0] @ to64(S)[0, 0] - Vf[-1])) <= 1e-4 * scale
