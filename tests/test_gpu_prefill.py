"""GPU parity of the chunked prefill (fused and staged schedules) against the
fp64 oracle, through the C ABI.  Needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_prefill, oracle_prefill, pick, to64

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


SEG_SHAPES = [(1, 64 * 12, 2, 3, True), (1, 64 * 13 + 17, 2, 4, True), (2, 64 * 20, 1, 5, False),
              (1, 64 * 9 + 1, 3, 3, True), (1, 64 * 40, 1, 8, True)]


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


def test_workload_fp32_B1_H2_T256(kda):
    """The fp32 workload at its full size (S0 = 0)."""
    inp = W.prefill_inputs(W.PREFILL_FP32_SMALL, device="cuda")
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.float32, "fp32 B1 H2 T256")
    print(st)


def test_workload_bf16_B1_H16_T4096(kda):
    """The H16 T4096 bf16 workload at full size, every head against the oracle."""
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda")
    o, S = _run(kda, inp)
    o_ref, S_ref = oracle_prefill(inp)
    st = check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, "bf16 B1 H16 T4096")
    print(st)


def test_workload_bf16_B8_H32_T8192_sampled(kda):
    """Full size (the benchmark's launch), sampled heads against the oracle."""
    cfg = W.PREFILL_BF16_B8_H32_T8K
    inp = W.prefill_inputs(cfg, device="cuda")
    o, S = _run(kda, inp)
    heads = [(0, 0), (3, 17), (7, 31), (5, 8)]
    o_ref, S_ref = oracle_prefill(inp, heads)
    o_s, S_s = pick(o, S, heads)
    st = check_prefill(o_s, S_s, o_ref, S_ref, torch.bfloat16, "bf16 B8 H32 T8192")
    print(st)
    assert torch.isfinite(o.float()).all()


def test_workload_bf16_long_T131072_sampled(kda):
    """Long-context slow-gate workload at full size: two heads vs the oracle."""
    cfg = W.PREFILL_BF16_LONG_T128K
    inp = W.prefill_inputs(cfg, device="cuda")
    o, S = _run(kda, inp)
    heads = [(0, 5), (0, 30)]
    o_ref, S_ref = oracle_prefill(inp, heads)
    o_s, S_s = pick(o, S, heads)
    st = check_prefill(o_s, S_s, o_ref, S_ref, torch.bfloat16, "bf16 T131072")
    print(st)


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
