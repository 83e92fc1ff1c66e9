"""GPU parity of the packed variable-length prefill (kda_chunk_fwd_varlen)
against the fp64 oracle run on each sequence alone, and of prefill that
continues from decode states ("Linear Attention Architecture Deep Dive: From
State Updates to Efficient Chunked Computation" §5 and §7: only the state is
carried, so input can be streamed piece by piece).  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_prefill, to64

pytestmark = pytest.mark.gpu

VARIANTS = [(False, True), (True, True), (False, False), (True, False)]
VIDS = ["kda", "scalar", "nodelta", "scalar-nodelta"]


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _packed(lengths, H, seed, scalar_gate=False, s0=True):
    """Tokens of len(lengths) sequences drawn as one [1, T_total, H, .] batch
    (the workload recipe), squeezed to the packed [T_total, H, .] layout."""
    Tt = int(sum(lengths))
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda", seed=seed, B=1, T=max(Tt, 1), H=H,
                           scalar_gate=scalar_gate)
    x = {n: inp[n][0, :Tt].contiguous() for n in ("q", "k", "v", "g", "beta")}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 1)
    x["S0"] = (torch.randn(len(lengths), H, 128, 128, device="cuda", generator=gen) * 0.02) if s0 else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x["cu"] = torch.tensor(cu, dtype=torch.int32, device="cuda")
    return x, cu


def _oracle_seq(x, a, b, i, scalar_gate, delta):
    sl = lambda t: None if t is None else to64(t[a:b])[None]
    S0 = None if x["S0"] is None else to64(x["S0"][i])[None]
    return oracle.recurrent_fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]),
                                sl(x["beta"]) if delta else None, S0, scalar_gate=scalar_gate, delta=delta)


def _run(kda, x, scalar_gate=False, delta=True):
    o, S = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"] if delta else None, x["cu"], x["S0"],
                                scalar_gate=scalar_gate, delta=delta)
    torch.cuda.synchronize()
    return o, S


def _check_all(x, cu, o, S, scalar_gate, delta, what):
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            ref = torch.zeros_like(S[i]) if x["S0"] is None else x["S0"][i]
            assert torch.equal(S[i], ref), f"{what}: empty sequence {i} must copy S0"
            continue
        o_ref, S_ref = _oracle_seq(x, a, b, i, scalar_gate, delta)
        check_prefill(to64(o[a:b])[None], to64(S[i])[None], o_ref, S_ref, torch.bfloat16, f"{what} seq {i} T={b - a}")


MIX = [0, 1, 63, 64, 65, 700, 130, 2]


@pytest.mark.parametrize("scalar_gate,delta", VARIANTS, ids=VIDS)
def test_mixed_lengths(kda, scalar_gate, delta):
    """Empty, single-token, exact, ragged and multi-chunk sequences in one call,
    each against the oracle on that sequence alone."""
    x, cu = _packed(MIX, 3, 41, scalar_gate)
    print(f"case varlen lengths={MIX} H3 scalar_gate={scalar_gate} delta={delta}", flush=True)
    o, S = _run(kda, x, scalar_gate, delta)
    _check_all(x, cu, o, S, scalar_gate, delta, "varlen")


def test_matches_separate_calls(kda, monkeypatch):
    """Each packed sequence gives bit-for-bit what a kda_chunk_fwd call on that
    sequence alone gives (same kernel, one pass)."""
    monkeypatch.setenv("KDA_SEGMENTS", "0")
    x, cu = _packed(MIX, 2, 43)
    o, S = _run(kda, x)
    for i in range(len(MIX)):
        a, b = int(cu[i]), int(cu[i + 1])
        part = lambda t: t[a:b][None].contiguous()
        o1, S1 = kda.chunk_fwd(*(part(x[n]) for n in ("q", "k", "v", "g", "beta")), x["S0"][i:i + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], o1[0]), i
        assert torch.equal(S[i], S1[0]), i


def test_no_initial_state_and_no_final_state(kda):
    x, cu = _packed([5, 64, 200], 2, 45, s0=False)
    o, S = _run(kda, x)
    _check_all(x, cu, o, S, False, True, "varlen S0=0")
    o2, S2 = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], None, want_state=False)
    torch.cuda.synchronize()
    assert S2 is None and torch.equal(o, o2)


def test_many_sequences(kda):
    """96 sequences of 1 .. 2048 tokens (a serving batch mix), 8 heads; every
    sequence against the oracle."""
    rng = np.random.default_rng(5)
    lengths = np.minimum(rng.geometric(1 / 300.0, size=96), 2048).tolist()
    x, cu = _packed(lengths, 8, 47)
    print(f"case varlen 96 sequences, T_total={cu[-1]}", flush=True)
    o, S = _run(kda, x)
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        o_ref, S_ref = _oracle_seq(x, a, b, i, False, True)
        check_prefill(to64(o[a:b])[None], to64(S[i])[None], o_ref, S_ref, torch.bfloat16, f"seq {i} T={b - a}")
    assert torch.isfinite(o.float()).all()


def test_prefill_continues_from_decode_states(kda):
    """Decode 6 tokens per sequence from a state, then prefill the next tokens
    of each sequence (different lengths, packed) from the decode states in
    place: the whole stream matches the oracle run over all tokens at once."""
    N, H, steps = 4, 2, 6
    lengths = [1, 64, 150, 33]
    x, cu = _packed(lengths, H, 49)
    dcfg = W.Decode("stream", N, H, 128, 128, steps, torch.bfloat16, 0.02)
    tok = W.decode_tokens(dcfg, device="cuda", seed=51)
    S = x["S0"].clone()
    o_dec = []
    for t in range(steps):
        o_dec.append(kda.recurrent_step(*(tok[n][t].contiguous() for n in ("q", "k", "v", "g", "beta")), S))
    o_pre, _ = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], S, S_T=S)
    torch.cuda.synchronize()
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        cat = lambda n: np.concatenate([to64(tok[n][:, i]), to64(x[n][a:b])], 0)[None]
        o_ref, S_ref = oracle.recurrent_fwd(cat("q"), cat("k"), cat("v"), cat("g"), cat("beta"),
                                            to64(x["S0"][i])[None])
        o_gpu = np.concatenate([np.stack([to64(od[i]) for od in o_dec], 0), to64(o_pre[a:b])], 0)[None]
        check_prefill(o_gpu, to64(S[i])[None], o_ref, S_ref, torch.bfloat16, f"decode+prefill seq {i}")


def test_out_of_range_offsets_are_clamped(kda):
    """Offsets outside [0, T_total] or decreasing are clamped on the device:
    sequence i covers [clamp(cu[i]), max(clamp(cu[i+1]), clamp(cu[i]))) -- no
    access outside the tensors, and rows outside every range are left alone."""
    x, _ = _packed([100], 2, 53)
    S0 = torch.randn(3, 2, 128, 128, device="cuda") * 0.02
    ref = lambda a, b, i: _oracle_seq(dict(x, S0=S0), a, b, i, False, True)
    run = lambda cu, o: kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                             torch.tensor(cu, dtype=torch.int32, device="cuda"),
                                             S0[:len(cu) - 1].contiguous(), o=o)
    # below 0 and past the end: [0, 30), [30, 30), [30, 100)
    o = torch.full((100, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o, S = run([-7, 30, 30, 10_000], o)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate([(0, 30), (30, 100)]):
        o_ref, S_ref = ref(a, b, 2 * i)
        check_prefill(to64(o[a:b])[None], to64(S[2 * i])[None], o_ref, S_ref, torch.bfloat16, f"clamped {a}:{b}")
    assert torch.equal(S[1], S0[1])
    # a sub-range: rows outside it keep their values
    o = torch.full((100, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o, S = run([10, 40], o)
    torch.cuda.synchronize()
    assert (o[:10] == 7.0).all() and (o[40:] == 7.0).all()
    o_ref, S_ref = ref(10, 40, 0)
    check_prefill(to64(o[10:40])[None], to64(S[0])[None], o_ref, S_ref, torch.bfloat16, "sub-range")
    # decreasing offsets: [0, 50), [50, 50), [30, 100); the overlapping output
    # rows 30..49 have two writers, the states and the other rows are defined
    o, S = run([0, 50, 30, 10_000], None)
    torch.cuda.synchronize()
    o_ref, S_ref = ref(0, 50, 0)
    check_prefill(to64(o[:30])[None], to64(S[0])[None], o_ref[:, :30], S_ref, torch.bfloat16, "decreasing seq 0")
    assert torch.equal(S[1], S0[1])
    o_ref, S_ref = ref(30, 100, 2)
    check_prefill(to64(o[50:])[None], to64(S[2])[None], o_ref[:, 20:], S_ref, torch.bfloat16, "decreasing seq 2")


def _expected_order(cu, T):
    cu = np.asarray(cu, dtype=np.int64)
    N = len(cu) - 1
    e0 = np.clip(cu[:-1], 0, T)
    e1 = np.minimum(np.maximum(cu[1:], e0), T)
    nch = (e1 - e0 + 63) // 64
    return sorted(range(N), key=lambda i: (-nch[i], i))


@pytest.mark.parametrize("N", [1, 8, 96, 1000, 16384])
def test_schedule_is_longest_first(kda, N):
    """kda_varlen_schedule sorts by decreasing chunk count, ties by index
    (also for clamped offsets), up to its 16384-sequence limit."""
    rng = np.random.default_rng(N)
    lengths = rng.integers(0, 400 if N <= 1000 else 40, size=N)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    if N == 96:
        cu[10] = -5
        cu[40] = T + 1000
    order = kda.varlen_schedule(torch.tensor(cu, device="cuda"), T)
    torch.cuda.synchronize()
    assert order.cpu().tolist() == _expected_order(cu, T)


def test_order_does_not_change_results(kda):
    """Longest-first order and index order give bit-identical results."""
    x, cu = _packed(MIX, 3, 55)
    o1, S1 = _run(kda, x)
    order = kda.varlen_schedule(x["cu"], int(cu[-1]))
    assert order.cpu().tolist() == _expected_order(cu, int(cu[-1]))
    o2, S2 = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["S0"], seq_order=order)
    rev = torch.arange(len(MIX) - 1, -1, -1, dtype=torch.int32, device="cuda")
    o3, S3 = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["S0"], seq_order=rev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, S3)


SEG_MIX = [64 * 60 + 5, 70, 0, 1, 64 * 12, 64 * 45 + 33]


@pytest.mark.parametrize("order", [False, True], ids=["index-order", "longest-first"])
@pytest.mark.parametrize("scalar_gate,delta", [VARIANTS[0], VARIANTS[3]], ids=[VIDS[0], VIDS[3]])
def test_segmented_packed(kda, scalar_gate, delta, order, monkeypatch):
    """The segmented schedule for packed sequences (kda_chunk_fwd_varlen_ws):
    with segments of ceil(T_total / 64 / 6) = 20 chunks the two longest
    sequences (61 and 46 chunks) run segmented and the others whole; every
    sequence against the oracle alone, and against the one-pass schedule."""
    monkeypatch.setenv("KDA_SEGMENTS", "6")
    x, cu = _packed(SEG_MIX, 2, 57, scalar_gate)
    N, Tt, H = len(SEG_MIX), int(cu[-1]), 2
    flags = (1 if scalar_gate else 0) | (0 if delta else 2)
    assert kda.lib().kda_chunk_fwd_varlen_workspace_size(N, Tt, H, 128, 128, 1, flags) > 0
    so = kda.varlen_schedule(x["cu"], Tt) if order else None
    print(f"case segmented varlen lengths={SEG_MIX} H2 scalar_gate={scalar_gate} delta={delta} order={order}", flush=True)
    o, S = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"] if delta else None, x["cu"], x["S0"],
                                seq_order=so, scalar_gate=scalar_gate, delta=delta)
    torch.cuda.synchronize()
    _check_all(x, cu, o, S, scalar_gate, delta, "segmented varlen")
    o1, S1 = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"] if delta else None, x["cu"], x["S0"],
                                  scalar_gate=scalar_gate, delta=delta, segmented=False)
    torch.cuda.synchronize()
    rel = (o.float() - o1.float()).norm() / o1.float().norm()
    assert rel < 5e-3, rel
    assert ((S - S1).norm() / S1.norm()) < 1e-3


def test_segmented_packed_default_heuristic(kda):
    """Without an override, 32 heads with one 25 600-token sequence beside a
    short one: segments of max(16, ceil((T/64 + N) H / CUs)) chunks split the
    long one; both sequences against the oracle, every head."""
    lengths = [64 * 400, 100]
    x, cu = _packed(lengths, 32, 58)
    N, Tt = len(lengths), int(cu[-1])
    assert kda.lib().kda_chunk_fwd_varlen_workspace_size(N, Tt, 32, 128, 128, 1, 0) > 0
    print(f"case segmented varlen default lengths={lengths} H32", flush=True)
    o, S = _run(kda, x)
    _check_all(x, cu, o, S, False, True, "segmented varlen default")
