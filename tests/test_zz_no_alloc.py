"""kda_chunk_fwd_noalloc (the prefill entry point for callers that cannot
allocate) through the C ABI against kda_chunk_fwd with a caller workspace:
the same kernels and schedule, so the results must match bit for bit, and
both within the bf16 bounds of the oracle.  Two calls in a row, the second
smaller (the scratch keeps the first call's contents), then sizes beyond
the scratch, which are refused before any launch."""
import pytest
import torch

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


def _both(kda, inp):
    B, T, H, d = inp["q"].shape
    dt = 1 if inp["q"].dtype == torch.bfloat16 else 0
    need = kda.lib().kda_chunk_fwd_workspace_size(B, T, H, d, d, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    o1, S1 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], workspace=ws)
    o2 = torch.full_like(o1, float("nan"))
    S2 = torch.full_like(S1, float("nan"))
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], o=o2, S_T=S2)
    torch.cuda.synchronize()
    return need, (o1, S1), (o2, S2)


def test_noalloc_matches_workspace_entry_point(kda):
    # 1) the H16 T4K workload (segmented: its schedule needs scratch);
    # 2) a smaller, ragged case right after it, also segmented
    for cfg, kw in ((W.PREFILL_BF16_H16_T4K, {}), (W.PREFILL_BF16_H16_T4K, dict(T=64 * 13 + 17, H=3, seed=57))):
        inp = W.prefill_inputs(cfg, device="cuda", **kw)
        B, T, H, _ = inp["q"].shape
        print(f"case noalloc B{B} T{T} H{H}", flush=True)
        need, (o1, S1), (o2, S2) = _both(kda, inp)
        assert need > 0, "the case must take the segmented schedule"
        assert need <= 64 << 20
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
        o_ref, S_ref = oracle_prefill(inp)
        check_prefill(to64(o2), to64(S2), o_ref, S_ref, torch.bfloat16, f"noalloc B{B}T{T}H{H}")


def test_noalloc_fp32_d128(kda):
    """fp32 at d = 128 takes its chunk blocks from the scratch: two calls in a
    row, the second smaller, each equal to the workspace entry point's."""
    for B, T, H, seed in ((2, 300, 3, 61), (1, 70, 2, 62)):
        cfg = W.Prefill("kda_fwd_fp32_d128", B, T, H, 128, 128, torch.float32, 0.05)
        inp = W.prefill_inputs(cfg, device="cuda", seed=seed)
        print(f"case noalloc fp32 d128 B{B} T{T} H{H}", flush=True)
        need, (o1, S1), (o2, S2) = _both(kda, inp)
        assert 0 < need <= 64 << 20
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
        o_ref, S_ref = oracle_prefill(inp)
        check_prefill(to64(o2), to64(S2), o_ref, S_ref, torch.float32, f"noalloc fp32 d128 B{B}T{T}H{H}")


def test_noalloc_one_pass_needs_no_scratch(kda):
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda", B=2, T=200, H=3, seed=58)
    need, (o1, S1), (o2, S2) = _both(kda, inp)
    assert need == 0
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_noalloc_refuses_sizes_beyond_its_scratch(kda):
    # 128 heads of 131 072 tokens: the segmented schedule's workspace is more
    # than the 64 MiB scratch; the call is refused on the host (the pointers
    # below are never dereferenced: nothing is launched)
    import ctypes
    L = kda.lib()
    need = L.kda_chunk_fwd_workspace_size(1, 131072, 128, 128, 128, 1)
    assert need > 64 << 20
    p = ctypes.c_void_p(256)
    st = L.kda_chunk_fwd_noalloc(p, p, p, p, p, None, p, None, 1, 131072, 128, 128, 128, 1, None)
    assert st == -8, st
