#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill over the B=8, H=32, T=8192, d=128 bf16
workload (kda_chunk_fwd, S0 = 0, o bf16 + S_T fp32) followed by 64 decode
tokens for 256 sequences x 32 heads (kda_recurrent_step, fp32 state updated
in place).  Inputs are synthetic (seeded, see workloads/) and resident in HBM
before timing starts.  Prints ONE JSON line:
  value         prefill tokens/s (B*T tokens per prefill call)
  decode        decode tokens/s (256 sequences x 64 tokens per step) + roofline
  roofline      the fused prefill kernel against the HBM bound
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same work
--variant runs the same step for a variant of the recurrence (scalar gate,
no delta rule, or both) on the same shapes; the default is KDA itself.
--packed runs the prefill on the same 65 536 tokens x 32 heads cut into
variable-length sequences (geometric lengths, mean 1024, seeded) through
kda_varlen_schedule + kda_chunk_fwd_varlen.
After the step loop (KDA only) the line also carries the backward on the
B8 H32 T8192 workload, a training step on it (the forward that keeps the
chunk states, then the backward on them), the two other bf16 prefill
workloads timed alone
(B1 H16 T4096 with S0, the cache evicted before each call; B1 H32 T131072
with slow forgetting, segmented schedule) and a device-to-device copy as
the achievable-bandwidth reference.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, TFLOP/s

# Algorithmic work per token and head (d_k = d_v = 128, chunk 64, bf16 I/O):
#   bytes: q, k, v, g (4 x 256) + beta (2) + o (256) = 1282
#   flops: 6 d^2 + (C+1) 4d + (C-1) d + C^2/3 + d^2/C  (triangles counted once)
D = 128
C = 64
PREFILL_BYTES_PER_TOKHEAD = 4 * D * 2 + 2 + D * 2
PREFILL_FLOPS_PER_TOKHEAD = 6 * D * D + (C + 1) * 4 * D + (C - 1) * D + C * C / 3 + D * D / C
STATE_BYTES = D * D * 4
DECODE_BYTES_PER_HEAD = 2 * STATE_BYTES + PREFILL_BYTES_PER_TOKHEAD   # state read + write + token I/O

# Backward: reads q, k, v, g (4 x 256), beta 2, dO 256; writes dq, dk, dv, dg
# (4 x 256), dbeta 2 -- the chunk states and adjoints it keeps in a workspace
# are not part of the algorithmic bytes.
BWD_BYTES_PER_TOKHEAD = 4 * D * 2 + 2 + D * 2 + 4 * D * 2 + 2

# Variants: (scalar_gate, delta).  A scalar gate reads one bf16 per token and
# head instead of d_k; without the delta rule beta is not read.
VARIANTS = {"kda": (False, True), "scalar": (True, True), "nodelta": (False, False),
            "scalar-nodelta": (True, False)}


def tok_bytes(scalar_gate: bool, delta: bool) -> int:
    """Algorithmic HBM bytes per token and head: q, k, v, g, beta in, o out."""
    return 3 * D * 2 + (2 if scalar_gate else D * 2) + (2 if delta else 0) + D * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (used for profiler runs)")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default="kda",
                    help="recurrence variant (default: KDA)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward (kda_chunk_bwd) measurement")
    ap.add_argument("--packed", action="store_true",
                    help="prefill over variable-length packed sequences of the same tokens")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing the H16 T4K and H32 T128K prefill workloads after the step loop")
    ap.add_argument("--only", choices=["t4k", "t128k"], default=None,
                    help="time only that prefill workload (for profiler runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


# Sources each measured kernel is compiled from (its counter record is valid
# only while they are unchanged).
KERNEL_SOURCES = {
    "prefill": ["kda_prefill.hip", "kda_device.hpp", "kda_launch.hpp"],
    "decode": ["kda_decode.hip", "kda_device.hpp", "kda_launch.hpp"],
    "backward": ["kda_backward.hip", "kda_prefill.hip", "kda_device.hpp", "kda_launch.hpp"],
}


def source_digest(family: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_61_amd", "csrc")
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, family: str = None):
    """HBM bytes per launch (or per call, for a record that sums several
    launches) from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if family is None:
        family = "decode" if kernel.startswith("decode") else "prefill"
    if not rec or rec.get("source_digest") != source_digest(family):
        return None
    t = rec.get("bytes_per_launch", rec.get("bytes_per_call"))
    return None if t is None else float(t)


def cpu_baseline(W, oracle, torch, scalar_gate=False, delta=True):
    """The fp64 oracle on the prefill workload's inputs (all 8 x 32 sequences
    of 8192 tokens), timed on the host cores."""
    cfg = W.PREFILL_BF16_B8_H32_T8K
    inp = W.prefill_inputs(cfg, device="cuda", scalar_gate=scalar_gate)
    f64 = lambda t: None if t is None else t.detach().cpu().double().numpy()
    args = [f64(inp[n]) for n in ("q", "k", "v", "g", "beta", "S0")]
    del inp
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.recurrent_fwd(*args, nthreads=threads, scalar_gate=scalar_gate, delta=delta)
    dt = time.perf_counter() - t0
    tokens = cfg.B * cfg.T
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpus_usable": affinity, "omp_threads": threads,
            "sample": f"the whole prefill workload (B={cfg.B}, H={cfg.H}, T={cfg.T}, d=128) once, "
                      f"fp64 token recurrence, {dt:.1f} s wall"}


def time_prefill_workload(kda, torch, cfg, iters, evict=None):
    """kda_chunk_fwd on one of the prefill workloads at full size, with the
    workspace its fastest schedule asks for: the median of `iters` calls, each
    timed alone with events on the launch stream.  evict: a device buffer
    written before every call (not timed), so that the inputs do not sit in
    the 256 MB last-level cache from the previous call."""
    import workloads as W
    inp = W.prefill_inputs(cfg, device="cuda")
    o = torch.empty_like(inp["v"])
    S_T = torch.empty(cfg.B, cfg.H, D, D, dtype=torch.float32, device="cuda")
    ws_bytes = kda.lib().kda_chunk_fwd_workspace_size(cfg.B, cfg.T, cfg.H, D, D, 1)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], o=o, S_T=S_T, workspace=ws)

    for _ in range(2):
        run()
    ms = []
    for _ in range(iters):
        if evict is not None:
            evict.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    med = ms[len(ms) // 2]
    BTH = cfg.B * cfg.T * cfg.H
    nbytes = BTH * PREFILL_BYTES_PER_TOKHEAD + cfg.B * cfg.H * STATE_BYTES * (2 if cfg.s0_std is not None else 1)
    gbs = nbytes / (med * 1e-3) / 1e9
    nseg = kda.lib().kda_chunk_fwd_workspace_size(cfg.B, cfg.T, cfg.H, D, D, 1) // max(cfg.B * cfg.H * 3 * STATE_BYTES, 1)
    del inp, o, S_T, ws
    return {"workload": f"kda_chunk_fwd B{cfg.B} H{cfg.H} T{cfg.T} d128 bf16"
                        + (" (S0 ~ N(0, 0.02))" if cfg.s0_std is not None else " (S0=0)")
                        + (f", log-gate mean mu={cfg.gate_mu:g}" if cfg.gate_mu != -3.0 else ""),
            "schedule": f"segmented, {nseg} segments" if nseg >= 3 else "one pass",
            "cache": "evicted before each call (1 GiB written)" if evict is not None else "warm",
            "ms": med, "ms_all": ms, "value": cfg.B * cfg.T / (med * 1e-3), "unit": "tokens/s",
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
                         "traffic": (measured_traffic(f"prefill_segmented[B{cfg.B} H{cfg.H} T{cfg.T}]")
                                     if nseg >= 3 else None),
                         "mfma_frac_algorithmic": BTH * PREFILL_FLOPS_PER_TOKHEAD / (med * 1e-3) / 1e12
                                                  / BF16_PEAK_TFLOPS}}


def copy_reference(torch, stream, nbytes=1 << 30, iters=5):
    """Bandwidth of a plain device-to-device copy (read + write bytes / time),
    the achievable-bandwidth reference beside the 8 TB/s peak."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        y.copy_(x)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del x, y
    return {"bytes_moved": 2 * nbytes, "ms": ms, "achieved_gbs": 2 * nbytes / (ms * 1e-3) / 1e9}


def measure_backward(kda, W, torch, pcfg, inp, args, stream):
    """kda_chunk_bwd on the prefill workload (adjoints dO ~ N(0,1) bf16,
    dS_T = 0), timed alone with events on the launch stream."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12345)
    dO = torch.randn(pcfg.B, pcfg.T, pcfg.H, D, device="cuda", generator=gen).to(torch.bfloat16)
    ws = torch.empty(kda.lib().kda_chunk_bwd_workspace_size(pcfg.B, pcfg.T, pcfg.H, D, D, 1),
                     dtype=torch.uint8, device="cuda")

    def bwd():
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], dO, None, want_dS0=False,
                      workspace=ws)

    for _ in range(max(args.warmup, 1)):
        bwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    BTH = pcfg.B * pcfg.T * pcfg.H
    alg = BTH * BWD_BYTES_PER_TOKHEAD
    gbs = alg / (ms * 1e-3) / 1e9
    del ws, dO
    return {"value": pcfg.B * pcfg.T / (ms * 1e-3), "unit": "tokens/s", "ms": ms,
            "workload": "kda_chunk_bwd B8 H32 T8192 d128 bf16 (S0=0, dS_T=0)",
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("backward", "backward"),
                         "kernel": "the whole backward: state pass (fused_pipe_kernel<4>) + bwd_prep_kernel + bwd_chain_kernel + bwd_grad_kernel"}}


def measure_train_step(kda, W, torch, pcfg, inp, args, stream):
    """One training step of the layer on the prefill workload: the forward
    that keeps the chunk states for its backward (kda_chunk_fwd_save) and the
    backward on them (KDA_STATES_SAVED), timed together with events."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12345)
    dO = torch.randn(pcfg.B, pcfg.T, pcfg.H, D, device="cuda", generator=gen).to(torch.bfloat16)
    ws = torch.empty(kda.lib().kda_chunk_bwd_workspace_size(pcfg.B, pcfg.T, pcfg.H, D, D, 1),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(inp["v"])
    S_T = torch.empty(pcfg.B, pcfg.H, D, D, dtype=torch.float32, device="cuda")

    def step():
        kda.chunk_fwd_save(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], o=o, S_T=S_T,
                           workspace=ws)
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], dO, None, want_dS0=False,
                      workspace=ws, states_saved=True)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    del ws, dO, o, S_T
    return {"value": pcfg.B * pcfg.T / (ms * 1e-3), "unit": "tokens/s", "ms": ms,
            "workload": "kda_chunk_fwd_save + kda_chunk_bwd_ex(KDA_STATES_SAVED) B8 H32 T8192 d128 bf16 "
                        "(S0=0, dS_T=0)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the kernels here are "
              "one GPU's share of a head-sharded job and have no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        x.fill_(1.0)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4}))
        return
    import gated_delta_rule_61_amd as kda
    import workloads as W

    if not os.path.exists(kda.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.only is not None:
        cfg = W.PREFILL_BF16_H16_T4K if args.only == "t4k" else W.PREFILL_BF16_LONG_T128K
        print(json.dumps(time_prefill_workload(kda, torch, cfg, args.steps)), flush=True)
        return

    scalar_gate, delta = VARIANTS[args.variant]
    flags = (1 if scalar_gate else 0) | (0 if delta else 2)
    pcfg = W.PREFILL_BF16_B8_H32_T8K
    dcfg = W.DECODE_256x32
    inp = W.prefill_inputs(pcfg, device="cuda", scalar_gate=scalar_gate)
    o = torch.empty_like(inp["v"])
    S_T = torch.empty(pcfg.B, pcfg.H, D, D, dtype=torch.float32, device="cuda")
    S = W.decode_state(dcfg, device="cuda")
    tok = W.decode_tokens(dcfg, device="cuda", scalar_gate=scalar_gate)
    if not delta:
        inp["beta"] = tok["beta"] = None
    steps_tok = [[None if tok[n] is None else tok[n][t] for n in ("q", "k", "v", "g", "beta")]
                 for t in range(dcfg.steps)]
    od = torch.empty(dcfg.N, dcfg.H, D, dtype=torch.bfloat16, device="cuda")
    vkw = dict(scalar_gate=scalar_gate, delta=delta)
    ws_bytes = kda.lib().kda_chunk_fwd_ex_workspace_size(pcfg.B, pcfg.T, pcfg.H, D, D, 1, flags)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def prefill():
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], o=o, S_T=S_T,
                      workspace=ws, **vkw)

    n_states = pcfg.B * pcfg.H
    if args.packed:
        lengths = W.packed_lengths(pcfg.B * pcfg.T, 1024.0, seed=11)
        cu_host = [0]
        for n in lengths:
            cu_host.append(cu_host[-1] + n)
        cu = torch.tensor(cu_host, dtype=torch.int32, device="cuda")
        flat = lambda t: None if t is None else t.reshape(pcfg.B * pcfg.T, pcfg.H, *t.shape[3:])
        pk = {n: flat(inp[n]) for n in ("q", "k", "v", "g", "beta")}
        o_flat = o.view(pcfg.B * pcfg.T, pcfg.H, D)
        S_T = torch.empty(len(lengths), pcfg.H, D, D, dtype=torch.float32, device="cuda")
        n_states = len(lengths) * pcfg.H

        order = torch.empty(len(lengths), dtype=torch.int32, device="cuda")

        def prefill():
            # the longest-first order is recomputed every step (it is timed)
            kda.varlen_schedule(cu, pcfg.B * pcfg.T, out=order)
            kda.chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], cu, None, seq_order=order,
                                 o=o_flat, S_T=S_T, **vkw)

    S_saved = S.clone()

    def decode():
        for t in range(dcfg.steps):
            kda.recurrent_step(*steps_tok[t], S, o=od, **vkw)

    for _ in range(args.warmup):
        prefill()
        S.copy_(S_saved)
        decode()
    torch.cuda.synchronize()

    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for e0, e1, e2, e3 in ev:
        e0.record(stream)
        prefill()
        e1.record(stream)
        # every timed decode run starts from the same state (the restore is
        # inside the step's wall time but outside both kernels' events)
        S.copy_(S_saved)
        e2.record(stream)
        decode()
        e3.record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    pre_ms = [e0.elapsed_time(e1) for e0, e1, _, _ in ev]
    dec_ms = [e2.elapsed_time(e3) for _, _, e2, e3 in ev]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)

    BTH = pcfg.B * pcfg.T * pcfg.H
    pre_bytes = BTH * tok_bytes(scalar_gate, delta) + n_states * STATE_BYTES   # + S_T write
    pre_flops = BTH * PREFILL_FLOPS_PER_TOKHEAD
    pre_gbs = pre_bytes / (pre_avg * 1e-3) / 1e9
    step_heads = dcfg.N * dcfg.H
    dec_step_ms = dec_avg / dcfg.steps
    dec_gbs = step_heads * (2 * STATE_BYTES + tok_bytes(scalar_gate, delta)) / (dec_step_ms * 1e-3) / 1e9
    pkn = "fused_pipe_kernel" if flags == 0 else f"fused_pipe_kernel<{flags}>"
    dk_name = "decode_kernel" if flags == 0 else f"decode_kernel<{flags}>"
    vname = {"kda": "", "scalar": " [scalar gate]", "nodelta": " [no delta rule]",
             "scalar-nodelta": " [scalar gate, no delta rule]"}[args.variant]

    def traffic(kernel):
        t = measured_traffic(kernel)
        return None if t is None else float(t)

    line = {
        "metric": "KDA prefill tokens/s and decode tokens/s, % of MFMA/HBM roofline",
        "value": pcfg.B * pcfg.T / (pre_avg * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta=sigmoid(N(0,1)), "
                "g=-softplus(N(-3,1)))",
        "config": {"workload": ((f"kda_chunk_fwd_varlen {n_states // pcfg.H} packed sequences "
                                 f"(geometric lengths, mean 1024) = 65536 tokens H32 d128 bf16 (S0=0) + ")
                                if args.packed else "kda_chunk_fwd B8 H32 T8192 d128 bf16 (S0=0) + ")
                               + "kda_recurrent_step 256x32 d128 x64 tokens" + vname,
                   "prefill_ms": pre_avg, "decode_ms_per_token_step": dec_step_ms},
        "roofline": {"bound": "hbm", "achieved": pre_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pre_gbs / HBM_PEAK_GBS, "traffic": traffic(pkn + ("[packed]" if args.packed else "")),
                     "kernel": pkn + " (bf16, d_k = d_v = 128)",
                     "mfma_frac_algorithmic": (pre_flops / (pre_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
                                               if flags == 0 else None)},
        "decode": {"value": dcfg.N * dcfg.steps / (dec_avg * 1e-3), "unit": "tokens/s",
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_gbs / HBM_PEAK_GBS, "traffic": traffic(dk_name),
                                "kernel": dk_name + " (bf16, 128 x 128)"}},
    }
    line["decode"]["state_restored_before_each_timed_run"] = True
    if not args.no_backward and flags == 0 and not args.packed:
        line["backward"] = measure_backward(kda, W, torch, pcfg, inp, args, stream)
        line["train_step"] = measure_train_step(kda, W, torch, pcfg, inp, args, stream)
    del inp, o, S, S_saved, tok, steps_tok
    if flags == 0 and not args.packed and not args.no_other_configs:
        # the other two prefill workloads, each timed alone after the step loop
        evict = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        line["prefill_B1_H16_T4096"] = time_prefill_workload(kda, torch, W.PREFILL_BF16_H16_T4K, 20, evict)
        del evict
        line["prefill_B1_H32_T131072"] = time_prefill_workload(kda, torch, W.PREFILL_BF16_LONG_T128K, 5)
        line["copy_reference"] = copy_reference(torch, stream)
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline(W, oracle, torch, scalar_gate, delta)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
