"""Benchmark of the Gated DeltaNet mixer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu-baseline]
                    [--copy-probe] [--decode-only]

One step = one gdn_prefill call over the whole batch of the headline workload
(default: the Qwen3.8-27B-shaped layer, B=1, T=262,144, 16 key / 48 value heads:
conv, L2 norm, gated delta rule over 4,096 chunks, gated RMSNorm), inputs already
resident in HBM.  Prints ONE JSON line.  `value` is prefill tokens/s of the layer;
mean, median and min per call are reported, and the workspace error word of every
input set is checked after the timed loop (a nonzero word fails the run).  The
roofline object carries the achieved algorithmic HBM bandwidth of the call, the
counter-measured HBM traffic and issued MFMA work of the same call (from the
committed counter summary, while the kernel sources still hash to the value it
records), and the useful-FLOP fraction of MFMA peak.  `detail` carries the other
prefill shapes (the 0.8B- and 4B-shaped layers, the tiny T=64 case in
microseconds), the decode step on the 27B-shaped B=256 batch (state GB/s, % of
HBM) and the same batch checking two tokens per sequence, the 4B-shaped layer's
tokens as 16 packed sequences, one GPU's share of the 27B-shaped layer under
16-way key-head sharding (two-level scan beside the plain sequential pass), and
the gate-logit entry point.  `cpu_baseline` is the fp64 CPU oracle timed on this
host on a bounded sample of the headline workload (a reported baseline, not a
target).

Inputs are synthetic and seeded (torch's generator on the GPU for the timed
runs, gdn_inputs for the CPU baseline) with the distributions of the pages'
workloads.  Several input sets are rotated when one set would fit in the
256 MB Infinity Cache, so the timed steps read from HBM.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_FP16_PEAK = 2.5e15    # FLOP/s dense fp16 / bf16 MFMA
D = 128
C = 64
# useful FLOPs per token per value head of the chunked form (triangles counted half):
# 6 d^2 + 5 C d + C^2 / 3
USEFUL_FLOP_PER_TOKEN_HEAD = 6 * D * D + 5 * C * D + C * C / 3

WORKLOADS = {
    # name: (B, T, Hk, Hv)
    "tiny_T64": (1, 64, 1, 1),  # no conv, no gated norm
    "qwen35_0p8b_prefill_T4096": (1, 4096, 16, 16),
    "qwen35_4b_prefill_B4_T16384": (4, 16384, 16, 32),
    "qwen38_27b_prefill_T262144": (1, 262144, 16, 48),
}
DECODE = ("qwen38_27b_decode_B256", (256, 16, 48))
NO_CONV_NORM = {"tiny_T64"}
HEADLINE = "qwen38_27b_prefill_T262144"
# packed sequences: the 4B-shaped layer's 65536 tokens as 16 sequences of mixed lengths
PACKED = ("qwen35_4b_prefill_packed_16seq_T65536", (16, 65536, 16, 32))


def packed_lengths(n, total, seed=3000):
    """n seeded sequence lengths summing to total, spread over a 1:8 range of weights."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([20261202, seed])))
    w = rng.uniform(0.25, 2.0, size=n)
    lens = np.maximum(1, np.floor(w / w.sum() * total)).astype(np.int64)
    lens[-1] += total - lens.sum()
    return lens.tolist()


def prefill_bytes(B, T, Hk, Hv, fused=True) -> int:
    """Algorithmic HBM bytes of one prefill: raw q,k; v, z, o; g, beta; final state;
    conv weights and conv tail (zero initial state and conv state are not read).
    Without conv and gated norm (the tiny case): no z, conv weights or conv tail."""
    Cc = 2 * Hk * D + Hv * D
    if not fused:
        return B * T * (2 * Hk * D * 2 + 2 * Hv * D * 2 + Hv * 8) + B * Hv * D * D * 4
    per_tok = 2 * Hk * D * 2 + 3 * Hv * D * 2 + Hv * 8
    return B * T * per_tok + B * Hv * D * D * 4 + Cc * 4 * 2 + B * 3 * Cc * 2 + D * 2


def decode_bytes(B, Hk, Hv) -> int:
    """Algorithmic HBM bytes of one decode step: state read + write, conv state
    read + write, q,k,v,z,g,beta in, o out, weights."""
    Cc = 2 * Hk * D + Hv * D
    return (2 * B * Hv * D * D * 4 + 2 * B * 3 * Cc * 2 + B * Hk * D * 2 * 2 + B * Hv * D * 2 * 3
            + B * Hv * 8 + Cc * 4 * 2 + D * 2)


def _gen(torch, gen, shape, kind):
    dev = "cuda"
    if kind == "normal_bf16":
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    if kind == "g":
        u = torch.rand(shape, generator=gen, device=dev, dtype=torch.float64) * (0.999 - 0.8) + 0.8
        return torch.log(u).to(torch.float32)
    if kind == "beta":
        return torch.sigmoid(torch.randn(shape, generator=gen, device=dev, dtype=torch.float64)).to(torch.float32)
    raise ValueError(kind)


def make_prefill_set(torch, gdn, B, T, Hk, Hv, seed, conv=True, norm=True, segments=0):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    Cc = 2 * Hk * D + Hv * D
    d = dict(
        q=_gen(torch, gen, (B, T, Hk, D), "normal_bf16"),
        k=_gen(torch, gen, (B, T, Hk, D), "normal_bf16"),
        v=_gen(torch, gen, (B, T, Hv, D), "normal_bf16"),
        z=_gen(torch, gen, (B, T, Hv, D), "normal_bf16"),
        g=_gen(torch, gen, (B, T, Hv), "g"),
        beta=_gen(torch, gen, (B, T, Hv), "beta"),
        conv_w=(torch.randn((Cc, 4), generator=gen, device="cuda") * 0.5).to(torch.bfloat16),
        norm_w=(1.0 + 0.02 * torch.randn((D,), generator=gen, device="cuda")).to(torch.bfloat16),
    )
    d["o"] = torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device="cuda")
    d["state_out"] = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    d["conv_state_out"] = torch.empty((B, 3, Cc), dtype=torch.bfloat16, device="cuda")
    if not conv:  # no conv: the boundary takes no conv weights and returns no conv tail
        d["conv_w"] = d["conv_state_out"] = None
    shape = gdn.make_shape(B, T, Hk, Hv, conv=conv, norm=norm, segments=segments)
    nws = gdn.gdn_prefill_workspace_size(shape)
    d["ws"] = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    d["shape"] = shape
    return d


def run_prefill(gdn, d):
    gdn.gdn_prefill(d["shape"], d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"], d["conv_w"], d["norm_w"],
                    None, None, d["o"], d["state_out"], d["conv_state_out"], d["ws"])


def add_gate_logits(torch, d, Hv, seed):
    """Gate logits in place of g and beta: a, b ~ N(0, 1), A_log = ln U(1, 16), dt_bias ~ U(-6.9, -2.3)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    d["a"] = torch.randn(d["g"].shape, generator=gen, device="cuda")
    d["b"] = torch.randn(d["beta"].shape, generator=gen, device="cuda")
    d["A_log"] = torch.log(torch.rand((Hv,), generator=gen, device="cuda") * 15.0 + 1.0)
    d["dt_bias"] = torch.rand((Hv,), generator=gen, device="cuda") * 4.6 - 6.9


def run_prefill_gate_logits(gdn, d):
    gdn.gdn_prefill_gate_logits(d["shape"], d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                d["z"], d["conv_w"], d["norm_w"], None, None, d["o"], d["state_out"],
                                d["conv_state_out"], d["ws"])


def time_calls(torch, fn, sets, steps, warmup):
    """Per-call times in ms over `steps` back-to-back calls (cycling the input sets), from
    HIP events recorded on the current stream (the stream the library launches on) between
    the calls, bracketed by device syncs.  Returns (mean, median, min, wall seconds)."""
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn(sets[i % len(sets)])
        ev[i + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mean = ev[0].elapsed_time(ev[steps]) / steps
    return mean, per[len(per) // 2], per[0], t_wall


def check_sets(gdn, sets):
    """The workspace error word of every input set after the timed calls: a timed-out wait
    between workgroups or a skipped packed sequence fails the run."""
    for d in sets:
        gdn.gdn_prefill_check(d["ws"])


def bench_prefill(torch, gdn, name, steps, warmup, gate_logits=False):
    B, T, Hk, Hv = WORKLOADS[name]
    fused = name not in NO_CONV_NORM
    per_set = prefill_bytes(B, T, Hk, Hv) + B * T * Hk * 2 * D * 2
    nsets = max(1, min(4, math.ceil(320e6 / per_set)))  # rotate past the 256 MB Infinity Cache
    sets = [make_prefill_set(torch, gdn, B, T, Hk, Hv, seed=1000 + i, conv=fused, norm=fused) for i in range(nsets)]
    if gate_logits:
        for i, d in enumerate(sets):
            add_gate_logits(torch, d, Hv, seed=2000 + i)
    torch.cuda.synchronize()
    run = run_prefill_gate_logits if gate_logits else run_prefill
    ms, med, mn, wall = time_calls(torch, lambda d: run(gdn, d), sets, steps, warmup)
    check_sets(gdn, sets)
    nbytes = prefill_bytes(B, T, Hk, Hv, fused)
    flops = USEFUL_FLOP_PER_TOKEN_HEAD * B * T * Hv
    res = {
        "workload": name + (" (gdn_prefill_gate_logits)" if gate_logits else ""), "B": B, "T": T, "Hk": Hk,
        "Hv": Hv, "conv_and_norm": fused, "ms_per_call": ms, "ms_median": med, "ms_min": mn,
        "tokens_per_s": B * T / (ms * 1e-3), "algorithmic_bytes": nbytes,
        "hbm_GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK,
        "useful_TFLOPs": flops / (ms * 1e-3) / 1e12, "mfma_useful_frac": flops / (ms * 1e-3) / MFMA_FP16_PEAK,
        "roof_frac": max(nbytes / HBM_PEAK, flops / MFMA_FP16_PEAK) / (ms * 1e-3),
        "input_sets": nsets, "steps": steps, "wall_s": wall, "error_word": 0,
    }
    if name in NO_CONV_NORM:
        res["us_per_call"] = ms * 1e3
    del sets
    torch.cuda.empty_cache()
    return res


def bench_prefill_packed(torch, gdn, steps, warmup):
    """One gdn_prefill_packed call over the 4B-shaped layer's tokens, split into
    sequences of mixed lengths (each restarts its state and conv window)."""
    name, (N, T, Hk, Hv) = PACKED
    lens = packed_lengths(N, T)
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32, device="cuda")
    Cc = 2 * Hk * D + Hv * D
    d = make_prefill_set(torch, gdn, 1, T, Hk, Hv, seed=1100)
    d["state_out"] = torch.empty((N, Hv, D, D), dtype=torch.float32, device="cuda")
    d["conv_state_out"] = torch.empty((N, 3, Cc), dtype=torch.bfloat16, device="cuda")
    d["shape"] = gdn.make_shape(N, T, Hk, Hv, packed=True)
    d["ws"] = torch.zeros(gdn.gdn_prefill_workspace_size(d["shape"]), dtype=torch.uint8, device="cuda")
    d["cu"] = cu
    torch.cuda.synchronize()

    def run(dd):
        gdn.gdn_prefill_packed(dd["shape"], dd["cu"], dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["z"],
                               dd["conv_w"], dd["norm_w"], None, None, dd["o"], dd["state_out"],
                               dd["conv_state_out"], dd["ws"])
    ms, med, mn, wall = time_calls(torch, run, [d], steps, warmup)
    check_sets(gdn, [d])
    # per-token bytes as the even batch; one final state and conv tail per sequence
    nbytes = prefill_bytes(1, T, Hk, Hv) + (N - 1) * (Hv * D * D * 4 + 3 * Cc * 2)
    flops = USEFUL_FLOP_PER_TOKEN_HEAD * T * Hv
    res = {
        "workload": name + " (gdn_prefill_packed)", "sequences": N, "T_total": T, "Hk": Hk, "Hv": Hv,
        "lengths_min_max": [min(lens), max(lens)], "ms_per_call": ms, "ms_median": med, "ms_min": mn,
        "tokens_per_s": T / (ms * 1e-3),
        "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / (ms * 1e-3) / 1e9,
        "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK, "useful_TFLOPs": flops / (ms * 1e-3) / 1e12,
        "mfma_useful_frac": flops / (ms * 1e-3) / MFMA_FP16_PEAK, "steps": steps, "wall_s": wall,
    }
    del d
    torch.cuda.empty_cache()
    return res


# one GPU's share of the 27B-shaped layer under 16-way key-head sharding: 1 key head, its 3 value heads
SHARD = ("qwen38_27b_prefill_T262144_keyhead_shard_1of16", (1, 262144, 1, 3))


def bench_prefill_shard(torch, gdn, steps, warmup):
    """The few-heads, long-sequence shape the two-level scan is for, timed as the library
    plans it (segments) and, for comparison, with the plain sequential pass forced through
    the shape's prefill_segments field (1)."""
    name, (B, T, Hk, Hv) = SHARD
    out = {"workload": name, "B": B, "T": T, "Hk": Hk, "Hv": Hv}
    for leg, segments in (("plain_sequential", 1), ("planned", 0)):
        d = make_prefill_set(torch, gdn, B, T, Hk, Hv, seed=1200, segments=segments)
        torch.cuda.synchronize()
        ms, med, mn, _ = time_calls(torch, lambda dd: run_prefill(gdn, dd), [d], steps, warmup)
        check_sets(gdn, [d])
        out[leg + "_ms_per_call"] = ms
        out[leg + "_ms_min"] = mn
        out[leg + "_workspace_MiB"] = d["ws"].numel() / 2 ** 20
        del d
        torch.cuda.empty_cache()
    ms = out["planned_ms_per_call"]
    nbytes = prefill_bytes(B, T, Hk, Hv)
    flops = USEFUL_FLOP_PER_TOKEN_HEAD * B * T * Hv
    out.update(tokens_per_s=B * T / (ms * 1e-3), algorithmic_bytes=nbytes, hbm_frac=nbytes / (ms * 1e-3) / HBM_PEAK,
               mfma_useful_frac=flops / (ms * 1e-3) / MFMA_FP16_PEAK,
               speedup_over_plain=out["plain_sequential_ms_per_call"] / ms, steps=steps)
    return out


def bench_decode(torch, gdn, steps, warmup):
    B, Hk, Hv = DECODE[1]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    Cc = 2 * Hk * D + Hv * D
    d = dict(
        q=_gen(torch, gen, (B, Hk, D), "normal_bf16"), k=_gen(torch, gen, (B, Hk, D), "normal_bf16"),
        v=_gen(torch, gen, (B, Hv, D), "normal_bf16"), z=_gen(torch, gen, (B, Hv, D), "normal_bf16"),
        g=_gen(torch, gen, (B, Hv), "g"), beta=_gen(torch, gen, (B, Hv), "beta"),
        conv_w=(torch.randn((Cc, 4), generator=gen, device="cuda") * 0.5).to(torch.bfloat16),
        norm_w=(1.0 + 0.02 * torch.randn((D,), generator=gen, device="cuda")).to(torch.bfloat16),
        state=torch.randn((B, Hv, D, D), generator=gen, device="cuda") * 0.1,
        conv_state=_gen(torch, gen, (B, 3, Cc), "normal_bf16"),
        o=torch.empty((B, Hv, D), dtype=torch.bfloat16, device="cuda"),
    )
    shape = gdn.make_shape(B, 1, Hk, Hv)

    def fn(dd):
        gdn.gdn_decode_step(shape, dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["z"], dd["conv_w"],
                            dd["norm_w"], dd["state"], dd["conv_state"], dd["o"])
    ms, med, mn, wall = time_calls(torch, fn, [d], steps, warmup)
    nbytes = decode_bytes(B, Hk, Hv)
    state_bytes = 2 * B * Hv * D * D * 4
    res = {"workload": DECODE[0], "B": B, "Hk": Hk, "Hv": Hv, "us_per_step": ms * 1e3,
           "us_median": med * 1e3, "us_min": mn * 1e3,
           "tokens_per_s": B / (ms * 1e-3), "algorithmic_bytes": nbytes,
           "hbm_GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK,
           "state_GBps": state_bytes / (ms * 1e-3) / 1e9, "steps": steps}
    del d
    torch.cuda.empty_cache()
    return res


def decode_multi_bytes(B, T, Hk, Hv) -> int:
    """Algorithmic HBM bytes of one T-token decode call with snapshots: the state read once and
    written T times (T - 1 snapshots and the final state), the conv window read once and written
    T times, T tokens of q,k,v,z,g,beta in and of o out, weights."""
    Cc = 2 * Hk * D + Hv * D
    return ((1 + T) * B * Hv * D * D * 4 + (1 + T) * B * 3 * Cc * 2
            + T * (B * Hk * D * 2 * 2 + B * Hv * D * 2 * 3 + B * Hv * 8) + Cc * 4 * 2 + D * 2)


def bench_decode_multi(torch, gdn, steps, warmup, T=2):
    """The 27B-shaped decode batch checking T tokens per sequence in one gdn_decode_multi call,
    with state and conv snapshots after every token but the last."""
    B, Hk, Hv = DECODE[1]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(78)
    Cc = 2 * Hk * D + Hv * D
    d = dict(
        q=_gen(torch, gen, (B, T, Hk, D), "normal_bf16"), k=_gen(torch, gen, (B, T, Hk, D), "normal_bf16"),
        v=_gen(torch, gen, (B, T, Hv, D), "normal_bf16"), z=_gen(torch, gen, (B, T, Hv, D), "normal_bf16"),
        g=_gen(torch, gen, (B, T, Hv), "g"), beta=_gen(torch, gen, (B, T, Hv), "beta"),
        conv_w=(torch.randn((Cc, 4), generator=gen, device="cuda") * 0.5).to(torch.bfloat16),
        norm_w=(1.0 + 0.02 * torch.randn((D,), generator=gen, device="cuda")).to(torch.bfloat16),
        state=torch.randn((B, Hv, D, D), generator=gen, device="cuda") * 0.1,
        conv_state=_gen(torch, gen, (B, 3, Cc), "normal_bf16"),
        o=torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device="cuda"),
        state_snaps=torch.empty((T - 1, B, Hv, D, D), device="cuda"),
        conv_snaps=torch.empty((T - 1, B, 3, Cc), dtype=torch.bfloat16, device="cuda"),
    )
    shape = gdn.make_shape(B, T, Hk, Hv)

    def fn(dd):
        gdn.gdn_decode_multi(shape, dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["z"], dd["conv_w"],
                             dd["norm_w"], dd["state"], dd["conv_state"], dd["o"], dd["state_snaps"],
                             dd["conv_snaps"])
    ms, med, mn, wall = time_calls(torch, fn, [d], steps, warmup)
    nbytes = decode_multi_bytes(B, T, Hk, Hv)
    res = {"workload": f"{DECODE[0]} checking T={T} tokens per sequence (gdn_decode_multi, snapshots)",
           "B": B, "T": T, "Hk": Hk, "Hv": Hv, "us_per_call": ms * 1e3, "tokens_per_s": B * T / (ms * 1e-3),
           "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK, "steps": steps}
    del d
    torch.cuda.empty_cache()
    return res


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, target_s=15.0, min_s=10.0):
    """The fp64 oracle (as it stands) on this host's cores, on a bounded sample of the
    headline workload: every (sequence, value-head) chain of the layer over its first Ts
    tokens, Ts sized from a one-chain calibration so that one pass takes about `target_s`
    seconds with all threads, repeated until `min_s` seconds have passed.  The recurrence
    does the same work for every token, so chain-tokens per second over the sample is the
    oracle's rate for the whole layer; the sample's inputs are drawn with the workload's
    distributions under a seed tag of their own."""
    import gdn_inputs as GI
    from oracle import oracle as O
    w = GI.WORKLOADS[name]
    threads = O.num_threads()
    nchains = w.B * w.Hv
    cal = GI.Workload(name + "_calibration", 1, min(1024, w.T), w.Hk, w.Hv, conv=w.conv, norm=w.norm, tag=w.tag + 200)
    ci = GI.make_inputs(cal)
    t = time.perf_counter()
    O.prefill(ci, 1, cal.T, w.Hk, w.Hv, w.conv, w.norm, chains=[0], threads=1, want_conv_state=False)
    per_chain_token = (time.perf_counter() - t) / cal.T
    used = max(1, min(threads, nchains))
    Ts = int(target_s * used / (nchains * per_chain_token))
    Ts = max(64, min(w.T, Ts // 64 * 64))
    sample = GI.Workload(name + "_sample", w.B, Ts, w.Hk, w.Hv, conv=w.conv, norm=w.norm, tag=w.tag + 100)
    inp = GI.make_inputs(sample)
    reps, el = 0, 0.0
    t = time.perf_counter()
    while reps == 0 or (el < min_s and reps < 200):
        O.prefill(inp, w.B, Ts, w.Hk, w.Hv, w.conv, w.norm, threads=threads, want_conv_state=False)
        reps += 1
        el = time.perf_counter() - t
    # tokens/s of the layer = chain-tokens/s divided by the layer's Hv chains per token
    return {"value": reps * nchains * Ts / el / w.Hv, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"all {nchains} (sequence, value-head) chains of {name} over their first {Ts} of {w.T} "
                      f"tokens, {reps} pass(es), {el:.1f} s wall; fp64 C oracle (conv, L2 norm, token-by-token "
                      f"recurrence, gated RMSNorm) with OpenMP over chains",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}


# Counter summaries taken with rocprofv3 on one MI355X (profiles/), per headline workload.
COUNTER_FILES = {"qwen38_27b_prefill_T262144": "profiles/prefill_qwen38_27b_T262144_counters.txt"}


def measured_counters(name):
    """Per-call figures of the committed counter summary of this workload (HBM traffic
    from FETCH_SIZE / WRITE_SIZE scaled by the copy-probe factors, issued MFMA work and
    MFMA-busy cycles), or None when there is none or the kernel sources changed since it
    was taken."""
    import hashlib
    rel = COUNTER_FILES.get(name)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    rec = {}
    for line in open(os.path.join(ROOT, rel)):
        if ":" in line:
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if not all(k in rec for k in ("traffic_bytes_per_call", "sources_sha256", "sources")):
        return None
    h = hashlib.sha256()
    for src in rec["sources"].split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    out = {"traffic": int(rec["traffic_bytes_per_call"])}
    for k in ("mfma_issued_flop_per_call", "mfma_busy_cycles_per_call", "calibration"):
        if k in rec:
            out[k] = rec[k] if k == "calibration" else float(rec[k])
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-extra", action="store_true", help="skip decode and the other prefill shapes")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the 27B-shaped B=256 decode step and print its record (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy three times (calibrates HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the mixer path here has no "
              "multi-GPU mode.", file=sys.stderr)
        return 2

    import torch
    import gated_deltanet_mixer_amd as gdn
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if args.decode_only:
        print(json.dumps({"decode": bench_decode(torch, gdn, args.steps, args.warmup)}), flush=True)
        return 0
    head = bench_prefill(torch, gdn, args.workload, args.steps, args.warmup)
    extra = {}
    if not args.no_extra:
        extra["decode"] = bench_decode(torch, gdn, max(20, args.steps // 4), 5)
        extra["decode_multi_T2"] = bench_decode_multi(torch, gdn, max(20, args.steps // 4), 5)
        for name in WORKLOADS:
            if name != args.workload:
                B, T, Hk, Hv = WORKLOADS[name]
                steps = max(3, min(200, int(2e8 // (B * T * Hv))))
                extra[name] = bench_prefill(torch, gdn, name, steps, 2)
        # few heads, long sequence: the two-level scan against the plain sequential pass
        extra[SHARD[0]] = bench_prefill_shard(torch, gdn, 5, 1)
        # the 4B-shaped layer's tokens as packed sequences of mixed lengths
        extra[PACKED[0]] = bench_prefill_packed(torch, gdn, 20, 2)
        # the same layer through the entry point that takes the gate logits
        extra[args.workload + "_gate_logits"] = bench_prefill(torch, gdn, args.workload, max(10, args.steps // 4), 3,
                                                              gate_logits=True)
    B, T, Hk, Hv = WORKLOADS[args.workload]
    ctr = measured_counters(args.workload)
    ms = head["ms_per_call"]
    roof = {
        "kernel": "one gdn_prefill call: chunk_prep_kernel then pass_kernel on the caller's stream, timed "
                  "together with HIP events on that stream",
        "bound": "hbm", "achieved": head["hbm_GBps"], "peak": HBM_PEAK / 1e9, "unit": "GB/s",
        "frac": head["hbm_frac"], "traffic": ctr["traffic"] if ctr else None,
        "algorithmic_bytes": head["algorithmic_bytes"],
        "mfma_useful_TFLOPs": head["useful_TFLOPs"], "mfma_useful_frac": head["mfma_useful_frac"],
    }
    if ctr:
        roof["traffic_over_algorithmic"] = ctr["traffic"] / head["algorithmic_bytes"]
        if "mfma_issued_flop_per_call" in ctr:
            roof["mfma_issued_TFLOPs"] = ctr["mfma_issued_flop_per_call"] / (ms * 1e-3) / 1e12
            roof["mfma_issued_frac"] = ctr["mfma_issued_flop_per_call"] / (ms * 1e-3) / MFMA_FP16_PEAK
        if "mfma_busy_cycles_per_call" in ctr:
            roof["mfma_busy_cycles_per_call"] = ctr["mfma_busy_cycles_per_call"]
        roof["counters"] = COUNTER_FILES[args.workload]
    out = {
        "metric": "GDN prefill tokens/s per layer (% MFMA peak); decode-step state GB/s (% HBM)",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_median": head["ms_median"],
        "ms_min": head["ms_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands, f32 accumulate and state, bf16 I/O",
        "data": "synthetic, seeded (torch generator on the GPU), distributions of the pages' workloads",
        "config": {"workload": args.workload, "B": B, "T": T, "Hk": Hk, "Hv": Hv, "Dk": D, "Dv": D,
                   "chunk": C, "conv_width": 0 if args.workload in NO_CONV_NORM else 4,
                   "gated_norm": args.workload not in NO_CONV_NORM, "parallelism": "single GPU"},
        "roofline": roof,
        "detail": {"headline": head, **extra},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
