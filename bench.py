"""Benchmark of the Gated DeltaNet mixer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu-baseline]

One step = one gdn_prefill call over the whole batch of the headline workload
(the Qwen3.5-0.8B-shaped layer, B=1, T=4096, 16 key / 16 value heads: conv,
L2 norm, gated delta rule, gated RMSNorm), inputs already resident in HBM.
Prints ONE JSON line.  `value` is prefill tokens/s of the layer.  Extra fields
carry the roofline of the timed call, the decode step on the 27B-shaped
B=256 workload (state GB/s, % of HBM) and the same batch checking two tokens per
sequence with snapshots, the other prefill shapes, the 4B-shaped
layer's tokens as 16 packed sequences of mixed lengths, one GPU's share of the
27B-shaped layer under 16-way key-head sharding (the two-level scan beside the
plain sequential pass), and the fp64
CPU oracle timed on this host (a reported baseline, not a target).

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
    "qwen35_0p8b_prefill_T4096": (1, 4096, 16, 16),
    "qwen35_4b_prefill_B4_T16384": (4, 16384, 16, 32),
    "qwen38_27b_prefill_T262144": (1, 262144, 16, 48),
}
DECODE = ("qwen38_27b_decode_B256", (256, 16, 48))
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


def prefill_bytes(B, T, Hk, Hv) -> int:
    """Algorithmic HBM bytes of one prefill: raw q,k; v, z, o; g, beta; final state;
    conv weights and conv tail (zero initial state and conv state are not read)."""
    Cc = 2 * Hk * D + Hv * D
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


def make_prefill_set(torch, gdn, B, T, Hk, Hv, seed):
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
    shape = gdn.make_shape(B, T, Hk, Hv)
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
    """Average ms per call over `steps` calls (cycling the input sets), with
    HIP events on the current stream, bracketed by device syncs."""
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(sets[i % len(sets)])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    return start.elapsed_time(end) / steps, t_wall


def bench_prefill(torch, gdn, name, steps, warmup, gate_logits=False):
    B, T, Hk, Hv = WORKLOADS[name]
    per_set = prefill_bytes(B, T, Hk, Hv) + B * T * Hk * 2 * D * 2
    nsets = max(1, min(4, math.ceil(320e6 / per_set)))  # rotate past the 256 MB Infinity Cache
    sets = [make_prefill_set(torch, gdn, B, T, Hk, Hv, seed=1000 + i) for i in range(nsets)]
    if gate_logits:
        for i, d in enumerate(sets):
            add_gate_logits(torch, d, Hv, seed=2000 + i)
    torch.cuda.synchronize()
    run = run_prefill_gate_logits if gate_logits else run_prefill
    ms, wall = time_calls(torch, lambda d: run(gdn, d), sets, steps, warmup)
    nbytes = prefill_bytes(B, T, Hk, Hv)
    flops = USEFUL_FLOP_PER_TOKEN_HEAD * B * T * Hv
    res = {
        "workload": name + (" (gdn_prefill_gate_logits)" if gate_logits else ""), "B": B, "T": T, "Hk": Hk,
        "Hv": Hv, "ms_per_call": ms,
        "tokens_per_s": B * T / (ms * 1e-3), "algorithmic_bytes": nbytes,
        "hbm_GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK,
        "useful_TFLOPs": flops / (ms * 1e-3) / 1e12, "mfma_useful_frac": flops / (ms * 1e-3) / MFMA_FP16_PEAK,
        "roof_frac": max(nbytes / HBM_PEAK, flops / MFMA_FP16_PEAK) / (ms * 1e-3),
        "input_sets": nsets, "steps": steps, "wall_s": wall,
    }
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
    ms, wall = time_calls(torch, run, [d], steps, warmup)
    # per-token bytes as the even batch; one final state and conv tail per sequence
    nbytes = prefill_bytes(1, T, Hk, Hv) + (N - 1) * (Hv * D * D * 4 + 3 * Cc * 2)
    flops = USEFUL_FLOP_PER_TOKEN_HEAD * T * Hv
    res = {
        "workload": name + " (gdn_prefill_packed)", "sequences": N, "T_total": T, "Hk": Hk, "Hv": Hv,
        "lengths_min_max": [min(lens), max(lens)], "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
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
    plans it (segments) and, for comparison, with the plain sequential pass
    (GDN_PREFILL_SEGMENTS=0)."""
    name, (B, T, Hk, Hv) = SHARD
    out = {"workload": name, "B": B, "T": T, "Hk": Hk, "Hv": Hv}
    old = os.environ.get("GDN_PREFILL_SEGMENTS")
    try:
        for leg, env in (("plain_sequential", "0"), ("planned", None)):
            if env is None:
                os.environ.pop("GDN_PREFILL_SEGMENTS", None)
            else:
                os.environ["GDN_PREFILL_SEGMENTS"] = env
            d = make_prefill_set(torch, gdn, B, T, Hk, Hv, seed=1200)
            torch.cuda.synchronize()
            ms, _ = time_calls(torch, lambda dd: run_prefill(gdn, dd), [d], steps, warmup)
            out[leg + "_ms_per_call"] = ms
            out[leg + "_workspace_MiB"] = d["ws"].numel() / 2 ** 20
            del d
            torch.cuda.empty_cache()
    finally:
        if old is None:
            os.environ.pop("GDN_PREFILL_SEGMENTS", None)
        else:
            os.environ["GDN_PREFILL_SEGMENTS"] = old
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
    ms, wall = time_calls(torch, fn, [d], steps, warmup)
    nbytes = decode_bytes(B, Hk, Hv)
    state_bytes = 2 * B * Hv * D * D * 4
    res = {"workload": DECODE[0], "B": B, "Hk": Hk, "Hv": Hv, "us_per_step": ms * 1e3,
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
    ms, wall = time_calls(torch, fn, [d], steps, warmup)
    nbytes = decode_multi_bytes(B, T, Hk, Hv)
    res = {"workload": f"{DECODE[0]} checking T={T} tokens per sequence (gdn_decode_multi, snapshots)",
           "B": B, "T": T, "Hk": Hk, "Hv": Hv, "us_per_call": ms * 1e3, "tokens_per_s": B * T / (ms * 1e-3),
           "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms * 1e-3) / HBM_PEAK, "steps": steps}
    del d
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, budget_s=20.0, min_s=10.0):
    """The fp64 oracle (as it stands) on this host's cores, on the headline
    workload: all of its (sequence, value-head) chains, repeated until about
    `min_s` seconds have passed, or as many whole chains as fit `budget_s` when
    one full pass would take longer."""
    import numpy as np
    import gdn_inputs as GI
    from oracle import oracle as O
    w = GI.WORKLOADS[name]
    inp = GI.make_inputs(w)
    nchains = w.B * w.Hv
    threads = O.num_threads()
    # calibrate on one chain
    t = time.perf_counter()
    O.prefill(inp, w.B, w.T, w.Hk, w.Hv, w.conv, w.norm, chains=[0], threads=1, want_conv_state=False)
    one = time.perf_counter() - t
    per_round = max(1, min(threads, nchains))
    full_est = one * math.ceil(nchains / per_round)
    if full_est <= budget_s:
        chains = np.arange(nchains)
    else:
        n = int(max(per_round, per_round * (budget_s // max(one, 1e-9))))
        chains = np.arange(min(n, nchains))
    reps, el = 0, 0.0
    t = time.perf_counter()
    while reps == 0 or (el < min_s and reps < 200):
        O.prefill(inp, w.B, w.T, w.Hk, w.Hv, w.conv, w.norm, chains=chains, threads=threads,
                  want_conv_state=False)
        reps += 1
        el = time.perf_counter() - t
    n = len(chains)
    used = min(threads, n)
    # tokens/s of the layer = chain-tokens/s divided by the layer's Hv chains per token
    return {"value": reps * n * w.T / el / w.Hv, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{n} of {nchains} (sequence, value-head) chains of {name}, all {w.T} tokens each, "
                      f"{reps} pass(es); fp64 C oracle (conv, L2 norm, token-by-token recurrence, gated "
                      f"RMSNorm) with OpenMP over chains; {el:.1f} s wall",
            "host_cpus": os.cpu_count()}


TRAFFIC_FILES = {"qwen35_0p8b_prefill_T4096": "profiles/prefill_qwen35_0p8b_T4096_hbm_traffic.txt"}


def measured_traffic(name):
    """HBM bytes per call from the committed counter summary of this workload,
    or None when there is none or the kernel sources changed since it was taken."""
    import hashlib
    rel = TRAFFIC_FILES.get(name)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    rec = {}
    for line in open(os.path.join(ROOT, rel)):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_call", "sources_sha256", "sources"):
            k, v = line.split(":", 1)
            rec[k] = v.strip()
    if not all(k in rec for k in ("traffic_bytes_per_call", "sources_sha256", "sources")):
        return None
    h = hashlib.sha256()
    for src in rec["sources"].split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return int(rec["traffic_bytes_per_call"]) if h.hexdigest() == rec["sources_sha256"] else None


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen35_0p8b_prefill_T4096", choices=sorted(WORKLOADS))
    ap.add_argument("--no-extra", action="store_true", help="skip decode and the other prefill shapes")
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
    head = bench_prefill(torch, gdn, args.workload, args.steps, args.warmup)
    extra = {}
    if not args.no_extra:
        extra["decode"] = bench_decode(torch, gdn, max(20, args.steps // 4), 5)
        extra["decode_multi_T2"] = bench_decode_multi(torch, gdn, max(20, args.steps // 4), 5)
        for name in WORKLOADS:
            if name != args.workload:
                B, T, Hk, Hv = WORKLOADS[name]
                steps = max(3, min(args.steps, int(2e8 // (B * T * Hv))))
                extra[name] = bench_prefill(torch, gdn, name, steps, 2)
        # few heads, long sequence: the two-level scan against the plain sequential pass
        extra[SHARD[0]] = bench_prefill_shard(torch, gdn, 5, 1)
        # the 4B-shaped layer's tokens as packed sequences of mixed lengths
        extra[PACKED[0]] = bench_prefill_packed(torch, gdn, 20, 2)
        # the same layer through the entry point that takes the gate logits
        extra[args.workload + "_gate_logits"] = bench_prefill(torch, gdn, args.workload, max(20, args.steps // 4), 5,
                                                              gate_logits=True)
    B, T, Hk, Hv = WORKLOADS[args.workload]
    out = {
        "metric": "GDN prefill tokens/s per layer (% MFMA peak); decode-step state GB/s (% HBM)",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 I/O, fp16 MFMA operands, fp32 accumulate and state",
        "data": "synthetic, seeded (torch generator on the GPU), distributions of the pages' workloads",
        "config": {"workload": args.workload, "B": B, "T": T, "Hk": Hk, "Hv": Hv, "Dk": D, "Dv": D,
                   "chunk": C, "conv_width": 4, "gated_norm": True, "parallelism": "single GPU"},
        "roofline": {
            "kernel": "one gdn_prefill call = chunk_prep_kernel + chain_kernel launches, timed together",
            "bound": "hbm", "achieved": head["hbm_GBps"], "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": head["hbm_frac"], "traffic": measured_traffic(args.workload),
            "mfma_useful_TFLOPs": head["useful_TFLOPs"], "mfma_useful_frac": head["mfma_useful_frac"],
        },
        "detail": {"headline": head, **extra},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
