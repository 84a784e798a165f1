"""Parity at the full sizes of the 4B- and 27B-shaped prefill layers, of one GPU's share of
the 27B-shaped layer under 16-way key-head sharding (which runs the two-level scan), and of
the packed 16-sequence batch: every (sequence, value head) chain against the oracle.

The GPU runs the whole layer in the launch configuration that bench.py times, on inputs of
the workloads' distributions drawn by torch's seeded generator on the device.  The input
bits the GPU consumed are copied to the host, and the fp64 oracle recomputes every chain
over all T tokens (OpenMP over chains, in batches of as many chains as the host has
threads), so that every output row, every final state and every conv-tail channel is
compared.  Host memory stays bounded: the oracle's fp64 outputs exist for one batch at a
time.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests.metrics import OUT_TOL, STATE_TOL, bf16_to_f64, out_errors, state_error

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


def _bg(gen, shape, kind):
    if kind == "x":
        return torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    if kind == "g":
        return torch.log(torch.rand(shape, generator=gen, device="cuda", dtype=torch.float64) * 0.199 + 0.8).float()
    return torch.sigmoid(torch.randn(shape, generator=gen, device="cuda", dtype=torch.float64)).float()


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _host_inputs(d):
    """The device inputs as the oracle's boundary-format arrays (the same bits)."""
    out = {n: _u16(d[n]) for n in ("q", "k", "v", "z", "conv_w", "norm_w")}
    out["g"] = d["g"].cpu().numpy()
    out["beta"] = d["beta"].cpu().numpy()
    if d.get("state_in") is not None:
        out["state"] = d["state_in"].cpu().numpy()
    if d.get("conv_state_in") is not None:
        out["conv_state"] = _u16(d["conv_state_in"])
    return out


def _make_layer(B, T, Hk, Hv, seed, states=False, rows=None):
    """Inputs of one layer drawn on the device; rows = token rows of the token-major tensors
    (B * T for an even batch, T for a packed batch)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    lead = (B, T) if rows is None else (rows,)
    Cc = 2 * Hk * D + Hv * D
    d = dict(q=_bg(gen, lead + (Hk, D), "x"), k=_bg(gen, lead + (Hk, D), "x"),
             v=_bg(gen, lead + (Hv, D), "x"), z=_bg(gen, lead + (Hv, D), "x"),
             g=_bg(gen, lead + (Hv,), "g"), beta=_bg(gen, lead + (Hv,), "b"),
             conv_w=(torch.randn((Cc, 4), generator=gen, device="cuda") * 0.5).to(torch.bfloat16),
             norm_w=(1.0 + 0.02 * torch.randn((D,), generator=gen, device="cuda")).to(torch.bfloat16))
    if states:
        d["state_in"] = torch.randn((B, Hv, D, D), generator=gen, device="cuda") * 0.1
        d["conv_state_in"] = torch.randn((B, 3, Cc), generator=gen, device="cuda").to(torch.bfloat16)
    return d


def _compare_chains(label, host, B, T, Hk, Hv, o_host, S_host, cs_host):
    """Oracle over every chain of an even batch, in batches of as many chains as the host has
    threads.  o_host [B*T, Hv, D] uint16, S_host [B, Hv, D, D], cs_host [B, 3, Cc] uint16."""
    threads = O.num_threads()
    worst_o = worst_s = 0.0
    n_large = 0
    nchains = B * Hv
    for i0 in range(0, nchains, threads):
        batch = list(range(i0, min(nchains, i0 + threads)))
        y_ref, S_ref, cs_ref = O.prefill(host, B, T, Hk, Hv, True, True, chains=batch, want_conv_state=(i0 == 0))
        if i0 == 0:
            np.testing.assert_array_equal(cs_host, cs_ref)  # every conv-tail channel, bit for bit
        for j, ch in enumerate(batch):
            b, h = ch // Hv, ch % Hv
            y = bf16_to_f64(o_host[b * T:(b + 1) * T, h])
            eo = out_errors(y[None], y_ref[j:j + 1])
            es = state_error(S_host[b, h][None], S_ref[j:j + 1])
            assert eo["nonfinite"] == 0, f"{label} chain {ch}: non-finite outputs"
            assert eo["e_out"] <= OUT_TOL, f"{label} chain {ch}: e_out {eo['e_out']:.3e}"
            assert es <= STATE_TOL, f"{label} chain {ch}: e_state {es:.3e}"
            worst_o, worst_s = max(worst_o, eo["e_out"]), max(worst_s, es)
            n_large += eo["n_large"]
        del y_ref, S_ref
        print(f"[fullsize] {label}: chains {i0}..{batch[-1]} of {nchains} match "
              f"(worst so far e_out={worst_o:.3e} e_state={worst_s:.3e})", flush=True)
    print(f"[fullsize] {label}: all {nchains} chains, worst e_out={worst_o:.3e} "
          f"e_state={worst_s:.3e}, outputs with |y_ref| >= 8: {n_large}", flush=True)


@pytest.mark.parametrize("B,T,Hk,Hv,segments", [
    (4, 16384, 16, 32, 0),   # the 4B-shaped layer
    (1, 262144, 16, 48, 0),  # the 27B-shaped layer
    (1, 262144, 1, 3, 0),    # one GPU's share of the 27B-shaped layer under 16-way key-head sharding (two-level scan)
], ids=["qwen35_4b_prefill_B4_T16384", "qwen38_27b_prefill_T262144", "qwen38_27b_keyhead_shard_1of16"])
def test_fullsize_every_chain(B, T, Hk, Hv, segments):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_mixer_amd as gdn
    label = f"B={B} T={T} {Hk}/{Hv}"
    print(f"[fullsize] {label}: generating", flush=True)
    d = _make_layer(B, T, Hk, Hv, seed=4242 + Hv)
    Cc = 2 * Hk * D + Hv * D
    o = torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device="cuda")
    state_out = torch.empty((B, Hv, D, D), device="cuda")
    conv_state_out = torch.empty((B, 3, Cc), dtype=torch.bfloat16, device="cuda")
    shape = gdn.make_shape(B, T, Hk, Hv, segments=segments)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(shape), dtype=torch.uint8, device="cuda")
    print(f"[fullsize] {label}: running the layer", flush=True)
    gdn.gdn_prefill(shape, d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"], d["conv_w"], d["norm_w"], None, None,
                    o, state_out, conv_state_out, ws)
    gdn.gdn_prefill_check(ws)
    del ws
    print(f"[fullsize] {label}: copying inputs and results to the host", flush=True)
    host = _host_inputs(d)
    del d
    o_host = _u16(o).reshape(B * T, Hv, D)
    del o
    S_host = state_out.cpu().numpy()
    cs_host = _u16(conv_state_out)
    torch.cuda.empty_cache()
    _compare_chains(label, host, B, T, Hk, Hv, o_host, S_host, cs_host)


def test_fullsize_packed_every_sequence():
    """The packed batch bench.py times: the 4B-shaped layer's 65,536 tokens as 16 sequences of
    1,793 to 6,656 tokens, each from its own random initial states.  The oracle runs every
    sequence alone (all 32 value heads) and every (sequence, head) chain is compared."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    import gated_deltanet_mixer_amd as gdn
    N, T, Hk, Hv = 16, 65536, 16, 32
    lens = bench.packed_lengths(N, T)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = _make_layer(N, T, Hk, Hv, seed=4343, states=True, rows=T)
    Cc = 2 * Hk * D + Hv * D
    o = torch.empty((T, Hv, D), dtype=torch.bfloat16, device="cuda")
    state_out = torch.empty((N, Hv, D, D), device="cuda")
    conv_state_out = torch.empty((N, 3, Cc), dtype=torch.bfloat16, device="cuda")
    shape = gdn.make_shape(N, T, Hk, Hv, packed=True)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(shape), dtype=torch.uint8, device="cuda")
    print("[fullsize] packed 16 sequences: running the layer", flush=True)
    gdn.gdn_prefill_packed(shape, torch.from_numpy(cu).cuda(), d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"],
                           d["conv_w"], d["norm_w"], d["state_in"], d["conv_state_in"], o, state_out, conv_state_out,
                           ws)
    gdn.gdn_prefill_check(ws)
    host = _host_inputs(d)
    o_host = _u16(o)
    S_host = state_out.cpu().numpy()
    cs_host = _u16(conv_state_out)
    for b in range(N):
        t0, L = int(cu[b]), int(lens[b])
        seq = {n: host[n][t0:t0 + L][None] for n in ("q", "k", "v", "z", "g", "beta")}
        seq.update(conv_w=host["conv_w"], norm_w=host["norm_w"], state=host["state"][b:b + 1],
                   conv_state=host["conv_state"][b:b + 1])
        y_ref, S_ref, cs_ref = O.prefill(seq, 1, L, Hk, Hv, True, True)
        np.testing.assert_array_equal(cs_host[b:b + 1], cs_ref)
        for h in range(Hv):
            y = bf16_to_f64(o_host[t0:t0 + L, h])
            eo = out_errors(y[None], y_ref[h:h + 1])
            es = state_error(S_host[b, h][None], S_ref[h:h + 1])
            assert eo["nonfinite"] == 0 and eo["e_out"] <= OUT_TOL and es <= STATE_TOL, \
                f"packed sequence {b} head {h}: e_out {eo['e_out']:.3e} e_state {es:.3e}"
        print(f"[fullsize] packed sequence {b} (T={L}): all {Hv} heads match", flush=True)
