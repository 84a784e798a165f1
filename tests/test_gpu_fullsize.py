"""Parity at the full sizes of the 4B- and 27B-shaped prefill layers, of one GPU's share of
the 27B-shaped layer under 16-way key-head sharding (which runs the two-level scan), and of
the packed 16-sequence batch.

The GPU runs the whole layer, every head, in the launch configuration that
bench.py times.  A few sampled (sequence, value head) pairs, each with its own
key head, carry inputs from the seeded generator (gdn_inputs); every other
head carries torch-generated inputs of the same distributions.  The oracle
recomputes the sampled heads over all T tokens, and their outputs, final state
and conv tail are compared.
"""
import numpy as np
import pytest

import gdn_inputs as GI
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


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


# one GPU's share of the 27B-shaped layer under 16-way key-head sharding: the library runs it
# through the two-level (segment-parallel) scan
SHARD = GI.Workload("qwen38_27b_prefill_T262144_keyhead_shard_1of16", 1, 262144, 1, 3)


@pytest.mark.parametrize("wname,picks", [
    ("qwen35_4b_prefill_B4_T16384", [(0, 0), (3, 31), (1, 13)]),
    ("qwen38_27b_prefill_T262144", [(0, 0), (0, 47), (0, 25)]),
    (SHARD.name, [(0, 1)]),
])
def test_fullsize_sampled_heads(wname, picks):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_mixer_amd as gdn
    w = SHARD if wname == SHARD.name else GI.WORKLOADS[wname]
    B, T, Hk, Hv = w.B, w.T, w.Hk, w.Hv
    r = Hv // Hk
    assert len({h // r for _, h in picks}) == len(picks)
    P = len(picks)
    print(f"[fullsize] {wname}: generating", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    q, k = _bg(gen, (B, T, Hk, D), "x"), _bg(gen, (B, T, Hk, D), "x")
    v, z = _bg(gen, (B, T, Hv, D), "x"), _bg(gen, (B, T, Hv, D), "x")
    g, beta = _bg(gen, (B, T, Hv), "g"), _bg(gen, (B, T, Hv), "b")
    Cc = 2 * Hk * D + Hv * D
    conv_w = (torch.randn((Cc, 4), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    # the sampled heads: P independent one-head sequences from the seeded generator
    sw = GI.Workload(f"{wname}_sampled", P, T, 1, 1, tag=800 + Hv)
    si = GI.make_inputs(sw)
    for i, (b, h) in enumerate(picks):
        kh = h // r
        q[b, :, kh] = _dev_bf16(si["q"][i, :, 0])
        k[b, :, kh] = _dev_bf16(si["k"][i, :, 0])
        v[b, :, h] = _dev_bf16(si["v"][i, :, 0])
        z[b, :, h] = _dev_bf16(si["z"][i, :, 0])
        g[b, :, h] = torch.from_numpy(si["g"][i, :, 0]).cuda()
        beta[b, :, h] = torch.from_numpy(si["beta"][i, :, 0]).cuda()
        cw = _dev_bf16(si["conv_w"])  # [3*128, 4]: q, k, v channels of the one-head layout
        conv_w[kh * D:(kh + 1) * D] = cw[0:D]
        conv_w[Hk * D + kh * D:Hk * D + (kh + 1) * D] = cw[D:2 * D]
        conv_w[2 * Hk * D + h * D:2 * Hk * D + (h + 1) * D] = cw[2 * D:3 * D]
    norm_w = _dev_bf16(si["norm_w"])
    o = torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device="cuda")
    state_out = torch.empty((B, Hv, D, D), device="cuda")
    conv_state_out = torch.empty((B, 3, Cc), dtype=torch.bfloat16, device="cuda")
    shape = gdn.make_shape(B, T, Hk, Hv)
    ws = torch.zeros(gdn.gdn_prefill_workspace_size(shape), dtype=torch.uint8, device="cuda")
    print(f"[fullsize] {wname}: running the layer", flush=True)
    gdn.gdn_prefill(shape, q, k, v, g, beta, z, conv_w, norm_w, None, None, o, state_out, conv_state_out, ws)
    torch.cuda.synchronize()
    assert int(ws[-256:-252].view(torch.int32).item()) == 0
    print(f"[fullsize] {wname}: oracle on {P} heads", flush=True)
    y_ref, S_ref, cs_ref = O.prefill(si, P, T, 1, 1, True, True)
    cs_all = conv_state_out.view(torch.int16).cpu().numpy().view(np.uint16)
    for i, (b, h) in enumerate(picks):
        kh = h // r
        y = bf16_to_f64(o[b, :, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        S = state_out[b, h].cpu().numpy()
        eo, es = out_errors(y[None], y_ref[i:i + 1]), state_error(S[None], S_ref[i:i + 1])
        print(f"[fullsize] {wname} (b={b}, h={h}): e_out={eo['e_out']:.3e} max_abs={eo['max_abs']:.3e} "
              f"n|y|>=8={eo['n_large']} e_state={es:.3e}", flush=True)
        assert eo["nonfinite"] == 0
        assert eo["e_out"] <= OUT_TOL
        assert es <= STATE_TOL
        tail = np.concatenate([cs_all[b, :, kh * D:(kh + 1) * D],
                               cs_all[b, :, Hk * D + kh * D:Hk * D + (kh + 1) * D],
                               cs_all[b, :, 2 * Hk * D + h * D:2 * Hk * D + (h + 1) * D]], axis=1)
        np.testing.assert_array_equal(tail, cs_ref[i])


def test_fullsize_packed_sampled_sequences():
    """The packed batch bench.py times: the 4B-shaped layer's 65,536 tokens as 16 sequences of
    1,793 to 6,656 tokens.  Three sampled (sequence, value head) pairs, each on its own key
    head, carry seeded inputs and random initial states; the oracle runs each of those
    sequences alone from its own states."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    import gated_deltanet_mixer_amd as gdn
    N, T, Hk, Hv = 16, 65536, 16, 32
    r = Hv // Hk
    lens = bench.packed_lengths(N, T)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    picks = [(0, 0), (7, 13), (15, 31)]  # (sequence, value head)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4343)
    q, k = _bg(gen, (T, Hk, D), "x"), _bg(gen, (T, Hk, D), "x")
    v, z = _bg(gen, (T, Hv, D), "x"), _bg(gen, (T, Hv, D), "x")
    g, beta = _bg(gen, (T, Hv), "g"), _bg(gen, (T, Hv), "b")
    Cc = 2 * Hk * D + Hv * D
    conv_w = (torch.randn((Cc, 4), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    state_in = torch.randn((N, Hv, D, D), generator=gen, device="cuda") * 0.1
    conv_state_in = torch.randn((N, 3, Cc), generator=gen, device="cuda").to(torch.bfloat16)
    seeded = []
    for i, (b, h) in enumerate(picks):
        L = int(lens[b])
        si = GI.make_inputs(GI.Workload(f"packed_full_{i}", 1, L, 1, 1, random_state=True, random_conv_state=True,
                                        tag=820 + i))
        seeded.append(si)
        kh, t0 = h // r, int(cu[b])
        q[t0:t0 + L, kh] = _dev_bf16(si["q"][0, :, 0])
        k[t0:t0 + L, kh] = _dev_bf16(si["k"][0, :, 0])
        v[t0:t0 + L, h] = _dev_bf16(si["v"][0, :, 0])
        z[t0:t0 + L, h] = _dev_bf16(si["z"][0, :, 0])
        g[t0:t0 + L, h] = torch.from_numpy(si["g"][0, :, 0]).cuda()
        beta[t0:t0 + L, h] = torch.from_numpy(si["beta"][0, :, 0]).cuda()
        cw = _dev_bf16(si["conv_w"])
        conv_w[kh * D:(kh + 1) * D] = cw[0:D]
        conv_w[Hk * D + kh * D:Hk * D + (kh + 1) * D] = cw[D:2 * D]
        conv_w[2 * Hk * D + h * D:2 * Hk * D + (h + 1) * D] = cw[2 * D:3 * D]
        state_in[b, h] = torch.from_numpy(si["state"][0, 0]).cuda()
        cs = _dev_bf16(si["conv_state"][0])  # [3, 3*128]: q, k, v channels of the one-head layout
        conv_state_in[b, :, kh * D:(kh + 1) * D] = cs[:, 0:D]
        conv_state_in[b, :, Hk * D + kh * D:Hk * D + (kh + 1) * D] = cs[:, D:2 * D]
        conv_state_in[b, :, 2 * Hk * D + h * D:2 * Hk * D + (h + 1) * D] = cs[:, 2 * D:3 * D]
    norm_w = _dev_bf16(seeded[0]["norm_w"])
    for si in seeded[1:]:
        si["norm_w"] = seeded[0]["norm_w"]
    o = torch.empty((T, Hv, D), dtype=torch.bfloat16, device="cuda")
    state_out = torch.empty((N, Hv, D, D), device="cuda")
    conv_state_out = torch.empty((N, 3, Cc), dtype=torch.bfloat16, device="cuda")
    shape = gdn.make_shape(N, T, Hk, Hv, packed=True)
    ws = torch.zeros(gdn.gdn_prefill_workspace_size(shape), dtype=torch.uint8, device="cuda")
    cu_dev = torch.from_numpy(cu).cuda()
    print("[fullsize] packed 16 sequences: running the layer", flush=True)
    gdn.gdn_prefill_packed(shape, cu_dev, q, k, v, g, beta, z, conv_w, norm_w, state_in, conv_state_in, o, state_out,
                           conv_state_out, ws)
    torch.cuda.synchronize()
    assert int(ws[-256:-252].view(torch.int32).item()) == 0
    cs_all = conv_state_out.view(torch.int16).cpu().numpy().view(np.uint16)
    for i, (b, h) in enumerate(picks):
        L, t0, kh = int(lens[b]), int(cu[b]), h // r
        y_ref, S_ref, cs_ref = O.prefill(seeded[i], 1, L, 1, 1, True, True)
        y = bf16_to_f64(o[t0:t0 + L, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        eo, es = out_errors(y[None], y_ref), state_error(state_out[b, h].cpu().numpy()[None], S_ref)
        print(f"[fullsize] packed sequence {b} (T={L}), head {h}: e_out={eo['e_out']:.3e} e_state={es:.3e}",
              flush=True)
        assert eo["nonfinite"] == 0
        assert eo["e_out"] <= OUT_TOL
        assert es <= STATE_TOL
        tail = np.concatenate([cs_all[b, :, kh * D:(kh + 1) * D],
                               cs_all[b, :, Hk * D + kh * D:Hk * D + (kh + 1) * D],
                               cs_all[b, :, 2 * Hk * D + h * D:2 * Hk * D + (h + 1) * D]], axis=1)
        np.testing.assert_array_equal(tail, cs_ref[0])
