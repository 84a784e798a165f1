"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each expected value is printed
on a page (tests/golden/), a closed form, a special case that reduces to a
library routine (numpy convolve), an independent algorithm from the pages (the
chunked form, the explicit product expansion), or an invariant.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O
import gdn_inputs as GI

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _unit_rows(rng, T, d):
    k = rng.standard_normal((T, d))
    return k / np.linalg.norm(k, axis=1, keepdims=True)


def _random_core(rng, T, dk=128, dv=128, s0=True):
    k = _unit_rows(rng, T, dk)
    q = rng.standard_normal((T, dk)) / np.sqrt(dk) * 0.3
    v = rng.standard_normal((T, dv))
    g = np.log(rng.uniform(0.8, 0.999, T))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((dk, dv)) * 0.1 if s0 else None
    return q, k, v, g, b, S0


# ---------------------------------------------------------------- worked examples

def test_worked_example_section_9_8():
    """How Qwen3.5 works, section 9.8: the 2x2 example printed on the page."""
    ex = json.load(open(os.path.join(GOLDEN, "hq_s9_8_worked_example.json")))
    toks = ex["tokens"]
    k = np.array([t["k"] for t in toks], float)
    v = np.array([t["v"] for t in toks], float)
    g = np.log([t["alpha"] for t in toks])
    b = np.array([t["beta"] for t in toks], float)
    q = np.array([ex["query"], ex["query"]], float) / np.sqrt(2.0)
    pr = ex["printed"]
    _, S1 = O.core_sequential(q[:1], k[:1], v[:1], g[:1], b[:1], np.array(ex["S0"], float))
    np.testing.assert_allclose(S1, pr["S1"], atol=1e-15)
    o, S2 = O.core_sequential(q, k, v, g, b, np.array(ex["S0"], float))
    np.testing.assert_allclose(S2, pr["S2"], atol=1e-15)
    # the correction written along k2 = e0 is row 0 of S2 - alpha2 * S1
    delta2 = (S2 - toks[1]["alpha"] * S1)[0]
    np.testing.assert_allclose(delta2, pr["delta2"], atol=1e-15)
    np.testing.assert_allclose(toks[1]["alpha"] * S1, pr["S2_decayed"], atol=1e-15)
    # o2 printed to 6 decimals; exactly (0.5, 2)/sqrt(2) from the printed S2
    np.testing.assert_allclose(o[1], pr["o2"], atol=0.5e-6)
    np.testing.assert_allclose(o[1], np.array([0.5, 2.0]) / np.sqrt(2.0), rtol=1e-15)


def test_walkthrough_d2_overwrite_and_fade():
    """Qwen3.5-4B architecture page, d = 2 walkthrough: the overwrite of slot A
    reads back exactly the new value and slot B fades by exactly 0.9."""
    ex = json.load(open(os.path.join(GOLDEN, "ad_d2_walkthrough.json")))
    slots = {n: np.array(vv, float) for n, vv in ex["slots"].items()}
    toks = ex["tokens"]
    k = np.array([slots[t["k"]] for t in toks])
    v = np.array([t["v"] for t in toks], float)
    g = np.log([t["alpha"] for t in toks])
    b = np.array([t["beta"] for t in toks], float)
    q = np.array([slots["A"]] * 3)  # read slot A after every token
    o, S = O.core_sequential(q, k, v, g, b, np.zeros((2, 2)))
    pr = ex["printed"]
    np.testing.assert_array_equal(o[1], pr["readout_A_before_overwrite"])
    np.testing.assert_allclose(o[2], pr["readout_A_after_overwrite"], rtol=1e-15)
    assert S[1, 1] == pytest.approx(pr["slot_B_after"], rel=1e-15)
    assert np.abs(S[1] - np.array([0.0, pr["slot_B_after"]])).max() < 1e-15


# ---------------------------------------------------------------- core invariants

def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(1)
    q, k, v, g, _, S0 = _random_core(rng, 37)
    b = np.zeros(37)
    G = np.cumsum(g)
    o_exp = np.exp(G)[:, None] * (q @ S0)
    S_exp = np.exp(G[-1]) * S0
    for fn in (O.core_sequential, lambda *a: O.core_chunked(*a, C=16)):
        o, S = fn(q, k, v, g, b, S0)
        np.testing.assert_allclose(S, S_exp, rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(o, o_exp, rtol=1e-13, atol=1e-15)


def test_exact_write_with_unit_keys():
    """g = 0, beta = 1, exactly unit keys: the state then returns v_t along k_t
    (reading with q_t = k_t gives o_t = S_t^T k_t = v_t)."""
    rng = np.random.default_rng(2)
    T = 50
    k = _unit_rows(rng, T, 128)
    v = rng.standard_normal((T, 128))
    S0 = rng.standard_normal((128, 128)) * 0.1
    o, _ = O.core_sequential(k, k, v, np.zeros(T), np.ones(T), S0)
    np.testing.assert_allclose(o, v, atol=1e-13)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 200])
def test_chunked_equals_sequential(C, T):
    rng = np.random.default_rng(100 + T + C)
    q, k, v, g, b, S0 = _random_core(rng, T)
    o1, S1 = O.core_sequential(q, k, v, g, b, S0)
    o2, S2 = O.core_chunked(q, k, v, g, b, S0, C=C)
    assert np.linalg.norm(S2 - S1) / np.linalg.norm(S1) < 1e-12
    assert np.abs(o2 - o1).max() <= 1e-12 * max(1.0, np.abs(o1).max())


@pytest.mark.parametrize("T,d", [(1, 128), (3, 16), (8, 128)])
def test_bruteforce_product_equals_sequential(T, d):
    rng = np.random.default_rng(7 + T)
    q, k, v, g, b, S0 = _random_core(rng, T, d, d)
    o1, S1 = O.core_sequential(q, k, v, g, b, S0)
    o2, S2 = O.core_bruteforce(q, k, v, g, b, S0)
    assert np.linalg.norm(S2 - S1) / np.linalg.norm(S1) < 1e-12
    assert np.abs(o2 - o1).max() <= 1e-12 * max(1.0, np.abs(o1).max())


def test_orthogonal_keys_do_not_interfere():
    """Distinct one-hot keys, g = 0, S0 = 0: every write lands in its own slot,
    S_T = sum_t beta_t k_t v_t^T exactly."""
    rng = np.random.default_rng(3)
    T = 100
    perm = rng.permutation(128)[:T]
    k = np.eye(128)[perm]
    v = rng.standard_normal((T, 128))
    b = rng.uniform(0.05, 1.0, T)
    _, S = O.core_sequential(k, k, v, np.zeros(T), b, None)
    expect = np.zeros((128, 128))
    expect[perm] = b[:, None] * v
    np.testing.assert_array_equal(S, expect)


def test_linear_in_v_from_zero_state():
    rng = np.random.default_rng(4)
    q, k, v1, g, b, _ = _random_core(rng, 40, s0=False)
    v2 = rng.standard_normal(v1.shape)
    o1, S1 = O.core_sequential(q, k, v1, g, b)
    o2, S2 = O.core_sequential(q, k, v2, g, b)
    o3, S3 = O.core_sequential(q, k, 2.0 * v1 - 3.0 * v2, g, b)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, atol=1e-13)
    np.testing.assert_allclose(S3, 2 * S1 - 3 * S2, atol=1e-13)


# ---------------------------------------------------------------- conv, l2norm, gated norm

def test_conv_delta_taps():
    """w = e3 leaves the current step; w = e0 takes the step three back
    (zero or the history before step 0)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20)
    hist = rng.standard_normal(3)
    np.testing.assert_allclose(O.conv_silu_channel(x, [0, 0, 0, 1]), _silu(x), rtol=1e-15)
    u = O.conv_silu_channel(x, [1, 0, 0, 0])
    np.testing.assert_array_equal(u[:3], 0.0)
    np.testing.assert_allclose(u[3:], _silu(x[:-3]), rtol=1e-15)
    u = O.conv_silu_channel(x, [1, 0, 0, 0], hist)
    np.testing.assert_allclose(u[:3], _silu(hist), rtol=1e-15)


def test_conv_matches_numpy_convolve():
    """Causal cross-correlation = numpy convolution with the reversed taps."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(50)
    w = rng.standard_normal(4)
    pre = np.convolve(x, w[::-1])[:50]
    np.testing.assert_allclose(O.conv_silu_channel(x, w), _silu(pre), rtol=1e-13, atol=1e-15)


def test_l2norm_closed_form_eps_inside_root():
    x = np.zeros(128)
    x[0], x[1] = 3.0, 4.0
    np.testing.assert_allclose(O.l2norm(x, 1e-6), x / np.sqrt(25.0 + 1e-6), rtol=1e-15)
    xs = x * 1e-4  # here eps is not negligible: sqrt(25e-8 + 1e-6)
    np.testing.assert_allclose(O.l2norm(xs, 1e-6, 0.5), 0.5 * xs / np.sqrt(25e-8 + 1e-6), rtol=1e-15)


def test_gated_norm_closed_forms():
    rng = np.random.default_rng(8)
    z = rng.standard_normal(128)
    c = 0.37
    o = np.full(128, c)
    y = O.gated_rmsnorm(o, z, np.ones(128))
    np.testing.assert_allclose(y, c / np.sqrt(c * c + 1e-6) * _silu(z), rtol=1e-14)
    # the weight multiplies as it is (w = 2 doubles the output; not 1 + w)
    np.testing.assert_allclose(O.gated_rmsnorm(o, z, np.full(128, 2.0)), 2 * y, rtol=1e-15)
    np.testing.assert_array_equal(O.gated_rmsnorm(rng.standard_normal(128), np.zeros(128), np.ones(128)), 0.0)
    o2 = rng.standard_normal(128)
    y1 = O.gated_rmsnorm(o2, z, np.ones(128), eps=0.0)
    y2 = O.gated_rmsnorm(5.0 * o2, z, np.ones(128), eps=0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-14)


# ---------------------------------------------------------------- the whole path

def _bf(x):
    return GI.f32_to_bf16_bits(np.asarray(x, np.float32))


def _path_inputs(B, T, Hk, Hv, tag, conv=True, norm=True, state=False, conv_state=False):
    w = GI.Workload("t", B, T, Hk, Hv, conv=conv, norm=norm, random_state=state,
                    random_conv_state=conv_state, tag=tag)
    return w, GI.make_inputs(w)


def test_gqa_value_head_reads_key_head_h_over_ratio():
    """Distinct one-hot key per key head: value head h writes only into the
    slot of key head h // r (not h % Hk)."""
    B, T, Hk, Hv = 1, 1, 2, 6
    w, inp = _path_inputs(B, T, Hk, Hv, 900, conv=False, norm=False)
    kf = np.zeros((B, T, Hk, 128), np.float32)
    for kh in range(Hk):
        kf[:, :, kh, 10 + kh] = 1.0
    inp["k"] = _bf(kf)
    inp["beta"] = np.ones((B, T, Hv), np.float32)
    inp["g"] = np.zeros((B, T, Hv), np.float32)
    _, S, _ = O.prefill(inp, B, T, Hk, Hv, conv=False, norm=False)
    vf = GI.bf16_bits_to_f32(inp["v"]).astype(np.float64)
    for h in range(Hv):
        nz = np.nonzero(np.abs(S[h]).sum(axis=1))[0]
        assert list(nz) == [10 + h // 3]
        np.testing.assert_allclose(S[h][10 + h // 3], vf[0, 0, h] / np.sqrt(1 + 1e-6), rtol=1e-15)


def test_query_scale_and_eps():
    """T = 1, S0 = 0, g = 0, beta = 1, q = k = 7 e0: o = v (k.q) with
    k = 7/sqrt(49 + eps), q = that / sqrt(128)."""
    B, T, Hk, Hv = 1, 1, 1, 1
    w, inp = _path_inputs(B, T, Hk, Hv, 901, conv=False, norm=False)
    e = np.zeros((1, 1, 1, 128), np.float32)
    e[..., 0] = 7.0
    inp["q"] = inp["k"] = _bf(e)
    inp["beta"][:] = 1.0
    inp["g"][:] = 0.0
    y, _, _ = O.prefill(inp, B, T, Hk, Hv, conv=False, norm=False)
    n = 7.0 / np.sqrt(49.0 + 1e-6)
    vf = GI.bf16_bits_to_f32(inp["v"]).astype(np.float64)[0, 0, 0]
    np.testing.assert_allclose(y[0, 0], vf * n * n / np.sqrt(128.0), rtol=1e-15)


def _compose_reference(inp, B, T, Hk, Hv, conv, norm, chain):
    """The path composed from pieces pinned above, with numpy's convolve for the
    conv and numpy indexing of the boundary layouts."""
    b, h = divmod(chain, Hv)
    kh = h // (Hv // Hk)
    f = lambda a: GI.bf16_bits_to_f32(a).astype(np.float64)
    qx, kx, vx = f(inp["q"])[b, :, kh], f(inp["k"])[b, :, kh], f(inp["v"])[b, :, h]
    if conv:
        Cc = 2 * Hk * 128 + Hv * 128
        cw = f(inp["conv_w"])
        cs = f(inp["conv_state"])[b] if inp.get("conv_state") is not None else np.zeros((3, Cc))
        chans = [kh * 128 + np.arange(128), Hk * 128 + kh * 128 + np.arange(128),
                 2 * Hk * 128 + h * 128 + np.arange(128)]
        outs = []
        for x, ch in zip((qx, kx, vx), chans):
            u = np.empty_like(x)
            for i, c in enumerate(ch):
                full = np.concatenate([cs[:, c], x[:, i]])
                u[:, i] = _silu(np.convolve(full, cw[c][::-1])[3:3 + T])
            outs.append(u)
        qx, kx, vx = outs
    qn = np.stack([O.l2norm(r, 1e-6, 1 / np.sqrt(128)) for r in qx])
    kn = np.stack([O.l2norm(r, 1e-6) for r in kx])
    S0 = inp["state"][b, h].astype(np.float64) if inp.get("state") is not None else None
    o, S = O.core_sequential(qn, kn, vx, inp["g"][b, :, h], inp["beta"][b, :, h], S0)
    if norm:
        z, w = f(inp["z"])[b, :, h], f(inp["norm_w"])
        o = np.stack([O.gated_rmsnorm(o[t], z[t], w) for t in range(T)])
    return o, S


@pytest.mark.parametrize("conv,norm,state", [(True, True, False), (False, False, True), (True, True, True)])
def test_path_composition(conv, norm, state):
    B, T, Hk, Hv = 2, 37, 2, 6
    w, inp = _path_inputs(B, T, Hk, Hv, 902, conv=conv, norm=norm, state=state, conv_state=state)
    chains = [0, 4, 7, 11]
    y, S, _ = O.prefill(inp, B, T, Hk, Hv, conv, norm, chains=chains)
    for i, c in enumerate(chains):
        yr, Sr = _compose_reference(inp, B, T, Hk, Hv, conv, norm, c)
        np.testing.assert_allclose(y[i], yr, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S[i], Sr, rtol=1e-12, atol=1e-13)


def test_conv_state_out_is_last_three_raw_inputs():
    B, T, Hk, Hv = 2, 5, 1, 2
    w, inp = _path_inputs(B, T, Hk, Hv, 903, conv_state=True)
    _, _, cs = O.prefill(inp, B, T, Hk, Hv, True, True)
    raw = np.concatenate([inp["q"].reshape(B, T, -1), inp["k"].reshape(B, T, -1),
                          inp["v"].reshape(B, T, -1)], axis=2)
    np.testing.assert_array_equal(cs, raw[:, T - 3:])
    # T = 2: the oldest entry comes from the incoming conv state
    _, _, cs2 = O.prefill({**inp, "q": inp["q"][:, :2].copy(), "k": inp["k"][:, :2].copy(),
                           "v": inp["v"][:, :2].copy(), "z": inp["z"][:, :2].copy(),
                           "g": inp["g"][:, :2].copy(), "beta": inp["beta"][:, :2].copy()},
                          B, 2, Hk, Hv, True, True)
    np.testing.assert_array_equal(cs2[:, 0], inp["conv_state"][:, 2])
    np.testing.assert_array_equal(cs2[:, 1:], raw[:, :2])


@pytest.mark.parametrize("T1", [1, 2, 3, 20])
def test_split_prefill_equals_whole(T1):
    """Running T1 tokens, then the rest from the returned state and conv state,
    equals one run over all tokens (conv and recurrent state hand-off)."""
    B, T, Hk, Hv = 1, 24, 1, 2
    w, inp = _path_inputs(B, T, Hk, Hv, 904, state=True, conv_state=True)
    y, S, cs = O.prefill(inp, B, T, Hk, Hv, True, True)
    cut = lambda a, s: np.ascontiguousarray(a[:, s])
    keys = ["q", "k", "v", "z", "g", "beta"]
    p1 = {**inp, **{n: cut(inp[n], slice(0, T1)) for n in keys}}
    y1, S1, cs1 = O.prefill(p1, B, T1, Hk, Hv, True, True)
    p2 = {**inp, **{n: cut(inp[n], slice(T1, T)) for n in keys}}
    y2, S2, cs2 = O.prefill(p2, B, T - T1, Hk, Hv, True, True,
                            state_in=S1.reshape(B, Hv, 128, 128).astype(np.float32), conv_state_in=cs1)
    # the hand-off state is rounded to fp32 (the boundary's state type)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(S2, S, rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(cs2, cs)


# --- gates from their logits ("How Qwen3.5 works" §9.5) ---------------------------------------

def _gates(a, b, A_log, dt_bias):
    return O.gate_logits(np.asarray(a, float), np.asarray(b, float), np.asarray(A_log, float),
                         np.asarray(dt_bias, float))


def test_gates_at_zero_logits():
    """softplus(0) = ln 2 and sigmoid(0) = 1/2, so g = -e^{A_log} ln 2."""
    g, beta = _gates(np.zeros((3, 2)), np.zeros((3, 2)), [0.0, np.log(5.0)], [0.0, 0.0])
    np.testing.assert_allclose(g[:, 0], -np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(g[:, 1], -5.0 * np.log(2.0), rtol=1e-14)
    np.testing.assert_allclose(beta, 0.5, rtol=1e-15)


def test_gate_identities():
    """softplus(x) - softplus(-x) = x; sigmoid(x) + sigmoid(-x) = 1; d softplus/dx = sigmoid;
    A_log scales g by e^{A_log}; dt_bias shifts the decay logit."""
    x = np.linspace(-12.0, 12.0, 49)[:, None]
    gp, bp = _gates(x, x, [0.0], [0.0])
    gm, bm = _gates(-x, -x, [0.0], [0.0])
    np.testing.assert_allclose(-(gp - gm), x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(bp + bm, 1.0, rtol=1e-15)
    h = 1e-5
    g1, _ = _gates(x + h, x, [0.0], [0.0])
    g0, _ = _gates(x - h, x, [0.0], [0.0])
    np.testing.assert_allclose(-(g1 - g0) / (2 * h), bp, rtol=1e-8, atol=1e-10)
    g3, _ = _gates(x, x, [np.log(3.0)], [0.0])
    np.testing.assert_allclose(g3, 3.0 * gp, rtol=1e-14)
    gs, _ = _gates(x - 0.75, x, [0.0], [0.75])
    np.testing.assert_allclose(gs, gp, rtol=1e-12)


def test_gate_extremes():
    """Large decay logits: softplus(x) -> x; very negative ones: softplus(x) -> e^x (no decay)."""
    g, beta = _gates([[50.0, -50.0]], [[40.0, -40.0]], [0.0, 0.0], [0.0, 0.0])
    assert g[0, 0] == pytest.approx(-50.0, rel=1e-15)
    assert g[0, 1] == pytest.approx(-np.exp(-50.0), rel=1e-12)
    assert beta[0, 0] == pytest.approx(1.0, abs=1e-15) and beta[0, 1] == pytest.approx(np.exp(-40.0), rel=1e-12)
    assert np.all(np.isfinite(_gates([[1e4]], [[-1e4]], [0.0], [0.0])[0]))
