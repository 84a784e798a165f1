"""GPU parity of multi-token decode with snapshots (gdn_decode_multi), through the C ABI.

T tokens per sequence go through the recurrence one after the other, so the
oracle is its token-by-token prefill over the same T tokens from the same
state and conv window.  Snapshot t (the state and conv window after token t,
"How Qwen3.5 works" §13.5: rolling back needs snapshots) is the oracle's final
state and conv tail after the first t + 1 tokens.  Same tolerances as every
other parity test; the conv windows are compared bit for bit.
"""
import numpy as np
import pytest

import gdn_inputs as GI
from oracle import oracle as O
from tests.metrics import OUT_TOL, STATE_TOL, bf16_to_f64, out_errors, state_error

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


def _R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gdn_run
    return gdn_run


def _prefix(inp, n):
    out = dict(inp)
    for k in ("q", "k", "v", "z", "g", "beta"):
        if inp.get(k) is not None:
            out[k] = np.ascontiguousarray(inp[k][:, :n])
    return out


class Multi:
    """Device buffers of one gdn_decode_multi call (state and conv state in place)."""

    def __init__(self, R, inp, B, T, Hk, Hv, conv, norm, snaps=True):
        import gated_deltanet_mixer_amd as gdn
        self.gdn, self.R = gdn, R
        self.shape = gdn.make_shape(B, T, Hk, Hv, conv=conv, norm=norm)
        self.d = {n: R.to_dev(inp.get(n)) for n in ("q", "k", "v", "g", "beta")}
        self.d["z"] = R.to_dev(inp.get("z")) if norm else None
        self.d["conv_w"] = R.to_dev(inp.get("conv_w")) if conv else None
        self.d["norm_w"] = R.to_dev(inp.get("norm_w")) if norm else None
        Cc = 2 * Hk * D + Hv * D
        st = inp.get("state")
        self.state = R.to_dev(st) if st is not None else torch.zeros((B, Hv, D, D), device="cuda")
        cs = inp.get("conv_state")
        self.conv_state = ((R.to_dev(cs) if cs is not None else torch.zeros((B, 3, Cc), dtype=torch.int16,
                                                                            device="cuda")) if conv else None)
        self.o = torch.empty((B, T, Hv, D), dtype=torch.int16, device="cuda")
        self.state_snaps = torch.full((T - 1, B, Hv, D, D), 7.0, device="cuda") if (snaps and T > 1) else None
        self.conv_snaps = (torch.full((T - 1, B, 3, Cc), 7, dtype=torch.int16, device="cuda")
                           if (snaps and conv and T > 1) else None)

    def run(self, gl=None):
        d = self.d
        if gl is None:
            self.gdn.gdn_decode_multi(self.shape, d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"], d["conv_w"],
                                      d["norm_w"], self.state, self.conv_state, self.o, self.state_snaps,
                                      self.conv_snaps)
        else:
            t = {n: self.R.to_dev(x) for n, x in gl.items()}
            self.gdn.gdn_decode_multi_gate_logits(self.shape, d["q"], d["k"], d["v"], t["a"], t["b"], t["A_log"],
                                                  t["dt_bias"], d["z"], d["conv_w"], d["norm_w"], self.state,
                                                  self.conv_state, self.o, self.state_snaps, self.conv_snaps)


def _check(label, y, y_ref, S, S_ref):
    eo, es = out_errors(y, y_ref), state_error(S, S_ref)
    assert eo["nonfinite"] == 0, label
    assert eo["e_out"] <= OUT_TOL, (label, eo)
    assert es <= STATE_TOL, (label, es)
    return eo["e_out"], es


def _against_oracle(R, m, inp, B, T, Hk, Hv, conv, norm, label):
    y_ref, S_ref, cs_ref = O.prefill(inp, B, T, Hk, Hv, conv, norm)
    o = R.bits(m.o)
    y = np.stack([bf16_to_f64(o[c // Hv, :, c % Hv]) for c in range(B * Hv)])
    worst = [_check(f"{label} tokens", y, y_ref, m.state.cpu().numpy().reshape(-1, D, D), S_ref)]
    if conv:
        np.testing.assert_array_equal(R.bits(m.conv_state), cs_ref, err_msg=f"{label}: conv window")
    for t in range(T - 1):
        if m.state_snaps is None:
            break
        _, St_ref, cst_ref = O.prefill(_prefix(inp, t + 1), B, t + 1, Hk, Hv, conv, norm)
        es = state_error(m.state_snaps[t].cpu().numpy().reshape(-1, D, D), St_ref)
        assert es <= STATE_TOL, (label, t, es)
        worst.append((0.0, es))
        if conv and m.conv_snaps is not None:
            np.testing.assert_array_equal(R.bits(m.conv_snaps[t]), cst_ref, err_msg=f"{label}: conv snapshot {t}")
    print(f"[decode multi] {label}: e_out={max(w[0] for w in worst):.3e} e_state={max(w[1] for w in worst):.3e}",
          flush=True)


@pytest.mark.parametrize("T", [2, 3, 4, 8])
def test_multi_token_decode_with_snapshots(T):
    R = _R()
    B, Hk, Hv = 5, 2, 6
    w = GI.Workload(f"multi_T{T}", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1400 + T)
    inp = GI.make_inputs(w)
    print(f"[decode multi] B={B} T={T} {Hk}/{Hv}", flush=True)
    m = Multi(R, inp, B, T, Hk, Hv, True, True)
    m.run()
    torch.cuda.synchronize()
    _against_oracle(R, m, inp, B, T, Hk, Hv, True, True, f"T={T}")


def test_multi_equals_repeated_steps():
    """T tokens in one call equal T gdn_decode_step calls bit for bit, and T = 1 is the step."""
    R = _R()
    B, T, Hk, Hv = 3, 4, 1, 3
    w = GI.Workload("multi_steps", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1410)
    inp = GI.make_inputs(w)
    m = Multi(R, inp, B, T, Hk, Hv, True, True)
    m.run()
    import gated_deltanet_mixer_amd as gdn
    step_shape = gdn.make_shape(B, 1, Hk, Hv)
    st = R.to_dev(inp["state"])
    cs = R.to_dev(inp["conv_state"])
    d = {n: R.to_dev(np.ascontiguousarray(inp[n])) for n in ("q", "k", "v", "z", "g", "beta")}
    cw, nw = R.to_dev(inp["conv_w"]), R.to_dev(inp["norm_w"])
    for t in range(T):
        o = torch.empty((B, Hv, D), dtype=torch.int16, device="cuda")
        one = {n: d[n][:, t].contiguous() for n in d}
        gdn.gdn_decode_step(step_shape, one["q"], one["k"], one["v"], one["g"], one["beta"], one["z"], cw, nw,
                            st, cs, o)
        torch.cuda.synchronize()
        assert torch.equal(o, m.o[:, t]), t
        if t < T - 1:
            assert torch.equal(st, m.state_snaps[t]), t
            assert torch.equal(cs, m.conv_snaps[t]), t
    assert torch.equal(st, m.state) and torch.equal(cs, m.conv_state)
    # T = 1 through gdn_decode_multi is the step itself
    one_shape = gdn.make_shape(B, 1, Hk, Hv)
    st2, cs2 = st.clone(), cs.clone()
    o1, o2 = (torch.empty((B, Hv, D), dtype=torch.int16, device="cuda") for _ in range(2))
    x = {n: d[n][:, 0].contiguous() for n in d}
    gdn.gdn_decode_step(one_shape, x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], cw, nw, st, cs, o1)
    gdn.gdn_decode_multi(one_shape, x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], cw, nw, st2, cs2, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st, st2) and torch.equal(cs, cs2)


def test_multi_without_snapshots_raw_path():
    R = _R()
    B, T, Hk, Hv = 4, 3, 2, 2
    w = GI.Workload("multi_raw", B, T, Hk, Hv, conv=False, norm=False, random_state=True, tag=1420)
    inp = GI.make_inputs(w)
    m = Multi(R, inp, B, T, Hk, Hv, False, False, snaps=False)
    m.run()
    torch.cuda.synchronize()
    _against_oracle(R, m, inp, B, T, Hk, Hv, False, False, "raw, no snapshots")


def test_multi_gate_logits():
    R = _R()
    B, T, Hk, Hv = 3, 2, 2, 4
    w = GI.Workload("multi_gl", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1430)
    inp = GI.make_inputs(w)
    gl = GI.make_gate_logits(w)
    g, beta = O.gate_logits(gl["a"], gl["b"], gl["A_log"], gl["dt_bias"])
    m = Multi(R, inp, B, T, Hk, Hv, True, True)
    m.run(gl)
    torch.cuda.synchronize()
    _against_oracle(R, m, dict(inp, g=g.astype(np.float32), beta=beta.astype(np.float32)), B, T, Hk, Hv, True,
                    True, "gate logits")


def test_multi_full_27b_decode_shape():
    """The 27B-shaped decode batch (B = 256, 16 key / 48 value heads) with T = 2 draft
    tokens and snapshots, every head against the oracle."""
    R = _R()
    B, T, Hk, Hv = 256, 2, 16, 48
    w = GI.Workload("multi_27b", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1440)
    inp = GI.make_inputs(w)
    m = Multi(R, inp, B, T, Hk, Hv, True, True)
    m.run()
    torch.cuda.synchronize()
    _against_oracle(R, m, inp, B, T, Hk, Hv, True, True, "27B-shaped B=256 T=2")


@pytest.mark.parametrize("B,T,Hk,Hv", [
    (2, 1, 1, 64),  # 64 value heads per key head: 1,056 conv items and 1,024 z pieces for 512 threads
    (2, 8, 1, 8),   # 8 tokens of 8 value heads: about 75 KB of LDS, above the default dynamic limit
    (1, 3, 2, 64),  # 32 per key head with 3 tokens: both of the above at once (about 89 KB)
])
def test_decode_many_value_heads_per_key_head(B, T, Hk, Hv):
    """Head ratios and token counts past one item per thread and past 64 KB of LDS: the
    second passes over conv items and z pieces and the raised LDS limit, against the oracle."""
    R = _R()
    w = GI.Workload(f"multi_wide_{B}_{T}_{Hk}_{Hv}", B, T, Hk, Hv, random_state=True, random_conv_state=True,
                    tag=1450 + T + Hv)
    inp = GI.make_inputs(w)
    print(f"[decode multi] wide B={B} T={T} {Hk}/{Hv}", flush=True)
    m = Multi(R, inp, B, T, Hk, Hv, True, True)
    m.run()
    torch.cuda.synchronize()
    _against_oracle(R, m, inp, B, T, Hk, Hv, True, True, f"{Hk}/{Hv} T={T}")
