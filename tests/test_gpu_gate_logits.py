"""GPU parity of the calls that take the raw gate logits ("How Qwen3.5 works" §9.5:
beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias)), through the C ABI.

The oracle turns the same fp32 logits into g and beta in fp64 (oracle.gate_logits,
pinned in test_oracle_pins.py) and runs its prefill on them; the GPU computes the
gates in fp32 inside its kernels.  Same tolerances as every other parity test.
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


def _with_gates(inp, gl):
    g, beta = O.gate_logits(gl["a"], gl["b"], gl["A_log"], gl["dt_bias"])
    out = dict(inp)
    out["g"], out["beta"] = g.astype(np.float32), beta.astype(np.float32)
    return out


def _check(name, y, y_ref, S, S_ref):
    eo, es = out_errors(y, y_ref), state_error(S, S_ref)
    print(f"[gate logits] {name}: e_out={eo['e_out']:.3e} e_state={es:.3e}", flush=True)
    assert eo["nonfinite"] == 0
    assert eo["e_out"] <= OUT_TOL
    assert es <= STATE_TOL


@pytest.mark.parametrize("B,T,Hk,Hv,rs", [(2, 100, 2, 4, True), (1, 257, 1, 3, False), (3, 64, 2, 2, True),
                                          (1, 4096, 16, 16, False)])
def test_prefill_gate_logits(B, T, Hk, Hv, rs):
    R = _R()
    w = GI.Workload(f"gl_{B}_{T}_{Hk}_{Hv}", B, T, Hk, Hv, random_state=rs, random_conv_state=rs,
                    tag=1000 + B * 7 + T + Hv)
    inp = GI.make_inputs(w)
    gl = GI.make_gate_logits(w)
    run = R.Prefill(inp, B, T, Hk, Hv, True, True)
    run.run_gate_logits(gl)
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    y_ref, S_ref, cs_ref = O.prefill(_with_gates(inp, gl), B, T, Hk, Hv, True, True)
    o = R.bits(run.o).reshape(B, T, Hv, D)
    y = np.stack([bf16_to_f64(o[c // Hv, :, c % Hv]) for c in range(B * Hv)])
    _check(f"prefill B={B} T={T} {Hk}/{Hv}", y, y_ref, run.state_out.cpu().numpy().reshape(-1, D, D), S_ref)
    np.testing.assert_array_equal(R.bits(run.conv_state_out), cs_ref)


def test_decode_gate_logits():
    R = _R()
    B, Hk, Hv = 5, 2, 6
    w = GI.Workload("gl_decode", B, 1, Hk, Hv, decode=True, random_state=True, random_conv_state=True, tag=1100)
    inp = GI.make_inputs(w)
    gl = GI.make_gate_logits(w)
    dec = R.Decode(inp, B, Hk, Hv, True, True)
    dec.run_gate_logits({"a": gl["a"][:, 0], "b": gl["b"][:, 0], "A_log": gl["A_log"], "dt_bias": gl["dt_bias"]})
    torch.cuda.synchronize()
    y_ref, S_ref, cs_ref = O.prefill(_with_gates(inp, gl), B, 1, Hk, Hv, True, True)
    y = bf16_to_f64(R.bits(dec.o)).reshape(B * Hv, 1, D)
    _check("decode", y, y_ref, dec.state.cpu().numpy().reshape(-1, D, D), S_ref)
    np.testing.assert_array_equal(R.bits(dec.conv_state), cs_ref)
