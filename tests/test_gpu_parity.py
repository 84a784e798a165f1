"""GPU parity of the mixer's HIP path against the fp64 oracle, through the C ABI.

Bars (tests/metrics.py): gated-norm / read-out outputs within 2e-2 beyond the
bf16 output rounding; final state within 1e-3 relative (Frobenius, per head);
conv state bit-exact (it is a copy of raw inputs).
"""
import numpy as np
import pytest

import gdn_inputs as GI
from oracle import oracle as O
from tests.metrics import OUT_TOL, STATE_TOL, bf16_to_f64, out_errors, state_error

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gdn_run
    return gdn_run


def _report(name, eo, es):
    print(f"[parity] {name}: e_out={eo['e_out']:.3e} max_abs={eo['max_abs']:.3e} "
          f"n|y|>=8={eo['n_large']} e_state={es:.3e}", flush=True)


def _check_prefill(w: GI.Workload, chains=None, inp=None, tag=""):
    R = _gpu()
    inp = GI.make_inputs(w) if inp is None else inp
    run = R.Prefill(inp, w.B, w.T, w.Hk, w.Hv, w.conv, w.norm)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    y_ref, S_ref, cs_ref = O.prefill(inp, w.B, w.T, w.Hk, w.Hv, w.conv, w.norm, chains=chains)
    ch = np.arange(w.B * w.Hv) if chains is None else np.asarray(chains)
    o = R.bits(run.o).reshape(w.B, w.T, w.Hv, 128)
    y = np.stack([bf16_to_f64(o[c // w.Hv, :, c % w.Hv]) for c in ch])
    S = run.state_out.cpu().numpy().reshape(w.B * w.Hv, 128, 128)[ch]
    eo, es = out_errors(y, y_ref), state_error(S, S_ref)
    _report(f"prefill {w.name} {tag}", eo, es)
    assert eo["nonfinite"] == 0
    assert eo["e_out"] <= OUT_TOL
    assert es <= STATE_TOL
    if w.conv:
        np.testing.assert_array_equal(R.bits(run.conv_state_out), cs_ref)
    return run, y_ref, S_ref


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("conv,norm", [(True, True), (False, False), (True, False)])
def test_decode_small(conv, norm):
    R = _gpu()
    w = GI.Workload("decode_small", 4, 1, 2, 6, conv=conv, norm=norm, decode=True,
                    random_state=True, random_conv_state=True, tag=200 + 2 * conv + norm)
    inp = GI.make_inputs(w)
    run = R.Decode(inp, w.B, w.Hk, w.Hv, conv, norm)
    run.run()
    torch.cuda.synchronize()
    y_ref, S_ref, cs_ref = O.prefill(inp, w.B, 1, w.Hk, w.Hv, conv, norm)
    y = bf16_to_f64(R.bits(run.o)).reshape(w.B * w.Hv, 1, 128)
    S = run.state.cpu().numpy().reshape(-1, 128, 128)
    eo, es = out_errors(y, y_ref), state_error(S, S_ref)
    _report(f"decode small conv={conv} norm={norm}", eo, es)
    assert eo["e_out"] <= OUT_TOL and es <= STATE_TOL
    if conv:
        np.testing.assert_array_equal(R.bits(run.conv_state), cs_ref)


def test_decode_27b_shape_B256():
    """The 27B-shaped decode workload at full size (all 12,288 heads)."""
    R = _gpu()
    w = GI.WORKLOADS["qwen38_27b_decode_B256"]
    inp = GI.make_inputs(w)
    run = R.Decode(inp, w.B, w.Hk, w.Hv, w.conv, w.norm)
    run.run()
    torch.cuda.synchronize()
    y_ref, S_ref, cs_ref = O.prefill(inp, w.B, 1, w.Hk, w.Hv, w.conv, w.norm)
    y = bf16_to_f64(R.bits(run.o)).reshape(w.B * w.Hv, 1, 128)
    S = run.state.cpu().numpy().reshape(-1, 128, 128)
    eo, es = out_errors(y, y_ref), state_error(S, S_ref)
    _report("decode 27b B256", eo, es)
    assert eo["e_out"] <= OUT_TOL and es <= STATE_TOL
    np.testing.assert_array_equal(R.bits(run.conv_state), cs_ref)


# ------------------------------------------------------------------ prefill

def test_prefill_tiny_T64():
    _check_prefill(GI.WORKLOADS["tiny_T64"])


@pytest.mark.parametrize("T", [1, 2, 3, 63, 64, 65, 127, 200])
@pytest.mark.parametrize("Hk,Hv", [(1, 1), (2, 4), (1, 3)])
def test_prefill_ragged(T, Hk, Hv):
    w = GI.Workload(f"ragged_T{T}_Hk{Hk}_Hv{Hv}", 2, T, Hk, Hv, random_state=True, random_conv_state=True,
                    tag=300 + T * 10 + Hv)
    _check_prefill(w)


@pytest.mark.parametrize("B,T,Hk,Hv", [
    (2, 150, 1, 16),  # 16 value heads per key head: the prep kernel's second pass over g and beta
    (1, 130, 1, 40),  # 40 per key head: 56 KB of prep LDS, 40 chains in two-tile slices
    (1, 200, 2, 64),  # 32 per key head on two key heads: the raised prep LDS limit (68 KB)
])
def test_prefill_many_value_heads_per_key_head(B, T, Hk, Hv):
    """Head ratios past the eight value heads whose gates one pass of the prep kernel's 256
    threads stages, and prep LDS past the default 64 KB limit, against the oracle."""
    w = GI.Workload(f"wide_B{B}_T{T}_Hk{Hk}_Hv{Hv}", B, T, Hk, Hv, random_state=True, random_conv_state=True,
                    tag=1900 + Hv)
    _check_prefill(w)


@pytest.mark.parametrize("conv,norm", [(False, True), (True, False), (False, False)])
def test_prefill_conv_norm_switches(conv, norm):
    w = GI.Workload(f"switch_c{conv}_n{norm}", 1, 150, 2, 4, conv=conv, norm=norm, tag=400 + 2 * conv + norm)
    _check_prefill(w)


def test_prefill_0p8b_T4096_full():
    """Qwen3.5-0.8B-shaped layer: B=1, T=4096, 16/16 heads, every head checked."""
    _check_prefill(GI.WORKLOADS["qwen35_0p8b_prefill_T4096"])
