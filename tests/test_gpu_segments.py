"""GPU parity of the two-level (segment-parallel) prefill, through the C ABI.

With few heads and long sequences the library splits every sequence into
segments: a first pass runs all segments at once, each from a zero state plus
128 transition columns (the map of a segment is affine in its start state),
a second pass chains the segment maps in fp32, and a third adds what the start
states contribute to the outputs and applies the gated RMSNorm.  The results
must match the oracle's token-by-token recurrence to the same tolerances as
the plain sequential pass.  The shape's prefill_segments field forces a segment
count (1: never split) so that small shapes exercise every part.

The long-memory cases (decay near 1: a state half-life of 200k tokens, far
longer than the sequence) check that nothing in either path loses precision
when the state keeps everything it has seen.
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


def _run_and_check(R, inp, B, T, Hk, Hv, conv, norm, nseg, label):
    run = R.Prefill(inp, B, T, Hk, Hv, conv, norm, segments=0 if nseg is None else nseg)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    y_ref, S_ref, cs_ref = O.prefill(inp, B, T, Hk, Hv, conv, norm)
    o = R.bits(run.o).reshape(B, T, Hv, D)
    y = np.stack([bf16_to_f64(o[c // Hv, :, c % Hv]) for c in range(B * Hv)])
    eo, es = out_errors(y, y_ref), state_error(run.state_out.cpu().numpy().reshape(-1, D, D), S_ref)
    print(f"[segments] {label}: e_out={eo['e_out']:.3e} max_abs={eo['max_abs']:.3e} e_state={es:.3e}", flush=True)
    assert eo["nonfinite"] == 0
    assert eo["e_out"] <= OUT_TOL
    assert es <= STATE_TOL
    if conv:
        np.testing.assert_array_equal(R.bits(run.conv_state_out), cs_ref)
    return run


@pytest.mark.parametrize("B,T,Hk,Hv,conv,norm,nseg", [
    (1, 1000, 1, 3, True, True, 4),      # ragged last segment and chunk
    (2, 300, 2, 4, True, True, 2),       # two sequences, segment boundary inside a chunk run
    (1, 327, 1, 1, False, False, 3),     # raw path
    (3, 200, 4, 12, True, True, 2),      # 36 heads: the 32-column slicing of the first pass
    (1, 4096, 1, 3, True, True, None),   # the library's own choice for few heads and a long sequence
    (3, 4100, 1, 3, True, True, None),   # 9 chains: two segments by the plan's own choice, the last one
                                         # a chunk shorter and ragged (65 chunks)
])
def test_segment_parallel_prefill(B, T, Hk, Hv, conv, norm, nseg):
    R = _R()
    w = GI.Workload(f"seg_{B}_{T}_{Hv}", B, T, Hk, Hv, conv=conv, norm=norm, random_state=True,
                    random_conv_state=conv, tag=1500 + B + T + Hv)
    inp = GI.make_inputs(w)
    print(f"[segments] B={B} T={T} {Hk}/{Hv} conv={conv} norm={norm} segments={nseg}", flush=True)
    _run_and_check(R, inp, B, T, Hk, Hv, conv, norm, nseg, f"B={B} T={T} {Hk}/{Hv}")


def test_segments_match_plain_pass_closely():
    """The same inputs through the plain sequential pass and the two-level scan: both
    meet the oracle, and they agree with each other to the state tolerance."""
    R = _R()
    B, T, Hk, Hv = 1, 2048, 1, 2
    w = GI.Workload("seg_vs_plain", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1520)
    inp = GI.make_inputs(w)
    a = _run_and_check(R, inp, B, T, Hk, Hv, True, True, 1, "plain")
    b = _run_and_check(R, inp, B, T, Hk, Hv, True, True, 8, "8 segments")
    assert b.ws_bytes > a.ws_bytes  # the segment plan ran (its read-outs and maps live in the workspace)
    print(f"[segments] outputs bit-equal: {torch.equal(a.o, b.o)}, states bit-equal: "
          f"{torch.equal(a.state_out, b.state_out)}", flush=True)
    sa, sb = a.state_out.cpu().numpy().reshape(-1, D, D), b.state_out.cpu().numpy().reshape(-1, D, D)
    assert state_error(sb, sa.astype(np.float64)) <= STATE_TOL


@pytest.mark.parametrize("nseg", [1, 8])
def test_long_memory_stress(nseg):
    """Decay near 1 (alpha = 2^(-1/200000): the state halves only after 200k tokens), T = 32768:
    the state keeps every write, through the plain pass and the two-level scan."""
    R = _R()
    B, T, Hk, Hv = 1, 32768, 1, 2
    w = GI.Workload("longmem", B, T, Hk, Hv, random_state=False, tag=1530)
    inp = dict(GI.make_inputs(w))
    inp["g"] = np.full((B, T, Hv), -np.log(2.0) / 200000.0, dtype=np.float32)
    print(f"[segments] long memory T={T} segments={nseg}", flush=True)
    _run_and_check(R, inp, B, T, Hk, Hv, True, True, nseg, f"long memory, segments={nseg}")


def test_segments_with_gate_logits():
    """The gate logits are turned into g and beta by the prep kernel, which both paths share."""
    R = _R()
    B, T, Hk, Hv = 1, 777, 1, 3
    w = GI.Workload("seg_gl", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1540)
    inp = GI.make_inputs(w)
    gl = GI.make_gate_logits(w)
    g, beta = O.gate_logits(gl["a"], gl["b"], gl["A_log"], gl["dt_bias"])
    run = R.Prefill(inp, B, T, Hk, Hv, True, True, segments=4)
    run.run_gate_logits(gl)
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    ref_inp = dict(inp, g=g.astype(np.float32), beta=beta.astype(np.float32))
    y_ref, S_ref, cs_ref = O.prefill(ref_inp, B, T, Hk, Hv, True, True)
    o = R.bits(run.o).reshape(B, T, Hv, D)
    y = np.stack([bf16_to_f64(o[c // Hv, :, c % Hv]) for c in range(B * Hv)])
    eo, es = out_errors(y, y_ref), state_error(run.state_out.cpu().numpy().reshape(-1, D, D), S_ref)
    print(f"[segments] gate logits, 4 segments: e_out={eo['e_out']:.3e} e_state={es:.3e}", flush=True)
    assert eo["e_out"] <= OUT_TOL and es <= STATE_TOL
    np.testing.assert_array_equal(R.bits(run.conv_state_out), cs_ref)

