"""GPU parity of packed-sequence prefill (gdn_prefill_packed), through the C ABI.

"How Qwen3.5 works" §12.2: when several samples share one packed sequence, the
conv and recurrent states must stop at every sample boundary, and the way to
check it is to run the samples one by one and compare with the packed run.  That
is what these tests do: the oracle runs every sequence alone (B = 1, its own
initial states) and each sequence's slice of the packed GPU output, its final
state and its conv state must match, to the same tolerances as every other
parity test.  A packed batch of one sequence must equal the even-batch call
bit for bit (same kernels, same chunking, same plan).
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


def _batch(lengths, Hk, Hv, conv, norm, tag):
    """Token tensors of the packed batch (one B = 1 input set of sum(lengths) rows) and
    per-sequence random initial states."""
    T = int(sum(lengths))
    tok = GI.make_inputs(GI.Workload(f"packed_tok_{tag}", 1, T, Hk, Hv, conv=conv, norm=norm, tag=tag))
    st = GI.make_inputs(GI.Workload(f"packed_st_{tag}", len(lengths), 1, Hk, Hv, conv=conv, norm=norm,
                                    random_state=True, random_conv_state=True, tag=tag + 1))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return tok, st["state"], st.get("conv_state"), cu, T


def _seq_inputs(tok, a, b):
    out = dict(tok)
    for n in ("q", "k", "v", "z", "g", "beta"):
        if tok.get(n) is not None:
            out[n] = tok[n][:, a:b]
    return out


def _check_against_oracle(run, tok, state, conv_state, cu, Hk, Hv, conv, norm, label, skip=()):
    o = _R().bits(run.o).reshape(-1, Hv, D)
    S = run.state_out.cpu().numpy()
    cs = _R().bits(run.conv_state_out) if conv else None
    worst_o, worst_s = 0.0, 0.0
    for i in range(len(cu) - 1):
        if i in skip:
            continue
        a, b = int(cu[i]), int(cu[i + 1])
        y_ref, S_ref, cs_ref = O.prefill(_seq_inputs(tok, a, b), 1, b - a, Hk, Hv, conv, norm,
                                         state_in=state[i:i + 1],
                                         conv_state_in=None if conv_state is None else conv_state[i:i + 1])
        y = np.stack([bf16_to_f64(o[a:b, h]) for h in range(Hv)])
        eo, es = out_errors(y, y_ref), state_error(S[i], S_ref)
        assert eo["nonfinite"] == 0, (label, i)
        assert eo["e_out"] <= OUT_TOL, (label, i, eo)
        assert es <= STATE_TOL, (label, i, es)
        worst_o, worst_s = max(worst_o, eo["e_out"]), max(worst_s, es)
        if conv:
            np.testing.assert_array_equal(cs[i], cs_ref[0], err_msg=f"{label}: conv state of sequence {i}")
    print(f"[packed] {label}: {len(cu) - 1 - len(skip)} sequences, e_out={worst_o:.3e} e_state={worst_s:.3e}",
          flush=True)


@pytest.mark.parametrize("lengths,Hk,Hv,conv,norm", [
    ([1, 63, 64, 65, 200, 3], 2, 4, True, True),     # lengths around the chunk size, a one-token sequence
    ([130, 2, 129], 1, 3, False, False),             # raw path (no conv, no norm)
    ([64, 64, 64, 64], 2, 2, True, True),            # whole chunks only: the slot ranges leave no gap
])
def test_packed_matches_sequences_run_alone(lengths, Hk, Hv, conv, norm):
    R = _R()
    tok, state, conv_state, cu, T = _batch(lengths, Hk, Hv, conv, norm, tag=1200 + len(lengths) * 10 + Hv)
    print(f"[packed] lengths={lengths} Hk={Hk} Hv={Hv} conv={conv} norm={norm}", flush=True)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, conv, norm, state_in=state, conv_state_in=conv_state)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    _check_against_oracle(run, tok, state, conv_state, cu, Hk, Hv, conv, norm, f"lengths={lengths}")


def test_packed_many_sequences():
    """More sequences than one wave's lanes (the slot search takes two rounds), with
    seeded random lengths from 1 to 300 tokens."""
    R = _R()
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([GI.SEED_BASE, 1300])))
    lengths = rng.integers(1, 301, size=70).tolist()
    Hk, Hv = 1, 2
    tok, state, conv_state, cu, T = _batch(lengths, Hk, Hv, True, True, tag=1300)
    print(f"[packed] 70 sequences, T={T}", flush=True)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, True, True, state_in=state, conv_state_in=conv_state)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    _check_against_oracle(run, tok, state, conv_state, cu, Hk, Hv, True, True, "70 sequences")


def test_one_packed_sequence_equals_even_batch():
    """B = 1 packed over T tokens is the even-batch call on the same tensors: bit-equal (the even
    batch held to the plain sequential pass, which packed sequences always take)."""
    R = _R()
    T, Hk, Hv = 4096, 16, 16
    w = GI.Workload("packed_one", 1, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1310)
    inp = GI.make_inputs(w)
    print(f"[packed] one sequence T={T} {Hk}/{Hv}", flush=True)
    even = R.Prefill(inp, 1, T, Hk, Hv, True, True, segments=1)
    even.run()
    pk = R.PackedPrefill(inp, [0, T], T, Hk, Hv, True, True, state_in=inp["state"], conv_state_in=inp["conv_state"])
    pk.run()
    torch.cuda.synchronize()
    assert torch.equal(even.o.reshape(-1), pk.o.reshape(-1))
    assert torch.equal(even.state_out, pk.state_out)
    assert torch.equal(even.conv_state_out, pk.conv_state_out)


def test_packed_gate_logits():
    R = _R()
    lengths, Hk, Hv = [100, 1, 190], 2, 4
    tok, state, conv_state, cu, T = _batch(lengths, Hk, Hv, True, True, tag=1320)
    gl = GI.make_gate_logits(GI.Workload("packed_gl", 1, T, Hk, Hv, tag=1322))
    g, beta = O.gate_logits(gl["a"], gl["b"], gl["A_log"], gl["dt_bias"])
    tok = dict(tok, g=g.astype(np.float32), beta=beta.astype(np.float32))
    print(f"[packed] gate logits lengths={lengths}", flush=True)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, True, True, state_in=state, conv_state_in=conv_state)
    run.run_gate_logits(gl)
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    _check_against_oracle(run, tok, state, conv_state, cu, Hk, Hv, True, True, "gate logits")


def test_packed_sequence_with_bad_bounds_is_skipped():
    """An empty sequence breaks the offsets' rule: the kernels skip it (its outputs keep
    what they held, the error word says why) and compute every other sequence."""
    R = _R()
    lengths, Hk, Hv = [70, 0, 90], 1, 2
    tok, state, conv_state, cu, T = _batch(lengths, Hk, Hv, True, True, tag=1330)
    print(f"[packed] bad bounds cu={cu.tolist()}", flush=True)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, True, True, state_in=state, conv_state_in=conv_state)
    run.state_out.fill_(7.0)
    run.conv_state_out.fill_(7)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 2
    assert bool((run.state_out[1] == 7.0).all())
    assert bool((run.conv_state_out[1] == 7).all())
    _check_against_oracle(run, tok, state, conv_state, cu, Hk, Hv, True, True, "bad bounds", skip=(1,))


def test_packed_with_decreasing_offsets_skips_everything():
    """Offsets that decrease somewhere cannot be placed: every sequence is skipped, nothing is
    written, and the error word says so."""
    R = _R()
    lengths, Hk, Hv = [70, 20, 90], 1, 2
    tok, state, conv_state, cu, T = _batch(lengths, Hk, Hv, True, True, tag=1335)
    cu = cu.copy()
    cu[1], cu[2] = cu[2], cu[1]  # [0, 90, 70, 180]: sequence 1 runs backwards
    print(f"[packed] decreasing offsets cu={cu.tolist()}", flush=True)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, True, True, state_in=state, conv_state_in=conv_state)
    run.state_out.fill_(7.0)
    run.conv_state_out.fill_(7)
    run.o.fill_(7)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 2
    assert bool((run.state_out == 7.0).all()) and bool((run.conv_state_out == 7).all())
    assert bool((run.o == 7).all())


def test_packed_from_zero_states():
    """No initial states (NULL state_in and conv_state_in): every sequence starts from zeros."""
    R = _R()
    lengths, Hk, Hv = [5, 130, 64], 1, 2
    tok, _, _, cu, T = _batch(lengths, Hk, Hv, True, True, tag=1340)
    zeros = np.zeros((len(lengths), Hv, D, D), dtype=np.float32)
    zcs = np.zeros((len(lengths), 3, 2 * Hk * D + Hv * D), dtype=np.uint16)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, True, True, state_in=None, conv_state_in=None)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    _check_against_oracle(run, tok, zeros, zcs, cu, Hk, Hv, True, True, "zero states")

