"""Non-finite inputs propagate; nothing is clamped or replaced.

Policy.  The kernels use IEEE arithmetic throughout and never test for, clamp or replace
a NaN or an infinity.  A non-finite value in q, k, v, z, g or beta therefore reaches every
output and state entry that depends on it in the recurrence's own definition (the oracle's
token-by-token order), as NaN or infinity.  The chunked form adds one effect of its own:
inside the chunk of 64 tokens that holds the value, block products multiply it by
coefficients that are exactly zero (the upper triangle of T, rows past a token in P), and
0 * inf is NaN, so outputs of that chunk at tokens before the value can turn NaN as well,
in the chains that read it.  Outputs of earlier chunks, and every output and state of the
chains that never read the value, are unaffected and match the oracle as usual.  The state
is non-finite exactly where the oracle's is (columns are independent in the update).

The cases plant one NaN or +infinity (bf16 bits for q, k, v; fp32 for g) and check: every
output the oracle makes non-finite is non-finite on the GPU; any further non-finite output
lies in the planted token's chunk of a chain the oracle shows affected; every other output
and every finite state matches the oracle to the usual tolerances; the state's non-finite
pattern equals the oracle's.
"""
import numpy as np
import pytest

import gdn_inputs as GI
from oracle import oracle as O
from tests.metrics import OUT_TOL, STATE_TOL, bf16_to_f64, ulp_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D, C = 128, 64
NAN16, INF16 = 0x7FC0, 0x7F80


def _R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gdn_run
    return gdn_run


def _plant(inp, tensor, idx, val):
    out = dict(inp)
    a = out[tensor].copy()
    a[idx] = val
    out[tensor] = a
    return out


def _check(y, y_ref, S, S_ref, t_planted, label):
    """y, y_ref [n, T, D]; S, S_ref [n, D, D]."""
    ref_bad, gpu_bad = ~np.isfinite(y_ref), ~np.isfinite(y)
    assert ref_bad.any(), f"{label}: the planted value reaches no output of the oracle"
    missing = ref_bad & ~gpu_bad
    assert not missing.any(), f"{label}: {int(missing.sum())} outputs non-finite in the oracle are finite here"
    affected = ref_bad.any(axis=(1, 2))  # chains that read the planted value
    extra = gpu_bad & ~ref_bad
    ch, tok = np.nonzero(extra.any(axis=2))
    c0 = t_planted // C
    assert affected[ch].all(), f"{label}: non-finite outputs in chains {sorted(set(ch[~affected[ch]]))} that never read it"
    assert ((tok // C) == c0).all(), f"{label}: extra non-finite outputs outside chunk {c0}: tokens {sorted(set(tok))[:8]}"
    ok = ~(ref_bad | gpu_bad)
    d = np.abs(np.where(ok, y, 0.0) - np.where(ok, y_ref, 0.0))
    half = 0.5 * ulp_bf16(np.maximum(np.abs(np.where(ok, y_ref, 0.0)), np.abs(np.where(ok, y, 0.0))))
    e_out = float(np.maximum(0.0, d - half).max())
    assert e_out <= OUT_TOL, f"{label}: e_out {e_out:.3e} on the finite outputs"
    np.testing.assert_array_equal(~np.isfinite(S), ~np.isfinite(S_ref), err_msg=f"{label}: state non-finite pattern")
    fin = np.isfinite(S_ref).all(axis=(1, 2))
    if fin.any():
        num = np.sqrt(((S[fin] - S_ref[fin]) ** 2).sum(axis=(1, 2)))
        den = np.sqrt((S_ref[fin] ** 2).sum(axis=(1, 2)))
        es = float((num / np.maximum(den, 1e-300)).max())
        assert es <= STATE_TOL, f"{label}: e_state {es:.3e} on the finite states"
    print(f"[nonfinite] {label}: oracle non-finite outputs {int(ref_bad.sum())}, GPU {int(gpu_bad.sum())} "
          f"(extra in chunk {c0}: {int(extra.sum())}), chains affected {int(affected.sum())} of {len(affected)}, "
          f"non-finite state entries {int((~np.isfinite(S)).sum())}", flush=True)


# (tensor, index, value): q/k [B,T,Hk,128], v [B,T,Hv,128] as bf16 bits; g [B,T,Hv] fp32
PREFILL_CASES = [
    ("q", (0, 100, 1, 5), NAN16),
    ("k", (1, 130, 0, 77), NAN16),
    ("v", (1, 70, 2, 3), INF16),
    ("g", (0, 150, 0), np.float32(np.nan)),
]


@pytest.mark.parametrize("tensor,idx,val", PREFILL_CASES, ids=[f"{c[0]}_{'nan' if c[0] != 'v' else 'inf'}" for c in PREFILL_CASES])
def test_prefill_nonfinite_propagates(tensor, idx, val):
    R = _R()
    B, T, Hk, Hv = 2, 200, 2, 4
    w = GI.Workload("nonfinite", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1700)
    inp = _plant(GI.make_inputs(w), tensor, idx, val)
    print(f"[nonfinite] prefill: {tensor}{list(idx)} <- {'NaN' if tensor != 'v' else '+inf'}", flush=True)
    run = R.Prefill(inp, B, T, Hk, Hv, True, True)
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    y_ref, S_ref, _ = O.prefill(inp, B, T, Hk, Hv, True, True)
    o = R.bits(run.o).reshape(B, T, Hv, D)
    y = np.stack([bf16_to_f64(o[c // Hv, :, c % Hv]) for c in range(B * Hv)])
    S = run.state_out.cpu().numpy().reshape(-1, D, D).astype(np.float64)
    _check(y, y_ref, S, S_ref, idx[1], f"prefill {tensor}")


def test_decode_nonfinite_propagates():
    """One step of a small decode batch with +inf in one sequence's v and NaN in another's g:
    those heads' outputs and state turn non-finite where the oracle's do, every other head
    is unaffected."""
    R = _R()
    w = GI.Workload("nonfinite_decode", 4, 1, 2, 6, decode=True, random_state=True, random_conv_state=True, tag=1710)
    inp = _plant(GI.make_inputs(w), "v", (1, 0, 4, 9), INF16)
    inp = _plant(inp, "g", (3, 0, 1), np.float32(np.nan))
    run = R.Decode(inp, w.B, w.Hk, w.Hv, True, True)
    run.run()
    torch.cuda.synchronize()
    y_ref, S_ref, _ = O.prefill(inp, w.B, 1, w.Hk, w.Hv, True, True)
    y = bf16_to_f64(R.bits(run.o)).reshape(w.B * w.Hv, 1, D)
    S = run.state.cpu().numpy().reshape(-1, D, D).astype(np.float64)
    _check(y, y_ref, S, S_ref, 0, "decode v/g")
    assert np.isfinite(y_ref[[c for c in range(w.B * w.Hv) if c not in (1 * 6 + 4, 3 * 6 + 1)]]).all()
