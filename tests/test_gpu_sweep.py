"""A seeded sweep of small configurations through every prefill and decode entry point,
each compared with the oracle (same tolerances as every other parity test).

The hand-picked cases elsewhere cover the edges one at a time; this sweep draws
combinations of them: head ratios, ragged lengths, the conv and norm switches,
random initial states or none, packed batches of random lengths, forced segment
counts of the two-level scan, and multi-token decode with snapshots.  The draws
come from two fixed seeds (the second with more and wider heads), so every run checks
the same configurations.
"""
import os

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


def _configs(n=12):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([GI.SEED_BASE, 1600])))
    out = []
    for i in range(n):
        Hk = int(rng.choice([1, 2, 4]))
        r = int(rng.choice([1, 2, 3]))
        out.append(dict(
            i=i, Hk=Hk, Hv=Hk * r, B=int(rng.integers(1, 4)), T=int(rng.integers(1, 400)),
            conv=bool(rng.random() < 0.8), norm=bool(rng.random() < 0.8), rs=bool(rng.random() < 0.6),
            nseg=int(rng.choice([0, 0, 2, 3, 5])),
            lengths=[int(x) for x in rng.integers(1, 200, size=int(rng.integers(1, 6)))],
            Tdec=int(rng.integers(1, 9))))
    return out


def _wide_configs(n=24):
    # wider draws: up to 8 key heads and 4 value heads per key head, so that B Hv crosses 32
    # (two-tile slices) and the sequential pass runs more items than one round of workgroups
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([GI.SEED_BASE, 1777])))
    out = []
    for i in range(n):
        Hk = int(rng.choice([1, 2, 4, 8]))
        r = int(rng.choice([1, 2, 3, 4]))
        out.append(dict(
            i=100 + i, Hk=Hk, Hv=Hk * r, B=int(rng.integers(1, 5)), T=int(rng.integers(1, 700)),
            conv=bool(rng.random() < 0.8), norm=bool(rng.random() < 0.8), rs=bool(rng.random() < 0.6),
            nseg=int(rng.choice([0, 0, 2, 3, 5])),
            lengths=[int(x) for x in rng.integers(1, 300, size=int(rng.integers(1, 7)))],
            Tdec=int(rng.integers(1, 9))))
    return out


CONFIGS = _configs() + _wide_configs()


def _ids(c):
    return f"c{c['i']}"


def _check(label, y, y_ref, S, S_ref):
    eo, es = out_errors(y, y_ref), state_error(S, S_ref)
    assert eo["nonfinite"] == 0, label
    assert eo["e_out"] <= OUT_TOL, (label, eo)
    assert es <= STATE_TOL, (label, es)
    return eo["e_out"], es


@pytest.mark.parametrize("c", CONFIGS, ids=_ids)
def test_sweep_prefill(c):
    """gdn_prefill with the drawn shape, switches and segment count."""
    R = _R()
    B, T, Hk, Hv, conv, norm = c["B"], c["T"], c["Hk"], c["Hv"], c["conv"], c["norm"]
    w = GI.Workload(f"sweep_{c['i']}", B, T, Hk, Hv, conv=conv, norm=norm, random_state=c["rs"],
                    random_conv_state=c["rs"] and conv, tag=1600 + c["i"])
    inp = GI.make_inputs(w)
    label = f"prefill {c}"
    print(f"[sweep] {label}", flush=True)
    # segment count: 0 draws the plain sequential pass (forced with 1), n >= 2 n segments
    run = R.Prefill(inp, B, T, Hk, Hv, conv, norm, segments=max(1, c["nseg"]))
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    y_ref, S_ref, cs_ref = O.prefill(inp, B, T, Hk, Hv, conv, norm)
    o = R.bits(run.o).reshape(B, T, Hv, D)
    y = np.stack([bf16_to_f64(o[i // Hv, :, i % Hv]) for i in range(B * Hv)])
    _check(label, y, y_ref, run.state_out.cpu().numpy().reshape(-1, D, D), S_ref)
    if conv:
        np.testing.assert_array_equal(R.bits(run.conv_state_out), cs_ref)


@pytest.mark.parametrize("c", CONFIGS, ids=_ids)
def test_sweep_packed(c):
    """gdn_prefill_packed over the drawn lengths; each sequence against the oracle run alone."""
    R = _R()
    Hk, Hv, conv, norm, lengths = c["Hk"], c["Hv"], c["conv"], c["norm"], c["lengths"]
    T = sum(lengths)
    tok = GI.make_inputs(GI.Workload(f"sweep_pk_{c['i']}", 1, T, Hk, Hv, conv=conv, norm=norm, tag=1650 + c["i"]))
    st = GI.make_inputs(GI.Workload(f"sweep_pks_{c['i']}", len(lengths), 1, Hk, Hv, conv=conv, norm=norm,
                                    random_state=True, random_conv_state=conv, tag=1700 + c["i"]))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    print(f"[sweep] packed {lengths} Hk={Hk} Hv={Hv} conv={conv} norm={norm}", flush=True)
    run = R.PackedPrefill(tok, cu, T, Hk, Hv, conv, norm, state_in=st["state"], conv_state_in=st.get("conv_state"))
    run.run()
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    o = R.bits(run.o).reshape(T, Hv, D)
    S = run.state_out.cpu().numpy()
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        seq = dict(tok)
        for n in ("q", "k", "v", "z", "g", "beta"):
            if tok.get(n) is not None:
                seq[n] = tok[n][:, a:b]
        y_ref, S_ref, cs_ref = O.prefill(seq, 1, b - a, Hk, Hv, conv, norm, state_in=st["state"][i:i + 1],
                                         conv_state_in=None if not conv else st["conv_state"][i:i + 1])
        y = np.stack([bf16_to_f64(o[a:b, h]) for h in range(Hv)])
        _check(f"packed {lengths} sequence {i}", y, y_ref, S[i], S_ref)
        if conv:
            np.testing.assert_array_equal(R.bits(run.conv_state_out)[i], cs_ref[0])


@pytest.mark.parametrize("c", CONFIGS, ids=_ids)
def test_sweep_decode_multi(c):
    """gdn_decode_multi with the drawn token count, snapshots included."""
    R = _R()
    import gated_deltanet_mixer_amd as gdn
    B, Hk, Hv, conv, norm, T = c["B"], c["Hk"], c["Hv"], c["conv"], c["norm"], c["Tdec"]
    w = GI.Workload(f"sweep_dec_{c['i']}", B, T, Hk, Hv, conv=conv, norm=norm, random_state=True,
                    random_conv_state=conv, tag=1750 + c["i"])
    inp = GI.make_inputs(w)
    print(f"[sweep] decode B={B} T={T} Hk={Hk} Hv={Hv} conv={conv} norm={norm}", flush=True)
    d = {n: R.to_dev(inp.get(n)) for n in ("q", "k", "v", "g", "beta")}
    z = R.to_dev(inp["z"]) if norm else None
    cw = R.to_dev(inp["conv_w"]) if conv else None
    nw = R.to_dev(inp["norm_w"]) if norm else None
    state = R.to_dev(inp["state"])
    Cc = 2 * Hk * D + Hv * D
    cs = R.to_dev(inp["conv_state"]) if conv else None
    o = torch.empty((B, T, Hv, D), dtype=torch.int16, device="cuda")
    snaps = torch.empty((max(T - 1, 1), B, Hv, D, D), device="cuda") if T > 1 else None
    csnaps = torch.empty((max(T - 1, 1), B, 3, Cc), dtype=torch.int16, device="cuda") if (T > 1 and conv) else None
    gdn.gdn_decode_multi(gdn.make_shape(B, T, Hk, Hv, conv=conv, norm=norm), d["q"], d["k"], d["v"], d["g"],
                         d["beta"], z, cw, nw, state, cs, o, snaps, csnaps)
    torch.cuda.synchronize()
    y_ref, S_ref, cs_ref = O.prefill(inp, B, T, Hk, Hv, conv, norm)
    ob = R.bits(o)
    y = np.stack([bf16_to_f64(ob[i // Hv, :, i % Hv]) for i in range(B * Hv)])
    _check(f"decode {c}", y, y_ref, state.cpu().numpy().reshape(-1, D, D), S_ref)
    if conv:
        np.testing.assert_array_equal(R.bits(cs), cs_ref)
    for t in range(T - 1):
        pre = dict(inp)
        for n in ("q", "k", "v", "z", "g", "beta"):
            if inp.get(n) is not None:
                pre[n] = np.ascontiguousarray(inp[n][:, :t + 1])
        _, St_ref, cst_ref = O.prefill(pre, B, t + 1, Hk, Hv, conv, norm)
        assert state_error(snaps[t].cpu().numpy().reshape(-1, D, D), St_ref) <= STATE_TOL, t
        if conv:
            np.testing.assert_array_equal(R.bits(csnaps[t]), cst_ref)
