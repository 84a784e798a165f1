"""gdn_prefill_no_workspace: the prefill on the library's static per-GPU scratch, called
through the C ABI, against gdn_prefill with a caller-provided workspace on the same
inputs (the same kernels run, so the results must be bit-identical) and against the
oracle.  Two calls in a row on one GPU, the second with a smaller input, so the second
starts from the first call's leftovers in the scratch; and a shape whose workspace exceeds
the scratch is rejected before any launch."""
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


def _no_workspace(R, run):
    """The same call as run.run(), through gdn_prefill_no_workspace, into fresh outputs."""
    import gated_deltanet_mixer_amd as gdn
    o = torch.full_like(run.o, 0x7fc0)
    state_out = torch.full_like(run.state_out, float("nan"))
    cs_out = torch.full_like(run.conv_state_out, 0x7fc0) if run.conv_state_out is not None else None
    d = run.d
    gdn.gdn_prefill_no_workspace(run.shape, d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"], d["conv_w"],
                                 d["norm_w"], d["state_in"], d["conv_state_in"], o, state_out, cs_out)
    return o, state_out, cs_out


@pytest.mark.parametrize("B,T,Hk,Hv,states", [
    (1, 4096, 16, 16, False),  # the 0.8B-shaped layer
    (2, 1000, 2, 4, True),     # then a smaller batch with initial states and a ragged last chunk
])
def test_no_workspace_matches_workspace_call(B, T, Hk, Hv, states):
    R = _R()
    import gated_deltanet_mixer_amd as gdn
    w = GI.Workload(f"noalloc_{B}_{T}", B, T, Hk, Hv, random_state=states, random_conv_state=states,
                    tag=1800 + B + Hv)
    inp = GI.make_inputs(w)
    print(f"[no_alloc] B={B} T={T} {Hk}/{Hv}: workspace {gdn.gdn_prefill_workspace_size(gdn.make_shape(B, T, Hk, Hv)) / 2**20:.1f} MiB "
          f"of {gdn.GDN_STATIC_SCRATCH_BYTES / 2**20:.0f}", flush=True)
    run = R.Prefill(inp, B, T, Hk, Hv, True, True)
    run.run()
    o, state_out, cs_out = _no_workspace(R, run)
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    assert torch.equal(o, run.o), "outputs differ from gdn_prefill's"
    assert torch.equal(state_out, run.state_out), "final states differ from gdn_prefill's"
    assert torch.equal(cs_out, run.conv_state_out), "conv tails differ from gdn_prefill's"
    y_ref, S_ref, cs_ref = O.prefill(inp, B, T, Hk, Hv, True, True)
    ob = R.bits(o).reshape(B, T, Hv, D)
    y = np.stack([bf16_to_f64(ob[c // Hv, :, c % Hv]) for c in range(B * Hv)])
    eo, es = out_errors(y, y_ref), state_error(state_out.cpu().numpy().reshape(-1, D, D), S_ref)
    print(f"[no_alloc] B={B} T={T}: bit-identical to gdn_prefill; e_out={eo['e_out']:.3e} e_state={es:.3e}",
          flush=True)
    assert eo["nonfinite"] == 0 and eo["e_out"] <= OUT_TOL and es <= STATE_TOL
    np.testing.assert_array_equal(R.bits(cs_out), cs_ref)


def test_no_workspace_falls_back_to_the_plain_pass():
    """The 0.8B-shaped layer at T = 8192: the library plans the two-level scan, whose workspace
    (about 190 MiB) exceeds the scratch, while the plain sequential pass's (about 120 MiB) fits.
    The allocation-free call then runs the plain pass: bit-identical to gdn_prefill held to the
    plain pass (prefill_segments = 1), and within the oracle's tolerance."""
    R = _R()
    import gated_deltanet_mixer_amd as gdn
    B, T, Hk, Hv = 1, 8192, 16, 16
    assert gdn.gdn_prefill_workspace_size(gdn.make_shape(B, T, Hk, Hv)) > gdn.GDN_STATIC_SCRATCH_BYTES
    assert gdn.gdn_prefill_workspace_size(gdn.make_shape(B, T, Hk, Hv, segments=1)) <= gdn.GDN_STATIC_SCRATCH_BYTES
    w = GI.Workload("noalloc_fallback", B, T, Hk, Hv, random_state=True, random_conv_state=True, tag=1830)
    inp = GI.make_inputs(w)
    print(f"[no_alloc] fallback B={B} T={T} {Hk}/{Hv}", flush=True)
    run = R.Prefill(inp, B, T, Hk, Hv, True, True, segments=1)
    run.run()
    # the library's own plan choice (prefill_segments = 0), not the plain-pass shape of `run`
    o = torch.full_like(run.o, 0x7fc0)
    state_out = torch.full_like(run.state_out, float("nan"))
    cs_out = torch.full_like(run.conv_state_out, 0x7fc0)
    d = run.d
    gdn.gdn_prefill_no_workspace(gdn.make_shape(B, T, Hk, Hv), d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"],
                                 d["conv_w"], d["norm_w"], d["state_in"], d["conv_state_in"], o, state_out, cs_out)
    torch.cuda.synchronize()
    assert run.exchange_error_word() == 0
    assert torch.equal(o, run.o) and torch.equal(state_out, run.state_out) and torch.equal(cs_out, run.conv_state_out)


def test_no_workspace_rejects_shapes_beyond_the_scratch():
    """A well-formed call whose workspace would exceed the scratch is rejected by a host check,
    before any HIP call (disjoint fake device addresses, never dereferenced)."""
    import ctypes as C
    import gated_deltanet_mixer_amd as gdn
    from tests.test_abi_host import _prefill_args
    shape = gdn.make_shape(1, 16384, 16, 32)
    assert gdn.gdn_prefill_workspace_size(shape) > gdn.GDN_STATIC_SCRATCH_BYTES
    a = _prefill_args(shape)
    rc = gdn._lib.gdn_prefill_no_workspace(C.byref(shape), a["q"], a["k"], a["v"], a["g"], a["beta"], a["z"],
                                           a["conv_w"], a["norm_w"], a["state_in"], a["conv_state_in"], a["o"],
                                           a["state_out"], a["conv_state_out"], None)
    assert rc == gdn.GDN_EWORKSPACE
    small = gdn.make_shape(1, 1024, 16, 16)
    a = _prefill_args(small)
    rc = gdn._lib.gdn_prefill_no_workspace(C.byref(small), None, a["k"], a["v"], a["g"], a["beta"], a["z"],
                                           a["conv_w"], a["norm_w"], a["state_in"], a["conv_state_in"], a["o"],
                                           a["state_out"], a["conv_state_out"], None)
    assert rc == gdn.GDN_EINVAL  # null q
