"""Host-side checks of the C ABI: the library loads, exports every entry point
include/gdn.h declares, and rejects bad arguments before any HIP call (so
these run without a GPU)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

gdn = pytest.importorskip("gated_deltanet_mixer_amd")

FAKE = 1 << 40  # a 256-byte aligned "device address"; never dereferenced by a rejected call
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["gdn_decode_step", "gdn_decode_step_gate_logits", "gdn_last_error", "gdn_prefill",
         "gdn_prefill_gate_logits", "gdn_prefill_packed", "gdn_prefill_packed_gate_logits",
         "gdn_decode_multi", "gdn_decode_multi_gate_logits", "gdn_prefill_check", "gdn_prefill_no_workspace",
         "gdn_prefill_workspace_size", "gdn_state_init", "gdn_status_string"])


def test_last_error_is_a_string_before_any_failure():
    assert isinstance(gdn.gdn_last_error(), str)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    for fn in declared_functions():
        assert fn in exported, fn
        assert hasattr(gdn._lib, fn)


def test_binding_names_match_the_abi():
    for fn in declared_functions():
        assert callable(getattr(gdn, fn)), fn


def test_status_strings():
    for code in (gdn.GDN_OK, gdn.GDN_EINVAL, gdn.GDN_EUNSUPPORTED, gdn.GDN_EHIP, gdn.GDN_EWORKSPACE):
        s = gdn.gdn_status_string(code)
        assert s and s != "unknown status"
    assert gdn.gdn_status_string(12345) == "unknown status"


def _prefill_args(shape, **over):
    """Arguments of a well-formed prefill on fake, disjoint device addresses."""
    B, T, Hk, Hv = shape.B, shape.T, shape.Hk, shape.Hv
    base = FAKE
    sizes = dict(q=B * T * Hk * 256, k=B * T * Hk * 256, v=B * T * Hv * 256, g=B * T * Hv * 4,
                 beta=B * T * Hv * 4, z=B * T * Hv * 256, conv_w=(2 * Hk + Hv) * 128 * 8, norm_w=256,
                 state_in=B * Hv * 65536, conv_state_in=B * 3 * (2 * Hk + Hv) * 256, o=B * T * Hv * 256,
                 state_out=B * Hv * 65536, conv_state_out=B * 3 * (2 * Hk + Hv) * 256)
    args = {}
    for n, sz in sizes.items():
        args[n] = base
        base += ((sz + MB - 1) // MB + 1) * MB
    args["workspace"] = base
    if "workspace_bytes" not in over:
        args["workspace_bytes"] = gdn.gdn_prefill_workspace_size(shape)
    args.update(over)
    return args


def _call_prefill(shape, **over):
    a = _prefill_args(shape, **over)
    return gdn._lib.gdn_prefill(C.byref(shape), a["q"], a["k"], a["v"], a["g"], a["beta"], a["z"], a["conv_w"],
                                a["norm_w"], a["state_in"], a["conv_state_in"], a["o"], a["state_out"],
                                a["conv_state_out"], a["workspace"], a["workspace_bytes"], None)


def _shape(**kw):
    s = dict(B=2, T=100, Hk=2, Hv=6, conv=True, norm=True)
    s.update(kw)
    return gdn.make_shape(**s)


def test_workspace_size_scales_with_tokens():
    a = gdn.gdn_prefill_workspace_size(_shape(T=64))
    b = gdn.gdn_prefill_workspace_size(_shape(T=6400))
    assert b > a > 0
    assert b >= 2 * 6400 * 2 * 2 * 128 * 2  # fp16 q/k operands


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, gdn.GDN_EINVAL), ("T", 0, gdn.GDN_EINVAL), ("Hv", 5, gdn.GDN_EINVAL),
    ("Dk", 64, gdn.GDN_EUNSUPPORTED), ("Dv", 256, gdn.GDN_EUNSUPPORTED),
    ("conv_width", 3, gdn.GDN_EUNSUPPORTED), ("flags", 8, gdn.GDN_EINVAL),
])
def test_bad_shapes_rejected(field, value, code):
    s = _shape()
    setattr(s, field, value)
    n = C.c_size_t(0)
    assert gdn._lib.gdn_prefill_workspace_size(C.byref(s), C.byref(n)) == code
    assert _call_prefill(s, workspace_bytes=1 << 40) == code


def test_null_and_misaligned_pointers_rejected():
    s = _shape()
    assert gdn._lib.gdn_prefill(None, *([FAKE] * 14), 1 << 30, None) == gdn.GDN_EINVAL
    for name in ("q", "k", "v", "g", "beta", "o", "state_out", "workspace"):
        assert _call_prefill(s, **{name: None}) == gdn.GDN_EINVAL, name
    assert _call_prefill(s, z=None) == gdn.GDN_EINVAL            # norm on needs z
    assert _call_prefill(s, conv_w=None) == gdn.GDN_EINVAL       # conv on needs weights
    assert _call_prefill(s, q=FAKE + 8) == gdn.GDN_EINVAL        # 16-byte alignment
    assert _call_prefill(s, g=FAKE + 2) == gdn.GDN_EINVAL        # 4-byte alignment


def test_overlaps_rejected():
    s = _shape()
    a = _prefill_args(s)
    assert _call_prefill(s, o=a["q"]) == gdn.GDN_EINVAL
    assert _call_prefill(s, conv_state_out=a["conv_state_in"]) == gdn.GDN_EINVAL
    assert _call_prefill(s, workspace=a["v"]) == gdn.GDN_EINVAL
    assert _call_prefill(s, state_out=a["state_in"] + 1024) == gdn.GDN_EINVAL


def test_small_workspace_rejected_last():
    s = _shape()
    ws = gdn.gdn_prefill_workspace_size(s)
    assert _call_prefill(s, workspace_bytes=ws - 1) == gdn.GDN_EWORKSPACE


def test_conv_state_without_conv_rejected():
    s = _shape(conv=False)
    assert _call_prefill(s, conv_w=None) == gdn.GDN_EINVAL  # conv_state_in/out given without conv


def test_decode_rejects_bad_arguments():
    s = _shape()
    # q, k, v, g, beta, z, conv_w, norm_w, state, conv_state, o
    ok = [FAKE + i * (64 * MB) for i in range(11)]
    f = gdn._lib.gdn_decode_step
    assert f(None, *ok, None) == gdn.GDN_EINVAL
    bad = list(ok)
    bad[0] = FAKE + 4
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    bad = list(ok)
    bad[9] = None  # conv state with conv on
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    bad = list(ok)
    bad[10] = ok[0]  # o on top of q
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    s2 = _shape(Hk=1, Hv=65)
    assert f(C.byref(s2), *ok, None) == gdn.GDN_EUNSUPPORTED


def _call_prefill_logits(shape, A_log, dt_bias, **over):
    a = _prefill_args(shape, **over)
    return gdn._lib.gdn_prefill_gate_logits(
        C.byref(shape), a["q"], a["k"], a["v"], a["g"], a["beta"], A_log, dt_bias, a["z"], a["conv_w"],
        a["norm_w"], a["state_in"], a["conv_state_in"], a["o"], a["state_out"], a["conv_state_out"],
        a["workspace"], a["workspace_bytes"], None)


def test_gate_logit_entry_points_reject_bad_arguments():
    s = _shape()
    a = _prefill_args(s)
    gates = a["workspace"] + (1 << 34)          # two fp32 [Hv] arrays far from everything else
    assert _call_prefill_logits(s, None, gates) == gdn.GDN_EINVAL
    assert _call_prefill_logits(s, gates, None) == gdn.GDN_EINVAL
    assert _call_prefill_logits(s, gates + 2, gates + 1024) == gdn.GDN_EINVAL   # 4-byte alignment
    assert _call_prefill_logits(s, a["o"], gates) == gdn.GDN_EINVAL             # A_log inside o
    assert _call_prefill_logits(s, gates, a["workspace"]) == gdn.GDN_EINVAL     # dt_bias inside the workspace
    assert _call_prefill_logits(s, gates, gates + 1024, q=None) == gdn.GDN_EINVAL
    ok = [FAKE + i * (64 * MB) for i in range(13)]  # q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state, conv_state, o
    f = gdn._lib.gdn_decode_step_gate_logits
    bad = list(ok)
    bad[5] = None
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    bad = list(ok)
    bad[6] = ok[12]  # dt_bias inside o
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL


def _call_packed(shape, cu, **over):
    a = _prefill_args(shape, **over)
    return gdn._lib.gdn_prefill_packed(C.byref(shape), cu, a["q"], a["k"], a["v"], a["g"], a["beta"], a["z"],
                                       a["conv_w"], a["norm_w"], a["state_in"], a["conv_state_in"], a["o"],
                                       a["state_out"], a["conv_state_out"], a["workspace"], a["workspace_bytes"],
                                       None)


def test_packed_workspace_covers_every_packing():
    """Slots for floor(T / 64) + B chunks: the most that B sequences of T tokens in all
    can have (each sequence's last chunk may be partial)."""
    even = gdn.gdn_prefill_workspace_size(_shape(B=1, T=6400))
    packed = gdn.gdn_prefill_workspace_size(_shape(B=100, T=6400, packed=True))
    assert packed > even
    many = gdn.gdn_prefill_workspace_size(_shape(B=6400, T=6400, packed=True))  # one token each
    assert many >= 6400 * 2 * (2 * 64 * 128 + 128 * 64) * 2


def test_packed_entry_points_reject_bad_arguments():
    s = _shape(B=3, T=300, packed=True)
    cu = FAKE + (1 << 36)                       # the [B + 1] offsets, far from everything else
    assert _call_packed(s, None) == gdn.GDN_EINVAL
    assert _call_packed(s, cu + 2) == gdn.GDN_EINVAL               # 4-byte alignment
    a = _prefill_args(s)
    assert _call_packed(s, a["o"]) == gdn.GDN_EINVAL               # offsets inside o
    assert _call_packed(s, a["workspace"]) == gdn.GDN_EINVAL       # offsets inside the workspace
    assert _call_packed(s, cu, q=None) == gdn.GDN_EINVAL
    assert _call_packed(s, cu, workspace_bytes=gdn.gdn_prefill_workspace_size(s) - 1) == gdn.GDN_EWORKSPACE
    even = _shape(B=3, T=300)
    assert _call_packed(even, cu) == gdn.GDN_EINVAL                # the shape must carry GDN_PACKED
    assert _call_prefill(s, workspace_bytes=1 << 40) == gdn.GDN_EINVAL   # and gdn_prefill refuses it
    f = gdn._lib.gdn_prefill_packed_gate_logits
    a = _prefill_args(s)
    gates = a["workspace"] + (1 << 34)
    args = [a["q"], a["k"], a["v"], a["g"], a["beta"]]
    rest = [a["z"], a["conv_w"], a["norm_w"], a["state_in"], a["conv_state_in"], a["o"], a["state_out"],
            a["conv_state_out"], a["workspace"], a["workspace_bytes"], None]
    assert f(C.byref(s), cu, *args, None, gates, *rest) == gdn.GDN_EINVAL
    assert f(C.byref(s), None, *args, gates, gates + 1024, *rest) == gdn.GDN_EINVAL
    ok = [FAKE + i * (64 * MB) for i in range(11)]
    assert gdn._lib.gdn_decode_step(C.byref(s), *ok, None) == gdn.GDN_EINVAL  # decode has nothing to pack


def test_decode_multi_rejects_bad_arguments():
    # q, k, v, g, beta, z, conv_w, norm_w, state, conv_state, o, state_snaps, conv_snaps
    ok = [FAKE + i * (256 * MB) for i in range(13)]
    f = gdn._lib.gdn_decode_multi
    for T, code in ((0, gdn.GDN_EINVAL), (9, gdn.GDN_EINVAL)):
        assert f(C.byref(_shape(T=T)), *ok, None) == code, T
    s = _shape(T=4)
    bad = list(ok)
    bad[11] = ok[8] + 65536             # snapshots inside the state
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    bad = list(ok)
    bad[12] = ok[0]                     # conv snapshots on top of q
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    bad = list(ok)
    bad[11] = ok[11] + 8                # 16-byte alignment
    assert f(C.byref(s), *bad, None) == gdn.GDN_EINVAL
    s0 = _shape(T=4, conv=False)        # conv snapshots without a conv
    bad = list(ok)
    bad[6] = bad[9] = None
    assert f(C.byref(s0), *bad, None) == gdn.GDN_EINVAL
    bad[12] = None
    assert f(C.byref(_shape(T=8, Hk=1, Hv=64)), *ok, None) == gdn.GDN_EUNSUPPORTED  # LDS of 8 tokens x 64 heads
    g = gdn._lib.gdn_decode_multi_gate_logits
    okg = ok[:5] + [FAKE + 13 * 256 * MB, FAKE + 14 * 256 * MB] + ok[5:]
    bad = list(okg)
    bad[5] = None                       # A_log missing
    assert g(C.byref(s), *bad, None) == gdn.GDN_EINVAL


def test_state_init_rejects_bad_arguments():
    s = _shape()
    f = gdn._lib.gdn_state_init
    assert f(C.byref(s), None, None, None) == gdn.GDN_EINVAL
    assert f(C.byref(s), FAKE + 4, None, None) == gdn.GDN_EINVAL
    s0 = _shape(conv=False)
    assert f(C.byref(s0), FAKE, FAKE + MB * 512, None) == gdn.GDN_EINVAL


def test_one_hip_runtime_per_process():
    """Importing the binding first must not load a second HIP runtime next to
    torch's (two runtimes each claim the device; the second sees none)."""
    code = ("import gated_deltanet_mixer_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT, check=True).stdout
    assert out.strip() == "1"


def test_two_level_plan_sizes_the_workspace():
    """Few heads and a long sequence: the plan splits the sequence into segments, and the
    workspace grows by their read-outs (32 KB per chunk and head) and segment maps.  Up to 16
    heads (whose sequential pass would fill at most half of the chip) take two segments from 64
    chunks on, the 0.8B-shaped layer among them; the larger benchmark shapes, shorter sequences
    of 16 heads and packed batches keep the plain sequential pass."""
    plain = gdn.gdn_prefill_workspace_size(_shape(B=1, T=262144, Hk=1, Hv=3, segments=1))
    planned = gdn.gdn_prefill_workspace_size(_shape(B=1, T=262144, Hk=1, Hv=3))
    assert planned - plain >= (262144 // 64) * 3 * 32 * 1024
    plain = gdn.gdn_prefill_workspace_size(_shape(B=1, T=4096, Hk=16, Hv=16, segments=1))
    planned = gdn.gdn_prefill_workspace_size(_shape(B=1, T=4096, Hk=16, Hv=16))
    assert planned == gdn.gdn_prefill_workspace_size(_shape(B=1, T=4096, Hk=16, Hv=16, segments=2))
    assert planned - plain >= 64 * 16 * 32 * 1024
    for kw in (dict(B=1, T=4032, Hk=16, Hv=16), dict(B=1, T=65536, Hk=16, Hv=48), dict(B=4, T=16384, Hk=16, Hv=32),
               dict(B=3, T=65536, Hk=1, Hv=3, packed=True)):
        assert gdn.gdn_prefill_workspace_size(_shape(**kw)) == gdn.gdn_prefill_workspace_size(_shape(**kw, segments=1))
    # a forced split asks for more only when the sequence has more than one chunk
    short_plain = gdn.gdn_prefill_workspace_size(_shape(B=1, T=1000, Hk=1, Hv=3, segments=1))
    assert gdn.gdn_prefill_workspace_size(_shape(B=1, T=1000, Hk=1, Hv=3, segments=4)) > short_plain
    one_chunk = gdn.gdn_prefill_workspace_size(_shape(B=1, T=64, Hk=1, Hv=3, segments=1))
    assert gdn.gdn_prefill_workspace_size(_shape(B=1, T=64, Hk=1, Hv=3, segments=4)) == one_chunk


def test_segment_field_is_checked():
    """prefill_segments must not be negative, and a packed batch takes no forced split."""
    n = C.c_size_t(0)
    assert gdn._lib.gdn_prefill_workspace_size(C.byref(_shape(segments=-1)), C.byref(n)) == gdn.GDN_EINVAL
    assert gdn._lib.gdn_prefill_workspace_size(C.byref(_shape(packed=True, segments=2)), C.byref(n)) == gdn.GDN_EINVAL
    assert gdn._lib.gdn_prefill_workspace_size(C.byref(_shape(packed=True, segments=1)), C.byref(n)) == gdn.GDN_OK