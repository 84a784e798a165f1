"""Python binding of the Gated DeltaNet mixer C ABI (include/gdn.h).

Argument marshalling only: every step of the mixer runs in the HIP kernels of
libgdn.so.  Tensors are torch tensors on the GPU (bf16 tensors may be
torch.bfloat16 or 16-bit integer views of the same bits); ``None`` passes a
NULL pointer.  Work is enqueued on torch's current stream unless ``stream`` is
given.  A non-zero status raises GdnError.  The import fails loudly when
libgdn.so has not been built (``python gated_deltanet_mixer_amd/build.py``).
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_EINVAL = -1
GDN_EUNSUPPORTED = -2
GDN_EHIP = -3
GDN_EWORKSPACE = -4
GDN_ETIMEOUT = -5
GDN_ESKIPPED = -6
GDN_NO_NORM = 1
GDN_PACKED = 2


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = f"{fn}: {gdn_status_string(status)} (status {status})"
        if status == GDN_EHIP:
            msg += f": {gdn_last_error()}"
        super().__init__(msg)
        self.status = status


class gdn_shape(C.Structure):
    _fields_ = [("B", C.c_int32), ("T", C.c_int32), ("Hk", C.c_int32), ("Hv", C.c_int32),
                ("Dk", C.c_int32), ("Dv", C.c_int32), ("conv_width", C.c_int32), ("flags", C.c_uint32),
                ("eps_l2", C.c_float), ("eps_norm", C.c_float), ("prefill_segments", C.c_int32)]


def make_shape(B: int, T: int, Hk: int, Hv: int, conv: bool = True, norm: bool = True,
               eps_l2: float = 1e-6, eps_norm: float = 1e-6, Dk: int = 128, Dv: int = 128,
               packed: bool = False, segments: int = 0) -> gdn_shape:
    """packed: B sequences of T tokens in all (gdn_prefill_packed).  segments: 0 lets the
    library choose between the plain sequential pass and the two-level scan, 1 forces the
    plain pass, n >= 2 asks for n segments."""
    flags = (0 if norm else GDN_NO_NORM) | (GDN_PACKED if packed else 0)
    return gdn_shape(B, T, Hk, Hv, Dk, Dv, 4 if conv else 0, flags, eps_l2, eps_norm, segments)


# torch ships its own copy of the HIP runtime under the same soname.  Loading
# torch first makes libgdn.so bind to that copy, so the process holds one HIP
# runtime and the library sees the device and the streams torch created.
try:
    import torch  # noqa: F401
except ImportError:  # host-only use (argument checks, symbol inspection)
    pass

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python gated_deltanet_mixer_amd/build.py`")
_lib = C.CDLL(LIB_PATH)
_vp = C.c_void_p
_sp = C.POINTER(gdn_shape)
_lib.gdn_status_string.argtypes = [C.c_int]
_lib.gdn_status_string.restype = C.c_char_p
_lib.gdn_last_error.argtypes = []
_lib.gdn_last_error.restype = C.c_char_p
_lib.gdn_state_init.argtypes = [_sp, _vp, _vp, _vp]
_lib.gdn_prefill_workspace_size.argtypes = [_sp, C.POINTER(C.c_size_t)]
_lib.gdn_prefill.argtypes = [_sp] + [_vp] * 14 + [C.c_size_t, _vp]
_lib.gdn_decode_step.argtypes = [_sp] + [_vp] * 12
_lib.gdn_prefill_gate_logits.argtypes = [_sp] + [_vp] * 16 + [C.c_size_t, _vp]
_lib.gdn_decode_step_gate_logits.argtypes = [_sp] + [_vp] * 14
_lib.gdn_prefill_packed.argtypes = [_sp] + [_vp] * 15 + [C.c_size_t, _vp]
_lib.gdn_decode_multi.argtypes = [_sp] + [_vp] * 14
_lib.gdn_decode_multi_gate_logits.argtypes = [_sp] + [_vp] * 16
_lib.gdn_prefill_packed_gate_logits.argtypes = [_sp] + [_vp] * 17 + [C.c_size_t, _vp]
_lib.gdn_prefill_check.argtypes = [_vp, C.c_size_t, _vp]
_lib.gdn_prefill_no_workspace.argtypes = [_sp] + [_vp] * 13 + [_vp]

EXPORTED = ("gdn_state_init", "gdn_prefill_workspace_size", "gdn_prefill", "gdn_decode_step",
            "gdn_prefill_gate_logits", "gdn_decode_step_gate_logits", "gdn_prefill_packed",
            "gdn_prefill_packed_gate_logits", "gdn_decode_multi", "gdn_decode_multi_gate_logits",
            "gdn_prefill_check", "gdn_prefill_no_workspace", "gdn_status_string", "gdn_last_error")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != GDN_OK:
        raise GdnError(fn, rc)


def gdn_status_string(status: int) -> str:
    return _lib.gdn_status_string(status).decode()


def gdn_last_error() -> str:
    return _lib.gdn_last_error().decode()


def gdn_state_init(shape: gdn_shape, state, conv_state=None, stream=None) -> None:
    _check("gdn_state_init", _lib.gdn_state_init(C.byref(shape), _ptr(state), _ptr(conv_state), _stream(stream)))


def gdn_prefill_workspace_size(shape: gdn_shape) -> int:
    n = C.c_size_t(0)
    _check("gdn_prefill_workspace_size", _lib.gdn_prefill_workspace_size(C.byref(shape), C.byref(n)))
    return int(n.value)


def gdn_prefill(shape: gdn_shape, q, k, v, g, beta, z, conv_w, norm_w, state_in, conv_state_in,
                o, state_out, conv_state_out, workspace, workspace_bytes: int | None = None,
                stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.gdn_prefill(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                          _ptr(conv_w), _ptr(norm_w), _ptr(state_in), _ptr(conv_state_in), _ptr(o),
                          _ptr(state_out), _ptr(conv_state_out), _ptr(workspace), int(workspace_bytes),
                          _stream(stream))
    _check("gdn_prefill", rc)


GDN_STATIC_SCRATCH_BYTES = 128 << 20


def gdn_prefill_no_workspace(shape: gdn_shape, q, k, v, g, beta, z, conv_w, norm_w, state_in, conv_state_in,
                             o, state_out, conv_state_out, stream=None) -> None:
    """gdn_prefill on the library's static per-GPU scratch (no workspace, no allocation;
    shapes up to GDN_STATIC_SCRATCH_BYTES of workspace; calls on one GPU must not overlap)."""
    rc = _lib.gdn_prefill_no_workspace(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                                       _ptr(conv_w), _ptr(norm_w), _ptr(state_in), _ptr(conv_state_in), _ptr(o),
                                       _ptr(state_out), _ptr(conv_state_out), _stream(stream))
    _check("gdn_prefill_no_workspace", rc)


def gdn_prefill_check(workspace, workspace_bytes: int | None = None, stream=None) -> None:
    """Wait for the stream and raise GdnError if the last prefill on this workspace left
    an error bit (a timed-out wait between workgroups, or a skipped packed sequence)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("gdn_prefill_check", _lib.gdn_prefill_check(_ptr(workspace), int(workspace_bytes), _stream(stream)))


def gdn_decode_step(shape: gdn_shape, q, k, v, g, beta, z, conv_w, norm_w, state, conv_state, o,
                    stream=None) -> None:
    rc = _lib.gdn_decode_step(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                              _ptr(conv_w), _ptr(norm_w), _ptr(state), _ptr(conv_state), _ptr(o),
                              _stream(stream))
    _check("gdn_decode_step", rc)


def gdn_prefill_gate_logits(shape: gdn_shape, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state_in,
                            conv_state_in, o, state_out, conv_state_out, workspace,
                            workspace_bytes: int | None = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.gdn_prefill_gate_logits(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                                      _ptr(dt_bias), _ptr(z), _ptr(conv_w), _ptr(norm_w), _ptr(state_in),
                                      _ptr(conv_state_in), _ptr(o), _ptr(state_out), _ptr(conv_state_out),
                                      _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("gdn_prefill_gate_logits", rc)


def gdn_decode_step_gate_logits(shape: gdn_shape, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state,
                                conv_state, o, stream=None) -> None:
    rc = _lib.gdn_decode_step_gate_logits(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                          _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(conv_w), _ptr(norm_w),
                                          _ptr(state), _ptr(conv_state), _ptr(o), _stream(stream))
    _check("gdn_decode_step_gate_logits", rc)


def gdn_prefill_packed(shape: gdn_shape, cu_seqlens, q, k, v, g, beta, z, conv_w, norm_w, state_in,
                       conv_state_in, o, state_out, conv_state_out, workspace,
                       workspace_bytes: int | None = None, stream=None) -> None:
    """cu_seqlens: int32 device tensor [B + 1]; the shape from make_shape(..., packed=True)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.gdn_prefill_packed(C.byref(shape), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                 _ptr(beta), _ptr(z), _ptr(conv_w), _ptr(norm_w), _ptr(state_in),
                                 _ptr(conv_state_in), _ptr(o), _ptr(state_out), _ptr(conv_state_out),
                                 _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("gdn_prefill_packed", rc)


def gdn_prefill_packed_gate_logits(shape: gdn_shape, cu_seqlens, q, k, v, a, b, A_log, dt_bias, z, conv_w,
                                   norm_w, state_in, conv_state_in, o, state_out, conv_state_out, workspace,
                                   workspace_bytes: int | None = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = _lib.gdn_prefill_packed_gate_logits(
        C.byref(shape), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), _ptr(z), _ptr(conv_w), _ptr(norm_w), _ptr(state_in), _ptr(conv_state_in), _ptr(o),
        _ptr(state_out), _ptr(conv_state_out), _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("gdn_prefill_packed_gate_logits", rc)


def gdn_decode_multi(shape: gdn_shape, q, k, v, g, beta, z, conv_w, norm_w, state, conv_state, o,
                     state_snaps=None, conv_snaps=None, stream=None) -> None:
    """shape.T tokens per sequence (1..8); state and conv_state are updated in place."""
    rc = _lib.gdn_decode_multi(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(z),
                               _ptr(conv_w), _ptr(norm_w), _ptr(state), _ptr(conv_state), _ptr(o),
                               _ptr(state_snaps), _ptr(conv_snaps), _stream(stream))
    _check("gdn_decode_multi", rc)


def gdn_decode_multi_gate_logits(shape: gdn_shape, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state,
                                 conv_state, o, state_snaps=None, conv_snaps=None, stream=None) -> None:
    rc = _lib.gdn_decode_multi_gate_logits(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                           _ptr(A_log), _ptr(dt_bias), _ptr(z), _ptr(conv_w), _ptr(norm_w),
                                           _ptr(state), _ptr(conv_state), _ptr(o), _ptr(state_snaps),
                                           _ptr(conv_snaps), _stream(stream))
    _check("gdn_decode_multi_gate_logits", rc)
