"""Run the mixer library on host-generated inputs (tests, smoke check, bench).

Uploads the boundary-format numpy arrays of gdn_inputs to the GPU as torch
tensors, allocates outputs and workspace, and calls the C ABI through the
binding.  No arithmetic of the mixer happens here.
"""
from __future__ import annotations

import numpy as np
import torch

import gated_deltanet_mixer_amd as gdn

DEV = "cuda"


def to_dev(a: np.ndarray | None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def bits(t) -> np.ndarray:
    """Device int16 tensor of bf16 bits -> host uint16 array."""
    return t.cpu().numpy().view(np.uint16)


class Prefill:
    """Device buffers of one prefill call: inputs, outputs and workspace."""

    def __init__(self, inp: dict, B: int, T: int, Hk: int, Hv: int, conv: bool, norm: bool,
                 state_in=None, conv_state_in=None, want_conv_state: bool = True, segments: int = 0):
        self.shape = gdn.make_shape(B, T, Hk, Hv, conv=conv, norm=norm, segments=segments)
        self.B, self.T, self.Hk, self.Hv, self.conv, self.norm = B, T, Hk, Hv, conv, norm
        self.d = {n: to_dev(inp.get(n)) for n in ("q", "k", "v", "g", "beta")}
        self.d["z"] = to_dev(inp.get("z")) if norm else None
        self.d["conv_w"] = to_dev(inp.get("conv_w")) if conv else None
        self.d["norm_w"] = to_dev(inp.get("norm_w")) if norm else None
        s_in = state_in if state_in is not None else inp.get("state")
        cs_in = conv_state_in if conv_state_in is not None else inp.get("conv_state")
        self.d["state_in"] = s_in if isinstance(s_in, torch.Tensor) else to_dev(s_in)
        self.d["conv_state_in"] = (cs_in if isinstance(cs_in, torch.Tensor) else to_dev(cs_in)) if conv else None
        Cc = 2 * Hk * 128 + Hv * 128
        self.o = torch.empty((B, T, Hv, 128), dtype=torch.int16, device=DEV)
        self.state_out = torch.empty((B, Hv, 128, 128), dtype=torch.float32, device=DEV)
        self.conv_state_out = (torch.empty((B, 3, Cc), dtype=torch.int16, device=DEV)
                               if (conv and want_conv_state) else None)
        self.ws_bytes = gdn.gdn_prefill_workspace_size(self.shape)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=DEV)

    def run(self, stream=None):
        d = self.d
        gdn.gdn_prefill(self.shape, d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"], d["conv_w"],
                        d["norm_w"], d["state_in"], d["conv_state_in"], self.o, self.state_out,
                        self.conv_state_out, self.ws, self.ws_bytes, stream=stream)

    def run_gate_logits(self, gl: dict, stream=None):
        """The same call through gdn_prefill_gate_logits; gl holds a, b, A_log, dt_bias
        as numpy arrays or device tensors (g and beta of the inputs are not used)."""
        t = {n: (x if isinstance(x, torch.Tensor) else to_dev(x)) for n, x in gl.items()}
        d = self.d
        gdn.gdn_prefill_gate_logits(self.shape, d["q"], d["k"], d["v"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                                    d["z"], d["conv_w"], d["norm_w"], d["state_in"], d["conv_state_in"], self.o,
                                    self.state_out, self.conv_state_out, self.ws, self.ws_bytes, stream=stream)

    def exchange_error_word(self) -> int:
        """The workspace's error word (its first 32-bit word): bit 0 a bounded wait timed out,
        bit 1 a packed sequence was skipped."""
        return int(self.ws[0:4].view(torch.int32).item())


class PackedPrefill:
    """Device buffers of one packed-sequence prefill: B sequences whose token rows
    cu_seqlens[b] .. cu_seqlens[b+1] - 1 share the token-major tensors of ``inp``
    (a B = 1 input set of T rows), and per-sequence states ``state_in`` [B,Hv,128,128]
    and ``conv_state_in`` [B,3,Cc] (numpy, device tensors or None)."""

    def __init__(self, inp: dict, cu_seqlens, T: int, Hk: int, Hv: int, conv: bool, norm: bool,
                 state_in=None, conv_state_in=None):
        cu = np.asarray(cu_seqlens, dtype=np.int32)
        B = len(cu) - 1
        self.shape = gdn.make_shape(B, T, Hk, Hv, conv=conv, norm=norm, packed=True)
        self.B, self.T, self.Hk, self.Hv = B, T, Hk, Hv
        self.cu = to_dev(cu)
        self.d = {n: to_dev(inp.get(n)) for n in ("q", "k", "v", "g", "beta")}
        self.d["z"] = to_dev(inp.get("z")) if norm else None
        self.d["conv_w"] = to_dev(inp.get("conv_w")) if conv else None
        self.d["norm_w"] = to_dev(inp.get("norm_w")) if norm else None
        self.d["state_in"] = state_in if (state_in is None or isinstance(state_in, torch.Tensor)) else to_dev(state_in)
        self.d["conv_state_in"] = ((conv_state_in if (conv_state_in is None or isinstance(conv_state_in, torch.Tensor))
                                    else to_dev(conv_state_in)) if conv else None)
        Cc = 2 * Hk * 128 + Hv * 128
        self.o = torch.empty((T, Hv, 128), dtype=torch.int16, device=DEV)
        self.state_out = torch.empty((B, Hv, 128, 128), dtype=torch.float32, device=DEV)
        self.conv_state_out = torch.empty((B, 3, Cc), dtype=torch.int16, device=DEV) if conv else None
        self.ws_bytes = gdn.gdn_prefill_workspace_size(self.shape)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=DEV)

    def run(self, stream=None):
        d = self.d
        gdn.gdn_prefill_packed(self.shape, self.cu, d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"],
                               d["conv_w"], d["norm_w"], d["state_in"], d["conv_state_in"], self.o,
                               self.state_out, self.conv_state_out, self.ws, self.ws_bytes, stream=stream)

    def run_gate_logits(self, gl: dict, stream=None):
        t = {n: (x if isinstance(x, torch.Tensor) else to_dev(x)) for n, x in gl.items()}
        d = self.d
        gdn.gdn_prefill_packed_gate_logits(self.shape, self.cu, d["q"], d["k"], d["v"], t["a"], t["b"],
                                           t["A_log"], t["dt_bias"], d["z"], d["conv_w"], d["norm_w"],
                                           d["state_in"], d["conv_state_in"], self.o, self.state_out,
                                           self.conv_state_out, self.ws, self.ws_bytes, stream=stream)

    def exchange_error_word(self) -> int:
        return int(self.ws[0:4].view(torch.int32).item())


class Decode:
    """Device buffers of one decode step (state and conv state are updated in place)."""

    def __init__(self, inp: dict, B: int, Hk: int, Hv: int, conv: bool, norm: bool):
        self.shape = gdn.make_shape(B, 1, Hk, Hv, conv=conv, norm=norm)
        self.d = {n: to_dev(inp.get(n)) for n in ("q", "k", "v", "g", "beta")}
        self.d["z"] = to_dev(inp.get("z")) if norm else None
        self.d["conv_w"] = to_dev(inp.get("conv_w")) if conv else None
        self.d["norm_w"] = to_dev(inp.get("norm_w")) if norm else None
        st = inp.get("state")
        self.state = to_dev(st) if st is not None else torch.zeros((B, Hv, 128, 128), device=DEV)
        Cc = 2 * Hk * 128 + Hv * 128
        cs = inp.get("conv_state")
        self.conv_state = (to_dev(cs) if cs is not None else torch.zeros((B, 3, Cc), dtype=torch.int16, device=DEV)) \
            if conv else None
        self.o = torch.empty((B, Hv, 128), dtype=torch.int16, device=DEV)

    def run(self, stream=None):
        d = self.d
        gdn.gdn_decode_step(self.shape, d["q"], d["k"], d["v"], d["g"], d["beta"], d["z"], d["conv_w"],
                            d["norm_w"], self.state, self.conv_state, self.o, stream=stream)

    def run_gate_logits(self, gl: dict, stream=None):
        """The step through gdn_decode_step_gate_logits (gl: a, b [B,Hv], A_log, dt_bias [Hv])."""
        t = {n: (x if isinstance(x, torch.Tensor) else to_dev(x)) for n, x in gl.items()}
        d = self.d
        gdn.gdn_decode_step_gate_logits(self.shape, d["q"], d["k"], d["v"], t["a"], t["b"], t["A_log"],
                                        t["dt_bias"], d["z"], d["conv_w"], d["norm_w"], self.state,
                                        self.conv_state, self.o, stream=stream)
