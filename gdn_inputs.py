"""Seeded synthetic inputs for the Gated DeltaNet mixer hot path.

This module draws random numbers and rounds them to the storage formats the
mixer boundary takes (bf16 bit patterns held in uint16, and fp32).  It holds
none of the mixer's own arithmetic: no convolution, normalisation, decay or
state update.  The GPU path's tests and bench and the CPU oracle both consume
the arrays it returns, bit for bit, so every comparison starts from identical
inputs.

Recipe (distributions follow the workloads the source pages shape the layer
on: Qwen3.5-0.8B, Qwen3.5-4B and Qwen3.8-27B Gated DeltaNet layers):

* q, k, v, z: N(0, 1) drawn in fp32, rounded to bf16 (round to nearest even).
* g (log-decay): ln(u), u ~ U(0.8, 0.999), computed in fp64, stored as fp32.
* beta (write strength): sigmoid(N(0, 1)), computed in fp64, stored as fp32.
* conv weights [Cc, 4]: N(0, 0.5) -> bf16 (0.5 is the standard deviation).
* gated-norm weight [128]: 1 + N(0, 0.02) -> bf16.
* initial recurrent state [B, Hv, 128, 128]: N(0, 0.1) fp32 (decode workload).
* conv state [B, 3, Cc]: N(0, 1) -> bf16 (decode workload; stands in for the
  raw pre-conv activations it holds).
* gate logits (make_gate_logits, for the calls that take them): a, b ~ N(0, 1)
  fp32 [B, T, Hv]; A_log = ln(U(1, 16)) and dt_bias ~ U(-6.9, -2.3) fp32 per
  value head (the usual initial ranges of these parameters: A in [1, 16], the
  softplus of dt_bias in [1e-3, 0.1]).

Every tensor is drawn in blocks of 2**24 elements; block ``j`` of tensor
``tid`` for workload tag ``tag`` uses
``Generator(PCG64(SeedSequence([20261202, tag, tid, j])))``, so the bits do
not depend on the number of threads used to draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202
BLOCK = 1 << 24
D = 128  # key and value head width of every shape here

TID = dict(q=0, k=1, v=2, z=3, g=4, beta=5, conv_w=6, norm_w=7, state=8, conv_state=9,
           gate_a=10, gate_b=11, A_log=12, dt_bias=13)


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic mixer workload."""
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    conv: bool = True
    norm: bool = True
    decode: bool = False
    random_state: bool = False       # initial state ~N(0, 0.1) instead of zeros
    random_conv_state: bool = False  # initial conv state ~N(0, 1) instead of zeros
    tag: int = 0                     # seed tag

    @property
    def Cc(self) -> int:
        return 2 * self.Hk * D + self.Hv * D

    @property
    def r(self) -> int:
        return self.Hv // self.Hk


# The five workloads, named by what they are.
WORKLOADS = {
    "tiny_T64": Workload("tiny_T64", 1, 64, 1, 1, conv=False, norm=False, tag=0),
    "qwen35_0p8b_prefill_T4096": Workload("qwen35_0p8b_prefill_T4096", 1, 4096, 16, 16, tag=1),
    "qwen35_4b_prefill_B4_T16384": Workload("qwen35_4b_prefill_B4_T16384", 4, 16384, 16, 32, tag=2),
    "qwen38_27b_prefill_T262144": Workload("qwen38_27b_prefill_T262144", 1, 262144, 16, 48, tag=3),
    "qwen38_27b_decode_B256": Workload("qwen38_27b_decode_B256", 256, 1, 16, 48, decode=True,
                                       random_state=True, random_conv_state=True, tag=4),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(tag: int, tid: int, blk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, tag, tid, blk])))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw(n: int, tag: int, tid: int, kind: str, out_dtype) -> np.ndarray:
    """Draw n values of distribution ``kind`` block by block (threaded for large n)."""
    out = np.empty(n, dtype=out_dtype)

    def one(blk: int) -> None:
        lo, hi = blk * BLOCK, min(n, (blk + 1) * BLOCK)
        g = _rng(tag, tid, blk)
        m = hi - lo
        if kind == "normal_bf16":
            out[lo:hi] = f32_to_bf16_bits(g.standard_normal(m, dtype=np.float32))
        elif kind == "convw_bf16":
            out[lo:hi] = f32_to_bf16_bits((g.standard_normal(m, dtype=np.float32) * np.float32(0.5)))
        elif kind == "normw_bf16":
            out[lo:hi] = f32_to_bf16_bits(np.float32(1.0) + g.standard_normal(m, dtype=np.float32) * np.float32(0.02))
        elif kind == "state_f32":
            out[lo:hi] = g.standard_normal(m, dtype=np.float32) * np.float32(0.1)
        elif kind == "logdecay_f32":
            u = g.uniform(0.8, 0.999, m)  # fp64
            out[lo:hi] = np.log(u).astype(np.float32)
        elif kind == "normal_f32":
            out[lo:hi] = g.standard_normal(m, dtype=np.float32)
        elif kind == "alog_f32":
            out[lo:hi] = np.log(g.uniform(1.0, 16.0, m)).astype(np.float32)
        elif kind == "dtbias_f32":
            out[lo:hi] = g.uniform(-6.9, -2.3, m).astype(np.float32)
        elif kind == "beta_f32":
            x = g.standard_normal(m)  # fp64
            out[lo:hi] = (1.0 / (1.0 + np.exp(-x))).astype(np.float32)
        else:  # pragma: no cover
            raise ValueError(kind)

    nblk = (n + BLOCK - 1) // BLOCK
    if nblk <= 1:
        one(0)
    else:
        with _cf.ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(one, range(nblk)))
    return out


def make_inputs(w: Workload) -> dict:
    """All inputs of workload ``w`` as numpy arrays (bf16 tensors as uint16 bits).

    Keys: q, k [B,T,Hk,128]; v, z [B,T,Hv,128]; g, beta [B,T,Hv];
    conv_w [Cc,4] or None; norm_w [128] or None; state [B,Hv,128,128] fp32 or None;
    conv_state [B,3,Cc] or None.  For decode workloads T == 1.
    """
    B, T, Hk, Hv = w.B, w.T, w.Hk, w.Hv
    t = w.tag
    out = {
        "q": _draw(B * T * Hk * D, t, TID["q"], "normal_bf16", np.uint16).reshape(B, T, Hk, D),
        "k": _draw(B * T * Hk * D, t, TID["k"], "normal_bf16", np.uint16).reshape(B, T, Hk, D),
        "v": _draw(B * T * Hv * D, t, TID["v"], "normal_bf16", np.uint16).reshape(B, T, Hv, D),
        "z": (_draw(B * T * Hv * D, t, TID["z"], "normal_bf16", np.uint16).reshape(B, T, Hv, D)
              if w.norm else None),
        "g": _draw(B * T * Hv, t, TID["g"], "logdecay_f32", np.float32).reshape(B, T, Hv),
        "beta": _draw(B * T * Hv, t, TID["beta"], "beta_f32", np.float32).reshape(B, T, Hv),
        "conv_w": (_draw(w.Cc * 4, t, TID["conv_w"], "convw_bf16", np.uint16).reshape(w.Cc, 4)
                   if w.conv else None),
        "norm_w": _draw(D, t, TID["norm_w"], "normw_bf16", np.uint16) if w.norm else None,
        "state": (_draw(B * Hv * D * D, t, TID["state"], "state_f32", np.float32).reshape(B, Hv, D, D)
                  if w.random_state else None),
        "conv_state": (_draw(B * 3 * w.Cc, t, TID["conv_state"], "normal_bf16", np.uint16).reshape(B, 3, w.Cc)
                       if (w.random_conv_state and w.conv) else None),
    }
    return out


def make_gate_logits(w: Workload) -> dict:
    """Gate inputs of workload ``w`` for the calls that take the raw logits: a, b
    [B,T,Hv] fp32 and A_log, dt_bias [Hv] fp32 (see the module docstring)."""
    B, T, Hv, t = w.B, w.T, w.Hv, w.tag
    return {
        "a": _draw(B * T * Hv, t, TID["gate_a"], "normal_f32", np.float32).reshape(B, T, Hv),
        "b": _draw(B * T * Hv, t, TID["gate_b"], "normal_f32", np.float32).reshape(B, T, Hv),
        "A_log": _draw(Hv, t, TID["A_log"], "alog_f32", np.float32),
        "dt_bias": _draw(Hv, t, TID["dt_bias"], "dtbias_f32", np.float32),
    }
