"""Seeded synthetic inputs for the gated delta-rule prefill.

This module draws random numbers and stores them; it holds none of the
method's arithmetic.  It is the only code shared by the tests' oracle side and
the HIP side: both receive the exact same values (bf16 tensors are produced
here by round-to-nearest-even from fp32 and kept as bit patterns, so the oracle
upcasts them exactly).

Workloads (the pages measure a 32k-token hybrid-model prefill with 48 value
heads of state 128, and a per-key-channel gated variant with a gate lower bound
of -5; no dataset is involved, so these synthetic draws stand in for them):

========  ===================================================================
name      recipe
========  ===================================================================
tiny      1 x 200 tokens, 4/4 heads, d=32, fp32 q/k/v, chunk 64, h0 ~ 0.1 N
single    1 x 4096 tokens, 16/16 heads, d=128, bf16, chunk 64, no h0
hybrid    1 x 32768 tokens, 16 key / 48 value heads, d=128, bf16, chunk 64, h0
kda       2 x 16384 tokens, 32/32 heads, d=128, bf16, per-channel gate
          U[-5, 0], chunk 32, no h0
packed    4 sequences 65536/32768/24576/8192 (131072 tokens), 16/48 heads,
          d=128, bf16, chunk 64, per-sequence h0
========  ===================================================================

Draw order per seed (numpy PCG64): q, k, v, beta logits, gate, h0.  With
``qk_same`` q is then replaced by a copy of k (same values, same bf16 bits).
q and k are N(0,1), L2-normalised per (token, head) in fp32; q is then scaled
by dk^-1/2 except in ``tiny``; v ~ N(0,1); beta = sigmoid(N(0,1)); the gate is
a natural-log decay (``clip5``: -softplus(N) clipped to [-5, 0]; ``half``:
-0.5 softplus(N); ``full``: -softplus(N); ``uniform5``: U[-5, 0] per key
channel; ``zero``: 0); h0 ~ 0.1 N(0,1), drawn per sequence.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Spec:
    name: str
    seq_lens: tuple
    hk: int
    hv: int
    dk: int
    dv: int
    qkv_dtype: str = "bf16"        # "bf16" | "f32"
    gate: str = "head"             # "head" ([tok, hv]) | "channel" ([tok, hv, dk])
    gate_law: str = "half"         # clip5 | half | full | uniform5 | uniform05 | zero
    q_scale: bool = True
    h0: bool = False
    chunk: int = 64
    packed: bool = False           # True: pass cu_seqlens; False: fixed-length batch
    o_dtype: str = "bf16"
    seed: int = 0
    beta_law: str = "sigmoid"      # sigmoid | one | zero | eps
    qk_same: bool = False          # q is a copy of k (after k's normalisation and cast)
    raw: bool = False              # keep the raw draws: q, k unnormalised (and q unscaled),
                                   # beta = the logits, g = the raw gate values (laws half, full)

    @property
    def tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def n_seq(self) -> int:
        return len(self.seq_lens)

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


CONFIGS = {
    "tiny": Spec("tiny", (200,), 4, 4, 32, 32, qkv_dtype="f32", gate_law="clip5", q_scale=False,
                 h0=True, chunk=64, o_dtype="f32", seed=1001),
    "single": Spec("single", (4096,), 16, 16, 128, 128, gate_law="clip5", chunk=64, seed=1002),
    "hybrid": Spec("hybrid", (32768,), 16, 48, 128, 128, gate_law="half", h0=True, chunk=64,
                   seed=1003),
    "kda": Spec("kda", (16384, 16384), 32, 32, 128, 128, gate="channel", gate_law="uniform5",
                chunk=32, seed=1004),
    "packed": Spec("packed", (65536, 32768, 24576, 8192), 16, 48, 128, 128, gate_law="full",
                   h0=True, chunk=64, packed=True, seed=1005),
    # the hybrid layer's draws before their preparation: raw q, k, beta logits, raw gate
    # values (for the raw-input entry point: q_scale 128^-1/2, gate_scale 1/2)
    "hybrid_raw": Spec("hybrid_raw", (32768,), 16, 48, 128, 128, gate_law="half", h0=True, chunk=64,
                       seed=1003, raw=True),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite input)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_in.size, step):
        u = flat_in[i:i + step]
        r = ((u >> 16) & 1) + np.uint32(0x7FFF)
        flat_out[i:i + step] = ((u + r) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    spec: Spec
    q: np.ndarray                  # fp32 values, or bf16 bit patterns (uint16)
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray                  # fp32
    beta: np.ndarray               # fp32
    h0: Optional[np.ndarray]       # fp32 or None
    cu_seqlens: np.ndarray         # int32 [n_seq+1]
    meta: dict = field(default_factory=dict)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if a is None:
            return None
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a

    def as_f64(self, name: str) -> np.ndarray:
        a = self.as_f32(name)
        return None if a is None else a.astype(np.float64)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2norm_rows(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x.astype(np.float64))


def make(spec, seed: Optional[int] = None) -> Inputs:
    """Draw the inputs of ``spec`` (a Spec or a CONFIGS name)."""
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    if seed is not None:
        spec = spec.with_(seed=seed)
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    tok, hk, hv, dk, dv = spec.tokens, spec.hk, spec.hv, spec.dk, spec.dv

    qd, kd = _normal(rng, (tok, hk, dk)), None
    q = qd if spec.raw else _l2norm_rows(qd)
    if spec.q_scale and not spec.raw:
        q *= np.float32(dk ** -0.5)
    kd = _normal(rng, (tok, hk, dk))
    k = kd if spec.raw else _l2norm_rows(kd)
    v = _normal(rng, (tok, hv, dv))
    blog = _normal(rng, (tok, hv))
    meta = {}
    if spec.raw:
        if spec.beta_law != "sigmoid" or spec.gate != "head" or spec.gate_law not in ("half", "full"):
            raise ValueError("raw draws: sigmoid beta law, per-head gate, gate law half or full")
        meta = dict(q_scale=float(np.float32(dk ** -0.5)) if spec.q_scale else 1.0,
                    gate_scale=0.5 if spec.gate_law == "half" else 1.0)
        beta = blog
    elif spec.beta_law == "sigmoid":
        beta = (1.0 / (1.0 + np.exp(-blog.astype(np.float64)))).astype(np.float32)
    elif spec.beta_law == "one":
        beta = np.ones((tok, hv), np.float32)
    elif spec.beta_law == "zero":
        beta = np.zeros((tok, hv), np.float32)
    elif spec.beta_law == "eps":
        beta = (1e-6 / (1.0 + np.exp(-blog.astype(np.float64)))).astype(np.float32)
    else:
        raise ValueError(spec.beta_law)

    gshape = (tok, hv) if spec.gate == "head" else (tok, hv, dk)
    law = spec.gate_law
    if law == "uniform5":
        g = rng.uniform(-5.0, 0.0, size=gshape).astype(np.float32)
    elif law == "uniform05":
        g = rng.uniform(-0.5, 0.0, size=gshape).astype(np.float32)
    else:
        graw = _normal(rng, gshape)
        if spec.raw:
            g = graw
        elif law == "clip5":
            g = np.clip(-_softplus(graw), -5.0, 0.0).astype(np.float32)
        elif law == "half":
            g = (-0.5 * _softplus(graw)).astype(np.float32)
        elif law == "full":
            g = (-_softplus(graw)).astype(np.float32)
        elif law == "zero":
            g = np.zeros(gshape, np.float32)
        else:
            raise ValueError(law)

    h0 = (np.float32(0.1) * _normal(rng, (spec.n_seq, hv, dk, dv))) if spec.h0 else None
    if spec.qk_same:  # (q's own draw above keeps the draw order of the other streams)
        q = k.copy()

    if spec.qkv_dtype == "bf16":
        q, k, v = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
    elif spec.qkv_dtype != "f32":
        raise ValueError(spec.qkv_dtype)
    cu = np.zeros(spec.n_seq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(spec.seq_lens, dtype=np.int64))
    return Inputs(spec, q, k, v, g, beta, h0, cu, meta)
