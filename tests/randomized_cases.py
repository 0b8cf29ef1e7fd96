"""Seeded random problems over the library's supported domain, for the randomized parity
test (tests/test_gpu_randomized.py) and its host-side check (tests/test_randomized_cpu.py);
and seeded one-token steps for gdn_decode_step.

Each case draws, from its own seed: the gate form and law, chunk, key/value widths, key
heads and grouping, a fixed-length batch or a packed batch (empty, one-token and ragged
sequences among them), beta's law (random, 1, 0, 1e-6), input and output dtypes, the
arithmetic arm, h0 or none, the solve's diagonal block, the composition (where it
applies) and, for the per-head gate, the raw-input entry point.  Sizes are capped so the
fp64 oracle finishes each case in well under a second."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from linear_attention_rnn_chunk_amd import inputs

N_CASES = 192
MAX_TOKEN_HEADS = 6000


@dataclass(frozen=True)
class Case:
    spec: inputs.Spec
    arm: str
    compose: str
    solve_block: int


def draw(i: int) -> Case:
    r = np.random.default_rng(5000 + i)
    while True:
        gate = str(r.choice(["head", "head", "channel"]))
        chunk = 32 if gate == "channel" else int(r.choice([32, 64]))
        dk, dv = int(r.choice([32, 64, 128])), int(r.choice([32, 64, 128]))
        hk = int(r.choice([1, 2, 4]))
        hv = hk * int(r.choice([1, 2, 3, 4]))
        packed = bool(r.integers(2))
        if packed:
            lens = tuple(int(x) for x in r.choice([0, 1, 7, 31, 64, 65, 100, 150, 257], size=int(r.integers(1, 5))))
        else:
            lens = (int(r.choice([1, 33, 64, 100, 200, 300])),) * int(r.integers(1, 4))
        if sum(lens) == 0 or sum(lens) * hv > MAX_TOKEN_HEADS:
            continue
        break
    law = str(r.choice(["uniform5", "uniform05"])) if gate == "channel" else str(r.choice(["clip5", "half", "full", "zero"]))
    beta_law = str(r.choice(["sigmoid", "sigmoid", "sigmoid", "one", "zero", "eps"]))
    qkv = str(r.choice(["bf16", "bf16", "f32"]))
    arm = str(r.choice(["bf16", "f32"]))
    o_dtype = "f32" if arm == "f32" else str(r.choice(["bf16", "f32"]))
    h0 = bool(r.integers(2))
    solve_block = int(r.choice([0, 8, 16, 32]))
    raw = gate == "head" and law in ("half", "full") and beta_law == "sigmoid" and r.random() < 0.6
    # compositions that apply to this problem (the fused and pipelined ones solve with
    # 16-row blocks only; raw inputs have no fused form; the sequence split needs dk == dv)
    options = ["auto", "split"]
    fixed = not packed and len(set(lens)) == 1
    sb16 = solve_block in (0, 16)
    if fixed and gate == "head" and sb16:
        options.append("pipelined")
    if fixed and gate == "head" and dk == dv and not raw:
        options.append("seqsplit")
    if gate == "head" and qkv == "bf16" and arm == "bf16" and sb16 and not raw:
        options.append("fused")
    compose = str(r.choice(options[1:])) if len(options) > 2 and r.random() < 0.7 else str(r.choice(options))
    spec = inputs.Spec("rand%d" % i, lens, hk, hv, dk, dv, qkv_dtype=qkv, gate=gate, gate_law=law, h0=h0,
                       chunk=chunk, packed=packed, o_dtype=o_dtype, seed=7000 + i, beta_law=beta_law, raw=raw)
    return Case(spec, arm, compose, solve_block)


CASES = [draw(i) for i in range(N_CASES)]


# one-token steps (gdn_decode_step): sequences of one token each, from a drawn state or zero
N_DECODE = 64


@dataclass(frozen=True)
class DecodeCase:
    spec: inputs.Spec
    o_dtype: str


def draw_decode(i: int) -> DecodeCase:
    r = np.random.default_rng(9000 + i)
    gate = str(r.choice(["head", "channel"]))
    law = str(r.choice(["uniform5", "uniform05"])) if gate == "channel" else str(r.choice(["clip5", "half", "full", "zero"]))
    hk = int(r.choice([1, 2, 4]))
    hv = hk * int(r.choice([1, 2, 3, 4]))
    dk, dv = int(r.choice([32, 64, 128])), int(r.choice([32, 64, 128]))
    B = int(r.choice([1, 2, 5, 17, 40]))
    qkv = str(r.choice(["bf16", "f32"]))
    o_dtype = "f32" if qkv == "f32" else str(r.choice(["bf16", "f32"]))
    spec = inputs.Spec("step%d" % i, (1,) * B, hk, hv, dk, dv, qkv_dtype=qkv, gate=gate, gate_law=law,
                       h0=bool(r.integers(4)), packed=True, seed=9500 + i,
                       beta_law=str(r.choice(["sigmoid", "sigmoid", "one", "zero", "eps"])))
    return DecodeCase(spec, o_dtype)


DECODE_CASES = [draw_decode(i) for i in range(N_DECODE)]
