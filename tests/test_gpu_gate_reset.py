"""Per-head gates far below the usual range: reset tokens and chunks whose gates add up
to thousands.  The in-chunk prefix is fp64, and a reset token (gate at most -200, where
every factor across the token is below fp32's resolution) enters it as -2^20, so every
factor across one is exactly zero and every arm keeps its bound however large the
gates.  An fp32 prefix lost the fp32 arm's bound from gates of -1e4 on, and the bf16
arm's from -1e6 (its difference of two in-chunk sums then has a grid of 1e-3 and 0.06).
Both arms, every composition that applies, the raw-input entry point, against the fp64
oracle."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import prepare
from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, device_inputs, oracle_ref, rel, to_np64

pytestmark = pytest.mark.gpu

T = 512


def _base(beta="sigmoid", raw=False):
    spec = inputs.Spec("reset", (T,), 2, 4, 64, 64, qkv_dtype="f32", gate="head", gate_law="half", h0=True,
                       chunk=64, o_dtype="f32", seed=21, beta_law=beta, raw=raw)
    return inputs.make(spec)


def _gates(kind, shape):
    g = np.full(shape, -0.01, np.float32)
    if kind.startswith("reset"):
        val, where = kind.split(":")[1:]
        g[int(where)::64] = np.float32(float(val))
    elif kind == "heavy":
        # 20 tokens of -150 at the start of every chunk, then small gates: the chunk's
        # sums reach -3000 while the later rows' differences stay small
        for c in range(0, shape[0], 64):
            g[c:c + 20] = -150.0
    elif kind == "edge":
        g[7::64] = -200.0          # exactly the reset threshold
        g[40::64] = -199.9         # just above it: an ordinary gate
    return g


KINDS = ["reset:-1e4:32", "reset:-1e4:0", "reset:-1e6:17", "reset:-1e30:63", "heavy", "edge"]
COMPOSE = [(a, c) for a in ("f32", "bf16") for c in ("split", "pipelined", "seqsplit")]


def _run(inp, arm, compose, raw=None):
    s = inp.spec
    d = device_inputs(inp)
    o, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], chunk=s.chunk,
                             arm=arm, o_dtype=torch.float32, compose=compose, raw=raw)
    return to_np64(o), to_np64(hT)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("arm,compose", COMPOSE)
def test_large_gates_keep_the_bound(kind, arm, compose):
    b = _base()
    inp = dataclasses.replace(b, g=_gates(kind, b.g.shape))
    o, hT = _run(inp, arm, compose)
    o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(o.reshape(o_ref.shape), o_ref), rel(hT, h_ref)
    print("%s arm=%s %s: rel o %.2e hT %.2e (bound %.0e)" % (kind, arm, compose, eo, eh, BOUND[arm]), flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm], (eo, eh)


@pytest.mark.parametrize("arm", ["f32", "bf16"])
def test_reset_with_no_later_writes_leaves_zero_state(arm):
    # beta = 0 throughout: the state only decays, and one reset token per chunk takes
    # it to exactly zero, as e^{-1e4} h0 is in fp32
    b = _base(beta="zero")
    inp = dataclasses.replace(b, g=_gates("reset:-1e4:32", b.g.shape))
    o, hT = _run(inp, arm, "split")
    assert np.all(hT == 0.0)
    o_ref, _ = oracle_ref(inp)
    assert rel(o.reshape(o_ref.shape), o_ref) <= BOUND[arm]


@pytest.mark.parametrize("arm", ["f32", "bf16"])
def test_raw_inputs_with_reset_gates(arm):
    # raw gate values of 1e4 give g = -gate_scale softplus(1e4), a reset token
    b = _base(raw=True)
    x = b.g.copy()
    x[32::64] = 1e4
    inp = dataclasses.replace(b, g=x)
    qs, gs = inp.meta["q_scale"], inp.meta["gate_scale"]
    o, hT = _run(inp, arm, "pipelined", raw=(qs, gs))
    o_ref, h_ref = prepare.raw_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.g.astype(np.float64),
                                   inp.beta.astype(np.float64), qs, gs, inp.as_f64("h0"), seq_start=inp.cu_seqlens)
    eo, eh = rel(o.reshape(o_ref.shape), o_ref), rel(hT, h_ref)
    print("raw reset arm=%s: rel o %.2e hT %.2e" % (arm, eo, eh), flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm], (eo, eh)
