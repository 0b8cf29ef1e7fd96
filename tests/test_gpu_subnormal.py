"""A state that decays into fp32's subnormal band (below 2^-126, where the grid has the
fixed spacing 2^-149).  With beta = 0 the rule only decays the state, so hT is
exp(sum of g) * h0 exactly; a gate summing to -90 .. -100 over the sequence puts hT
between about 1e-40 and 1e-44.  The library must keep those values (no flush to zero)
to within a couple of grid steps, on both arms and in every composition that applies,
and the whole-tensor figure must meet the arm's bound with the metric's subnormal
allowance.  Also the seeded problem that first drew such a state: one packed 257-token
sequence whose per-head gate sums to -95 .. -104, beta = 0."""
import dataclasses

import numpy as np
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, device_inputs, oracle_ref, rel, to_np64
from tests.randomized_cases import draw

pytestmark = pytest.mark.gpu

STEP = 2.0 ** -149
T = 256


def _decay_inputs(gate, total):
    chunk = 64 if gate == "head" else 32
    spec = inputs.Spec("decay", (T,), 1, 2, 64, 64, qkv_dtype="bf16", gate=gate,
                       gate_law="half" if gate == "head" else "uniform5", h0=True, chunk=chunk,
                       o_dtype="f32", seed=11, beta_law="zero")
    base = inputs.make(spec)
    if gate == "head":
        # value head 1 decays 4 further than head 0
        tot = np.array([total, total - 4.0])
        g = np.broadcast_to((tot / T).astype(np.float32), base.g.shape).copy()
    else:
        # key channels spread over 12 units of decay, so rows of the state sit at
        # different depths in the band
        tot = total + np.linspace(3.0, -9.0, spec.dk)
        g = np.broadcast_to((tot / T).astype(np.float32), base.g.shape).copy()
    return dataclasses.replace(base, g=g)


def _check(inp, arm, compose, solve_block=0):
    s = inp.spec
    d = device_inputs(inp)
    o, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                             chunk=s.chunk, arm=arm, o_dtype=torch.float32, compose=compose,
                             solve_block=solve_block)
    o_ref, h_ref = oracle_ref(inp)
    x = to_np64(hT)
    steps = np.abs(x - h_ref) / STEP
    kept = np.abs(x - h_ref) <= 2 * STEP + 1e-5 * np.abs(h_ref)
    eo, eh = rel(to_np64(o).reshape(o_ref.shape), o_ref), rel(x, h_ref)
    print("%s arm=%s %s: |hT|max %.2e, error max %.2f steps (rms %.2f); rel o %.2e hT %.2e"
          % (s.name, arm, compose, np.abs(h_ref).max(), steps.max(), np.sqrt((steps ** 2).mean()), eo, eh),
          flush=True)
    assert np.abs(h_ref).max() < 2.0 ** -126          # the case does reach the band
    assert kept.all(), int((~kept).sum())
    assert eo <= BOUND[arm] and eh <= BOUND[arm], (eo, eh)


HEAD_COMPOSE = [(arm, c) for arm in ("f32", "bf16") for c in ("auto", "split", "pipelined", "seqsplit")]
HEAD_COMPOSE += [("bf16", "fused")]


@pytest.mark.parametrize("total", [-90.0, -95.0, -100.0])
@pytest.mark.parametrize("arm,compose", HEAD_COMPOSE)
def test_head_gate_state_in_subnormal_band(total, arm, compose):
    _check(_decay_inputs("head", total), arm, compose)


@pytest.mark.parametrize("total", [-90.0, -95.0, -100.0])
@pytest.mark.parametrize("arm,compose", [(a, c) for a in ("f32", "bf16") for c in ("auto", "split")])
def test_channel_gate_state_in_subnormal_band(total, arm, compose):
    _check(_decay_inputs("channel", total), arm, compose)


@pytest.mark.parametrize("arm", ["f32", "bf16"])
def test_drawn_problem_in_subnormal_band(arm):
    c = draw(311)
    assert c.spec.beta_law == "zero" and c.spec.h0 and c.spec.seq_lens == (257,)
    _check(inputs.make(c.spec), arm, "split", solve_block=8)
