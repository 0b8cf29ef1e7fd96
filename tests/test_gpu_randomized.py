"""Randomized parity: 192 seeded problems drawn over the supported domain
(tests/randomized_cases.py: gate form and law, chunk 32/64, widths 32-128, grouped heads,
fixed-length and packed batches with empty, one-token and ragged sequences, beta random /
1 / 0 / 1e-6, bf16 or fp32 inputs and outputs, both arms, h0 or none, the solve's diagonal
block, every composition that applies, and the raw-input entry point) against the fp64
token-serial oracle (with the input-side oracle in front for raw inputs), at each arm's
bound.  Each case prints what it drew, so a failure names its problem."""
import numpy as np
import pytest
import torch

from oracle import prepare
from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, device_inputs, oracle_ref, rel, to_np64
from tests.randomized_cases import CASES, DECODE_CASES

pytestmark = pytest.mark.gpu

ODT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _describe(c):
    s = c.spec
    return ("lens=%s hk=%d hv=%d dk=%d dv=%d gate=%s/%s chunk=%d qkv=%s o=%s beta=%s h0=%s raw=%s arm=%s "
            "compose=%s solve_block=%d" % (s.seq_lens, s.hk, s.hv, s.dk, s.dv, s.gate, s.gate_law, s.chunk,
                                           s.qkv_dtype, s.o_dtype, s.beta_law, s.h0, s.raw, c.arm, c.compose,
                                           c.solve_block))


@pytest.mark.parametrize("i", range(len(CASES)))
def test_randomized_case(i):
    c = CASES[i]
    print("case %d: %s" % (i, _describe(c)), flush=True)
    inp = inputs.make(c.spec)
    d = device_inputs(inp)
    raw = (inp.meta["q_scale"], inp.meta["gate_scale"]) if c.spec.raw else None
    o, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                             chunk=c.spec.chunk, arm=c.arm, o_dtype=ODT[c.spec.o_dtype], compose=c.compose,
                             solve_block=c.solve_block, raw=raw)
    o = o.reshape(c.spec.tokens, c.spec.hv, c.spec.dv)
    if c.spec.raw:
        o_ref, h_ref = prepare.raw_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                       inp.g.astype(np.float64), inp.beta.astype(np.float64),
                                       inp.meta["q_scale"], inp.meta["gate_scale"], inp.as_f64("h0"),
                                       seq_start=inp.cu_seqlens)
    else:
        o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(hT), h_ref)
    print("case %d rel-L2 o=%.3e hT=%.3e (bound %.0e)" % (i, eo, eh, BOUND[c.arm]), flush=True)
    assert eo <= BOUND[c.arm] and eh <= BOUND[c.arm], (eo, eh)


# one-token steps: fp32 throughout, so h_out and an fp32 o within 1e-5, a bf16 o within 4e-3
# (its own rounding, at most 2^-9 per element), as in tests/test_gpu_decode.py
STEP_BOUND = {"h": 1e-5, "f32": 1e-5, "bf16": 4e-3}


@pytest.mark.parametrize("i", range(len(DECODE_CASES)))
def test_randomized_step(i):
    c = DECODE_CASES[i]
    s = c.spec
    print("step case %d: B=%d hk=%d hv=%d dk=%d dv=%d gate=%s/%s qkv=%s o=%s beta=%s h0=%s"
          % (i, s.n_seq, s.hk, s.hv, s.dk, s.dv, s.gate, s.gate_law, s.qkv_dtype, c.o_dtype, s.beta_law, s.h0),
          flush=True)
    inp = inputs.make(s)
    d = device_inputs(inp)
    sq = lambda x: x.squeeze(0)
    h_in = d["h0"]
    h_keep = None if h_in is None else h_in.clone()
    o, h_out, _ = gdn.decode_step(sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["g"]), sq(d["beta"]), h_in,
                                  o_dtype=ODT[c.o_dtype])
    o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(to_np64(o), o_ref.reshape(o.shape)), rel(to_np64(h_out), h_ref)
    print("step case %d rel-L2 o=%.3e h=%.3e" % (i, eo, eh), flush=True)
    assert eo <= STEP_BOUND[c.o_dtype] and eh <= STEP_BOUND["h"], (eo, eh)
    if h_keep is not None:
        assert torch.equal(h_in, h_keep)  # the input state is never written
