"""A packed batch of 4,000 sequences whose lengths mix empty, one-token, chunk-edge and
multi-chunk cases (0, 1, 7, 31, 32, 33, 63, 64, 65, 127, 300 tokens), so the chunk
table is built over many 256-sequence blocks and every chunk is located among 4,000
bounds.  Each composition that takes a packed batch, both arms and both gate forms,
against the fp64 oracle over every (sequence, value head) unit: o and hT within the
arm's bound as a whole and unit by unit, and an empty sequence's final state equal to
its initial one."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests._util import rel_l2_axes
from tests.gpu_util import BOUND, device_inputs, oracle_ref, rel, to_np64

pytestmark = pytest.mark.gpu

N_SEQ = 4000
LENS = (0, 1, 7, 31, 32, 33, 63, 64, 65, 127, 300)


def _spec(gate):
    r = np.random.default_rng(4000)
    lens = tuple(int(x) for x in r.choice(LENS, size=N_SEQ))
    return inputs.Spec("many", lens, 2, 4, 64, 64, qkv_dtype="bf16", gate=gate,
                       gate_law="half" if gate == "head" else "uniform5", h0=True,
                       chunk=64 if gate == "head" else 32, packed=True, o_dtype="f32", seed=4001)


_CACHE = {}


def _problem(gate):
    if gate not in _CACHE:
        inp = inputs.make(_spec(gate))
        _CACHE[gate] = (inp, oracle_ref(inp))
    return _CACHE[gate]


CASES = [("head", "bf16", "auto"), ("head", "bf16", "fused"), ("head", "f32", "split"),
         ("channel", "bf16", "split"), ("channel", "f32", "split")]


@pytest.mark.parametrize("gate,arm,compose", CASES)
def test_many_packed_sequences(gate, arm, compose):
    inp, (o_ref, h_ref) = _problem(gate)
    s = inp.spec
    print("%d sequences, %d tokens, gate=%s arm=%s %s" % (N_SEQ, s.tokens, gate, arm, compose), flush=True)
    d = device_inputs(inp)
    o, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                             chunk=s.chunk, arm=arm, o_dtype=torch.float32, compose=compose)
    o = to_np64(o).reshape(o_ref.shape)
    hT = to_np64(hT)
    eo, eh = rel(o, o_ref), rel(hT, h_ref)
    # unit by unit: each sequence's o over its tokens and heads' columns, and each final state
    cu = inp.cu_seqlens
    worst_o = max(rel(o[cu[n]:cu[n + 1]], o_ref[cu[n]:cu[n + 1]]) for n in range(N_SEQ) if cu[n + 1] > cu[n])
    worst_h = float(np.max(rel_l2_axes(hT, h_ref.astype(np.float32).astype(np.float64), (2, 3))))
    print("rel-L2 o %.3e hT %.3e; worst sequence o %.3e, worst state %.3e" % (eo, eh, worst_o, worst_h), flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm]
    assert worst_o <= BOUND[arm] and worst_h <= BOUND[arm]
    empty = [n for n in range(N_SEQ) if cu[n + 1] == cu[n]]
    assert empty and np.array_equal(hT[empty], to_np64(d["h0"])[empty])
