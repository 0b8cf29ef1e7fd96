"""The library against the examples of the rule worked by hand in tests/golden/, with no
oracle in between.  Each example is zero-padded to the smallest supported widths (dk = dv
= 32): padded key channels carry zero k and q, so the rows of H they index stay zero, and
padded value columns carry zero v and h0, so their columns of H and o stay zero; nothing
else changes.  It runs as a packed batch on the fp32-fold arm with fp32 inputs and outputs.
The unpadded part of o and hT must equal the hand values to fp32 rounding, and the padded
part must be exactly zero."""
import json
import pathlib

import numpy as np
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn

pytestmark = pytest.mark.gpu

GOLDEN = pathlib.Path(__file__).parent / "golden"
EX = json.loads((GOLDEN / "delta_rule_by_hand.json").read_text())["examples"]
RAW = json.loads((GOLDEN / "input_side_by_hand.json").read_text())["examples"]
D = 32
TOL = 1e-5  # fp32 arithmetic on values of order 1..10


def _padded(e, qn="q", kn="k", gn="g", bn="beta"):
    q0, k0, v0 = (np.asarray(e[n], np.float64) for n in (qn, kn, "v"))
    T, hk, dk = q0.shape
    hv, dv = v0.shape[1], v0.shape[2]
    q = np.zeros((T, hk, D)); q[:, :, :dk] = q0
    k = np.zeros((T, hk, D)); k[:, :, :dk] = k0
    v = np.zeros((T, hv, D)); v[:, :, :dv] = v0
    g0 = np.asarray(e[gn], np.float64)
    per_channel = g0.ndim == 3
    if per_channel:
        g = np.zeros((T, hv, D)); g[:, :, :dk] = g0
    else:
        g = g0
    ss = np.asarray(e["seq_start"], np.int32)
    h0 = np.zeros((len(ss) - 1, hv, D, D))
    if e["h0"] is not None:
        h0[:, :, :dk, :dv] = np.asarray(e["h0"], np.float64)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    args = dict(q=dev(q)[None], k=dev(k)[None], v=dev(v)[None], g=dev(g)[None],
                beta=dev(np.asarray(e[bn], np.float64))[None], h0=dev(h0),
                cu=torch.from_numpy(ss).cuda())
    return args, per_channel, dk, dv


def _check(e, o, hT, dk, dv):
    o = o.float().cpu().numpy().reshape(len(e["o"]), -1, D)
    hT = hT.float().cpu().numpy()
    want_o, want_h = np.asarray(e["o"], np.float64), np.asarray(e["hT"], np.float64)
    print("%s: o %s hT %s" % (e["name"][:48], o[:, :, :dv].ravel()[:6], hT[:, :, :dk, :dv].ravel()[:6]), flush=True)
    assert np.allclose(o[:, :, :dv], want_o, rtol=0, atol=TOL)
    assert np.allclose(hT[:, :, :dk, :dv], want_h, rtol=0, atol=TOL)
    assert not o[:, :, dv:].any() and not hT[:, :, dk:, :].any() and not hT[:, :, :, dv:].any()


@pytest.mark.parametrize("i", range(len(EX)), ids=["ex%d" % i for i in range(len(EX))])
def test_library_by_hand(i):
    e = EX[i]
    a, per_channel, dk, dv = _padded(e)
    o, hT, _ = gdn.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                             chunk=32 if per_channel else 64, arm="f32", o_dtype=torch.float32)
    _check(e, o, hT, dk, dv)


@pytest.mark.parametrize("i", range(len(RAW)))
def test_library_input_side_by_hand(i):
    e = RAW[i]
    a, _, dk, dv = _padded(e, qn="q_raw", kn="k_raw", gn="gate_x", bn="beta_logit")
    o, hT, _ = gdn.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], chunk=64, arm="f32",
                             o_dtype=torch.float32, raw=(e["q_scale"], e["gate_scale"]))
    _check(e, o, hT, dk, dv)


ONE_TOKEN = [i for i, e in enumerate(EX) if all(b - a == 1 for a, b in zip(e["seq_start"], e["seq_start"][1:]))]


@pytest.mark.parametrize("i", ONE_TOKEN, ids=["ex%d" % i for i in ONE_TOKEN])
def test_decode_step_by_hand(i):
    """The one-token step (gdn_decode_step) on the examples whose sequences are one token
    each: the batch is the examples' tokens, each continuing from its own state."""
    e = EX[i]
    a, _, dk, dv = _padded(e)
    o, h_out, _ = gdn.decode_step(a["q"][0].contiguous(), a["k"][0].contiguous(), a["v"][0].contiguous(),
                                  a["g"][0].contiguous(), a["beta"][0].contiguous(), a["h0"], o_dtype=torch.float32)
    _check(e, o, h_out, dk, dv)
