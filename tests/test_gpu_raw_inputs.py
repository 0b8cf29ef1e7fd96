"""gdn_chunk_fwd_raw_inputs on the GPU against the fp64 oracle of the input side
(oracle/prepare.py: raw q/k normalised per row and q scaled, beta = sigmoid(logit),
g = -a softplus(x), then the token-serial rule), at the arms' bounds (fp32-fold 1e-4,
bf16-MFMA 2e-2, relative L2): widths, chunk sizes, ragged and packed lengths, both arms,
fp32 inputs, zero rows, saturating logits and gate values, the pipelined composition (bit
for bit against split), the status bits, and every unit of the hybrid layer's raw draws."""
import numpy as np
import pytest
import torch

from oracle import prepare
from linear_attention_rnn_chunk_amd import gdn, inputs
from tests._util import chunk_rel_l2, rel_l2_axes
from tests.gpu_util import BOUND, ODT, device_inputs, rel, to_np64

pytestmark = pytest.mark.gpu


def run_raw(inp, arm="bf16", compose="auto", d=None, check=True):
    d = d or device_inputs(inp)
    m = inp.meta
    o, hT, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              chunk=inp.spec.chunk, arm=arm, o_dtype=ODT[arm], compose=compose, check=check,
                              raw=(m["q_scale"], m["gate_scale"]))
    return o.reshape(inp.spec.tokens, inp.spec.hv, inp.spec.dv), hT, st


def oracle_raw(inp):
    m = inp.meta
    return prepare.raw_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.g.astype(np.float64),
                           inp.beta.astype(np.float64), m["q_scale"], m["gate_scale"], inp.as_f64("h0"),
                           seq_start=inp.cu_seqlens)


def _check(inp, arm, label, compose="auto"):
    o, hT, _ = run_raw(inp, arm, compose)
    o_ref, h_ref = oracle_raw(inp)
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(hT), h_ref)
    print("raw %s arm=%s rel-L2 o=%.3e hT=%.3e" % (label, arm, eo, eh), flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm], (eo, eh)
    return o, hT


@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("law", ["half", "full"])
@pytest.mark.parametrize("C", [32, 64])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_raw_inputs_sweep(T, C, law, arm):
    spec = inputs.Spec("raw", (T,), 2, 4, 64, 64, gate_law=law, h0=True, chunk=C, raw=True, seed=900 + T + C)
    _check(inputs.make(spec), arm, "T=%d C=%d %s" % (T, C, law))


@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
def test_raw_inputs_widths_packed_and_edges(dk, dv, arm):
    spec = inputs.Spec("raw-edges", (100, 0, 1, 64, 157), 2, 6, dk, dv, gate_law="full", h0=True, chunk=64,
                       packed=True, raw=True, seed=dk + 3 * dv)
    inp = inputs.make(spec)
    # zero rows of q and k stay zero; saturating logits and gate values stay finite
    inp.q[10, 1] = 0
    inp.k[11, 0] = 0
    inp.k[130, 1] = 0
    inp.beta[20:24] = np.float32(60.0)
    inp.beta[40:44] = np.float32(-60.0)
    inp.g[50:53] = np.float32(80.0)
    inp.g[60:63] = np.float32(-80.0)
    _check(inp, arm, "dk=%d dv=%d packed" % (dk, dv))


@pytest.mark.parametrize("arm", ["f32", "bf16"])
def test_raw_fp32_inputs(arm):
    spec = inputs.Spec("raw-f32", (300,), 2, 2, 128, 128, qkv_dtype="f32", gate_law="half", h0=True, chunk=64,
                       o_dtype="f32", raw=True, seed=31)
    _check(inputs.make(spec), arm, "fp32 inputs")


def test_raw_pipelined_equals_split_bitwise():
    spec = inputs.Spec("raw-pipe", (9000,), 8, 16, 128, 128, gate_law="half", h0=True, chunk=64, raw=True, seed=77)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    op, hp, _ = run_raw(inp, compose="pipelined", d=d)
    os_, hs, _ = run_raw(inp, compose="split", d=d)
    assert torch.equal(op, os_) and torch.equal(hp, hs)
    o_ref, h_ref = oracle_raw(inp)
    assert rel(to_np64(op), o_ref) <= BOUND["bf16"] and rel(to_np64(hp), h_ref) <= BOUND["bf16"]


def test_raw_status_bits_and_refusals():
    spec = inputs.Spec("raw-st", (90,), 2, 4, 64, 64, gate_law="half", h0=True, chunk=64, raw=True, seed=5)
    inp = inputs.make(spec)
    inp.beta[7, 1] = np.float32(np.nan)
    _, _, st = run_raw(inp, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    inp = inputs.make(spec)
    inp.g[3, 0] = np.float32(np.inf)
    _, _, st = run_raw(inp, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    # the per-key-channel gate and the fused composition are refused
    kda = inputs.make(inputs.Spec("k", (40,), 2, 2, 64, 64, gate="channel", gate_law="uniform5", chunk=32))
    d = device_inputs(kda)
    with pytest.raises(gdn.GdnError):
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None, chunk=32, raw=(1.0, 1.0))
    inp = inputs.make(spec)
    with pytest.raises(gdn.GdnError):
        run_raw(inp, compose="fused")


def test_raw_hybrid_layer_every_unit():
    inp = inputs.make("hybrid_raw")
    o, hT, _ = run_raw(inp)
    o_ref, h_ref = oracle_raw(inp)
    o_ref = o_ref.astype(np.float32).astype(np.float64)
    h_ref = h_ref.astype(np.float32).astype(np.float64)
    og = o.float().cpu().numpy().astype(np.float64)
    eo = rel_l2_axes(og, o_ref, (0, 2))
    eh = rel_l2_axes(hT[0].cpu().numpy().astype(np.float64), h_ref[0], (1, 2))
    ec = chunk_rel_l2(og, o_ref, 64)
    print("hybrid raw inputs, every unit: worst o %.3e hT %.3e chunk %.3e (bound 2e-02)"
          % (eo.max(), eh.max(), ec.max()), flush=True)
    assert eo.max() <= BOUND["bf16"] and eh.max() <= BOUND["bf16"] and ec.max() <= BOUND["bf16"]
