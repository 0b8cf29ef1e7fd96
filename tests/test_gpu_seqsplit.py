"""The sequence-split composition (each sequence cut into parts scanned side by side, the
parts' starting states chained in fp32 through their transitions) against the fp64
token-serial oracle, within the arm's bound.  It is not bit-identical to the other
compositions (the chained states round differently), so every case goes to the oracle;
an error in a part's own state, its transition or the chaining would show in the
outputs of the parts after it, which are most of the tokens."""
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, device_inputs, oracle_ref, rel, run_gpu, to_np64

pytestmark = pytest.mark.gpu


def _check(inp, arm="bf16", chunk=None, label=""):
    o, hT, _ = run_gpu(inp, arm=arm, chunk=chunk, compose="seqsplit")
    o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(hT), h_ref)
    print("seqsplit %s arm=%s rel-L2 o=%.3e hT=%.3e" % (label, arm, eo, eh), flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm], (eo, eh)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [32, 64])
def test_seqsplit_widths_and_chunks(d, chunk):
    spec = inputs.Spec("seqs", (2000, 2000), 2, 4, d, d, qkv_dtype="bf16", gate_law="half", h0=True,
                       chunk=chunk, seed=40 + d + chunk)
    _check(inputs.make(spec), chunk=chunk, label="d=%d C=%d" % (d, chunk))


@pytest.mark.parametrize("T", [1, 100, 257, 2049, 4099])
def test_seqsplit_lengths(T):
    """One chunk (empty parts pass their state through), parts of one chunk, a partial
    last chunk, long parts."""
    spec = inputs.Spec("seqsT", (T,), 2, 4, 128, 128, qkv_dtype="bf16", gate_law="clip5", h0=True,
                       chunk=64, seed=700 + T)
    _check(inputs.make(spec), label="T=%d" % T)


@pytest.mark.parametrize("qkv", ["bf16", "f32"])
def test_seqsplit_fp32_arm(qkv):
    spec = inputs.Spec("seqsf32", (1500, 1500), 2, 4, 64, 64, qkv_dtype=qkv, gate_law="half", h0=True,
                       chunk=64, o_dtype="f32", seed=33)
    _check(inputs.make(spec), arm="f32", label="%s inputs" % qkv)


def test_seqsplit_without_h0_or_hT():
    spec = inputs.Spec("seqsnh", (3000,), 2, 6, 128, 128, qkv_dtype="bf16", gate_law="full", h0=False,
                       chunk=64, seed=14)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    o, hT, _ = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, compose="seqsplit", want_hT=False)
    assert hT is None
    o_ref, _ = oracle_ref(inp)
    assert rel(to_np64(o.reshape(3000, 6, 128)), o_ref) <= BOUND["bf16"]


def test_seqsplit_status_bits():
    spec = inputs.Spec("seqsst", (2048,), 2, 4, 128, 128, qkv_dtype="bf16", gate_law="half", h0=True,
                       chunk=64, seed=6)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    h_bad = d["h0"].clone()
    h_bad[0, 2, 9, 4] = float("nan")
    _, _, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h_bad, compose="seqsplit", check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    v_bad = d["v"].clone()
    v_bad[0, 2000, 3, 1] = float("inf")  # in the last part
    _, _, st = gdn.chunk_fwd(d["q"], d["k"], v_bad, d["g"], d["beta"], d["h0"], compose="seqsplit", check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    _, _, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], compose="seqsplit")
    torch.cuda.synchronize()
    assert int(st.item()) == 0
