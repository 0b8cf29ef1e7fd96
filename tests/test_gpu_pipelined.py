"""The pipelined composition (the scan in chunk-aligned segments of 2,048 tokens carrying
the state through the workspace, each segment's launch also running the next segment's
prep) against the plain split one: every chunk's tiles and every step of the recurrence
are the same instructions on the same values, and the state crosses a segment boundary
as exact fp32, so o and hT must agree bit for bit; and against the oracle within the
arm's bound.  The shapes below span one to five segments."""
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, device_inputs, oracle_ref, rel, run_gpu, to_np64

pytestmark = pytest.mark.gpu


def _both(inp, arm="bf16", chunk=None, other="pipelined"):
    d = device_inputs(inp)
    o_s, h_s, _ = run_gpu(inp, arm=arm, chunk=chunk, compose="split", d=d)
    o_p, h_p, _ = run_gpu(inp, arm=arm, chunk=chunk, compose=other, d=d)
    return (o_s, h_s), (o_p, h_p)


def _check(inp, arm, o_p, h_p, label):
    o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(to_np64(o_p), o_ref), rel(to_np64(h_p), h_ref)
    print("%s rel-L2 o=%.2e hT=%.2e" % (label, eo, eh), flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm]


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_pipelined_bitwise_equals_split(dk, dv, chunk):
    # 2,500 tokens: 40 chunks of 64 (segments of 32 and 8), 79 chunks of 32 (64 and 15)
    spec = inputs.Spec("pipe", (2500, 2500), 2, 6, dk, dv, qkv_dtype="bf16", gate_law="half", h0=True,
                       chunk=chunk, seed=7 * dk + dv + chunk)
    inp = inputs.make(spec)
    (o_s, h_s), (o_p, h_p) = _both(inp, chunk=chunk)
    assert torch.equal(o_s, o_p) and torch.equal(h_s, h_p)
    _check(inp, "bf16", o_p, h_p, "pipelined dk=%d dv=%d C=%d" % (dk, dv, chunk))


@pytest.mark.parametrize("T", [1, 37, 65, 2048, 2049, 4099])
def test_pipelined_lengths(T):
    """One segment (short sequences, exactly 32 chunks), a segment of a single partial
    chunk after a full one (2,049 tokens), three segments ending in a partial chunk."""
    spec = inputs.Spec("pipeT", (T, T, T), 2, 4, 128, 128, qkv_dtype="bf16", gate_law="clip5", h0=True,
                       chunk=64, seed=900 + T)
    inp = inputs.make(spec)
    (o_s, h_s), (o_p, h_p) = _both(inp)
    assert torch.equal(o_s, o_p) and torch.equal(h_s, h_p)
    _check(inp, "bf16", o_p, h_p, "pipelined T=%d" % T)


@pytest.mark.parametrize("qkv", ["bf16", "f32"])
def test_pipelined_fp32_arm(qkv):
    spec = inputs.Spec("pipef32", (2200, 2200), 2, 4, 128, 64, qkv_dtype=qkv, gate_law="half", h0=True,
                       chunk=64, o_dtype="f32", seed=31)
    inp = inputs.make(spec)
    (o_s, h_s), (o_p, h_p) = _both(inp, arm="f32")
    assert torch.equal(o_s, o_p) and torch.equal(h_s, h_p)
    _check(inp, "f32", o_p, h_p, "pipelined fp32 arm, %s inputs" % qkv)


def test_pipelined_without_h0_or_hT():
    spec = inputs.Spec("pipenh", (4200,), 2, 6, 128, 128, qkv_dtype="bf16", gate_law="full", h0=False,
                       chunk=64, seed=12)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    outs = []
    for compose in ("split", "pipelined"):
        o, hT, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, compose=compose,
                                  want_hT=False)
        assert hT is None
        outs.append(o)
    assert torch.equal(outs[0], outs[1])


def test_pipelined_status_bits():
    """Inf/NaN in h0 (read by the first segment only) and in a key of the third segment
    (seen by the prep that runs beside the second segment's scan) still set the bit."""
    spec = inputs.Spec("pipest", (6144,), 2, 4, 128, 128, qkv_dtype="bf16", gate_law="half", h0=True,
                       chunk=64, seed=5)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    h_bad = d["h0"].clone()
    h_bad[0, 1, 5, 7] = float("inf")
    _, _, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h_bad, compose="pipelined", check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    k_bad = d["k"].clone()
    k_bad[0, 5000, 1, 3] = float("nan")
    _, _, st = gdn.chunk_fwd(d["q"], k_bad, d["v"], d["g"], d["beta"], d["h0"], compose="pipelined", check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    _, _, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], compose="pipelined")
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_library_choice_bitwise_equals_split():
    """The hybrid layer at full size: the library's choice (the pipelined composition on a
    device whose scan grid leaves compute units idle) agrees with the split composition
    bit for bit over the whole output and final state."""
    inp = inputs.make("hybrid")
    (o_s, h_s), (o_a, h_a) = _both(inp, other="auto")
    assert torch.equal(o_s, o_a) and torch.equal(h_s, h_a)


def test_library_choice_on_this_device():
    """On MI355X (256 compute units) the hybrid layer's scan grid (192 workgroups) leaves
    64 units idle, so the library pipelines it; the 4,096-token single-sequence layer is
    below the four-segment minimum and stays split."""
    import torch as _t
    if _t.cuda.get_device_properties(0).multi_processor_count < 256:
        pytest.skip("the choice below is stated for a 256-unit device")
    mk = lambda spec: gdn.make_problem(spec.n_seq, spec.tokens, spec.seq_lens[0], spec.hk, spec.hv, spec.dk,
                                       spec.dv, gdn.GATE_HEAD, spec.chunk)
    assert gdn.plan_compose(mk(inputs.CONFIGS["hybrid"])) == gdn.COMPOSE_PIPELINED
    assert gdn.plan_compose(mk(inputs.CONFIGS["single"])) == gdn.COMPOSE_SPLIT
