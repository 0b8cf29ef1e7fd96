"""The library's calls inside a captured HIP graph (torch.cuda.graph): nothing on their
launch path allocates, synchronises or records a memset, so a graph of a call replays
it.  Each case is captured once and replayed four times; before each replay new inputs
are copied into the captured tensors, and between replays the program runs eager work of
its own (another library call, checked and synchronised).  Every replay must equal the
eager call on the same inputs bit for bit, with a clear status: the pipelined
composition's 17 launches, a packed batch (chunk table, dispatch order, prep, scan) and
the one-token step."""
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu


def _sets(spec, seeds):
    out = []
    for s in seeds:
        d = device_inputs(inputs.make(spec, seed=s))
        out.append(d)
    return out


def _eager_side_work():
    # the program's own work between replays: a different library call, checked
    d = device_inputs(inputs.make("tiny"))
    gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], check=True)
    torch.cuda.synchronize()


def _replay_case(spec, compose):
    sets = _sets(spec, (11, 12, 13))
    keys = ("q", "k", "v", "g", "beta", "h0")
    call = lambda d: gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                                   chunk=spec.chunk, compose=compose, check=False)
    refs = []
    for d in sets:
        o, hT, st = call(d)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        refs.append((o.clone(), hT.clone()))
    static = {k: sets[0][k].clone() for k in keys}
    static["cu_seqlens"] = sets[0]["cu_seqlens"]
    call(static)  # warm-up outside the capture (kernel attributes are set on first use)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, hT, st = call(static)
    for r, i in enumerate((1, 0, 2, 1)):
        for k in keys:
            static[k].copy_(sets[i][k])
        g.replay()
        torch.cuda.synchronize()
        print("%s %s replay %d (inputs %d): status %d" % (spec.name, compose, r, i, int(st.item())), flush=True)
        assert int(st.item()) == 0
        assert torch.equal(o, refs[i][0]) and torch.equal(hT, refs[i][1])
        _eager_side_work()


def test_graph_pipelined_layer():
    spec = inputs.Spec("graph_fixed", (16384,), 8, 24, 128, 128, gate_law="half", h0=True, chunk=64, seed=0)
    _replay_case(spec, "pipelined")


def test_graph_packed_batch():
    spec = inputs.Spec("graph_packed", (3000, 17, 0, 5000, 64), 2, 6, 64, 64, gate_law="full", h0=True,
                       chunk=64, packed=True, seed=0)
    _replay_case(spec, "auto")


def test_graph_one_token_step():
    spec = inputs.Spec("graph_step", (1,) * 40, 4, 12, 128, 128, gate_law="half", h0=True, packed=True, seed=0)
    sq = lambda x: x.squeeze(0)
    sets = [{k: (sq(v) if k != "h0" else v) for k, v in device_inputs(inputs.make(spec, seed=s)).items()
             if k != "cu_seqlens"} for s in (21, 22)]
    keys = ("q", "k", "v", "g", "beta", "h0")
    call = lambda d: gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                     o_dtype=torch.float32, check=False)
    refs = []
    for d in sets:
        o, h, st = call(d)
        torch.cuda.synchronize()
        refs.append((o.clone(), h.clone()))
    static = {k: sets[0][k].clone() for k in keys}
    call(static)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, h, st = call(static)
    for r, i in enumerate((1, 0, 1, 0)):
        for k in keys:
            static[k].copy_(sets[i][k])
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(o, refs[i][0]) and torch.equal(h, refs[i][1])
        _eager_side_work()
