"""Library calls running at the same time: two calls on two streams of one device (a
pipelined layer beside a packed batch, each with its own workspace), issued from one host
thread and from two, must each equal the same call run alone, bit for bit.  Nothing a
call uses outside its own arguments and workspace may be shared between calls in flight
(the entry point without allocation, whose fixed array is shared by design, is not
covered here)."""
import threading

import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu

SPECS = [inputs.Spec("conc_fixed", (16384,), 8, 24, 128, 128, gate_law="half", h0=True, chunk=64, seed=31),
         inputs.Spec("conc_packed", (5000, 300, 0, 9000), 4, 12, 128, 64, gate_law="full", h0=True, chunk=64,
                     packed=True, seed=32)]
COMPOSE = ["pipelined", "auto"]


def _call(d, spec, compose):
    return gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], chunk=spec.chunk,
                         compose=compose, check=False)


def _alone():
    ins = [device_inputs(inputs.make(s)) for s in SPECS]
    refs = []
    for d, s, c in zip(ins, SPECS, COMPOSE):
        o, hT, st = _call(d, s, c)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        refs.append((o.clone(), hT.clone()))
    return ins, refs


def test_two_streams_one_thread():
    ins, refs = _alone()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        outs = []
        for d, s, c, st in zip(ins, SPECS, COMPOSE, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs.append(_call(d, s, c))
        torch.cuda.synchronize()
        for (o, hT, status), (ro, rh) in zip(outs, refs):
            assert int(status.item()) == 0
            assert torch.equal(o, ro) and torch.equal(hT, rh)
        print("round %d: both calls equal their lone runs" % rep, flush=True)


def test_two_streams_two_threads():
    ins, refs = _alone()
    outs = [None, None]
    errors = []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(3):
                    o, hT, status = _call(ins[i], SPECS[i], COMPOSE[i])
                st.synchronize()
                outs[i] = (o, hT, status)
        except Exception as e:  # reported on the main thread
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for (o, hT, status), (ro, rh) in zip(outs, refs):
        assert int(status.item()) == 0
        assert torch.equal(o, ro) and torch.equal(hT, rh)
