"""gdn_chunk_fwd_noalloc (the library's own per-device workspace, nothing allocated)
against gdn_chunk_fwd with a caller-owned workspace, through the C ABI, on the same
problem and inputs: the same kernels on the same values, so o and hT must agree bit for
bit.  Two calls in a row, the second on a smaller problem (the array keeps the first
call's contents, which the second must not depend on), the second also against the fp64
oracle at the bf16 arm's bound."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, device_inputs, is_packed, oracle_ref, rel, to_np64

pytestmark = pytest.mark.gpu


def _problem(spec, compose):
    packed = is_packed(spec)
    gate = gdn.GATE_KEY_CHANNEL if spec.gate == "channel" else gdn.GATE_HEAD
    return gdn.make_problem(spec.n_seq, spec.tokens, 0 if packed else spec.seq_lens[0], spec.hk, spec.hv,
                            spec.dk, spec.dv, gate, spec.chunk, gdn.BF16, gdn.BF16, gdn.ARM_MFMA_BF16, compose)


def _both(inp, compose=gdn.COMPOSE_AUTO):
    spec = inp.spec
    d = device_inputs(inp)
    prob = _problem(spec, compose)
    outs = []
    for noalloc in (False, True):
        o = torch.full((spec.tokens, spec.hv, spec.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
        hT = torch.full((spec.n_seq, spec.hv, spec.dk, spec.dv), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], o, hT, st)
        if noalloc:
            rc = gdn.chunk_fwd_noalloc_raw(prob, *args)
        else:
            ws = torch.empty(max(1, gdn.workspace_bytes(prob)), dtype=torch.uint8, device="cuda")
            rc = gdn.chunk_fwd_raw(prob, *args, ws)
        torch.cuda.synchronize()
        assert rc == gdn.GDN_OK, gdn.error_string(rc)
        assert int(st.item()) == 0, gdn.status_string(int(st.item()))
        outs.append((o, hT))
    (o1, h1), (o2, h2) = outs
    print("%s (%s): noalloc equal to the workspace entry point: o %s hT %s"
          % (spec.name, ("auto", "split", "fused", "pipelined", "seqsplit")[gdn.plan_compose(prob)],
             torch.equal(o1, o2), torch.equal(h1, h2)), flush=True)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    return o2, h2


def test_noalloc_equals_workspace_entry_point_two_calls_smaller_second():
    big = inputs.make("hybrid")  # 32,768 tokens, 16/48 heads: pipelined, about 39 MiB of workspace
    small = inputs.make(inputs.Spec("small", (700, 0, 333), 2, 6, 128, 128, gate_law="full", h0=True,
                                    chunk=64, packed=True, seed=17))  # packed, split
    _both(big)
    o, hT = _both(small)
    o_ref, h_ref = oracle_ref(small)
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(hT), h_ref)
    print("small: rel-L2 against the oracle o %.3e hT %.3e" % (eo, eh), flush=True)
    assert eo <= BOUND["bf16"] and eh <= BOUND["bf16"]


def test_noalloc_refuses_a_problem_beyond_its_array():
    spec = inputs.CONFIGS["packed"]  # 131,072 tokens: far more tiles than the array holds
    prob = _problem(spec, gdn.COMPOSE_AUTO)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")  # never read: refused first
    assert gdn.workspace_bytes(prob) > gdn.NOALLOC_WORKSPACE_BYTES
    rc = gdn.chunk_fwd_noalloc_raw(prob, fake, fake, fake, fake, fake, None, fake, fake, None, st)
    assert rc == gdn.GDN_E_WORKSPACE
