"""GPU parity: the HIP path against the fp64 token-serial oracle, element by element
on the same seeded inputs, within the bounds recorded before the kernels were
written (fp32-fold arm 1e-4, bf16-MFMA arm 2e-2, relative L2, NaN-aware)."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_chunk_amd import inputs
from tests.gpu_util import BOUND, oracle_ref, rel, run_gpu, to_np64

pytestmark = pytest.mark.gpu


def _check(inp, arm, chunk=None, label="", solve_block=0):
    o, hT, _ = run_gpu(inp, arm=arm, chunk=chunk, solve_block=solve_block)
    o_ref, h_ref = oracle_ref(inp)
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(hT), h_ref)
    print("%s arm=%s chunk=%s rel-L2 o=%.3e hT=%.3e" % (label or inp.spec.name, arm, chunk, eo, eh),
          flush=True)
    assert eo <= BOUND[arm] and eh <= BOUND[arm], (eo, eh)
    return eo, eh


@pytest.mark.parametrize("arm", ["f32", "bf16"])
def test_tiny_config(arm):
    _check(inputs.make("tiny"), arm)


GATE_MODES = {
    "zero": dict(gate="head", gate_law="zero"),
    "scalar": dict(gate="head", gate_law="clip5"),
    "kda5": dict(gate="channel", gate_law="uniform5"),
    "kda05": dict(gate="channel", gate_law="uniform05"),
}


@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("mode", list(GATE_MODES))
@pytest.mark.parametrize("T", [1, 37, 64, 65, 200, 4099])
def test_length_and_gate_sweep(T, mode, arm):
    kw = GATE_MODES[mode]
    chunk = 32 if kw["gate"] == "channel" else 64
    spec = inputs.Spec("sweep", (T,), 2, 4, 64, 64, qkv_dtype="bf16", h0=True, chunk=chunk,
                       seed=100 + T, **kw)
    _check(inputs.make(spec), arm, label="T=%d %s" % (T, mode))


# beta at its edges: 0 (no write: pure decay of h0, T = I), 1 (full erase: the largest
# off-diagonal A, the hardest solve) and 1e-6 (the write at first order: decayed linear
# attention scaled by 1e-6; no h0, so the outputs are that small term alone)
@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("gate,law", [("head", "half"), ("channel", "uniform5"), ("channel", "uniform05")])
@pytest.mark.parametrize("beta_law", ["zero", "one", "eps"])
@pytest.mark.parametrize("T", [1, 65, 4099])
def test_beta_edge_sweep(T, beta_law, gate, law, arm):
    spec = inputs.Spec("beta", (T,), 2, 4, 64, 64, qkv_dtype="bf16", gate=gate, gate_law=law,
                       h0=beta_law != "eps", chunk=32 if gate == "channel" else 64, beta_law=beta_law,
                       seed=700 + T)
    _check(inputs.make(spec), arm, label="T=%d beta=%s %s/%s" % (T, beta_law, gate, law))


# The delta rule stores v exactly: with beta = 1, unit keys and q = k, o_t = v_t for every
# token whatever the gate and h0 (the state's read along k_t after the write is v_t).  On
# fp32 inputs (|k| = 1 to fp32 rounding) the GPU's o is checked against v itself, at the
# arm's bound: the identity is exact, so any excess is the kernel's own error.
@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("gate,law", [("head", "half"), ("head", "clip5"), ("channel", "uniform5"),
                                      ("channel", "uniform05")])
@pytest.mark.parametrize("T", [1, 65, 4099])
def test_unit_key_equal_query_returns_value(T, gate, law, arm):
    spec = inputs.Spec("o=v", (T,), 2, 4, 64, 64, qkv_dtype="f32", gate=gate, gate_law=law, h0=True,
                       chunk=32 if gate == "channel" else 64, beta_law="one", qk_same=True,
                       q_scale=False, o_dtype="f32", seed=800 + T)
    inp = inputs.make(spec)
    assert np.array_equal(inp.q, inp.k) and np.all(inp.beta == 1.0)
    o, hT, _ = run_gpu(inp, arm=arm, o_dtype=torch.float32)
    ev = rel(to_np64(o), inp.v.astype(np.float64))
    o_ref, h_ref = oracle_ref(inp)
    assert rel(o_ref, inp.v.astype(np.float64)) < 1e-6   # the identity, on these inputs
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(hT), h_ref)
    print("o=v T=%d %s/%s arm=%s: rel-L2 o-v %.3e, vs oracle o %.3e hT %.3e" % (T, gate, law, arm, ev, eo, eh),
          flush=True)
    assert ev <= BOUND[arm] and eo <= BOUND[arm] and eh <= BOUND[arm], (ev, eo, eh)


# The triangular solve's diagonal block (8, 16, 32 rows) changes only the rounding: every
# size against the oracle, on packed ragged sequences (an empty one, chunk tails of 7 and 1
# rows) with beta at 1 (the largest off-diagonal entries of A) and at its random law.
@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("gate,law,C", [("head", "clip5", 64), ("head", "full", 32), ("channel", "uniform5", 32)])
@pytest.mark.parametrize("beta_law", ["one", "sigmoid"])
@pytest.mark.parametrize("sb", [8, 16, 32])
def test_solve_block_sweep(sb, beta_law, gate, law, C, arm):
    spec = inputs.Spec("solve-block", (199, 0, 1, 71), 2, 4, 64, 64, qkv_dtype="bf16", gate=gate, gate_law=law,
                       h0=True, chunk=C, packed=True, beta_law=beta_law, seed=1200 + sb + C)
    _check(inputs.make(spec), arm, label="solve_block=%d C=%d %s/%s beta=%s" % (sb, C, gate, law, beta_law),
           solve_block=sb)


@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 128), (64, 64), (128, 32), (128, 64), (128, 128)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_widths_and_chunks(dk, dv, chunk, arm):
    spec = inputs.Spec("widths", (150,), 1, 2, dk, dv, qkv_dtype="bf16", gate_law="clip5", h0=True,
                       chunk=chunk, seed=dk * 7 + dv + chunk)
    _check(inputs.make(spec), arm, chunk=chunk, label="dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_packed_sequences_with_empty_and_short(arm, gate):
    law = "uniform5" if gate == "channel" else "full"
    spec = inputs.Spec("packed-small", (100, 0, 1, 64, 257, 31), 2, 6, 128, 128, qkv_dtype="bf16",
                       gate=gate, gate_law=law, h0=True, chunk=32 if gate == "channel" else 64,
                       packed=True, seed=55)
    _check(inputs.make(spec), arm, label="packed %s" % gate)


@pytest.mark.parametrize("arm", ["f32", "bf16"])
def test_fp32_inputs_and_outputs(arm):
    spec = inputs.Spec("f32io", (300,), 2, 2, 128, 128, qkv_dtype="f32", gate_law="half", h0=True,
                       chunk=64, o_dtype="f32", seed=31)
    _check(inputs.make(spec), arm)


def test_single_sequence_config():
    _check(inputs.make("single"), "bf16")


def test_stage_calls_equal_one_full_call_bitwise():
    """PREP then SCAN on one workspace is the same work as one call: same bits."""
    import ctypes
    from linear_attention_rnn_chunk_amd import gdn
    from tests.gpu_util import device_inputs
    spec = inputs.Spec("stages", (64, 100, 7), 2, 4, 128, 128, qkv_dtype="bf16", gate_law="half",
                       h0=True, chunk=64, packed=True, seed=3)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    outs = []
    for stages_list in ([gdn.STAGE_ALL], [gdn.STAGE_PREP, gdn.STAGE_SCAN]):
        o = torch.empty((1, spec.tokens, spec.hv, spec.dv), dtype=torch.bfloat16, device="cuda")
        hT = torch.empty((spec.n_seq, spec.hv, spec.dk, spec.dv), dtype=torch.float32, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = None
        for stages in stages_list:
            prob = gdn.make_problem(spec.n_seq, spec.tokens, 0, spec.hk, spec.hv, spec.dk, spec.dv,
                                    gdn.GATE_HEAD, 64, gdn.BF16, gdn.BF16, gdn.ARM_MFMA_BF16,
                                    gdn.COMPOSE_SPLIT, stages)
            if ws is None:
                ws = torch.empty(gdn.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
            assert gdn.chunk_fwd_raw(prob, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                     d["cu_seqlens"], o, hT, st, ws) == gdn.GDN_OK
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        outs.append((o.clone(), hT.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
