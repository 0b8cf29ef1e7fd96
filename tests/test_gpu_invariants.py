"""GPU checks beyond element-wise parity:

* the solve pinned tile by tile (T and P in the workspace vs the dense chunk oracle),
* negative controls that must FAIL the bounds (each mistake is planted in the oracle,
  on the CPU, never in GPU code),
* bitwise contracts between GPU runs (determinism, grouped vs repeated heads, packed vs
  per-sequence, chunk-aligned continuation, causality, immutable h0),
* device status bits forced from the host (non-finite inputs, gate domain, malformed
  cu_seqlens, non-finite outputs), all without a fault.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import chunked
from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import (BOUND, device_inputs, oracle_ref, rel, run_gpu, to_np64,
                            workspace_tile_views)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ tile level -----
# every diagonal block of the solve (8, 16, 32 rows); 8 rows is the size at which a missing
# wait between one lane's LDS write and another lane's read shows first
@pytest.mark.parametrize("arm,tol", [("bf16", 1e-2), ("f32", 1e-5)])
@pytest.mark.parametrize("gate,law,C", [("head", "clip5", 64), ("head", "clip5", 32), ("channel", "uniform5", 32),
                                        ("channel", "uniform05", 32)])
@pytest.mark.parametrize("sb", [8, 16, 32])
def test_solve_and_P_tiles_match_chunk_oracle(sb, arm, tol, gate, law, C):
    spec = inputs.Spec("tiles", (150,), 1, 2, 64, 64, qkv_dtype="bf16", gate=gate, gate_law=law,
                       h0=True, chunk=C, seed=21)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    prob = gdn.make_problem(1, spec.tokens, spec.tokens, 1, 2, 64, 64,
                            gdn.GATE_KEY_CHANNEL if gate == "channel" else gdn.GATE_HEAD, C,
                            gdn.BF16, gdn.F32 if arm == "f32" else gdn.BF16,
                            gdn.ARM_FOLD_F32 if arm == "f32" else gdn.ARM_MFMA_BF16,
                            gdn.COMPOSE_SPLIT, gdn.STAGE_PREP, solve_block=sb)
    ws = torch.zeros(gdn.workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty((1, spec.tokens, 2, 64), dtype=torch.float32 if arm == "f32" else torch.bfloat16,
                    device="cuda")
    assert gdn.chunk_fwd_raw(prob, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, o,
                             None, st, ws) == gdn.GDN_OK
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    Tg, Pg = workspace_tile_views(prob, ws, arm == "f32")
    _, _, tiles = chunked.chunked_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                      inp.as_f64("g"), inp.as_f64("beta"), inp.as_f64("h0"),
                                      chunk=C, pad_to=True, want_tiles=True)
    worst_t = worst_p = 0.0
    for (n, h, ci), t in tiles.items():
        et = rel(Tg[ci, h].float().cpu().numpy(), t["T"])
        ep = rel(Pg[ci, h].float().cpu().numpy(), t["P"])
        worst_t, worst_p = max(worst_t, et), max(worst_p, ep)
    print("tiles solve_block=%d C=%d %s %s: worst rel-L2 T %.3e P %.3e" % (sb, C, arm, law, worst_t, worst_p),
          flush=True)
    assert worst_t <= tol and worst_p <= tol


# ------------------------------------------------------- negative controls -----
def _gpu_and_ref(spec, arm="bf16"):
    inp = inputs.make(spec)
    o, hT, _ = run_gpu(inp, arm=arm)
    return inp, to_np64(o), to_np64(hT)


def test_nc1_checker_fails_a_result_at_two_and_a_half_bounds():
    inp, o, hT = _gpu_and_ref(inputs.CONFIGS["tiny"])
    o_ref, _ = oracle_ref(inp)
    z = np.random.default_rng(0).standard_normal(o.shape)
    bad = o_ref + 2.5 * BOUND["bf16"] * np.linalg.norm(o_ref) * z / np.linalg.norm(z)
    assert rel(bad, o_ref) > BOUND["bf16"]
    assert rel(o, o_ref) <= BOUND["bf16"]


@pytest.mark.parametrize("gate,law,C", [("head", "half", 64), ("channel", "uniform5", 32)])
def test_nc2_gate_read_one_token_late_fails(gate, law, C):
    spec = inputs.Spec("nc2", (300,), 2, 4, 64, 64, gate=gate, gate_law=law, h0=True, chunk=C, seed=5)
    inp, o, hT = _gpu_and_ref(spec)
    o_bad, h_bad = oracle_ref(inp, mutant=oracle.MUT_GATE_NEXT_TOKEN)
    o_ref, h_ref = oracle_ref(inp)
    assert rel(o, o_ref) <= BOUND["bf16"]
    assert max(rel(o, o_bad), rel(hT, h_bad)) > BOUND["bf16"]


def test_nc4_skipped_solve_fails_with_per_head_gate():
    spec = inputs.Spec("nc4", (300,), 2, 4, 128, 128, gate_law="half", h0=True, chunk=64, seed=6)
    inp, o, hT = _gpu_and_ref(spec)
    o_bad, h_bad = chunked.chunked_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                       inp.as_f64("g"), inp.as_f64("beta"), inp.as_f64("h0"),
                                       chunk=64, mutant="skip_solve")
    print("NC4 skipped solve: o %.3e hT %.3e" % (rel(o, o_bad), rel(hT, h_bad)))
    assert max(rel(o, o_bad), rel(hT, h_bad)) > BOUND["bf16"]


def test_nc5_missing_state_reset_fails_the_first_chunk_metric():
    spec = inputs.Spec("nc5", (200, 130, 90), 2, 4, 64, 64, gate_law="half", h0=True, chunk=64,
                       packed=True, seed=8)
    inp, o, hT = _gpu_and_ref(spec)
    o_bad, _ = chunked.chunked_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                   inp.as_f64("g"), inp.as_f64("beta"), inp.as_f64("h0"),
                                   seq_start=inp.cu_seqlens, chunk=64, mutant="no_reset")
    o_ref, _ = oracle_ref(inp)
    cu = inp.cu_seqlens
    for n in (1, 2):
        fc = slice(int(cu[n]), int(cu[n]) + 64)
        assert rel(o[fc], o_ref[fc]) <= BOUND["bf16"]
        assert rel(o[fc], o_bad[fc]) > BOUND["bf16"]


def test_nc6_debug_arm_bound_sees_bf16_rounding():
    spec = inputs.Spec("nc6", (256,), 2, 2, 128, 128, gate_law="half", h0=True, chunk=64, seed=9)
    inp = inputs.make(spec)
    o32, h32, _ = run_gpu(inp, arm="f32")
    o16, h16, _ = run_gpu(inp, arm="bf16", o_dtype=torch.float32)
    o_ref, h_ref = oracle_ref(inp)
    assert rel(to_np64(o32), o_ref) <= BOUND["f32"]
    assert rel(to_np64(o16), to_np64(o32)) > BOUND["f32"]


# ------------------------------------------------------ bitwise contracts -----
def _run(spec_or_inp, **kw):
    inp = inputs.make(spec_or_inp) if not isinstance(spec_or_inp, inputs.Inputs) else spec_or_inp
    o, hT, _ = run_gpu(inp, **kw)
    return o.clone(), hT.clone()


def test_run_to_run_bitwise_determinism():
    inp = inputs.make(inputs.CONFIGS["single"].with_(seq_lens=(1000,)))
    a = _run(inp)
    b = _run(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_grouped_heads_equal_repeated_key_heads_bitwise():
    spec = inputs.Spec("grp", (333,), 2, 6, 128, 128, gate_law="half", h0=True, chunk=64, seed=12)
    inp = inputs.make(spec)
    a = _run(inp)
    rep = inputs.Inputs(spec.with_(hk=6), np.repeat(inp.q, 3, axis=1), np.repeat(inp.k, 3, axis=1),
                        inp.v, inp.g, inp.beta, inp.h0, inp.cu_seqlens)
    b = _run(rep)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("gate,law,C", [("head", "full", 64), ("channel", "uniform5", 32)])
def test_packed_equals_per_sequence_bitwise(gate, law, C):
    lens = (128, 0, 77, 192, 5)
    spec = inputs.Spec("pk", lens, 2, 4, 128, 64, gate=gate, gate_law=law, h0=True, chunk=C,
                       packed=True, seed=13)
    inp = inputs.make(spec)
    o, hT = _run(inp)
    cu = inp.cu_seqlens
    for n, L in enumerate(lens):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        one = inputs.Inputs(spec.with_(seq_lens=(L,), packed=True), inp.q[sl], inp.k[sl], inp.v[sl],
                            inp.g[sl], inp.beta[sl], inp.h0[n:n + 1], np.array([0, L], np.int32))
        o1, h1 = _run(one)
        assert torch.equal(o[sl], o1), n
        assert torch.equal(hT[n], h1[0]), n


def test_chunk_aligned_continuation_bitwise():
    spec = inputs.Spec("cont", (320,), 2, 4, 128, 128, gate_law="half", h0=True, chunk=64, seed=14)
    inp = inputs.make(spec)
    o, hT = _run(inp)
    cut = 128
    part = lambda a, sl: a[sl]
    first = inputs.Inputs(spec.with_(seq_lens=(cut,)), inp.q[:cut], inp.k[:cut], inp.v[:cut],
                          inp.g[:cut], inp.beta[:cut], inp.h0, np.array([0, cut], np.int32))
    o1, h1 = _run(first)
    second = inputs.Inputs(spec.with_(seq_lens=(320 - cut,)), inp.q[cut:], inp.k[cut:], inp.v[cut:],
                           inp.g[cut:], inp.beta[cut:], h1.cpu().numpy(),
                           np.array([0, 320 - cut], np.int32))
    o2, h2 = _run(second)
    assert torch.equal(torch.cat([o1, o2]), o)
    assert torch.equal(h2, hT)


@pytest.mark.parametrize("t", [0, 70, 199])
def test_causality_bitwise(t):
    spec = inputs.Spec("caus", (200,), 2, 4, 64, 64, gate_law="half", h0=True, chunk=64, seed=15)
    inp = inputs.make(spec)
    o, _ = _run(inp)
    q, k, v, g, b = (x.copy() for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    v[t] = inputs.bf16_round_bits(inputs.bf16_bits_to_f32(v[t]) + 1.0)
    g[t] -= 0.3
    b[t] = 0.9
    pert = inputs.Inputs(spec, q, k, v, g, b, inp.h0, inp.cu_seqlens)
    o2, _ = _run(pert)
    assert torch.equal(o[:t], o2[:t])
    assert not torch.equal(o[t], o2[t])


def test_h0_is_never_written():
    inp = inputs.make(inputs.CONFIGS["tiny"])
    d = device_inputs(inp)
    before = d["h0"].clone()
    gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, arm="bf16")
    assert torch.equal(before, d["h0"])


# ------------------------------------------------------------- status bits -----
def _status(inp, arm="bf16", cu=None):
    d = device_inputs(inp)
    if cu is not None:
        d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device="cuda")
        d = {k_: (v_.reshape((1, -1) + tuple(v_.shape[2:])) if k_ in ("q", "k", "v", "g", "beta") else v_)
             for k_, v_ in d.items()}
    o, hT, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              chunk=inp.spec.chunk, arm=arm, check=False)
    torch.cuda.synchronize()
    return int(st.item()) & 0xFFFFFFFF


def _small(**kw):
    base = dict(seq_lens=(100,), hk=1, hv=2, dk=64, dv=64, gate_law="half", h0=True, chunk=64, seed=30)
    base.update(kw)
    return inputs.Spec("st", **base)


def test_clean_inputs_set_no_status():
    assert _status(inputs.make(_small())) == 0


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "beta", "h0"])
def test_nonfinite_input_is_flagged(field):
    inp = inputs.make(_small())
    a = getattr(inp, field).copy()
    flat = a.reshape(-1)
    flat[7] = 0x7FC0 if a.dtype == np.uint16 else np.float32(np.nan)
    setattr(inp, field, a)
    assert _status(inp) & gdn.ST_NONFINITE_INPUT


def test_positive_gate_is_outside_the_domain():
    inp = inputs.make(_small())
    inp.g[5, 1] = 0.25
    assert _status(inp) & gdn.ST_GATE_DOMAIN


def test_channel_gate_below_minus_five_is_outside_the_domain():
    inp = inputs.make(_small(gate="channel", gate_law="uniform5", chunk=32))
    inp.g[3, 0, 9] = -7.0
    st = _status(inp)
    assert st & gdn.ST_GATE_DOMAIN and not st & gdn.ST_NONFINITE_OUTPUT


@pytest.mark.parametrize("cu", [[0, 60, 40, 100], [5, 60, 100], [0, 60, 90], [0, 60, 130]])
def test_malformed_cu_seqlens_flagged_without_fault(cu):
    inp = inputs.make(_small(seq_lens=(100,)))
    # three or two sequences over the same 100 tokens; h0 per sequence
    n = len(cu) - 1
    inp.h0 = np.repeat(inp.h0, n, axis=0)
    assert _status(inp, cu=cu) & gdn.ST_BAD_SEQLENS


def test_overflowing_output_is_flagged():
    inp = inputs.make(_small())
    inp.h0 = np.full_like(inp.h0, 3.0e38)
    assert _status(inp) & gdn.ST_NONFINITE_OUTPUT


def test_all_empty_sequences_return_h0():
    spec = inputs.Spec("empty", (0, 0, 0), 1, 2, 64, 64, gate_law="half", h0=True, chunk=64,
                       packed=True, seed=31)
    inp = inputs.make(spec)
    d = device_inputs(inp)
    o, hT, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    assert torch.equal(hT, d["h0"])
