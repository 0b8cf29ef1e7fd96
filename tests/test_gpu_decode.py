"""GPU parity of the one-token recurrent step (gdn_decode_step) against the fp64
token-serial oracle run on one-token sequences, and of prefill followed by steps
against the oracle on the whole sequences.

Bounds (relative L2, NaN-aware), derived from the step's arithmetic: everything is
fp32 with two dot products of length dk <= 128 per state column, so the relative
error of h_out and of an fp32 o is a few units of 2^-24 times sqrt(dk), about 1e-6;
1e-5 leaves a margin of ten.  A bf16 o adds its own rounding, at most 2^-9 relative
per element, so 4e-3.  A step that continues a GPU prefill inherits the prefill's
state error, so there the prefill's bounds apply (fp32-fold arm 1e-4, bf16 arm 2e-2).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_rnn_chunk_amd import gdn, inputs
from tests.gpu_util import BOUND, dev_tensor, oracle_units, rel, to_np64

pytestmark = pytest.mark.gpu

STEP_BOUND = {"h": 1e-5, "f32": 1e-5, "bf16": 4e-3}
ODT = {"f32": torch.float32, "bf16": torch.bfloat16}


def decode_spec(B, hk, hv, dk, dv, gate="head", qkv="bf16", h0=True, seed=0, **kw):
    law = "uniform5" if gate == "channel" else "half"
    return inputs.Spec("decode", (1,) * B, hk, hv, dk, dv, qkv_dtype=qkv, gate=gate, gate_law=law,
                       h0=h0, packed=True, seed=seed, **kw)


def step_args(inp):
    return tuple(dev_tensor(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta", "h0"))


def oracle_step(inp):
    return oracle.serial_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                             inp.as_f64("beta"), inp.as_f64("h0"), seq_start=inp.cu_seqlens)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("qkv,odt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_step_matches_oracle(dk, dv, gate, qkv, odt):
    inp = inputs.make(decode_spec(5, 2, 6, dk, dv, gate=gate, qkv=qkv, seed=dk + dv))
    q, k, v, g, b, h_in = step_args(inp)
    h_keep = h_in.clone()
    o, h_out, _ = gdn.decode_step(q, k, v, g, b, h_in, o_dtype=ODT[odt])
    o_ref, h_ref = oracle_step(inp)
    eo, eh = rel(to_np64(o), o_ref), rel(to_np64(h_out), h_ref)
    print("step dk=%d dv=%d %s %s/%s rel-L2 o=%.2e h=%.2e" % (dk, dv, gate, qkv, odt, eo, eh), flush=True)
    assert eo <= STEP_BOUND[odt] and eh <= STEP_BOUND["h"], (eo, eh)
    assert torch.equal(h_in, h_keep)  # the input state is never written


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_step_from_zero_state(gate):
    inp = inputs.make(decode_spec(3, 1, 4, 128, 128, gate=gate, h0=False, seed=7))
    q, k, v, g, b, _ = step_args(inp)
    o, h_out, _ = gdn.decode_step(q, k, v, g, b, None, o_dtype=torch.float32)
    o_ref, h_ref = oracle_step(inp)
    assert rel(to_np64(o), o_ref) <= STEP_BOUND["f32"]
    assert rel(to_np64(h_out), h_ref) <= STEP_BOUND["h"]
    zeros = torch.zeros_like(h_out)
    o2, h2, _ = gdn.decode_step(q, k, v, g, b, zeros, o_dtype=torch.float32)
    assert torch.equal(o, o2) and torch.equal(h_out, h2)  # NULL state == zero state, bitwise


def test_step_deterministic():
    inp = inputs.make(decode_spec(8, 4, 12, 128, 128, seed=11))
    args = step_args(inp)
    o1, h1, _ = gdn.decode_step(*args)
    o2, h2, _ = gdn.decode_step(*args)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_step_at_serving_batch_sampled():
    """The timed decode workload (256 sequences of the hybrid layer: 16 key / 48 value
    heads, d = 128, bf16): 64 sampled (sequence, head) units against the oracle, and
    every state finite and moved by the step."""
    inp = inputs.make(decode_spec(256, 16, 48, 128, 128, seed=2003))
    q, k, v, g, b, h_in = step_args(inp)
    o, h_out, _ = gdn.decode_step(q, k, v, g, b, h_in)
    rng = np.random.default_rng(5)
    units = sorted({(int(n), int(h)) for n, h in zip(rng.integers(0, 256, 64), rng.integers(0, 48, 64))})
    units += [(0, 0), (255, 47)]
    ref = oracle_units(inp, units)
    on, hn = to_np64(o), h_out
    for n, h in units:
        o_ref, h_ref = ref[(n, h)]
        eo = rel(on[n, h], o_ref[0])
        eh = rel(to_np64(hn[n, h]), h_ref)
        assert eo <= STEP_BOUND["bf16"] and eh <= STEP_BOUND["h"], ((n, h), eo, eh)
    assert torch.isfinite(h_out).all()


@pytest.mark.parametrize("arm", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prefill_then_steps(arm, gate):
    """Prefill of T tokens (gdn_chunk_fwd), then three steps, each from the previous
    state: the steps' outputs and final state against the oracle on T + 3 tokens."""
    B, T, S = 2, 130, 3
    law = "uniform05" if gate == "channel" else "half"
    spec = inputs.Spec("cont", (T + S,) * B, 2, 6, 128, 128, qkv_dtype="bf16", gate=gate,
                       gate_law=law, h0=True, chunk=32 if gate == "channel" else 64, seed=77)
    inp = inputs.make(spec)
    o_ref, h_ref = oracle.serial_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                     inp.as_f64("g"), inp.as_f64("beta"), inp.as_f64("h0"),
                                     seq_start=inp.cu_seqlens)
    full = {n: dev_tensor(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta")}
    per_seq = {n: t.reshape((B, T + S) + tuple(t.shape[1:])) for n, t in full.items()}
    h0 = dev_tensor(inp.h0)
    pre = {n: t[:, :T].contiguous() for n, t in per_seq.items()}
    odt = ODT[arm]
    o_pre, state, _ = gdn.chunk_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], h0,
                                    arm=arm, o_dtype=odt)
    o_ref = o_ref.reshape(B, T + S, 6, 128)
    assert rel(to_np64(o_pre), o_ref[:, :T]) <= BOUND[arm]
    for s in range(S):
        tok = {n: t[:, T + s].contiguous() for n, t in per_seq.items()}
        o, nxt, _ = gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], state,
                                    o_dtype=odt)
        eo = rel(to_np64(o), o_ref[:, T + s])
        print("arm=%s gate=%s step %d rel-L2 o=%.2e" % (arm, gate, s, eo), flush=True)
        assert eo <= BOUND[arm]
        state = nxt
    eh = rel(to_np64(state), h_ref)
    print("arm=%s gate=%s final state rel-L2 %.2e" % (arm, gate, eh), flush=True)
    assert eh <= BOUND[arm]


def test_step_status_bits():
    inp = inputs.make(decode_spec(4, 2, 4, 64, 64, seed=3))
    q, k, v, g, b, h_in = step_args(inp)
    _, _, st = gdn.decode_step(q, k, v, g, b, h_in, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    v_bad = v.clone()
    v_bad[2, 1, 5] = float("nan")
    _, _, st = gdn.decode_step(q, k, v_bad, g, b, h_in, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    h_bad = h_in.clone()
    h_bad[3, 0, 17, 9] = float("inf")
    _, _, st = gdn.decode_step(q, k, v, g, b, h_bad, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) & gdn.ST_NONFINITE_INPUT
    g_bad = g.clone()
    g_bad[1, 2] = 0.25
    _, _, st = gdn.decode_step(q, k, v, g_bad, b, h_in, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == gdn.ST_GATE_DOMAIN
    with pytest.raises(gdn.GdnStatusError):
        gdn.decode_step(q, k, v, g_bad, b, h_in)
    with pytest.raises(gdn.GdnError):
        gdn.decode_step(q, k, v, g, b, h_in, h_out=h_in)  # in-place state is refused
