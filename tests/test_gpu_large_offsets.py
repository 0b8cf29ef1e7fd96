"""A layer whose value and output tensors hold more than 2^31 elements: one sequence of
360,448 tokens with the hybrid layer's heads (16 key / 48 value, d = 128), so every
element offset past token 349,526 of v and o needs more than 31 bits.  The whole call
must equal, bit for bit, its two halves run one after the other through the final
state (the second half then sits at small offsets of tensors of its own); and the last
value head, whose rows lie highest in memory, is checked against the fp64 oracle over
the whole sequence.  The same for the per-channel gate, whose gate tensor and gated
operands pass 2^31 elements, and for the one-token step over a batch whose states do.
Inputs are drawn on the device with a seeded generator, with the workloads'
distributions (unit-norm rows, q scaled by dk^-1/2, v ~ N(0,1), beta = sigmoid(N),
g = -0.5 softplus(N) or U[-5, 0] per key channel, h0 ~ 0.1 N)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from linear_attention_rnn_chunk_amd import gdn
from tests.gpu_util import BOUND, rel

pytestmark = pytest.mark.gpu

T, HK, HV, D = 360_448, 16, 48, 128   # 5,632 chunks of 64


def _inputs():
    gen = torch.Generator(device="cuda").manual_seed(20241203)
    dev = "cuda"
    def unit_rows(shape, scale):
        x = torch.randn(shape, device=dev, generator=gen)
        return (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12) * scale).to(torch.bfloat16)
    q = unit_rows((1, T, HK, D), D ** -0.5)
    k = unit_rows((1, T, HK, D), 1.0)
    v = torch.empty((1, T, HV, D), dtype=torch.bfloat16, device=dev)
    for a in range(0, T, 32768):  # fp32 draws a slab at a time
        b = min(T, a + 32768)
        v[:, a:b] = torch.randn((1, b - a, HV, D), device=dev, generator=gen).to(torch.bfloat16)
    g = -0.5 * F.softplus(torch.randn((1, T, HV), device=dev, generator=gen))
    beta = torch.sigmoid(torch.randn((1, T, HV), device=dev, generator=gen))
    h0 = 0.1 * torch.randn((1, HV, D, D), device=dev, generator=gen)
    return q, k, v, g.contiguous(), beta.contiguous(), h0


def test_offsets_beyond_31_bits():
    assert T * HV * D > 2 ** 31
    print("inputs: %d tokens, %d/%d heads, d=%d" % (T, HK, HV, D), flush=True)
    q, k, v, g, beta, h0 = _inputs()
    print("whole call (library composition)", flush=True)
    o, hT, _ = gdn.chunk_fwd(q, k, v, g, beta, h0)
    half = T // 2   # 2,816 chunks each
    print("two halves through the final state", flush=True)
    o1, h1, _ = gdn.chunk_fwd(q[:, :half], k[:, :half], v[:, :half], g[:, :half], beta[:, :half], h0)
    o2, h2, _ = gdn.chunk_fwd(q[:, half:], k[:, half:], v[:, half:], g[:, half:], beta[:, half:], h1)
    assert torch.equal(o[:, :half], o1)
    assert torch.equal(o[:, half:], o2)
    assert torch.equal(hT, h2)
    del o1, o2, h1, h2
    # the last value head (key head 15) against the oracle, over the whole sequence
    h, kh = HV - 1, HK - 1
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    print("oracle: value head %d over %d tokens" % (h, T), flush=True)
    o_ref, h_ref = oracle.serial_fwd(f64(q[0, :, kh:kh + 1]), f64(k[0, :, kh:kh + 1]), f64(v[0, :, h:h + 1]),
                                     f64(g[0, :, h:h + 1]), f64(beta[0, :, h:h + 1]), f64(h0[:, h:h + 1]))
    og = f64(o[0, :, h:h + 1])
    eo, eh = rel(og, o_ref), rel(f64(hT[:, h:h + 1]), h_ref)
    eo_last = rel(og[-64:], o_ref[-64:])
    print("rel-L2 o %.3e (last chunk %.3e) hT %.3e" % (eo, eo_last, eh), flush=True)
    assert eo <= BOUND["bf16"] and eh <= BOUND["bf16"] and eo_last <= BOUND["bf16"]


def test_per_channel_gate_offsets_beyond_31_bits():
    # the per-channel gate g [T, hv, dk] fp32 and the prep's gated operands (three
    # [C][dk] tiles per chunk and head) pass 2^31 elements: 540,672 tokens, 32/32 heads
    Tc, H = 540_672, 32   # 16,896 chunks of 32
    assert Tc * H * D > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(20241204)
    def unit_rows(scale):
        out = torch.empty((1, Tc, H, D), dtype=torch.bfloat16, device="cuda")
        for a in range(0, Tc, 65536):
            b = min(Tc, a + 65536)
            x = torch.randn((1, b - a, H, D), device="cuda", generator=gen)
            out[:, a:b] = (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12) * scale).to(torch.bfloat16)
        return out
    print("inputs: %d tokens, %d/%d heads, per-channel gate U[-5, 0]" % (Tc, H, H), flush=True)
    q, k = unit_rows(D ** -0.5), unit_rows(1.0)
    v = torch.empty((1, Tc, H, D), dtype=torch.bfloat16, device="cuda")
    for a in range(0, Tc, 65536):
        b = min(Tc, a + 65536)
        v[:, a:b] = torch.randn((1, b - a, H, D), device="cuda", generator=gen).to(torch.bfloat16)
    g = torch.empty((1, Tc, H, D), dtype=torch.float32, device="cuda")
    for a in range(0, Tc, 65536):
        b = min(Tc, a + 65536)
        g[:, a:b] = -5.0 * torch.rand((1, b - a, H, D), device="cuda", generator=gen)
    beta = torch.sigmoid(torch.randn((1, Tc, H), device="cuda", generator=gen))
    o, hT, _ = gdn.chunk_fwd(q, k, v, g, beta, None, chunk=32)
    half = Tc // 2
    print("two halves through the final state", flush=True)
    o1, h1, _ = gdn.chunk_fwd(q[:, :half], k[:, :half], v[:, :half], g[:, :half], beta[:, :half], None, chunk=32)
    o2, h2, _ = gdn.chunk_fwd(q[:, half:], k[:, half:], v[:, half:], g[:, half:], beta[:, half:], h1, chunk=32)
    assert torch.equal(o[:, :half], o1) and torch.equal(o[:, half:], o2) and torch.equal(hT, h2)
    del o1, o2, h1, h2
    h = H - 1
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    print("oracle: value head %d over %d tokens" % (h, Tc), flush=True)
    o_ref, h_ref = oracle.serial_fwd(f64(q[0, :, h:h + 1]), f64(k[0, :, h:h + 1]), f64(v[0, :, h:h + 1]),
                                     f64(g[0, :, h:h + 1]), f64(beta[0, :, h:h + 1]), None)
    og = f64(o[0, :, h:h + 1])
    eo, eh, eo_last = rel(og, o_ref), rel(f64(hT[:, h:h + 1]), h_ref), rel(og[-32:], o_ref[-32:])
    print("rel-L2 o %.3e (last chunk %.3e) hT %.3e" % (eo, eo_last, eh), flush=True)
    assert eo <= BOUND["bf16"] and eh <= BOUND["bf16"] and eo_last <= BOUND["bf16"]


def test_one_token_step_states_beyond_31_bits():
    # 2,816 sequences x 48 value heads of 128 x 128 fp32 states: 2.2e9 state elements
    B = 2816
    assert B * HV * D * D > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(20241205)
    x = torch.randn((B, HK, D), device="cuda", generator=gen)
    k = (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    x = torch.randn((B, HK, D), device="cuda", generator=gen)
    q = (x / x.norm(dim=-1, keepdim=True) * D ** -0.5).to(torch.bfloat16)
    v = torch.randn((B, HV, D), device="cuda", generator=gen).to(torch.bfloat16)
    g = -0.5 * F.softplus(torch.randn((B, HV), device="cuda", generator=gen))
    beta = torch.sigmoid(torch.randn((B, HV), device="cuda", generator=gen))
    h_in = torch.empty((B, HV, D, D), dtype=torch.float32, device="cuda")
    for a in range(0, B, 256):
        h_in[a:a + 256] = 0.1 * torch.randn((min(B, a + 256) - a, HV, D, D), device="cuda", generator=gen)
    print("one-token step: %d sequences, %d/%d heads, d=%d" % (B, HK, HV, D), flush=True)
    o, h_out, _ = gdn.decode_step(q, k, v, g, beta, h_in, o_dtype=torch.float32)
    b0 = B // 2
    o2, h2, _ = gdn.decode_step(q[b0:], k[b0:], v[b0:], g[b0:], beta[b0:], h_in[b0:].contiguous(),
                                o_dtype=torch.float32)
    assert torch.equal(o[b0:], o2) and torch.equal(h_out[b0:], h2)
    n = B - 1   # the last sequence, highest in memory, every head, against the oracle
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    o_ref, h_ref = oracle.serial_fwd(f64(q[n:n + 1]), f64(k[n:n + 1]), f64(v[n:n + 1]), f64(g[n:n + 1]),
                                     f64(beta[n:n + 1]), f64(h_in[n:n + 1]))
    eo, eh = rel(f64(o[n:n + 1]), o_ref), rel(f64(h_out[n:n + 1]), h_ref)
    print("last sequence rel-L2 o %.3e h_out %.3e" % (eo, eh), flush=True)
    assert eo <= 1e-5 and eh <= 1e-5
