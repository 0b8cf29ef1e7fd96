"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its binding, and evaluate the oracle on the same values."""
import numpy as np
import torch

import oracle
from linear_attention_rnn_chunk_amd import gdn, inputs

BOUND = {"f32": 1e-4, "bf16": 2e-2}
ODT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev_tensor(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def is_packed(spec):
    return spec.packed or len(set(spec.seq_lens)) > 1


def device_inputs(inp):
    spec = inp.spec
    q, k, v, g, b = (dev_tensor(getattr(inp, n)) for n in ("q", "k", "v", "g", "beta"))
    h0 = dev_tensor(inp.h0)
    if is_packed(spec):
        shp = lambda x: x.unsqueeze(0)
        cu = torch.from_numpy(inp.cu_seqlens).to("cuda")
    else:
        B, T = spec.n_seq, spec.seq_lens[0]
        shp = lambda x: x.reshape((B, T) + tuple(x.shape[1:]))
        cu = None
    return dict(q=shp(q), k=shp(k), v=shp(v), g=shp(g), beta=shp(b), h0=h0, cu_seqlens=cu)


def run_gpu(inp, arm="bf16", chunk=None, compose="auto", o_dtype=None, d=None, check=True, solve_block=0):
    d = d or device_inputs(inp)
    odt = o_dtype or ODT[arm]
    o, hT, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              chunk=chunk if chunk is not None else inp.spec.chunk, arm=arm,
                              o_dtype=odt, compose=compose, check=check, solve_block=solve_block)
    tok = inp.spec.tokens
    o = o.reshape(tok, inp.spec.hv, inp.spec.dv)
    return o, hT, st


def to_np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_ref(inp, units=None, want_o=True, mutant=oracle.CORRECT):
    return oracle.serial_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                             inp.as_f64("beta"), inp.as_f64("h0"), seq_start=inp.cu_seqlens,
                             units=units, want_o=want_o, mutant=mutant)


# fp32's grid below 2^-126 (its subnormals) has the fixed spacing 2^-149, so there a value
# is held to an absolute, not a relative, resolution: a state decayed into that band by
# e^-90 .. e^-103 carries an error of a grid step or so from its last few fp32 roundings
# however exactly it was computed.  Each element's error counts only beyond 16 such steps;
# against a normal fp32 value (>= 2^-126) that allowance is at most 2^-19 of the value.
SUBNORMAL_ALLOWANCE = 16 * 2.0 ** -149


def rel(x, ref):
    """NaN-aware relative L2 of a GPU result x against the fp64 oracle's ref.  ref is first
    taken to fp32 (the exponent range of every output, fp32 or bf16): a value below that
    range (a state decayed by e^-160, say) has no representation but zero there, so it
    cannot count as error; and each element's error counts beyond SUBNORMAL_ALLOWANCE."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64).astype(np.float32).astype(np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    err = np.maximum(np.abs(x - ref) - SUBNORMAL_ALLOWANCE, 0.0)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm(err.ravel()) / den) if den > 0 else float(np.linalg.norm(err.ravel()))


def oracle_units(inp, units, want_o=True):
    """fp64 oracle on selected (sequence, value head) units only; returns
    {(n, h): (o [len, dv] or None, hT [dk, dv])}.  Each unit becomes one sequence of a
    packed single-head problem (its key head's q/k, its value head's v/g/beta, its h0),
    so large workloads stay cheap and the units run in parallel."""
    spec = inp.spec
    group = spec.hv // spec.hk
    cu = inp.cu_seqlens
    q32, k32, v32 = inp.as_f32("q"), inp.as_f32("k"), inp.as_f32("v")
    qs, ks, vs, gs, bs, h0s, starts = [], [], [], [], [], [], [0]
    for n, h in units:
        kh = h // group
        sl = slice(int(cu[n]), int(cu[n + 1]))
        qs.append(q32[sl, kh:kh + 1])
        ks.append(k32[sl, kh:kh + 1])
        vs.append(v32[sl, h:h + 1])
        gs.append(inp.g[sl, h:h + 1])
        bs.append(inp.beta[sl, h:h + 1])
        h0s.append(np.zeros((1, spec.dk, spec.dv)) if inp.h0 is None else inp.h0[n, h:h + 1])
        starts.append(starts[-1] + (sl.stop - sl.start))
    cat = lambda xs: np.concatenate(xs).astype(np.float64)
    o, hT = oracle.serial_fwd(cat(qs), cat(ks), cat(vs), cat(gs), cat(bs),
                              np.stack(h0s).astype(np.float64), seq_start=np.array(starts),
                              want_o=want_o)
    out = {}
    for i, u in enumerate(units):
        out[tuple(u)] = (None if o is None else o[starts[i]:starts[i + 1], 0], hT[i, 0])
    return out


def tile_frags(C):
    """(mt, sb) of the stored fragments of a C x C lower-triangular tile, in order."""
    return [(mt, sb) for mt in range(C // 16) for sb in range(mt // 2 + 1)]


def decode_tiles(frag, C):
    """Dense [..., C, C] tiles from stored fragments [..., n_frag, 64, 8]: fragment (mt, sb),
    lane l = 16 g + i, element e holds row 16 mt + i, column 32 sb + 4 g + e (e < 4) or
    32 sb + 16 + 4 g + e - 4 (e >= 4); entries no fragment covers are zero."""
    import torch
    out = torch.zeros(frag.shape[:-3] + (C, C), dtype=frag.dtype, device=frag.device)
    lane = torch.arange(64)
    i, g = lane % 16, lane // 16
    for f, (mt, sb) in enumerate(tile_frags(C)):
        for e in range(8):
            col = 32 * sb + 4 * g + (e if e < 4 else 16 + e - 4)
            out[..., 16 * mt + i, col] = frag[..., f, :, e]
    return out


def workspace_tile_views(prob, ws, arm_f32):
    """T and P tiles inside the library's workspace for a fixed-length problem, decoded to
    dense [slot][hv][C][C] (layout: T fragments [slot][hv][n_frag][64][8], then P
    fragments, each region 256-byte aligned)."""
    import torch
    C = prob.chunk
    esz = 4 if arm_f32 else 2
    nf = len(tile_frags(C))
    cps = (prob.seq_len + C - 1) // C
    slots = prob.n_seq * cps
    n = slots * prob.hv * nf * 512
    tile_bytes = n * esz
    off_p = (tile_bytes + 255) // 256 * 256
    dt = torch.float32 if arm_f32 else torch.bfloat16
    T = ws[:tile_bytes].view(dt).view(slots, prob.hv, nf, 64, 8)
    P = ws[off_p:off_p + tile_bytes].view(dt).view(slots, prob.hv, nf, 64, 8)
    return decode_tiles(T, C), decode_tiles(P, C)
