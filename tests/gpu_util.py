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


def run_gpu(inp, arm="bf16", chunk=None, compose="auto", o_dtype=None, d=None, check=True):
    d = d or device_inputs(inp)
    odt = o_dtype or ODT[arm]
    o, hT, st = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              chunk=chunk if chunk is not None else inp.spec.chunk, arm=arm,
                              o_dtype=odt, compose=compose, check=check)
    tok = inp.spec.tokens
    o = o.reshape(tok, inp.spec.hv, inp.spec.dv)
    return o, hT, st


def to_np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_ref(inp, units=None, want_o=True, mutant=oracle.CORRECT):
    return oracle.serial_fwd(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.as_f64("g"),
                             inp.as_f64("beta"), inp.as_f64("h0"), seq_start=inp.cu_seqlens,
                             units=units, want_o=want_o, mutant=mutant)


def rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((x - ref).ravel()) / den) if den > 0 else float(np.linalg.norm(x.ravel()))
