"""Thin ctypes binding of the C ABI in ``include/gdn.h`` (libgdn_mi355x.so).

Argument marshalling only: shapes and dtypes are checked, device pointers and
the current HIP stream are passed through, and every step of the computation
runs in the library's kernels.  There is no CPU fallback: a missing library,
a CPU tensor or a host-side refusal raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libgdn_mi355x.so")
# the measurement build (built on request: python -m linear_attention_rnn_chunk_amd.build
# --stamps), the same library plus per-phase timestamps of the scan
STAMPS_LIBRARY_PATH = os.path.join(_HERE, "libgdn_mi355x_stamps.so")

GDN_OK, GDN_E_NULL, GDN_E_SHAPE, GDN_E_UNSUPPORTED, GDN_E_ALIAS, GDN_E_WORKSPACE, GDN_E_LAUNCH = range(7)
ST_NONFINITE_INPUT = 0x1
ST_GATE_DOMAIN = 0x2
ST_BAD_SEQLENS = 0x4
ST_NONFINITE_OUTPUT = 0x8
GATE_HEAD, GATE_KEY_CHANNEL = 0, 1
BF16, F32 = 0, 1
ARM_MFMA_BF16, ARM_FOLD_F32 = 0, 1
COMPOSE_AUTO, COMPOSE_SPLIT, COMPOSE_FUSED, COMPOSE_PIPELINED, COMPOSE_SEQSPLIT = 0, 1, 2, 3, 4
STAGE_ALL, STAGE_PREP, STAGE_SCAN = 0, 1, 2

# every symbol include/gdn.h declares
EXPORTS = ("gdn_validate", "gdn_workspace_bytes", "gdn_plan_compose", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc",
           "gdn_raw_workspace_bytes", "gdn_chunk_fwd_raw_inputs", "gdn_decode_step", "gdn_error_string",
           "gdn_status_string", "gdn_abi_version")
# the largest workspace gdn_chunk_fwd_noalloc serves (its per-device array)
NOALLOC_WORKSPACE_BYTES = 64 << 20
ABI_VERSION = 2  # the gdn_problem layout above (GDN_ABI_VERSION)


class Problem(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("seq_len", ctypes.c_int32), ("hk", ctypes.c_int32), ("hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("arm", ctypes.c_int32), ("compose", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("solve_block", ctypes.c_int32)]


class RawInputs(ctypes.Structure):
    """gdn_raw_inputs: q rows scaled by q_scale after normalisation; g = -gate_scale softplus(x)."""
    _fields_ = [("q_scale", ctypes.c_float), ("gate_scale", ctypes.c_float)]


class GdnError(RuntimeError):
    """A host-side refusal (gdn_status != GDN_OK); nothing was launched."""

    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__("%s%s (code %d)" % (where + ": " if where else "", error_string(code), code))


class GdnStatusError(RuntimeError):
    """Device status bits were set during a call."""

    def __init__(self, bits: int):
        self.bits = bits
        super().__init__("device status: %s (0x%x)" % (status_string(bits), bits))


_lock = threading.Lock()
_lib = None
_path = LIBRARY_PATH


def use_library(path: str) -> None:
    """Load `path` (e.g. STAMPS_LIBRARY_PATH) instead of the product library; only before
    the first call that loads one."""
    global _path
    with _lock:
        if _lib is not None and path != _path:
            raise RuntimeError("a library is already loaded: %s" % _path)
        _path = path


def load():
    """Load libgdn_mi355x.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_path):
                raise RuntimeError("%s is not built (run __graft_entry__.build())" % os.path.basename(_path))
            lib = ctypes.CDLL(_path)
            P = ctypes.POINTER(Problem)
            vp = ctypes.c_void_p
            lib.gdn_validate.argtypes = [P]
            lib.gdn_validate.restype = ctypes.c_int
            lib.gdn_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn_workspace_bytes.restype = ctypes.c_int
            lib.gdn_plan_compose.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
            lib.gdn_plan_compose.restype = ctypes.c_int
            lib.gdn_chunk_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.c_size_t, vp]
            lib.gdn_chunk_fwd.restype = ctypes.c_int
            lib.gdn_chunk_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
            lib.gdn_raw_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn_raw_workspace_bytes.restype = ctypes.c_int
            lib.gdn_chunk_fwd_raw_inputs.argtypes = [P, ctypes.POINTER(RawInputs), vp, vp, vp, vp, vp, vp, vp, vp,
                                                     vp, vp, vp, ctypes.c_size_t, vp]
            lib.gdn_chunk_fwd_raw_inputs.restype = ctypes.c_int
            lib.gdn_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.gdn_decode_step.restype = ctypes.c_int
            lib.gdn_error_string.argtypes = [ctypes.c_int32]
            lib.gdn_error_string.restype = ctypes.c_char_p
            lib.gdn_status_string.argtypes = [ctypes.c_uint32]
            lib.gdn_status_string.restype = ctypes.c_char_p
            lib.gdn_abi_version.restype = ctypes.c_int32
            if lib.gdn_abi_version() != ABI_VERSION:
                raise RuntimeError("%s has ABI version %d, this binding expects %d: rebuild it"
                                   % (_path, lib.gdn_abi_version(), ABI_VERSION))
            _lib = lib
    return _lib


def error_string(code: int) -> str:
    return load().gdn_error_string(int(code)).decode()


def status_string(bits: int) -> str:
    return load().gdn_status_string(int(bits) & 0xFFFFFFFF).decode()


def abi_version() -> int:
    return int(load().gdn_abi_version())


def make_problem(n_seq, total_tokens, seq_len, hk, hv, dk, dv, gate=GATE_HEAD, chunk=0,
                 qkv_dtype=BF16, o_dtype=BF16, arm=ARM_MFMA_BF16, compose=COMPOSE_AUTO,
                 stages=STAGE_ALL, solve_block=0) -> Problem:
    return Problem(int(n_seq), int(total_tokens), int(seq_len), int(hk), int(hv), int(dk), int(dv),
                   int(gate), int(chunk), int(qkv_dtype), int(o_dtype), int(arm), int(compose),
                   int(stages), int(solve_block))


def validate(prob: Problem) -> int:
    return int(load().gdn_validate(ctypes.byref(prob)))


def workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    rc = load().gdn_workspace_bytes(ctypes.byref(prob), ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_workspace_bytes")
    return int(n.value)


def raw_workspace_bytes(prob: Problem) -> int:
    """Workspace bytes of gdn_chunk_fwd_raw_inputs for `prob`."""
    n = ctypes.c_size_t(0)
    rc = load().gdn_raw_workspace_bytes(ctypes.byref(prob), ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_raw_workspace_bytes")
    return int(n.value)


def plan_compose(prob: Problem) -> int:
    """The composition gdn_chunk_fwd runs for `prob` on the current device (COMPOSE_*)."""
    c = ctypes.c_int32(-1)
    rc = load().gdn_plan_compose(ctypes.byref(prob), ctypes.byref(c))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_plan_compose")
    return int(c.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_DT = {torch.bfloat16: BF16, torch.float32: F32}
_ARM = {"bf16": ARM_MFMA_BF16, "f32": ARM_FOLD_F32}
_COMPOSE = {"auto": COMPOSE_AUTO, "split": COMPOSE_SPLIT, "fused": COMPOSE_FUSED,
            "pipelined": COMPOSE_PIPELINED, "seqsplit": COMPOSE_SEQSPLIT}


def chunk_fwd_raw(prob: Problem, q, k, v, g, beta, h0, cu_seqlens, o, hT, status, workspace,
                  stream=None) -> int:
    """Direct call of gdn_chunk_fwd with caller-owned tensors; returns the host code."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(load().gdn_chunk_fwd(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
        _ptr(cu_seqlens), _ptr(o), _ptr(hT), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_bytes),
        ctypes.c_void_p(int(stream))))


def chunk_fwd_raw_inputs_raw(prob: Problem, q_scale, gate_scale, q, k, v, gate_x, beta_logit, h0, cu_seqlens, o, hT,
                             status, workspace, stream=None) -> int:
    """Direct call of gdn_chunk_fwd_raw_inputs with caller-owned tensors; returns the host code."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    raw = RawInputs(float(q_scale), float(gate_scale))
    return int(load().gdn_chunk_fwd_raw_inputs(
        ctypes.byref(prob), ctypes.byref(raw), _ptr(q), _ptr(k), _ptr(v), _ptr(gate_x), _ptr(beta_logit), _ptr(h0),
        _ptr(cu_seqlens), _ptr(o), _ptr(hT), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_bytes),
        ctypes.c_void_p(int(stream))))


def chunk_fwd_noalloc_raw(prob: Problem, q, k, v, g, beta, h0, cu_seqlens, o, hT, status,
                          stream=None) -> int:
    """Direct call of gdn_chunk_fwd_noalloc (the library's own per-device workspace, no
    allocation); returns the host code."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load().gdn_chunk_fwd_noalloc(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
        _ptr(cu_seqlens), _ptr(o), _ptr(hT), _ptr(status), ctypes.c_void_p(int(stream))))


def chunk_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, *, chunk: int = 0, arm: str = "bf16",
              o_dtype: Optional[torch.dtype] = None, compose: str = "auto", want_hT: bool = True,
              check: bool = True, workspace: Optional[torch.Tensor] = None, raw: Optional[tuple] = None,
              solve_block: int = 0):
    """Chunkwise gated delta-rule prefill on the current device and stream.

    With ``raw = (q_scale, gate_scale)`` the inputs are the raw per-token values
    (gdn_chunk_fwd_raw_inputs): q, k raw rows (normalised inside, q then scaled), beta the
    logits (beta = sigmoid), g the raw gate values (g = -gate_scale softplus), per-head gate.

    Fixed-length batch: q, k [B, T, HK, DK]; v [B, T, HV, DV]; g [B, T, HV] (per-head
    gate) or [B, T, HV, DK] (per-key-channel gate); beta [B, T, HV]; h0 [B, HV, DK, DV].
    Packed batch (cu_seqlens int32 [N+1]): the same with B = 1 (or no batch axis) and
    h0 [N, HV, DK, DV].  Returns (o [..., HV, DV], hT [N, HV, DK, DV] or None, status
    int32[1] on the device).  With ``check`` the stream is synchronised and any device
    status bit raises GdnStatusError.  ``solve_block`` (8, 16, 32; 0 = library choice) sets the
    rows of the triangular solve's diagonal blocks.
    """
    if q.dim() == 3:
        q, k, v, g, beta = (x.unsqueeze(0) for x in (q, k, v, g, beta))
        squeeze = True
    else:
        squeeze = False
    B, T, HK, DK = q.shape
    HV, DV = v.shape[2], v.shape[3]
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share dtype bfloat16 or float32")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("h0", h0)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous device tensor" % name)
    if k.shape != q.shape or v.shape[:2] != (B, T) or beta.shape != (B, T, HV):
        raise ValueError("inconsistent q/k/v/beta shapes")
    if g.shape == (B, T, HV):
        gate = GATE_HEAD
    elif g.shape == (B, T, HV, DK):
        gate = GATE_KEY_CHANNEL
    else:
        raise ValueError("g must be [B, T, HV] or [B, T, HV, DK]")
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("cu_seqlens describes one packed batch (B = 1)")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
            raise TypeError("cu_seqlens must be an int32 device tensor")
        n_seq, seq_len = cu_seqlens.numel() - 1, 0
    else:
        n_seq, seq_len = B, T
    if h0 is not None and (h0.dtype != torch.float32 or h0.shape != (n_seq, HV, DK, DV)):
        raise ValueError("h0 must be float32 [N, HV, DK, DV]")
    odt = o_dtype or q.dtype
    prob = make_problem(n_seq, B * T, seq_len, HK, HV, DK, DV, gate, chunk, _DT[q.dtype], _DT[odt],
                        _ARM[arm], _COMPOSE[compose], solve_block=solve_block)
    rc = validate(prob)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_validate")
    if raw is not None and gate != GATE_HEAD:
        raise GdnError(GDN_E_UNSUPPORTED, "raw inputs: per-head gate only")
    dev = q.device
    o = torch.empty((B, T, HV, DV), dtype=odt, device=dev)
    hT = torch.empty((n_seq, HV, DK, DV), dtype=torch.float32, device=dev) if want_hT else None
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    need = raw_workspace_bytes(prob) if raw is not None else workspace_bytes(prob)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if raw is not None:
        rc = chunk_fwd_raw_inputs_raw(prob, raw[0], raw[1], q, k, v, g, beta, h0, cu_seqlens, o, hT, status,
                                      workspace)
    else:
        rc = chunk_fwd_raw(prob, q, k, v, g, beta, h0, cu_seqlens, o, hT, status, workspace)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_raw_inputs" if raw is not None else "gdn_chunk_fwd")
    if check:
        torch.cuda.current_stream().synchronize()
        bits = int(status.item()) & 0xFFFFFFFF
        if bits:
            raise GdnStatusError(bits)
    if squeeze:
        o = o.squeeze(0)
    return o, hT, status


def decode_step_raw(prob: Problem, q, k, v, g, beta, h_in, o, h_out, status, stream=None) -> int:
    """Direct call of gdn_decode_step with caller-owned tensors; returns the host code."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load().gdn_decode_step(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h_in), _ptr(o),
        _ptr(h_out), _ptr(status), ctypes.c_void_p(int(stream))))


def decode_step(q, k, v, g, beta, h_in=None, *, o_dtype: Optional[torch.dtype] = None,
                h_out: Optional[torch.Tensor] = None, check: bool = True):
    """One recurrent step (one new token per sequence) on the current device and stream.

    q, k [B, HK, DK]; v [B, HV, DV]; g [B, HV] (per-head gate) or [B, HV, DK]
    (per-key-channel gate); beta [B, HV]; h_in [B, HV, DK, DV] float32 or None (zeros).
    Returns (o [B, HV, DV], h_out [B, HV, DK, DV] float32, status int32[1] on the
    device); h_in is never written.  With ``check`` the stream is synchronised and any
    device status bit raises GdnStatusError.
    """
    B, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share dtype bfloat16 or float32")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("h_in", h_in),
                    ("h_out", h_out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous device tensor" % name)
    if k.shape != q.shape or v.shape[0] != B or beta.shape != (B, HV):
        raise ValueError("inconsistent q/k/v/beta shapes")
    if g.shape == (B, HV):
        gate = GATE_HEAD
    elif g.shape == (B, HV, DK):
        gate = GATE_KEY_CHANNEL
    else:
        raise ValueError("g must be [B, HV] or [B, HV, DK]")
    for name, t in (("h_in", h_in), ("h_out", h_out)):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, HV, DK, DV)):
            raise ValueError("%s must be float32 [B, HV, DK, DV]" % name)
    odt = o_dtype or q.dtype
    prob = make_problem(B, B, 1, HK, HV, DK, DV, gate, 0, _DT[q.dtype], _DT[odt])
    dev = q.device
    o = torch.empty((B, HV, DV), dtype=odt, device=dev)
    if h_out is None:
        h_out = torch.empty((B, HV, DK, DV), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    rc = decode_step_raw(prob, q, k, v, g, beta, h_in, o, h_out, status)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_step")
    if check:
        torch.cuda.current_stream().synchronize()
        bits = int(status.item()) & 0xFFFFFFFF
        if bits:
            raise GdnStatusError(bits)
    return o, h_out, status
