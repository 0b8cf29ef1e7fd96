"""CPU oracles for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it, and it imports nothing from them.

Two independent evaluations live here:

* :func:`serial_fwd` -- the fp64 token-serial rule (C, OpenMP), one token at a
  time and never chunked, following the ROCm/rocm-libraries KDA chunkwise page
  (section "Correctness", the token-serial oracle) in the K-first orientation of
  the logismos issue #46 page (activity of Sep 6 and Sep 8).
* :mod:`oracle.chunked` -- a dense numpy fp64 evaluation of the chunk (WY) form
  that builds every gate factor from pairwise exponent differences, following
  the same page's tile oracle (no midpoint factoring), with a LAPACK solve.

* :mod:`oracle.prepare` -- the input side next to the recurrence (raw q/k normalised per
  row and scaled, beta = sigmoid(logit), g = -a softplus(x)), plainly in fp64, feeding
  :func:`serial_fwd`.

Parity status: all pinned (tests/test_oracle_pins.py, tests/test_oracle_prepare.py); the
first two also pin each other.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None

CORRECT = 0
MUT_DECAY_AFTER_WRITE = 1
MUT_NO_BETA_ERASE = 2
MUT_TRANSPOSED_READ = 3
MUT_GATE_NEXT_TOKEN = 4
MUT_OUTPUT_BEFORE_WRITE = 5


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.gdn_oracle_fwd.argtypes = [
                ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int,
                ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                dp, dp, dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                ctypes.c_int, ctypes.c_int]
            lib.gdn_oracle_fwd.restype = ctypes.c_int
            lib.gdn_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def serial_fwd(q, k, v, g, beta, h0=None, seq_start=None, head_map=None, units=None,
               want_o=True, n_threads=0, mutant=CORRECT):
    """Token-serial fp64 gated delta rule.

    q, k: [tok, hk, dk]; v: [tok, hv, dv]; g: [tok, hv] or [tok, hv, dk];
    beta: [tok, hv]; h0: [n_seq, hv, dk, dv] or None; seq_start: [n_seq+1]
    token offsets (default: one sequence of all tokens).  Every input is read
    exactly as float64.  Returns (o [tok, hv, dv] float64 or None,
    hT [n_seq, hv, dk, dv] float64).
    """
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    tok, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    if q.shape != k.shape or v.shape[0] != tok or beta.shape != (tok, hv):
        raise ValueError("inconsistent shapes")
    per_channel = 1 if g.ndim == 3 else 0
    if g.shape != ((tok, hv, dk) if per_channel else (tok, hv)):
        raise ValueError("bad gate shape")
    if seq_start is None:
        seq_start = np.array([0, tok], dtype=np.int64)
    seq_start = np.ascontiguousarray(seq_start, dtype=np.int64)
    n_seq = seq_start.shape[0] - 1
    if h0 is not None and h0.shape != (n_seq, hv, dk, dv):
        raise ValueError("bad h0 shape")
    hm = None if head_map is None else np.ascontiguousarray(head_map, dtype=np.int32)
    un = None
    n_units = 0
    if units is not None:
        un = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = un.shape[0]
    o = np.zeros((tok, hv, dv), dtype=np.float64) if want_o else None
    hT = np.zeros((n_seq, hv, dk, dv), dtype=np.float64)
    rc = _load().gdn_oracle_fwd(
        n_seq, _ptr(seq_start, ctypes.c_int64), hk, hv, _ptr(hm, ctypes.c_int32), dk, dv,
        per_channel, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
        _ptr(un, ctypes.c_int32), n_units, int(n_threads), int(mutant))
    if rc != 0:
        raise ValueError("gdn_oracle_fwd rejected its arguments (code %d)" % rc)
    return o, hT
