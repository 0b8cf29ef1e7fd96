"""CPU oracle of the input side adjacent to the recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the HIP library never uses it.

The logismos issue #46 page (section "Remaining work") keeps model-specific gating
separate from the generic operation, which takes q, k already normalised, beta and the
natural-log decay g already formed.  The workloads of the problem statement fix how those
are formed from raw per-token values, and this module states exactly that, in fp64:

* q, k: each (token, head) row is divided by its L2 norm (a zero row stays zero), and q is
  then multiplied by a per-call scale (the single-sequence workload's dk^-1/2);
* beta = sigmoid(logit) = 1 / (1 + e^-logit);
* g = -a softplus(x) = -a log(1 + e^x), a > 0 per call (the hybrid layer's a = 1/2, the
  packed batch's a = 1).

``raw_fwd`` then hands the prepared values to the token-serial oracle unchanged.

Parity status: pinned (tests/test_oracle_prepare.py): unit norms, scale invariance, the
closed forms sigmoid(0) = 1/2 and softplus(0) = ln 2, the reflections sigmoid(x) +
sigmoid(-x) = 1 and softplus(x) - softplus(-x) = x, and planted mistakes that fail them.
"""
from __future__ import annotations

import numpy as np

from . import serial_fwd

CORRECT = 0
MUT_NORM_SQUARED = 1      # divides by the squared norm
MUT_GATE_SIGN = 2         # g = +a softplus(x)
MUT_SIGMOID_FLIP = 3      # beta = sigmoid(-logit)
MUT_SCALE_BOTH = 4        # scales k as well as q


def l2_normalize_rows(x, scale=1.0, mutant=CORRECT):
    """Each row (last axis) of x divided by its L2 norm, times `scale`; zero rows stay zero."""
    x = np.asarray(x, dtype=np.float64)
    n2 = np.sum(x * x, axis=-1, keepdims=True)
    n = np.sqrt(n2)
    den = n2 if mutant == MUT_NORM_SQUARED else n
    inv = np.zeros_like(den)
    np.divide(1.0, den, out=inv, where=den > 0)
    return x * inv * scale


def sigmoid(x, mutant=CORRECT):
    x = np.asarray(x, dtype=np.float64)
    if mutant == MUT_SIGMOID_FLIP:
        x = -x
    # 1 / (1 + e^-x), evaluated without overflow on either side
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + e^x) = max(x, 0) + log(1 + e^-|x|), without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gate_from_raw(x, a, mutant=CORRECT):
    return (1.0 if mutant == MUT_GATE_SIGN else -1.0) * a * softplus(x)


def prepare(q_raw, k_raw, gate_x, beta_logit, q_scale, gate_scale, mutant=CORRECT):
    """The prepared (q, k, g, beta) of the raw per-token values, all fp64."""
    q = l2_normalize_rows(q_raw, q_scale, mutant)
    k = l2_normalize_rows(k_raw, q_scale if mutant == MUT_SCALE_BOTH else 1.0, mutant)
    return q, k, gate_from_raw(gate_x, gate_scale, mutant), sigmoid(beta_logit, mutant)


def raw_fwd(q_raw, k_raw, v, gate_x, beta_logit, q_scale, gate_scale, h0=None, seq_start=None,
            mutant=CORRECT, **kw):
    """Token-serial fp64 rule on the prepared inputs (see serial_fwd for shapes)."""
    q, k, g, b = prepare(q_raw, k_raw, gate_x, beta_logit, q_scale, gate_scale, mutant)
    return serial_fwd(q, k, v, g, b, h0, seq_start=seq_start, **kw)
