"""Pins of the input-side oracle (oracle/prepare.py) against what the mathematics fixes:
unit row norms, invariance to the scale of a raw row, zero rows staying zero, the closed
forms sigmoid(0) = 1/2 and softplus(0) = ln 2, the reflections sigmoid(x) + sigmoid(-x) = 1
and softplus(x) - softplus(-x) = x, and the input generator's own fp32 normalisation (code
written separately) agreeing to fp32 rounding.  Each planted mistake fails one of them."""
import math

import numpy as np
import pytest

import oracle
from oracle import prepare as P
from linear_attention_rnn_chunk_amd import inputs


def _rows(seed, shape=(50, 3, 16)):
    return np.random.default_rng(seed).standard_normal(shape) * 3.0


def check_normalize(mutant=P.CORRECT):
    x = _rows(1)
    x[7, 1] = 0.0                                   # a zero row
    y = P.l2_normalize_rows(x, 1.0, mutant)
    n = np.linalg.norm(y, axis=-1)
    live = np.linalg.norm(x, axis=-1) > 0
    assert np.allclose(n[live], 1.0, atol=1e-14), "unit norms"
    assert np.all(y[7, 1] == 0.0), "zero row"
    # same direction: y . x = |y| |x|
    assert np.allclose(np.sum(y * x, axis=-1)[live], np.linalg.norm(x, axis=-1)[live], rtol=1e-13)
    for c in (3.7, 1e-20, 1e20):                    # invariant to the raw row's scale
        assert np.allclose(P.l2_normalize_rows(c * x, 1.0, mutant), y, atol=1e-14)
    ys = P.l2_normalize_rows(x, 0.125, mutant)
    assert np.allclose(np.linalg.norm(ys, axis=-1)[live], 0.125, atol=1e-15), "scaled norms"


def check_sigmoid(mutant=P.CORRECT):
    assert P.sigmoid(0.0, mutant) == 0.5
    x = np.linspace(-40, 40, 161)
    s = P.sigmoid(x, mutant)
    assert np.allclose(s + P.sigmoid(-x, mutant), 1.0, atol=1e-15)
    assert np.all(np.diff(s) >= 0) and np.all(np.diff(s[np.abs(x) <= 30]) > 0), "increasing"
    assert np.all((s >= 0) & (s <= 1))
    m = np.abs(x) <= 20                             # e^x / (1 + e^x), another form of the same function
    assert np.allclose(s[m], np.exp(x[m]) / (1.0 + np.exp(x[m])), rtol=1e-14)


def check_gate(mutant=P.CORRECT):
    assert abs(P.softplus(0.0) - math.log(2.0)) < 1e-16
    x = np.linspace(-40, 40, 161)
    sp = P.softplus(x)
    assert np.allclose(sp - P.softplus(-x), x, atol=1e-13)
    assert np.all(sp >= np.maximum(x, 0.0)) and np.all((sp > np.maximum(x, 0.0))[np.abs(x) <= 30])
    assert abs(P.softplus(40.0) - (40.0 + math.exp(-40.0))) < 1e-14
    for a in (0.5, 1.0):
        g = P.gate_from_raw(x, a, mutant)
        assert np.all(g <= 0.0), "natural-log decay is never positive"
        assert abs(P.gate_from_raw(0.0, a, mutant) + a * math.log(2.0)) < 1e-15


def check_prepare_matches_generator(mutant=P.CORRECT):
    # the input generator's own fp32 normalisation and scale (written separately)
    rng = np.random.default_rng(5)
    qr = rng.standard_normal((40, 2, 32)).astype(np.float32)
    kr = rng.standard_normal((40, 2, 32)).astype(np.float32)
    q, k, _, _ = P.prepare(qr, kr, np.zeros((40, 4)), np.zeros((40, 4)), 32 ** -0.5, 1.0, mutant)
    gq = inputs._l2norm_rows(qr) * np.float32(32 ** -0.5)
    gk = inputs._l2norm_rows(kr)
    assert np.max(np.abs(q - gq)) < 1e-6 and np.max(np.abs(k - gk)) < 1e-6


PINS = [check_normalize, check_sigmoid, check_gate, check_prepare_matches_generator]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_raw_fwd_is_the_rule_on_prepared_inputs():
    rng = np.random.default_rng(9)
    T, hk, hv, dk, dv = 37, 1, 2, 8, 6
    qr, kr = rng.standard_normal((T, hk, dk)) * 2, rng.standard_normal((T, hk, dk)) * 0.3
    v = rng.standard_normal((T, hv, dv))
    x, bl = rng.standard_normal((T, hv)), rng.standard_normal((T, hv))
    o, hT = P.raw_fwd(qr, kr, v, x, bl, 0.5, 0.7)
    q, k, g, b = P.prepare(qr, kr, x, bl, 0.5, 0.7)
    o2, h2 = oracle.serial_fwd(q, k, v, g, b)
    assert np.array_equal(o, o2) and np.array_equal(hT, h2)
    # delta-rule exact storage holds for prepared inputs: q = k (same raw rows, scale 1),
    # beta logits -> 1 (large), so o_t = v_t
    o3, _ = P.raw_fwd(kr, kr, v, x, np.full((T, hv), 40.0), 1.0, 0.7)
    assert np.max(np.abs(o3 - v)) < 1e-12


@pytest.mark.parametrize("mutant", [P.MUT_NORM_SQUARED, P.MUT_GATE_SIGN, P.MUT_SIGMOID_FLIP, P.MUT_SCALE_BOTH])
def test_planted_prepare_mistakes_fail_a_pin(mutant):
    failed = 0
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1
