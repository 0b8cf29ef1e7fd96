"""Pins of the CPU oracles against what the pages and the mathematics fix.

No page prints a worked numeric example, so every pin is a closed form, an
invariant, a library special case, or the two independent oracles checking
each other.  Each planted mistake in the oracles (``mutant``) must fail at
least one of these pins (see the end of this file).

Citations: the recurrence and its closed-form checks (single token, beta = 0,
orthonormal keys, exact storage of v) are the problem statement of the
chunk-parallel GDN pages; the state orientation (K-first), natural-log decay,
grouped heads, chunk composition and causality are the logismos issue #46 page
(activity of Sep 6/8/10: K-first state, all nonempty chunk cuts, partition
continuation, mixed-length packing, grouped shapes, causality); the two
independent fp64 oracles are the ROCm/rocm-libraries KDA chunkwise page
(section "Correctness").
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import chunked
from tests._util import rel_l2, unit_rows


def _draw(rng, T, hk, hv, dk, dv, gate="head", glo=-1.0, beta=None, h0=True, unit_keys=True):
    q = unit_rows(rng, (T, hk, dk)) if unit_keys else rng.standard_normal((T, hk, dk))
    k = unit_rows(rng, (T, hk, dk)) if unit_keys else rng.standard_normal((T, hk, dk))
    v = rng.standard_normal((T, hv, dv))
    gs = (T, hv) if gate == "head" else (T, hv, dk)
    g = rng.uniform(glo, 0.0, gs)
    b = rng.uniform(0.05, 1.0, (T, hv)) if beta is None else np.full((T, hv), float(beta))
    H0 = 0.3 * rng.standard_normal((1, hv, dk, dv)) if h0 else None
    return q, k, v, g, b, H0


def _dense_S_form(q, k, v, g, b, H0, per_channel):
    """The defining recurrence in the value-by-key orientation S = H^T:
    S_t = S_{t-1} D_t (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t,
    with D_t = exp(g_t) I for the per-head gate (the problem statement's
    S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + ...) and diag(exp(g_t)) per key channel.
    Dense matrices, one value head, written independently of the oracle."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if H0 is None else H0.T.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        D = np.diag(np.exp(g[t])) if per_channel else np.exp(g[t]) * np.eye(dk)
        E = np.eye(dk) - b[t] * np.outer(k[t], k[t])
        S = S @ D @ E + b[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S.T


# ---------------------------------------------------------------- P1 ------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_P1_single_token_closed_form(gate):
    rng = np.random.default_rng(11)
    dk, dv = 8, 6
    q, k, v, g, b, H0 = _draw(rng, 1, 1, 1, dk, dv, gate=gate, glo=-2.0)
    o, hT = oracle.serial_fwd(q, k, v, g, b, H0)
    # o = H0^T D (I - b k k^T) q + b v (k . q)
    D = np.diag(np.exp(g[0, 0])) if gate == "channel" else np.exp(g[0, 0]) * np.eye(dk)
    kk, qq, vv, bb = k[0, 0], q[0, 0], v[0, 0], b[0, 0]
    o_ref = H0[0, 0].T @ D @ (np.eye(dk) - bb * np.outer(kk, kk)) @ qq + bb * vv * (kk @ qq)
    h_ref = (np.eye(dk) - bb * np.outer(kk, kk)) @ D @ H0[0, 0] + bb * np.outer(kk, vv)
    assert rel_l2(o[0, 0], o_ref) < 1e-14
    assert rel_l2(hT[0, 0], h_ref) < 1e-14


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_P1b_defining_recurrence_dense(gate):
    """Whole sequences against the defining recurrence in the S orientation."""
    rng = np.random.default_rng(12)
    T, dk, dv = 23, 6, 5
    q, k, v, g, b, H0 = _draw(rng, T, 1, 1, dk, dv, gate=gate, glo=-1.5, unit_keys=False)
    o, hT = oracle.serial_fwd(q, k, v, g, b, H0)
    o_ref, h_ref = _dense_S_form(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], H0[0, 0],
                                 gate == "channel")
    assert rel_l2(o[:, 0], o_ref) < 1e-13
    assert rel_l2(hT[0, 0], h_ref) < 1e-13


# ---------------------------------------------------------------- P2 ------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_P2_beta_zero_is_pure_decay(gate):
    rng = np.random.default_rng(21)
    T, dk, dv = 37, 8, 4
    q, k, v, g, b, H0 = _draw(rng, T, 2, 2, dk, dv, gate=gate, glo=-0.7, beta=0.0)
    o, hT = oracle.serial_fwd(q, k, v, g, b, H0)
    G = np.cumsum(g, axis=0)
    for h in range(2):
        for t in range(T):
            scale = np.exp(G[t, h]) if gate == "channel" else np.exp(G[t, h]) * np.ones(dk)
            ref = (scale[:, None] * H0[0, h]).T @ q[t, h]
            assert rel_l2(o[t, h], ref) < 1e-13
        scale = np.exp(G[-1, h]) if gate == "channel" else np.exp(G[-1, h]) * np.ones(dk)
        assert rel_l2(hT[0, h], scale[:, None] * H0[0, h]) < 1e-13


# ---------------------------------------------------------------- P3 ------
def test_P3_small_beta_is_decayed_linear_attention():
    rng = np.random.default_rng(31)
    T, dk, dv, eps = 40, 16, 8, 1e-8
    q, k, v, g, b, _ = _draw(rng, T, 1, 1, dk, dv, glo=-0.3, h0=False)
    bhat = b.copy()
    o, _ = oracle.serial_fwd(q, k, v, g, eps * bhat, None)
    G = np.cumsum(g[:, 0])
    ref = np.zeros((T, dv))
    for t in range(T):
        for s in range(t + 1):
            ref[t] += np.exp(G[t] - G[s]) * bhat[s, 0] * (k[s, 0] @ q[t, 0]) * v[s, 0]
    assert rel_l2(o[:, 0] / eps, ref) < 1e-5


# ---------------------------------------------------------------- P4 ------
def test_P4_orthonormal_keys_give_exact_linear_attention():
    rng = np.random.default_rng(41)
    dk, dv, T = 24, 7, 24
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][:, None, :]                           # mutually orthonormal keys
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = rng.uniform(-1.0, 0.0, (T, 1))
    b = rng.uniform(0.1, 1.0, (T, 1))
    o, hT = oracle.serial_fwd(q, k, v, g, b, None)
    G = np.cumsum(g[:, 0])
    H = np.zeros((dk, dv))
    for t in range(T):
        H = np.exp(g[t, 0]) * H + b[t, 0] * np.outer(k[t, 0], v[t, 0])
        assert rel_l2(o[t, 0], H.T @ q[t, 0]) < 1e-13
    assert rel_l2(hT[0, 0], H) < 1e-13
    # closed form of the state: sum_s exp(G_T - G_s) b_s k_s v_s^T
    Hc = sum(np.exp(G[-1] - G[s]) * b[s, 0] * np.outer(k[s, 0], v[s, 0]) for s in range(T))
    assert rel_l2(hT[0, 0], Hc) < 1e-13


# ---------------------------------------------------------------- P5 ------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_P5_unit_query_equal_key_returns_value(gate):
    rng = np.random.default_rng(51)
    T, dk, dv = 50, 12, 9
    _, k, v, g, _, H0 = _draw(rng, T, 1, 1, dk, dv, gate=gate, glo=-2.0)
    b = np.ones((T, 1))
    o, _ = oracle.serial_fwd(k, k, v, g, b, H0)
    assert rel_l2(o[:, 0], v[:, 0]) < 1e-14 * T


def test_P5b_orthonormal_store_then_retrieve():
    rng = np.random.default_rng(52)
    dk, dv, T = 16, 5, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][:, None, :]
    v = rng.standard_normal((T, 1, dv))
    o, hT = oracle.serial_fwd(k, k, v, np.zeros((T, 1)), np.ones((T, 1)), None)
    retrieved = hT[0, 0].T @ k[:, 0].T               # column s = H_T^T k_s
    assert rel_l2(retrieved.T, v[:, 0]) < 1e-14


# ---------------------------------------------------------------- P6 ------
def test_P6_householder_product_is_orthogonal():
    rng = np.random.default_rng(61)
    d, T = 10, 31
    k = unit_rows(rng, (T, 1, d))
    o, hT = oracle.serial_fwd(k, k, np.zeros((T, 1, d)), np.zeros((T, 1)), 2.0 * np.ones((T, 1)),
                              np.eye(d)[None, None])
    M = hT[0, 0]
    assert np.linalg.norm(M.T @ M - np.eye(d)) < 1e-13
    # in general (any beta, g = 0, v = 0): H_T = prod_t (I - b_t k_t k_t^T) H_0
    b = rng.uniform(0.0, 2.0, (T, 1))
    H0 = rng.standard_normal((1, 1, d, 3))
    _, hT = oracle.serial_fwd(k, k, np.zeros((T, 1, 3)), np.zeros((T, 1)), b, H0)
    P = np.eye(d)
    for t in range(T):
        P = (np.eye(d) - b[t, 0] * np.outer(k[t, 0], k[t, 0])) @ P
    assert rel_l2(hT[0, 0], P @ H0[0, 0]) < 1e-13


# ---------------------------------------------------------------- P7 ------
SWEEP_T = [1, 37, 64, 65, 200]
GATES = [("zero", "head", 0.0), ("scalar", "head", -1.0), ("kda5", "channel", -5.0),
         ("kda05", "channel", -0.5)]


@pytest.mark.parametrize("C", [1, 2, 7, 32, 64])
@pytest.mark.parametrize("T", SWEEP_T)
@pytest.mark.parametrize("gname,gate,glo", GATES)
def test_P7_chunk_form_matches_token_serial(C, T, gname, gate, glo):
    rng = np.random.default_rng(700 + C * 7 + T)
    dk, dv = 16, 8
    q, k, v, g, b, H0 = _draw(rng, T, 2, 4, dk, dv, gate=gate, glo=glo)
    if gname == "zero":
        g = np.zeros_like(g)
    o_s, h_s = oracle.serial_fwd(q, k, v, g, b, H0)
    o_c, h_c = chunked.chunked_fwd(q, k, v, g, b, H0, chunk=C)
    assert rel_l2(o_c, o_s) < 1e-10
    assert rel_l2(h_c, h_s) < 1e-10


@pytest.mark.parametrize("gname,gate,glo", GATES)
def test_P7_long_sequence(gname, gate, glo):
    rng = np.random.default_rng(4099)
    T, dk, dv = 4099, 16, 8
    q, k, v, g, b, H0 = _draw(rng, T, 1, 1, dk, dv, gate=gate, glo=glo)
    if gname == "zero":
        g = np.zeros_like(g)
    o_s, h_s = oracle.serial_fwd(q, k, v, g, b, H0)
    C = 32 if gate == "channel" else 64
    o_c, h_c = chunked.chunked_fwd(q, k, v, g, b, H0, chunk=C)
    assert rel_l2(o_c, o_s) < 1e-10
    assert rel_l2(h_c, h_s) < 1e-10


@pytest.mark.parametrize("gate,C", [("head", 64), ("channel", 32)])
def test_zero_filled_partial_chunk_is_exact(gate, C):
    rng = np.random.default_rng(77)
    q, k, v, g, b, H0 = _draw(rng, 70, 1, 2, 8, 8, gate=gate, glo=-2.0)
    a = chunked.chunked_fwd(q, k, v, g, b, H0, chunk=C)
    p = chunked.chunked_fwd(q, k, v, g, b, H0, chunk=C, pad_to=True)
    assert rel_l2(p[0], a[0]) < 1e-14 and rel_l2(p[1], a[1]) < 1e-14


# ---------------------------------------------------------------- P8 ------
def test_P8_every_chunk_cut_continues_exactly():
    rng = np.random.default_rng(81)
    T, dk, dv = 19, 6, 5
    q, k, v, g, b, H0 = _draw(rng, T, 1, 2, dk, dv, glo=-1.0)
    o, hT = oracle.serial_fwd(q, k, v, g, b, H0)
    for cut in range(1, T):
        o1, h1 = oracle.serial_fwd(q[:cut], k[:cut], v[:cut], g[:cut], b[:cut], H0)
        o2, h2 = oracle.serial_fwd(q[cut:], k[cut:], v[cut:], g[cut:], b[cut:], h1)
        assert rel_l2(np.concatenate([o1, o2]), o) < 1e-13
        assert rel_l2(h2, hT) < 1e-13


# ---------------------------------------------------------------- P9 ------
def test_P9_packed_sequences_equal_independent_runs():
    rng = np.random.default_rng(91)
    lens = [13, 0, 40, 1, 29]
    tot = sum(lens)
    q, k, v, g, b, _ = _draw(rng, tot, 2, 4, 8, 6, glo=-1.0)
    H0 = rng.standard_normal((len(lens), 4, 8, 6))
    starts = np.concatenate([[0], np.cumsum(lens)])
    o, hT = oracle.serial_fwd(q, k, v, g, b, H0, seq_start=starts)
    o_c, h_c = chunked.chunked_fwd(q, k, v, g, b, H0, seq_start=starts, chunk=8)
    for n in range(len(lens)):
        sl = slice(starts[n], starts[n + 1])
        o1, h1 = oracle.serial_fwd(q[sl], k[sl], v[sl], g[sl], b[sl], H0[n:n + 1])
        assert np.array_equal(o[sl], o1)
        assert np.array_equal(hT[n], h1[0])
    assert np.array_equal(hT[1], H0[1])                 # empty sequence: hT = h0
    assert rel_l2(o_c, o) < 1e-12 and rel_l2(h_c, hT) < 1e-12


def test_oracle_unit_selection_computes_exactly_the_listed_units():
    """The oracle's `units` argument (evaluate only listed (sequence, value head) pairs):
    every listed unit equals the same unit of a full run bit for bit, and the rows of
    every unit not listed are left as the caller passed them (zeros here)."""
    rng = np.random.default_rng(92)
    lens = [21, 0, 37]
    tot = sum(lens)
    q, k, v, g, b, _ = _draw(rng, tot, 2, 6, 8, 5, glo=-1.0)
    H0 = rng.standard_normal((len(lens), 6, 8, 5))
    starts = np.concatenate([[0], np.cumsum(lens)])
    o, hT = oracle.serial_fwd(q, k, v, g, b, H0, seq_start=starts)
    units = [(0, 5), (2, 0), (2, 3), (1, 4)]
    o_u, h_u = oracle.serial_fwd(q, k, v, g, b, H0, seq_start=starts, units=units)
    listed = set(units)
    for n in range(len(lens)):
        sl = slice(starts[n], starts[n + 1])
        for h in range(6):
            if (n, h) in listed:
                assert np.array_equal(o_u[sl, h], o[sl, h])
                assert np.array_equal(h_u[n, h], hT[n, h])
            else:
                assert not np.any(o_u[sl, h]) and not np.any(h_u[n, h])
    with pytest.raises(ValueError):
        oracle.serial_fwd(q, k, v, g, b, H0, seq_start=starts, units=[(3, 0)])
    with pytest.raises(ValueError):
        oracle.serial_fwd(q, k, v, g, b, H0, seq_start=starts, units=[(0, 6)])


# ---------------------------------------------------------------- P10 -----
def test_P10_channel_gate_constant_over_channels_equals_head_gate():
    rng = np.random.default_rng(101)
    T, dk, dv = 45, 8, 8
    q, k, v, g, b, H0 = _draw(rng, T, 1, 2, dk, dv, glo=-1.3)
    gc = np.repeat(g[:, :, None], dk, axis=2)
    o1, h1 = oracle.serial_fwd(q, k, v, g, b, H0)
    o2, h2 = oracle.serial_fwd(q, k, v, gc, b, H0)
    assert rel_l2(o2, o1) < 1e-13 and rel_l2(h2, h1) < 1e-13


# ---------------------------------------------------------------- P11 -----
def test_P11_grouped_heads_equal_repeated_key_heads():
    rng = np.random.default_rng(111)
    T, hk, hv = 30, 2, 6
    q, k, v, g, b, H0 = _draw(rng, T, hk, hv, 8, 4, glo=-1.0)
    o1, h1 = oracle.serial_fwd(q, k, v, g, b, H0)
    rep = hv // hk
    qr, kr = np.repeat(q, rep, axis=1), np.repeat(k, rep, axis=1)
    o2, h2 = oracle.serial_fwd(qr, kr, v, g, b, H0)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    # an explicit map equal to the contiguous grouping gives the same bits
    o3, h3 = oracle.serial_fwd(q, k, v, g, b, H0, head_map=np.arange(hv) // rep)
    assert np.array_equal(o1, o3) and np.array_equal(h1, h3)


# ---------------------------------------------------------------- P12 -----
def test_P12_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(121)
    T = 33
    q, k, v, g, b, H0 = _draw(rng, T, 1, 1, 8, 5, glo=-1.0)
    v2 = rng.standard_normal(v.shape)
    H02 = rng.standard_normal(H0.shape)
    a1, a2 = 0.7, -1.9
    o1, h1 = oracle.serial_fwd(q, k, v, g, b, H0)
    o2, h2 = oracle.serial_fwd(q, k, v2, g, b, H02)
    o3, h3 = oracle.serial_fwd(q, k, a1 * v + a2 * v2, g, b, a1 * H0 + a2 * H02)
    assert rel_l2(o3, a1 * o1 + a2 * o2) < 1e-13
    assert rel_l2(h3, a1 * h1 + a2 * h2) < 1e-13


def test_P12_causality():
    rng = np.random.default_rng(122)
    T = 40
    q, k, v, g, b, H0 = _draw(rng, T, 1, 2, 8, 5, glo=-1.0)
    o1, _ = oracle.serial_fwd(q, k, v, g, b, H0)
    for t in (0, 17, 39):
        q2, k2, v2, g2, b2 = (x.copy() for x in (q, k, v, g, b))
        q2[t] += 1.0
        k2[t] *= -0.5
        v2[t] += 3.0
        g2[t] -= 0.4
        b2[t] = 0.9
        o2, _ = oracle.serial_fwd(q2, k2, v2, g2, b2, H0)
        assert np.array_equal(o1[:t], o2[:t])
        assert not np.array_equal(o1[t], o2[t])


# ---------------------------------------------------------------- P13 -----
@pytest.mark.parametrize("gate,C", [("head", 64), ("channel", 32)])
def test_P13_chunk_solve_against_triangular_solver(gate, C):
    rng = np.random.default_rng(131)
    q, k, v, g, b, H0 = _draw(rng, C, 1, 1, 16, 8, gate=gate, glo=-2.0)
    _, _, tiles = chunked.chunked_fwd(q, k, v, g, b, H0, chunk=C, want_tiles=True)
    A, T = tiles[(0, 0, 0)]["A"], tiles[(0, 0, 0)]["T"]
    assert np.all(np.triu(A) == 0.0)
    T2 = scipy.linalg.solve_triangular(np.eye(C) + A, np.eye(C), lower=True, unit_diagonal=True)
    assert np.linalg.norm(T - T2) / np.linalg.norm(T2) < 1e-12
    assert np.allclose(np.triu(T), np.eye(C), atol=1e-14, rtol=0)


# ------------------------------------------------- planted mistakes -------
def _pin_errors(mutant):
    """Run the pins that can see each planted token-serial mistake; return the
    largest relative error among them (must exceed every pin tolerance)."""
    rng = np.random.default_rng(900)
    errs = []
    dk = dv = 6
    q, k, v, g, b, H0 = _draw(rng, 1, 1, 1, dk, dv, glo=-2.0)
    o, _ = oracle.serial_fwd(q, k, v, g, b, H0, mutant=mutant)
    D = np.exp(g[0, 0]) * np.eye(dk)
    kk, qq, vv, bb = k[0, 0], q[0, 0], v[0, 0], b[0, 0]
    o_ref = H0[0, 0].T @ D @ (np.eye(dk) - bb * np.outer(kk, kk)) @ qq + bb * vv * (kk @ qq)
    errs.append(rel_l2(o[0, 0], o_ref))
    q, k, v, g, b, H0 = _draw(rng, 20, 1, 1, dk, dv, glo=-0.7, beta=0.0)
    o, _ = oracle.serial_fwd(q, k, v, g, b, H0, mutant=mutant)
    G = np.cumsum(g[:, 0])
    ref = np.stack([(np.exp(G[t]) * H0[0, 0]).T @ q[t, 0] for t in range(20)])
    errs.append(rel_l2(o[:, 0], ref))
    _, k, v, g, _, H0 = _draw(rng, 20, 1, 1, dk, dv, glo=-1.0)
    o, _ = oracle.serial_fwd(k, k, v, g, np.ones((20, 1)), H0, mutant=mutant)
    errs.append(rel_l2(o[:, 0], v[:, 0]))
    return max(errs)


@pytest.mark.parametrize("mutant", [oracle.MUT_DECAY_AFTER_WRITE, oracle.MUT_NO_BETA_ERASE,
                                    oracle.MUT_TRANSPOSED_READ, oracle.MUT_GATE_NEXT_TOKEN,
                                    oracle.MUT_OUTPUT_BEFORE_WRITE])
def test_planted_token_serial_mistakes_fail_the_pins(mutant):
    assert _pin_errors(oracle.CORRECT) < 1e-13
    assert _pin_errors(mutant) > 1e-6


@pytest.mark.parametrize("mutant", ["skip_solve", "gate_off_by_one", "drop_diag"])
def test_planted_chunk_form_mistakes_fail_P7(mutant):
    rng = np.random.default_rng(901)
    q, k, v, g, b, H0 = _draw(rng, 130, 1, 2, 16, 8, glo=-1.0)
    o_s, h_s = oracle.serial_fwd(q, k, v, g, b, H0)
    o_c, h_c = chunked.chunked_fwd(q, k, v, g, b, H0, chunk=64, mutant=mutant)
    assert max(rel_l2(o_c, o_s), rel_l2(h_c, h_s)) > 1e-4


def test_planted_missing_reset_fails_P9():
    rng = np.random.default_rng(902)
    lens = [20, 30]
    q, k, v, g, b, _ = _draw(rng, 50, 1, 1, 8, 8, glo=-0.05)
    H0 = rng.standard_normal((2, 1, 8, 8))
    starts = np.array([0, 20, 50])
    o_s, h_s = oracle.serial_fwd(q, k, v, g, b, H0, seq_start=starts)
    o_c, h_c = chunked.chunked_fwd(q, k, v, g, b, H0, seq_start=starts, chunk=8, mutant="no_reset")
    assert rel_l2(o_c[20:], o_s[20:]) > 1e-4
