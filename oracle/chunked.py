"""Dense fp64 numpy evaluation of the chunk (WY) form -- TEST INFRASTRUCTURE ONLY.

Second, independent oracle (see ``oracle/__init__.py`` for who may import it).
It follows the tile oracle described on the ROCm/rocm-libraries KDA chunkwise
page (section "Correctness"): every gate factor is formed from the pairwise
exponent difference exp(G_r - G_s) directly, never through a midpoint
factoring, and the per-chunk unit-lower-triangular system is solved with LAPACK
(``numpy.linalg.solve``).  The chunk equations are the WY form named on the
stratat.com page "hip: chunk-parallel GDN recurrence (WY form)" (section "What
this is": per chunk one C x C unit-lower-triangular solve plus GEMM-shaped
folds), written out for a chunk of rows r = 1..n entering with state H0
(K-first, [dk, dv]) and in-chunk cumulative gate G_r = sum_{s<=r} g_s
(per key channel for the per-channel gate):

    A_rs = beta_r * sum_c k_r[c] k_s[c] exp(G_r[c] - G_s[c])      (s < r, else 0)
    T    = (I + A)^-1
    W    = T diag(beta) (K * exp(G));   U' = T diag(beta) V
    R    = U' - W H0                                            (true per-token deltas)
    P_rs = sum_c q_r[c] k_s[c] exp(G_r[c] - G_s[c])              (s <= r, else 0)
    O    = (Q * exp(G)) H0 + P R
    H_n  = diag(exp(G_n)) H0 + Ktil^T R,   Ktil_s = k_s * exp(G_n - G_s)

These follow from unrolling the token-serial rule inside one chunk; the
equivalence is what ``tests/test_oracle_pins.py`` checks against the
token-serial oracle.  A short last chunk is evaluated at its own length;
``pad_to`` instead zero-fills it (q = k = v = 0, beta = 0, g = 0), which must
give the same result.

Parity status: pinned (token-serial agreement, LAPACK triangular solve,
closed forms).
"""
from __future__ import annotations

import numpy as np

MUTANTS = ("skip_solve", "gate_off_by_one", "drop_diag", "no_reset")


def _gate_factors(G):
    """Pairwise exp(G_r - G_s) for s <= r (zero above the diagonal).

    G is [n] (scalar gate) or [n, dk] (per-channel gate); the result is
    [n, n] or [n, n, dk].
    """
    n = G.shape[0]
    keep = np.tril(np.ones((n, n), dtype=bool))
    if G.ndim == 1:
        D = G[:, None] - G[None, :]
        return np.where(keep, np.exp(np.where(keep, D, 0.0)), 0.0)
    D = G[:, None, :] - G[None, :, :]
    return np.where(keep[:, :, None], np.exp(np.where(keep[:, :, None], D, 0.0)), 0.0)


def chunk_step(q, k, v, g, beta, H0, mutant=None, want_tiles=False):
    """One chunk of n rows: q, k [n, dk]; v [n, dv]; g [n] or [n, dk]; beta [n]."""
    n, dk = k.shape
    G = np.cumsum(g, axis=0)
    if mutant == "gate_off_by_one":
        G = np.concatenate([np.zeros_like(G[:1]), G[:-1]], axis=0)
    F = _gate_factors(G)
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    if G.ndim == 1:
        KK = k @ k.T
        QK = q @ k.T
        A = np.where(strict, beta[:, None] * F * KK, 0.0)
        P = F * QK
        eG = np.exp(G)[:, None]
        dec = np.full(dk, np.exp(G[-1]))
        Ktil = k * np.exp(G[-1] - G)[:, None]
    else:
        A = np.where(strict, beta[:, None] * np.einsum("rc,sc,rsc->rs", k, k, F), 0.0)
        P = np.einsum("rc,sc,rsc->rs", q, k, F)
        eG = np.exp(G)
        dec = np.exp(G[-1])
        Ktil = k * np.exp(G[-1][None, :] - G)
    if mutant == "drop_diag":
        P = np.tril(P, -1)
    eye = np.eye(n)
    T = eye if mutant == "skip_solve" else np.linalg.solve(eye + A, eye)
    W = T @ (beta[:, None] * (k * eG))
    U = T @ (beta[:, None] * v)
    R = U - W @ H0
    O = (q * eG) @ H0 + P @ R
    H = dec[:, None] * H0 + Ktil.T @ R
    if want_tiles:
        return O, H, {"A": A, "T": T, "P": P, "W": W, "U": U}
    return O, H


def chunked_fwd(q, k, v, g, beta, h0=None, seq_start=None, chunk=64, head_map=None,
                pad_to=False, mutant=None, units=None, want_tiles=False):
    """Chunk-form evaluation over packed sequences (same argument layout as
    ``oracle.serial_fwd``).  Returns (o [tok, hv, dv], hT [n_seq, hv, dk, dv])
    and, with ``want_tiles``, a dict {(seq, head, chunk_index): tiles}."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    tok, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    if seq_start is None:
        seq_start = np.array([0, tok], dtype=np.int64)
    seq_start = np.asarray(seq_start, dtype=np.int64)
    n_seq = len(seq_start) - 1
    if head_map is None:
        head_map = np.arange(hv) // (hv // hk)
    o = np.zeros((tok, hv, dv))
    hT = np.zeros((n_seq, hv, dk, dv))
    tiles = {}
    pairs = [(n, h) for n in range(n_seq) for h in range(hv)] if units is None else \
        [tuple(u) for u in np.asarray(units).reshape(-1, 2)]
    carried = {}
    for n, h in pairs:
        kh = int(head_map[h])
        if mutant == "no_reset" and n > 0 and (n - 1, h) in carried:
            H = carried[(n - 1, h)].copy()
        else:
            H = np.zeros((dk, dv)) if h0 is None else np.asarray(h0[n, h], dtype=np.float64).copy()
        t0, t1 = int(seq_start[n]), int(seq_start[n + 1])
        for ci, c0 in enumerate(range(t0, t1, chunk)):
            c1 = min(c0 + chunk, t1)
            sl = slice(c0, c1)
            qc, kc, vc = q[sl, kh], k[sl, kh], v[sl, h]
            gc = g[sl, h]
            bc = beta[sl, h]
            m = c1 - c0
            if pad_to and m < chunk:
                pad = chunk - m
                qc = np.concatenate([qc, np.zeros((pad, dk))])
                kc = np.concatenate([kc, np.zeros((pad, dk))])
                vc = np.concatenate([vc, np.zeros((pad, dv))])
                gc = np.concatenate([gc, np.zeros((pad,) + gc.shape[1:])])
                bc = np.concatenate([bc, np.zeros(pad)])
            res = chunk_step(qc, kc, vc, gc, bc, H, mutant=mutant, want_tiles=want_tiles)
            O, H = res[0], res[1]
            if want_tiles:
                tiles[(n, h, ci)] = res[2]
            o[sl, h] = O[:m]
        hT[n, h] = H
        carried[(n, h)] = H
    if want_tiles:
        return o, hT, tiles
    return o, hT
