"""Small numeric helpers shared by the tests (no method arithmetic)."""
import numpy as np


def rel_l2(x, ref):
    """NaN-aware relative L2 error ||x - ref|| / ||ref||; inf when x is not finite."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64)))) if np.size(x) else 0.0


def unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rel_l2_axes(x, ref, axes):
    """rel_l2 reduced over `axes` only (one figure per remaining index); inf where x has
    a non-finite element, the absolute error where ref is zero."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return np.where(np.all(np.isfinite(x), axis=axes), out, np.inf)


def chunk_rel_l2(x, ref, C):
    """rel_l2 of every (chunk, head) of token-major x, ref [L, H, D]: chunk c covers tokens
    c C .. c C + C - 1 (the last chunk may be partial).  Returns [ceil(L / C), H]."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    L, H, D = ref.shape
    nch = (L + C - 1) // C
    pad = nch * C - L
    if pad:
        z = np.zeros((pad, H, D))
        x, ref = np.concatenate([x, z]), np.concatenate([ref, z])
    return rel_l2_axes(x.reshape(nch, C, H, D), ref.reshape(nch, C, H, D), (1, 3))
