"""The parity metrics themselves (CPU): the per-(chunk, head) relative L2 that the
full-size GPU tests apply to every chunk sees a single wrong token row, which the
whole-unit figure of a long sequence does not; and the whole-tensor figure of the GPU
tests excuses a state's last grid steps in fp32's subnormal band but nothing above it."""
import numpy as np

from tests._util import chunk_rel_l2, rel_l2, rel_l2_axes
from tests.gpu_util import SUBNORMAL_ALLOWANCE, rel

STEP = 2.0 ** -149      # fp32's spacing below 2^-126


def test_chunk_metric_equals_rel_l2_of_each_chunk():
    rng = np.random.default_rng(3)
    L, H, D, C = 150, 3, 8, 64
    ref = rng.standard_normal((L, H, D))
    x = ref + 1e-3 * rng.standard_normal((L, H, D))
    m = chunk_rel_l2(x, ref, C)
    assert m.shape == (3, H)
    for c in range(3):
        for h in range(H):
            sl = slice(c * C, min(L, c * C + C))
            assert abs(m[c, h] - rel_l2(x[sl, h], ref[sl, h])) < 1e-15
    assert np.allclose(rel_l2_axes(x, ref, (0, 2)), [rel_l2(x[:, h], ref[:, h]) for h in range(H)])


def test_one_wrong_row_fails_its_chunk_but_not_a_long_unit():
    rng = np.random.default_rng(4)
    L, H, D, C = 32768, 1, 128, 64
    ref = rng.standard_normal((L, H, D))
    x = ref.copy()
    x[1000, 0] = rng.standard_normal(D)          # one token row replaced
    assert rel_l2(x, ref) < 2e-2                  # the whole-unit figure does not see it
    m = chunk_rel_l2(x, ref, C)
    assert m.max() > 0.1 and int(np.argmax(m[:, 0])) == 1000 // C


def test_non_finite_scores_inf():
    ref = np.ones((70, 2, 4))
    x = ref.copy()
    x[65, 1, 2] = np.nan
    m = chunk_rel_l2(x, ref, 64)
    assert np.isinf(m[1, 1]) and np.all(np.isfinite(m[0])) and np.isfinite(m[1, 0])


def test_subnormal_state_one_step_off_passes():
    # a state decayed into the subnormal band (about 1,500 grid steps tall), every element
    # one step off its exact value: relative L2 would read ~1e-3, above the fp32 arm's 1e-4
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((3, 32, 32)) * 1500 * STEP
    x = ref.astype(np.float32).astype(np.float64) + STEP * rng.choice([-1.0, 1.0], size=ref.shape)
    assert rel_l2(x, ref) > 1e-4
    assert rel(x, ref) == 0.0


def test_subnormal_state_flushed_to_zero_fails():
    rng = np.random.default_rng(6)
    ref = rng.standard_normal((3, 32, 32)) * 1500 * STEP
    r = rel(np.zeros_like(ref), ref)
    assert 0.95 < r <= 1.0


def test_allowance_leaves_normal_range_errors():
    # at and above the smallest normal value the allowance is at most 2^-19 of a value
    assert SUBNORMAL_ALLOWANCE / 2.0 ** -126 <= 2.0 ** -19
    rng = np.random.default_rng(7)
    for scale in (1.0, 2.0 ** -126):
        ref = rng.standard_normal(4096) * scale
        x = ref * (1 + 1e-3 * rng.standard_normal(4096))
        assert abs(rel(x, ref) - rel_l2(x, ref)) <= 0.02 * rel_l2(x, ref)


def test_rel_scores_non_finite_inf():
    ref = np.ones(10)
    x = ref.copy()
    x[3] = np.inf
    assert np.isinf(rel(x, ref))
