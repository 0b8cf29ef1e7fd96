"""Host logic of the seeded input generator (no method arithmetic)."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_chunk_amd import inputs


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 100000),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 0.0], np.float32)])
    x = x.astype(np.float32)
    ours = inputs.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny"])
def test_generator_is_deterministic_and_follows_its_recipe(name):
    a = inputs.make(name)
    b = inputs.make(name)
    for f in ("q", "k", "v", "g", "beta", "h0"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    s = a.spec
    q, k = a.as_f64("q"), a.as_f64("k")
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-5)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-5)       # tiny: no q scale
    assert np.all(a.g <= 0) and np.all(a.g >= -5)
    assert np.all((a.beta > 0) & (a.beta < 1))
    assert a.h0.shape == (s.n_seq, s.hv, s.dk, s.dv)
    assert list(a.cu_seqlens) == [0, 200]


def test_small_bf16_spec_rounds_and_scales_q():
    spec = inputs.CONFIGS["single"].with_(seq_lens=(70,), hk=2, hv=6)
    a = inputs.make(spec)
    assert a.q.dtype == np.uint16 and a.k.dtype == np.uint16 and a.v.dtype == np.uint16
    qn = np.linalg.norm(a.as_f64("q"), axis=-1)
    assert np.allclose(qn, 128 ** -0.5, rtol=1e-2)
    assert a.h0 is None
    assert a.g.shape == (70, 6)


def test_raw_draws_are_the_prepared_workloads_draws_before_preparation():
    spec = inputs.CONFIGS["hybrid"].with_(seq_lens=(70,), hk=2, hv=6, qkv_dtype="f32")
    a, r = inputs.make(spec), inputs.make(spec.with_(raw=True))
    assert r.meta == dict(q_scale=float(np.float32(128 ** -0.5)), gate_scale=0.5)
    assert np.array_equal(inputs._l2norm_rows(r.k), a.k)
    assert np.array_equal(inputs._l2norm_rows(r.q) * np.float32(128 ** -0.5), a.q)
    assert np.allclose(1.0 / (1.0 + np.exp(-r.beta.astype(np.float64))), a.beta, rtol=1e-6)
    assert np.allclose(-0.5 * np.logaddexp(0.0, r.g.astype(np.float64)), a.g, rtol=1e-6)
    assert np.array_equal(r.v, a.v) and np.array_equal(r.h0, a.h0)
    with pytest.raises(ValueError):
        inputs.make(inputs.CONFIGS["tiny"].with_(raw=True))   # clip5 gate law: no raw form
