"""The seeded input generator: shapes, bf16 exactness and gate ranges (CPU)."""
import numpy as np

from linear_attention_scan_amd import workloads as wl


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1).
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], dtype=np.float32)
    got = wl.round_to_bf16(x)
    assert got.tolist() == [1.0, 1.0 + 2 * 2.0 ** -7, -2.5, 0.0]
    y = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    r = wl.round_to_bf16(y)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    assert np.max(np.abs(r - y) / np.abs(y)) <= 2.0 ** -8


def test_small_delta_recipe():
    w = wl.delta_bf16(seed=1, B=2, H=3, T=50, d=32)
    assert w.q.shape == (2, 3, 50, 32) and w.v.shape == (2, 3, 50, 32)
    assert np.all((w.k.view(np.uint32) & 0xFFFF) == 0)
    assert np.allclose(np.linalg.norm(w.k, axis=-1), 1.0, atol=1e-2)
    assert np.all((w.beta > 0) & (w.beta < 2)) and np.all(w.lam > 0)
    again = wl.delta_bf16(seed=1, B=2, H=3, T=50, d=32)
    assert np.array_equal(w.q, again.q) and np.array_equal(w.lam, again.lam)


def test_additive_and_per_channel_recipes():
    a = wl.additive_bf16(seed=0, B=1, H=2, T=40, d=16)
    assert a.beta is None and a.rule == wl.RULE_ADDITIVE and a.phi == wl.PHI_ELU1
    assert np.all((a.lam > 0) & (a.lam < 1))
    p = wl.delta_long_pc(seed=0, B=1, H=2, T=40, d=16)
    assert p.lam.shape == (1, 2, 40, 16) and p.per_channel


def test_decode_steps_are_reproducible():
    s0 = wl.decode_step(3, 7, B=2, H=2, d=16)
    s1 = wl.decode_step(3, 7, B=2, H=2, d=16)
    s2 = wl.decode_step(3, 8, B=2, H=2, d=16)
    assert np.array_equal(s0.q, s1.q) and not np.array_equal(s0.q, s2.q)
    S0 = wl.decode_state0(0, B=2, H=2, d=16)
    assert S0.shape == (2, 2, 16, 16) and abs(float(S0.std()) - 0.02) < 0.005


def test_inner_recipe():
    w = wl.inner_bf16(seed=2, B=1, H=2, T=30, d=16)
    d = wl.delta_bf16(seed=2, B=1, H=2, T=30, d=16)
    assert w.rule == wl.RULE_INNER and w.name == "inner_bf16"
    assert np.array_equal(w.k, d.k) and np.array_equal(w.beta, d.beta) and np.array_equal(w.lam, d.lam)
