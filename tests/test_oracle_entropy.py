"""Pins for the oracle's row entropy and argmax (CPU only).

Checked against closed forms (uniform and two-level rows), 50-digit brute
force, and properties the definitions imply (bounds, monotonicity in the
temperature, the low-temperature limit, invariance under a constant logit
shift, padded rows taking no part, lowest-index ties).
"""

import math

import mpmath
import numpy as np
import pytest

import oracle
from workloads import synth


def bits(a):
    u = np.asarray(a, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not bf16-exact"
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("V", [4096, 151936])
@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_uniform_row(V, temperature):
    # Zero weights: every logit 0, p = 1/V, entropy ln V; every index ties, so
    # the argmax is the first one.
    x = synth.tiny_case(T=3, H=16, V=8).x_bits
    w = np.zeros((V, 16), np.uint16)
    lp, lse, ent, am = oracle.score_stats(x, w, np.array([0, 1, V - 1]), temperature)
    assert np.allclose(ent, math.log(V), rtol=0, atol=1e-11)
    assert np.array_equal(am, [0, 0, 0])
    assert np.allclose(lp, -math.log(V), atol=1e-12)


@pytest.mark.parametrize("temperature", [1.0, 0.5, 2.0])
def test_two_level_closed_form(temperature):
    # One logit a at `target`, V - 1 logits b elsewhere.
    V, H, k, target, a, b = 1000, 32, 3, 417, 1.5, -0.25
    x = np.zeros((1, H), np.float32); x[0, k] = 1.0
    w = np.zeros((V, H), np.float32); w[:, k] = b; w[target, k] = a
    _, _, ent, am = oracle.score_stats(bits(x), bits(w), np.array([0]), temperature)
    za, zb = a / temperature, b / temperature
    Z = math.exp(za) + (V - 1) * math.exp(zb)
    p1, p2 = math.exp(za) / Z, math.exp(zb) / Z
    assert abs(ent[0] - (-p1 * math.log(p1) - (V - 1) * p2 * math.log(p2))) < 1e-12
    assert am[0] == target
    # Swap the roles: the single logit is now the smallest; the argmax is the
    # first of the tied largest ones.
    w[:, k] = a; w[target, k] = b
    _, _, _, am2 = oracle.score_stats(bits(x), bits(w), np.array([0]), temperature)
    assert am2[0] == 0


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_50_digits(seed):
    rng = np.random.default_rng(100 + seed)
    T, H, V = rng.integers(1, 4), rng.integers(1, 13), rng.integers(2, 25)
    x = synth.bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    w = synth.bf16_bits_from_f32(rng.standard_normal((V, H)).astype(np.float32))
    temperature = float(rng.choice([1.0, 0.6, 1.7]))
    v_true = int(rng.integers(1, V + 1))
    _, _, ent, am = oracle.score_stats(x, w, np.zeros(T, np.int64), temperature, v_true)
    mpmath.mp.dps = 50
    xf, wf = oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(w)
    for t in range(T):
        z = [mpmath.fsum(mpmath.mpf(xf[t, h]) * mpmath.mpf(wf[v, h]) for h in range(H))
             for v in range(v_true)]
        s = [zv / mpmath.mpf(temperature) for zv in z]
        Zs = mpmath.fsum(mpmath.exp(sv) for sv in s)
        p = [mpmath.exp(sv) / Zs for sv in s]
        H_ = -mpmath.fsum(pv * mpmath.log(pv) for pv in p)
        assert abs(float(H_) - ent[t]) < 1e-12
        best = max(z)
        assert am[t] == min(v for v in range(v_true) if z[v] == best)


def test_bounds_and_temperature_monotonic():
    c = synth.tiny_case(T=6, H=64, V=700)
    z = oracle.logits(c.x_bits, c.w_bits)
    prev = None
    for T_ in (0.3, 0.7, 1.0, 2.0, 5.0):
        ent, _ = oracle.entropy_argmax(z, T_)
        assert np.all(ent >= 0) and np.all(ent <= math.log(700) + 1e-12)
        if prev is not None:
            assert np.all(ent >= prev - 1e-12)        # dH/dT >= 0
        prev = ent
    ent_cold, am_cold = oracle.entropy_argmax(z, 1e-4)
    assert np.all(ent_cold < 1e-6)                    # all mass on the argmax
    assert np.array_equal(am_cold, np.argmax(z, axis=1))


def test_shift_invariance_and_padding():
    c0 = synth.tiny_case(T=5, H=64, V=300)
    x = synth.f32_from_bf16_bits(c0.x_bits).copy()
    w = synth.f32_from_bf16_bits(c0.w_bits).copy()
    x[:, 3] = 0.0; w[:, 3] = 0.0
    _, _, e0, a0 = oracle.score_stats(bits(x), bits(w), c0.ids % 300, 0.9)
    x[:, 3] = 1.0; w[:, 3] = 2.5                      # every logit + 2.5
    _, _, e1, a1 = oracle.score_stats(bits(x), bits(w), c0.ids % 300, 0.9)
    assert np.allclose(e0, e1, rtol=0, atol=1e-12) and np.array_equal(a0, a1)
    # Padded rows past v_true with huge logits change neither.
    wp = np.zeros((320, 64), np.float32); wp[:300] = w; wp[300:, 3] = 64.0
    _, _, e2, a2 = oracle.score_stats(bits(x), bits(wp), c0.ids % 300, 0.9, v_true=300)
    assert np.allclose(e1, e2, rtol=0, atol=1e-12) and np.array_equal(a1, a2)
