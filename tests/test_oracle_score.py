"""Pins for the fp64 selected-token-logprob oracle (CPU only).

Each test checks the oracle against something other than itself: a closed form,
an invariant the definition implies, 50-digit brute force, or a value printed
on the pages.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
from workloads import synth


def bits(a):
    """fp32 values that are exactly representable in bf16 -> bf16 bits."""
    u = np.asarray(a, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not bf16-exact"
    return (u >> 16).astype(np.uint16)


def test_bf16_decode_is_exact():
    b = np.array([0x3F80, 0xC020, 0x0001, 0x7F80, 0x8000, 0x3DCD], np.uint16)
    v = oracle.bf16_bits_to_f64(b)
    assert v[0] == 1.0 and v[1] == -2.5
    assert v[2] == 2.0 ** -133                     # smallest bf16 subnormal
    assert v[3] == math.inf and math.copysign(1, v[4]) == -1.0
    assert v[5] == 0.10009765625                   # 0x3DCD0000


@pytest.mark.parametrize("V", [4096, 151936])
@pytest.mark.parametrize("temperature", [1.0, 0.7, 3.0])
def test_zero_weights_give_minus_log_v(V, temperature):
    # All logits are 0, so every token has probability 1/V at any temperature.
    x = synth.tiny_case(T=3, H=16, V=8).x_bits
    w = np.zeros((V, 16), np.uint16)
    lp, lse = oracle.score(x, w, np.array([0, V // 2, V - 1]), temperature)
    assert np.allclose(lp, -math.log(V), rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-12)


def test_true_vocab_range_excludes_padded_rows():
    # Rows at and past v_true are padding: huge logits there must not count.
    V, v_true, H = 64, 50, 8
    w = np.zeros((V, H), np.uint16)
    w[v_true:, :] = bits(np.full((V - v_true, H), 8.0))
    x = bits(np.ones((2, H)))
    lp, _ = oracle.score(x, w, np.array([0, v_true - 1]), 1.0, v_true=v_true)
    assert np.allclose(lp, -math.log(v_true), atol=1e-12)
    with pytest.raises(ValueError):
        oracle.score(x, w, np.array([0, v_true]), 1.0, v_true=v_true)


@pytest.mark.parametrize("temperature", [1.0, 0.7, 2.5])
def test_two_level_closed_form(temperature):
    # x = e_k; w[:, k] = b for every row except w[target, k] = a.
    # logprob(target) = a/T - ln(exp(a/T) + (V - 1) exp(b/T)).
    V, H, k, target = 1000, 32, 5, 321
    a, b = 1.5, -0.25
    x = np.zeros((1, H), np.float32); x[0, k] = 1.0
    w = np.zeros((V, H), np.float32); w[:, k] = b; w[target, k] = a
    w[:, k + 1] = 0.75                           # ignored: x is 0 there
    lp, _ = oracle.score(bits(x), bits(w), np.array([target]), temperature)
    expect = a / temperature - math.log(math.exp(a / temperature)
                                        + (V - 1) * math.exp(b / temperature))
    assert abs(lp[0] - expect) < 1e-13
    # The other tokens: b/T - same normaliser.
    lp2, _ = oracle.score(bits(x), bits(w), np.array([7]), temperature)
    assert abs(lp2[0] - (expect - (a - b) / temperature)) < 1e-13
    if temperature != 1.0:
        # Dividing a finished logprob by T is not the tempered score
        # (AMD blog, "How this differs from a real temperature mismatch").
        lp1, _ = oracle.score(bits(x), bits(w), np.array([target]), 1.0)
        assert abs(lp1[0] / temperature - lp[0]) > 1e-3


def test_normalisation_sums_to_one():
    c = synth.tiny_case(T=4, H=64, V=512)
    for t in range(c.T):
        row = np.repeat(c.x_bits[t:t + 1], c.V, axis=0)
        lp, lse = oracle.score(row, c.w_bits, np.arange(c.V), 0.8)
        assert abs(math.fsum(np.exp(lp)) - 1.0) < 1e-12
        assert np.all(lse == lse[0])


def test_constant_logit_shift_cancels():
    # Give x a constant-1 column and every weight row the same value c in it:
    # every logit moves by c and the logprobs do not change.
    c0 = synth.tiny_case(T=5, H=64, V=300)
    x = synth.f32_from_bf16_bits(c0.x_bits).copy()
    w = synth.f32_from_bf16_bits(c0.w_bits).copy()
    x[:, 3] = 0.0
    w[:, 3] = 0.0
    lp0, lse0 = oracle.score(bits(x), bits(w), c0.ids % 300, 0.9)
    x[:, 3] = 1.0
    w[:, 3] = 2.5
    lp1, lse1 = oracle.score(bits(x), bits(w), c0.ids % 300, 0.9)
    assert np.allclose(lp0, lp1, rtol=0, atol=1e-13)
    assert np.allclose(lse1 - lse0, 2.5 / 0.9, rtol=0, atol=1e-12)


def test_high_temperature_tends_to_uniform():
    c = synth.tiny_case(T=3, H=64, V=777)
    lp, _ = oracle.score(c.x_bits, c.w_bits, c.ids % 777, 1e7)
    assert np.allclose(lp, -math.log(777), atol=1e-5)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_50_digits(seed):
    rng = np.random.default_rng(seed)
    T, H, V = rng.integers(1, 5), rng.integers(1, 17), rng.integers(2, 33)
    x = synth.bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    w = synth.bf16_bits_from_f32(rng.standard_normal((V, H)).astype(np.float32))
    ids = rng.integers(0, V, T)
    temperature = float(rng.choice([1.0, 0.7, 1.3]))
    v_true = int(rng.integers(1, V + 1))
    ids = ids % v_true
    lp, lse = oracle.score(x, w, ids, temperature, v_true=v_true)
    mpmath.mp.dps = 50
    xf, wf = oracle.bf16_bits_to_f64(x), oracle.bf16_bits_to_f64(w)
    for t in range(T):
        z = [mpmath.fsum(mpmath.mpf(xf[t, h]) * mpmath.mpf(wf[v, h]) for h in range(H))
             / mpmath.mpf(temperature) for v in range(v_true)]
        norm = mpmath.log(mpmath.fsum(mpmath.exp(zv) for zv in z))
        assert abs(float(z[ids[t]] - norm) - lp[t]) < 1e-12
        assert abs(float(norm) - lse[t]) < 1e-12


def test_page_uniform_score_within_one_ulp(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "uniform_score.json")))
    V = g["vocab_rows"]
    lp, _ = oracle.score(np.zeros((1, 8), np.uint16), np.zeros((V, 8), np.uint16),
                         np.array([0]))
    ours = np.float32(lp[0]).view(np.int32)
    page = np.float32(g["printed_A"]).view(np.int32)
    assert abs(int(ours) - int(page)) <= 1


def test_rejects_bad_arguments():
    c = synth.tiny_case(T=2, H=8, V=16)
    with pytest.raises(ValueError):
        oracle.score(c.x_bits, c.w_bits, np.array([0, 16]))
    with pytest.raises(ValueError):
        oracle.score(c.x_bits, c.w_bits, np.array([0, -1]))
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            oracle.score(c.x_bits, c.w_bits, np.array([0, 1]), bad)
    lp, lse = oracle.score(c.x_bits[:0], c.w_bits, np.array([], np.int64))
    assert lp.shape == (0,) and lse.shape == (0,)
