"""Pins of the bf16-logit scoring mode of the oracle (round_to_bf16 and
score(..., bf16_logits=True)): hand-checked roundings (ties to even both
ways, signs, tiny and huge values), agreement with PyTorch's own fp32 ->
bf16 conversion, closed forms that tell round-to-even from truncation and
half-up, and the plain PyTorch CPU path of a trainer that keeps bf16 logits
(bf16 LM-head product, fp32 log-softmax)."""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import synth


def test_hand_checked_roundings():
    cases = [
        (1.0, 1.0),
        (1 + 2**-8, 1.0),                 # tie, kept part even: stays
        (1 + 3 * 2**-8, 1 + 2**-6),       # tie, kept part odd: rounds up to even
        (1 + 2**-8 + 2**-20, 1 + 2**-7),  # just above the tie
        (1 + 2**-8 - 2**-20, 1.0),        # just below
        (1 + 3 * 2**-9, 1 + 2**-7),
        (-(1 + 3 * 2**-8), -(1 + 2**-6)),  # sign-magnitude: the same on the negative side
        (0.0, 0.0),
        (2.0**-133, 2.0**-133),           # subnormal fp32, exact in bf16
        (3.0e38, 2.0**127 * 226 / 128),   # 3e38 / 2^127 = 1.763: mantissa 97.7 -> 98
    ]
    z = np.array([c[0] for c in cases])
    got = oracle.round_to_bf16(z)
    assert list(got) == [c[1] for c in cases]


def test_matches_torch_conversion():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 3, 20000).astype(np.float32)
    # plant exact ties and near-ties
    bits = x.view(np.uint32)
    bits[:2000] = (bits[:2000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    bits[2000:4000] = (bits[2000:4000] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    x = bits.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), want)


def test_closed_form_tells_rounding_rules_apart():
    # x = (1, 1) on two hidden units; row v of W holds (1, b_v) so z_v = 1 + b_v.
    # b = 2^-8 is a tie (-> 1.0), 3 * 2^-9 rounds up (-> 1 + 2^-7), 2^-10
    # rounds down (-> 1.0). Round-half-up or truncation would give other sets.
    H = 64
    bs = [2.0**-8, 3 * 2.0**-9, 2.0**-10, 0.0]
    w = np.zeros((4, H), np.float32)
    w[:, 0] = 1.0
    w[:, 1] = bs
    x = np.zeros((1, H), np.float32)
    x[0, :2] = 1.0
    xb, wb = synth.bf16_bits_from_f32(x), synth.bf16_bits_from_f32(w)
    zr = np.array([1.0, 1 + 2**-7, 1.0, 1.0])
    for T in (1.0, 0.5):
        lse = math.log(np.exp(zr / T).sum())
        for t in range(4):
            got, _ = oracle.score(xb, wb, [t], T, bf16_logits=True)
            assert abs(got[0] - (zr[t] / T - lse)) < 1e-14
        plain, _ = oracle.score(xb, wb, [0], T)
        assert abs(plain[0] - got[0]) > 1e-4            # the modes differ here


def test_representable_logits_unchanged():
    # Zero weights and one-hot rows give bf16-exact logits: both modes agree
    # exactly, and zero weights still give -ln V.
    c = synth.tiny_case(T=8, H=64, V=300)
    wz = np.zeros_like(c.w_bits)
    got, _ = oracle.score(c.x_bits, wz, c.ids, 0.7, bf16_logits=True)
    assert np.allclose(got, -math.log(300), atol=1e-14)
    x = np.zeros((3, 64), np.float32)
    x[np.arange(3), [0, 5, 9]] = 1.0
    xb = synth.bf16_bits_from_f32(x)
    a, _ = oracle.score(xb, c.w_bits, c.ids[:3], 1.3, bf16_logits=True)
    b, _ = oracle.score(xb, c.w_bits, c.ids[:3], 1.3)
    assert np.array_equal(a, b)


def test_plain_torch_trainer_path():
    # A trainer that keeps bf16 logits: PyTorch CPU bf16 matmul (fp32
    # accumulation, bf16 result), then float(), / T, log_softmax, gather.
    c = synth.tiny_case(T=64, H=256, V=4096, seed=2)
    T_ = 0.8
    x = torch.from_numpy(c.x_bits.view(np.int16)).view(torch.bfloat16)
    w = torch.from_numpy(c.w_bits.view(np.int16)).view(torch.bfloat16)
    logits = x @ w.T                                   # bf16
    ref = torch.log_softmax(logits.float() / T_, dim=-1)[torch.arange(64), torch.from_numpy(c.ids)]
    got, _ = oracle.score(c.x_bits, c.w_bits, c.ids, T_, bf16_logits=True)
    plain, _ = oracle.score(c.x_bits, c.w_bits, c.ids, T_)
    # A logit whose fp32 sum sits at a bf16 rounding boundary may round the
    # other way in PyTorch's summation order: one bf16 ulp (<= 2^-8 |z|) on
    # the target, a far smaller change through the normaliser.
    z = oracle.logits(c.x_bits, c.w_bits)[np.arange(64), c.ids]
    slack = 2.0**-8 * np.abs(z) / T_ + 1e-5
    d = np.abs(got - ref.double().numpy())
    assert (d <= slack).all()
    assert np.mean(d <= 1e-5) > 0.9                    # almost every row agrees tightly
    assert np.max(np.abs(got - plain)) > 1e-4          # and the mode matters
