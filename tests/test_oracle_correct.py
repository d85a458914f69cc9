"""Pins of the correction-consumer oracle (oracle.correct): the pages' worked
numbers, closed forms, the estimators' series, bounds, and a token-by-token
brute force written independently of the vectorised oracle."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import REJECT_K1, REJECT_K3, REJECT_NONE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
INF = math.inf


def one_token(rollout_p, train_p):
    r = np.array([[math.log(rollout_p)]], np.float32)
    t = np.array([[math.log(train_p)]], np.float32)
    return r, t, np.ones((1, 1), np.uint8)


def test_figure1_correction_weight():
    # [TII] Figure 1: q = 0.20, pi_0 = p_v = 0.21 -> w = 1.05.
    g = json.load(open(os.path.join(GOLDEN, "eq1_split.json")))
    r, t, m = one_token(g["rollout_probability_q_v"], g["trainer_same_version_p_v"])
    w_page = g["printed"]["correction_w"]
    w, s = oracle.correct(r, t, m, tis_clip=2.0)
    assert abs(w[0, 0] / w_page - 1) < 3e-7          # fp32 logprobs, fp32 weight
    assert s["kept"][0] == 1 and s["capped"][0] == 0
    w, s = oracle.correct(r, t, m, tis_clip=1.02)     # TIS: min(w, C)
    assert w[0, 0] == np.float32(1.02) and s["capped"][0] == 1
    w, s = oracle.correct(r, t, m, mis_log_lo=math.log(0.5), mis_log_hi=math.log(2.0))
    assert abs(w[0, 0] / w_page - 1) < 3e-7          # MIS: inside [l, u] keeps w
    w, s = oracle.correct(r, t, m, mis_log_lo=math.log(1.1), mis_log_hi=math.log(2.0))
    assert w[0, 0] == 0 and s["kept"][0] == 0          # outside: dropped
    # K1 of that token is -log w, K3 = w - 1 - log w.
    _, s1 = oracle.correct(r, t, m, reject=REJECT_K1)
    _, s3 = oracle.correct(r, t, m, reject=REJECT_K3)
    d = float(t[0, 0]) - float(r[0, 0])
    assert abs(s1["stat"][0] + math.log(w_page)) < 3e-7
    assert s1["stat"][0] == -d
    assert abs(s3["stat"][0] - (w_page - 1 - math.log(w_page))) < 3e-7


def test_identical_scores_closed_form():
    rng = np.random.default_rng(1)
    r = np.log(rng.random((4, 50))).astype(np.float32)
    m = (rng.random((4, 50)) < 0.7).astype(np.uint8)
    for kind in (REJECT_NONE, REJECT_K1, REJECT_K3):
        w, s = oracle.correct(r, r, m, tis_clip=2.0, reject=kind, reject_hi=0.0)
        assert np.array_equal(w, m.astype(np.float32))   # r = 1 on every active token
        assert (s["stat"] == 0).all() and (s["accepted"] == 1).all()
        assert np.array_equal(s["kept"], m.sum(1)) and (s["capped"] == 0).all()
        assert np.array_equal(s["sum_weight"], m.sum(1).astype(float))


@pytest.mark.parametrize("delta", [0.25, -0.5, 1.5])
def test_constant_offset_closed_form(delta):
    # rollout = -2, train = -2 + delta: both exact in fp32, so d = delta.
    N, L = 3, 40
    r = np.full((N, L), -2.0, np.float32)
    t = (r + np.float32(delta)).astype(np.float32)
    m = np.ones((N, L), np.uint8)
    m[1, 10:] = 0
    cnt = m.sum(1)
    _, s1 = oracle.correct(r, t, m, reject=REJECT_K1)
    np.testing.assert_allclose(s1["stat"], -delta * cnt, rtol=1e-15)
    _, s3 = oracle.correct(r, t, m, reject=REJECT_K3)
    np.testing.assert_allclose(s3["stat"], cnt * (math.exp(delta) - 1 - delta), rtol=1e-14)
    w, s = oracle.correct(r, t, m, tis_clip=2.0)
    want = min(math.exp(delta), 2.0)
    assert np.array_equal(w[m != 0], np.full(cnt.sum(), np.float32(want)))
    assert np.array_equal(s["capped"], cnt if math.exp(delta) >= 2 else 0 * cnt)


def test_rejection_by_accumulated_mismatch():
    # Sequences with offsets 0, 0.01, 0.1, 1 on 100 tokens: sum K3 =
    # 100 (e^d - 1 - d); a bound between the second and third rejects the
    # last two, and their weights are all zero.
    deltas = np.array([0.0, 0.01, 0.1, 1.0], np.float32)
    r = np.full((4, 100), -1.0, np.float32)
    t = (r + deltas[:, None]).astype(np.float32)
    m = np.ones_like(r, np.uint8)
    d64 = t.astype(np.float64)[:, 0] - r.astype(np.float64)[:, 0]
    stat = 100 * (np.exp(d64) - 1 - d64)
    bound = 0.5 * (stat[1] + stat[2])
    w, s = oracle.correct(r, t, m, reject=REJECT_K3, reject_hi=bound)
    assert list(s["accepted"]) == [1, 1, 0, 0]
    assert (w[2:] == 0).all() and (w[:2] > 0).all()
    assert list(s["kept"]) == [100] * 4               # kept does not depend on rejection
    assert (s["sum_weight"][2:] == 0).all()
    # K1 with a two-sided range: |sum K1| small.
    _, s = oracle.correct(r, -(-t), m, reject=REJECT_K1, reject_lo=-5.0, reject_hi=5.0)
    assert list(s["accepted"]) == [1, 1, 0, 0]


def test_k3_series_and_sign():
    rng = np.random.default_rng(3)
    d = rng.normal(0, 0.01, 2000)
    r = np.full((1, d.size), -3.0, np.float32)
    t = (r + d.astype(np.float32)).astype(np.float32)
    m = np.ones_like(r, np.uint8)
    dd = t.astype(np.float64) - r.astype(np.float64)
    _, s = oracle.correct(r, t, m, reject=REJECT_K3)
    series = np.sum(dd ** 2 / 2 + dd ** 3 / 6 + dd ** 4 / 24)
    assert s["stat"][0] >= 0
    assert abs(s["stat"][0] - series) <= np.sum(np.abs(dd) ** 5) + 1e-18


def test_overflow_rejects_and_cap_bounds_the_weight():
    r = np.full((2, 4), -800.0, np.float32)
    t = r.copy()
    t[0, 1] = -60.0                                    # d = 740: e^d overflows fp64
    m = np.ones_like(r, np.uint8)
    w, s = oracle.correct(r, t, m, tis_clip=2.0, reject=REJECT_K3, reject_hi=1e6)
    assert s["stat"][0] == INF and s["accepted"][0] == 0 and s["accepted"][1] == 1
    assert (w[0] == 0).all() and (w[1] == 1).all()
    w, s = oracle.correct(r, t, m, tis_clip=2.0)      # no rejection: the cap holds
    assert w[0, 1] == 2.0 and s["capped"][0] == 1


def test_masked_and_nonfinite_tokens():
    r = np.array([[-1.0, np.nan, -1.0, -np.inf, -1.0]], np.float32)
    t = np.array([[-1.0, -1.0, np.inf, -1.0, -0.5]], np.float32)
    m = np.array([[1, 1, 1, 1, 0]], np.uint8)
    w, s = oracle.correct(r, t, m, reject=REJECT_K1)
    assert list(w[0]) == [1.0, 0.0, 0.0, 0.0, 0.0]
    assert s["valid"][0] == 4 and s["nonfinite"][0] == 3 and s["kept"][0] == 1
    assert s["stat"][0] == 0.0


def brute(r, t, m, C, lo, hi, kind, rlo, rhi):
    """Token-by-token Python floats, independent of the vectorised oracle."""
    N, L = r.shape
    W = np.zeros((N, L), np.float32)
    rows = []
    for n in range(N):
        terms, inside = [], []
        valid = nonfin = 0
        for i in range(L):
            if not m[n, i]:
                continue
            valid += 1
            a, b = float(r[n, i]), float(t[n, i])
            if not (math.isfinite(a) and math.isfinite(b)):
                nonfin += 1
                continue
            d = b - a
            if kind == 1:
                terms.append(-d)
            elif kind == 3:
                try:
                    terms.append(math.expm1(d) - d)
                except OverflowError:
                    terms.append(math.inf)
            if lo <= d <= hi:
                inside.append((i, d))
        stat = math.fsum(terms) if terms else 0.0
        acc = rlo <= stat <= rhi
        capped = 0
        for i, d in inside:
            if d >= math.log(C):
                capped += 1
                v = C
            else:
                v = math.exp(d)
            if acc:
                W[n, i] = np.float32(v)
        rows.append((valid, nonfin, len(inside), capped, int(acc), stat))
    return W, rows


@pytest.mark.parametrize("seed", range(4))
def test_brute_force(seed):
    rng = np.random.default_rng(70 + seed)
    N, L = 6, int(rng.integers(1, 60))
    r = np.log(rng.random((N, L))).astype(np.float32)
    t = (r + rng.normal(0, 0.3, (N, L))).astype(np.float32)
    t[rng.random((N, L)) < 0.05] = np.nan
    m = (rng.random((N, L)) < 0.8).astype(np.uint8)
    C, lo, hi = 1.5, -0.4, 0.6
    for kind in (0, 1, 3):
        rlo, rhi = (-1.0, 1.0) if kind == 1 else (-INF, 0.3)
        w, s = oracle.correct(r, t, m, C, lo, hi, kind, rlo, rhi)
        bw, rows = brute(r, t, m, C, lo, hi, kind, rlo, rhi)
        assert np.array_equal(w, bw)
        for n, row in enumerate(rows):
            assert tuple(int(s[f][n]) for f in ("valid", "nonfinite", "kept", "capped", "accepted")) \
                == row[:5]
            # numpy's and libm's expm1 may differ in the last bit.
            assert abs(s["stat"][n] - row[5]) <= 1e-14 * max(1.0, abs(row[5]))


def test_weight_bounds():
    rng = np.random.default_rng(9)
    r = np.log(rng.random((5, 300))).astype(np.float32)
    t = (r + rng.normal(0, 1.0, r.shape)).astype(np.float32)
    m = np.ones_like(r, np.uint8)
    lo, hi, C = math.log(0.5), math.log(3.0), 2.0
    w, _ = oracle.correct(r, t, m, C, lo, hi)
    nz = w[w != 0]
    assert nz.max() <= C and nz.min() >= np.float32(0.5) * (1 - 1e-7)
    w, _ = oracle.correct(r, t, m, INF, lo, hi)       # MIS only: w itself, up to u
    nz = w[w != 0]
    assert nz.max() <= np.float32(3.0) * (1 + 1e-7) and nz.max() > 2.0


def test_rejects_bad_parameters():
    z = np.zeros((1, 1), np.float32)
    m = np.ones((1, 1), np.uint8)
    for kw in ({"tis_clip": 0.0}, {"mis_log_lo": 1.0, "mis_log_hi": 0.0},
               {"reject_lo": 1.0, "reject_hi": 0.0}, {"reject": 2}):
        with pytest.raises(ValueError):
            oracle.correct(z, z, m, **kw)
