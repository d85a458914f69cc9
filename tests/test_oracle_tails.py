"""Pins for the oracle's tail statistics (CPU only): the quantile rule
against numpy's np.quantile at its default settings (the estimator the AMD
blog's compare() uses) on random and heavily tied data, hand-worked lists,
the one-token and two-token cases, closed forms for identical and offset
scores, the probability difference of the AMD blog's worked example,
first-occurrence maxima, position profiles that add up to the batch totals,
and per-sequence quantiles against np.quantile on each record alone."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import synth

PROBS = oracle.QUANTILE_PROBS


@pytest.mark.parametrize("seed", range(8))
def test_quantile_rule_is_numpys_default(seed):
    # [AMD] "Case 1: A Changes; B and C Stay Close": compare() returns
    # np.quantile(error, .95) and np.quantile(error, .99); numpy's routine on
    # the same sorted values must give the same bits.
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 700))
    vals = np.abs(rng.standard_normal(n)) * 10.0 ** rng.integers(-6, 2, n)
    if seed % 2:
        vals = np.round(vals, 1)                     # many ties
    if seed % 4 == 3:
        vals[: n // 2] = 0.0                         # a block of exact zeros
    srt = np.sort(vals)
    for p in PROBS + (0.0, 0.25, 0.75, 1.0):
        got = oracle.quantile_linear(srt, p)
        ref = float(np.quantile(vals, p))
        assert got == ref, (n, p, got, ref)
        assert float(np.percentile(vals, 100 * p)) == pytest.approx(got, rel=1e-15, abs=0)


def test_hand_worked_lists():
    v = np.array([0.0, 1.0, 2.0, 3.0])               # h = 3p
    assert oracle.quantile_linear(v, 0.5) == 1.5
    assert abs(oracle.quantile_linear(v, 0.95) - 2.85) < 1e-15
    assert abs(oracle.quantile_linear(v, 0.99) - 2.97) < 1e-15
    v5 = np.array([10.0, 20.0, 30.0, 40.0, 50.0])    # h = 4p: 2, 3.8, 3.96
    assert oracle.quantile_linear(v5, 0.5) == 30.0
    assert abs(oracle.quantile_linear(v5, 0.95) - 48.0) < 1e-12
    assert abs(oracle.quantile_linear(v5, 0.99) - 49.6) < 1e-12
    v20 = np.arange(20.0)                             # h = 19p: 9.5, 18.05, 18.81
    assert oracle.quantile_linear(v20, 0.5) == 9.5
    assert abs(oracle.quantile_linear(v20, 0.95) - 18.05) < 1e-12
    assert abs(oracle.quantile_linear(v20, 0.99) - 18.81) < 1e-12
    assert oracle.quantile_linear(np.zeros(0), 0.5) == 0.0


def test_one_and_two_tokens():
    # The blog: with one active token every percentile equals its |Delta|.
    for x in (0.0, 2.0 ** -23, 0.017098, 5.5):
        for p in PROBS:
            assert oracle.quantile_linear(np.array([x]), p) == x
    # Two values: the straight line between them, q_p = a + p (b - a).
    a, b = 0.25, 1.75
    for p in PROBS:
        assert abs(oracle.quantile_linear(np.array([a, b]), p) - (a + p * (b - a))) < 1e-15


def test_quantile_is_monotone_and_bounded():
    rng = np.random.default_rng(11)
    srt = np.sort(np.abs(rng.standard_normal(333)))
    qs = [oracle.quantile_linear(srt, p) for p in np.linspace(0, 1, 101)]
    assert all(x <= y for x, y in zip(qs, qs[1:]))
    assert qs[0] == srt[0] and qs[-1] == srt[-1]


def test_identical_scores_closed_form():
    c = synth.compare_case(N=5, max_resp=200, prompt=16, seed=3)
    t, pos_sum, pos_count = oracle.tails(c.A, c.B, c.B.copy(), c.mask)
    n_active = int((c.mask != 0).sum())
    first = np.argwhere(c.mask != 0)[0]
    for p in ("AB", "BC", "AC"):
        r = t[p]
        assert r["count"] == n_active
        assert r["q50"] == r["q95"] == r["q99"] == r["max_abs"] == 0.0
        assert (r["max_seq"], r["max_pos"]) == (int(first[0]), int(first[1]))
        assert r["sum_abs"] == 0.0 and r["sum_prob_abs"] == 0.0
    assert np.all(pos_sum == 0.0) and pos_count.sum() == 3 * n_active


def test_offset_closed_form():
    # [AMD] Case 1: A = B - 0.10 on every active token except each sequence's
    # first; |A - B| is then 0 on N tokens and one rounded offset elsewhere.
    c = synth.compare_case(N=6, max_resp=300, prompt=16, seed=4)
    A = c.B.copy()
    act = c.mask != 0
    first_cols = act.argmax(axis=1)
    for n in range(6):
        row = act[n].copy(); row[first_cols[n]] = False
        A[n, row] = (A[n, row].astype(np.float64) - 0.10).astype(np.float32)
    t, _, _ = oracle.tails(A, c.B, c.B, c.mask)
    d = np.abs(A.astype(np.float64) - c.B.astype(np.float64))[act]
    n = d.size
    srt = np.sort(d)
    assert t["AB"]["count"] == n and np.count_nonzero(srt == 0) == 6
    # Six zeros then n - 6 tokens at 0.10 rounded through fp32 scores: every
    # quantile's two neighbours lie among the offsets (h = (n - 1) p >= 6), so
    # each quantile lies within the offsets' range, one fp32 rounding of 0.10.
    offs = np.unique(srt[6:])
    assert np.all(np.abs(offs - 0.10) < 4e-6)
    for name, p in zip(("q50", "q95", "q99"), PROBS):
        j = math.floor((n - 1) * p)
        assert j >= 6
        assert offs[0] <= t["AB"][name] <= offs[-1]
        assert t["AB"][name] == float(np.quantile(d, p))
    assert t["BC"]["max_abs"] == 0.0 and t["AC"]["max_abs"] == t["AB"]["max_abs"]


def test_probability_difference_of_the_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ratio_example.json")))
    pa, pb = g["rollout_probability"], g["trainer_probability"]
    A = np.array([[np.float32(math.log(pa))]], np.float32)
    B = np.array([[np.float32(math.log(pb))]], np.float32)
    t, _, _ = oracle.tails(A, B, B, np.ones((1, 1), np.uint8))
    assert abs(t["AB"]["sum_prob_abs"] - abs(pa - pb)) < 1e-7
    assert abs(t["AB"]["sum_abs"] - abs(math.log(pa) - math.log(pb))) < 1e-6


def test_first_occurrence_of_the_maximum_and_nonfinite_tokens():
    A = np.zeros((3, 5), np.float32)
    B = np.zeros((3, 5), np.float32)
    mask = np.ones((3, 5), np.uint8)
    A[1, 3] = -2.0; A[2, 0] = -2.0; A[0, 4] = -1.0
    A[0, 1] = np.nan; mask[2, 2] = 0; A[2, 2] = -9.0   # non-finite / masked: not counted
    t, pos_sum, pos_count = oracle.tails(A, B, B, mask)
    r = t["AB"]
    assert (r["max_abs"], r["max_seq"], r["max_pos"]) == (2.0, 1, 3)
    assert r["count"] == 13
    assert pos_count[0].tolist() == [3, 2, 2, 3, 3] and pos_sum[0, 4] == 1.0


def test_position_profile_adds_up():
    c = synth.compare_case(N=7, max_resp=250, prompt=8, seed=9)
    C = synth.noise_scores(c.C, c.mask, 1e-3, seed=9)
    t, pos_sum, pos_count = oracle.tails(c.A, c.B, C, c.mask)
    for p, name in enumerate(("AB", "BC", "AC")):
        assert pos_count[p].sum() == t[name]["count"]
        assert abs(math.fsum(pos_sum[p].tolist()) - t[name]["sum_abs"]) <= 1e-12 * max(1.0, t[name]["sum_abs"])


# ---------------------------------------------------------------------------
# Worst tokens: pinned to a brute force with Python's own tuple ordering,
# to the maximum and its position, to the order statistics, and to planted
# ties that only the row-major rule orders.
# ---------------------------------------------------------------------------

def brute_worst(A, B, C, mask, k):
    sides = {"A": A, "B": B, "C": C}
    out = {}
    for ln, rn in oracle.PAIRS:
        items = []
        for n in range(A.shape[0]):
            for i in range(A.shape[1]):
                l, r = float(sides[ln][n, i]), float(sides[rn][n, i])
                if mask[n, i] and math.isfinite(l) and math.isfinite(r):
                    items.append((-abs(l - r), n, i))
        items.sort()
        out[ln + rn] = [(-d, n, i) for d, n, i in items[:k]]
    return out


@pytest.mark.parametrize("seed", range(4))
def test_worst_tokens_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    N, L = int(rng.integers(1, 6)), int(rng.integers(1, 40))
    A = rng.standard_normal((N, L)).astype(np.float32)
    B = (A + rng.integers(-3, 4, (N, L)) * 0.25).astype(np.float32)   # many equal |Delta|
    C = (B + 1e-3 * rng.standard_normal((N, L))).astype(np.float32)
    mask = (rng.random((N, L)) < 0.8).astype(np.uint8)
    C[0, 0] = np.nan
    for k in (0, 1, 5, N * L + 3):
        got = oracle.worst_tokens(A, B, C, mask, k)
        assert got == brute_worst(A, B, C, mask, k)


def test_worst_one_is_the_tail_maximum():
    r = synth.compare_case(N=6, max_resp=300, prompt=16, seed=8)
    C = synth.noise_scores(r.C, r.mask, 1e-3, seed=8)
    tails, _, _ = oracle.tails(r.A, r.B, C, r.mask)
    worst = oracle.worst_tokens(r.A, r.B, C, r.mask, 1)
    for p in ("AB", "BC", "AC"):
        t = tails[p]
        if t["count"]:
            assert worst[p] == [(t["max_abs"], t["max_seq"], t["max_pos"])]
        else:
            assert worst[p] == []


def test_worst_values_are_the_top_order_statistics():
    r = synth.compare_case(N=5, max_resp=200, prompt=16, seed=9)
    C = synth.noise_scores(r.C, r.mask, 1e-2, seed=9)
    k = 37
    worst = oracle.worst_tokens(r.A, r.B, C, r.mask, k)["BC"]
    d = np.abs(r.B.astype(np.float64) - C.astype(np.float64))[r.mask != 0]
    top = np.sort(d)[::-1][:k]
    assert [w[0] for w in worst] == top.tolist()


def test_worst_ties_follow_row_major_order():
    N, L = 3, 5
    A = np.zeros((N, L), np.float32)
    B = np.zeros((N, L), np.float32)
    B[2, 1] = B[0, 3] = B[1, 0] = B[0, 1] = 0.5     # four equal |Delta|
    B[1, 4] = 0.75
    mask = np.ones((N, L), np.uint8)
    w = oracle.worst_tokens(A, B, B.copy(), mask, 4)["AB"]
    assert w == [(0.75, 1, 4), (0.5, 0, 1), (0.5, 0, 3), (0.5, 1, 0)]
    assert oracle.worst_tokens(A, B, B.copy(), mask, 40)["BC"][:2] == [(0.0, 0, 0), (0.0, 0, 1)]


# ---------------------------------------------------------------------------
# Per-sequence quantiles: the blog's compare() on one record's arrays.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_seq_quantiles_are_np_quantile_per_record(seed):
    r = synth.compare_case(N=6, max_resp=300, prompt=16, seed=20 + seed)
    C = synth.noise_scores(r.C, r.mask, 1e-3, seed=seed)
    A = r.A.copy()
    A[1, 20] = np.nan                                  # not counted
    mask = r.mask.copy()
    mask[2, 16:40] = 0                                 # a hole in the record
    q = oracle.seq_quantiles(A, r.B, C, mask)
    sides = {"A": A, "B": r.B, "C": C}
    for ln, rn in oracle.PAIRS:
        for n in range(A.shape[0]):
            left = sides[ln][n].astype(np.float64)
            right = sides[rn][n].astype(np.float64)
            keep = (mask[n] != 0) & np.isfinite(left) & np.isfinite(right)
            err = np.abs(left[keep] - right[keep])
            want = [float(np.quantile(err, p)) for p in PROBS] if err.size else [0.0] * 3
            assert q[ln + rn][n].tolist() == want, (ln + rn, n)


def test_seq_quantiles_worked_token(golden_dir):
    # One active token (the blog's outlier): p50 = p95 = p99 = |A - B0|.
    g = json.load(open(os.path.join(golden_dir, "amd_worked_token.json")))["scores"]
    A = np.array([[np.float32(g["A"]), 0.0]], np.float32)
    B = np.array([[np.float32(g["B0"]), 5.0]], np.float32)
    mask = np.array([[1, 0]], np.uint8)
    q = oracle.seq_quantiles(A, B, B, mask)["AB"][0]
    d = abs(float(np.float32(g["A"])) - float(np.float32(g["B0"])))
    assert q.tolist() == [d, d, d] and f"{d:.6f}" == "0.017098"
    q0 = oracle.seq_quantiles(A, B, B, np.zeros((1, 2), np.uint8))["AB"][0]
    assert q0.tolist() == [0.0, 0.0, 0.0]


def test_batch_quantiles_pool_the_records():
    # The batch quantile is the quantile of all records' counted tokens
    # together, not a mean of per-record quantiles.
    r = synth.compare_case(N=5, max_resp=200, prompt=8, seed=31)
    C = synth.noise_scores(r.C, r.mask, 1e-2, seed=31)
    t, _, _ = oracle.tails(r.A, r.B, C, r.mask)
    d = np.abs(r.B.astype(np.float64) - C.astype(np.float64))[r.mask != 0]
    for name, p in zip(("q50", "q95", "q99"), PROBS):
        assert t["BC"][name] == float(np.quantile(d, p))
