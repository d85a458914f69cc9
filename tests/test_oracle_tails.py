"""Pins for the oracle's batch tail statistics (CPU only): the nearest-rank
quantile against numpy's inverted-CDF percentile, hand-counted ranks, closed
forms for identical and offset scores, the probability difference of the
AMD blog's worked example, first-occurrence maxima and position profiles that
add up to the batch totals."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import synth


@pytest.mark.parametrize("seed", range(6))
def test_nearest_rank_is_the_inverted_cdf_percentile(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    vals = np.sort(np.abs(rng.standard_normal(n)) * 10.0 ** rng.integers(-6, 2, n))
    if seed % 2:
        vals = np.sort(np.round(vals, 1))            # many ties
    for pct in (50, 95, 99):
        assert oracle.nearest_rank(vals, pct) == np.percentile(vals, pct, method="inverted_cdf")


def test_hand_counted_ranks():
    v = np.array([0.0, 1.0, 2.0, 3.0])
    assert oracle.nearest_rank(v, 50) == 1.0          # rank ceil(2)   = 2
    assert oracle.nearest_rank(v, 95) == 3.0          # rank ceil(3.8) = 4
    v20 = np.arange(20.0)
    assert oracle.nearest_rank(v20, 95) == 18.0       # rank 95*20/100 = 19 exactly
    assert oracle.nearest_rank(v20, 99) == 19.0       # rank ceil(19.8) = 20
    assert oracle.nearest_rank(np.zeros(0), 50) == 0.0


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
    for pct in (50, 95, 99):
        rank = -(-pct * n // 100)
        assert t["AB"][f"q{pct}"] == srt[rank - 1] and srt[rank - 1] > 0.09
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
