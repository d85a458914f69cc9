"""Pins for the three-way comparison oracle (CPU only).

Sources of truth other than the oracle itself: values the pages print, the
closed forms of the injected faults, identities the definitions imply, and a
token-by-token brute-force recount on tiny inputs.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import synth

f32 = np.float32


def one_token(left, right, **kw):
    a = np.array([[left]], f32)
    b = np.array([[right]], f32)
    return oracle.compare(a, b, b, np.ones((1, 1), np.uint8), **kw)["AB"]


def test_blog_worked_token(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "amd_worked_token.json")))
    s = g["scores"]
    for k in ("B0", "B1", "C0", "C1"):          # printed fp32 values
        assert float(f32(s[k])) == s[k]
    v = {k: f32(x) for k, x in s.items()}       # A is rounded to fp32 here
    pairs = {"A-B0": ("A", "B0"), "B0-C0": ("B0", "C0"), "A-C0": ("A", "C0"),
             "B0-B1": ("B0", "B1"), "B1-C0": ("B1", "C0"), "C0-C1": ("C0", "C1")}
    for label, (l, r) in pairs.items():
        st = one_token(v[l], v[r])
        n = st["valid"][0]
        assert f"{st['sum_signed'][0] / n:+.6f}" == g["printed_differences"][label]["signed"]
        assert f"{st['sum_abs'][0] / n:.6f}" == g["printed_differences"][label]["mae"]
    # "A displayed zero need not be exact zero": B1 and C0 are one fp32 ulp
    # apart, so the bitwise comparison counts a mismatch.
    st = one_token(v["B1"], v["C0"])
    assert st["mismatch"][0] == 1 and st["first_div"][0] == 0
    assert st["max_abs"][0] == 2.0 ** -23
    st = one_token(v["C0"], v["C1"])
    assert st["mismatch"][0] == 0 and st["max_abs"][0] == 0.0


def test_blog_ratio_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ratio_example.json")))
    lr, lt = f32(math.log(g["rollout_probability"])), f32(math.log(g["trainer_probability"]))
    p = g["printed"]
    assert round(float(lr), 4) == p["rollout_logprob"]
    assert round(float(lt), 4) == p["trainer_logprob"]
    st = one_token(lr, lt)          # left = rollout, right = trainer
    assert round(st["sum_d"][0], 4) == p["trainer_minus_rollout"]
    assert round(st["sum_tok_tis"][0], 2) == p["probability_ratio"]
    r = g["trainer_probability"] / g["rollout_probability"]
    assert abs(st["sum_k3"][0] - (r - 1 - math.log(r))) < 1e-6   # k3 = r - 1 - ln r
    assert abs(st["seq_tis"][0] - r) < 1e-6
    st = one_token(lr, lt, tis_clip=1.1)                             # clipped
    assert st["sum_tok_tis"][0] == 1.1 and st["seq_tis"][0] == 1.1


def test_eq1_log_ratio_split(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "eq1_split.json")))
    q, pv, pk = (g[k] for k in ("rollout_probability_q_v", "trainer_same_version_p_v",
                                "trainer_current_p_k"))
    A = np.array([[math.log(q)]], f32)
    B = np.array([[math.log(pv)]], f32)
    C = np.array([[math.log(pk)]], f32)
    res = oracle.compare(A, B, C, np.ones((1, 1), np.uint8), tis_clip=10.0)
    w, r = g["printed"]["correction_w"], g["printed"]["movement_r"]
    assert abs(res["AB"]["sum_tok_tis"][0] - w) < 1e-6       # same-version term
    assert abs(res["BC"]["sum_tok_tis"][0] - r) < 1e-6       # weight movement
    # Eq. (1): log(p_k/q_v) = log(p_k/p_v) + log(p_v/q_v), exactly per token.
    assert res["AC"]["sum_d"][0] == res["AB"]["sum_d"][0] + res["BC"]["sum_d"][0]
    assert abs(res["AC"]["sum_d"][0] - math.log(pk / q)) < 1e-6


@pytest.fixture(scope="module")
def record():
    return synth.compare_case(N=8, max_resp=2048, prompt=256, seed=0)


def test_identical_arrays(record):
    res = oracle.compare(record.A, record.B, record.B, record.mask)
    for p in ("AB", "BC", "AC"):
        s = res[p]
        assert np.array_equal(s["valid"], record.resp_len)
        assert not s["mismatch"].any() and not s["longest_run"].any()
        assert np.all(s["first_div"] == -1)
        assert not s["max_abs"].any() and not s["sum_k3"].any()
        assert np.array_equal(s["sum_tok_tis"], record.resp_len.astype(float))
        assert np.all(s["seq_tis"] == 1.0)


def test_case1_offset_on_a(record):
    # Blog Case 1: 0.10 nat subtracted from stored A at response positions >= 1.
    A = synth.offset_scores(record.A, record.mask, 0.10, first_pos=1)
    s = oracle.compare(A, record.B, record.C, record.mask)["AB"]
    n = record.resp_len
    has2 = n >= 2
    assert np.array_equal(s["first_div"], np.where(has2, 1, -1))
    assert np.array_equal(s["mismatch"], n - 1)
    assert np.array_equal(s["longest_run"], n - 1)
    assert np.all(np.abs(s["max_abs"][has2] - 0.10) < 1e-6)
    assert np.all(np.abs(s["sum_signed"] + 0.10 * (n - 1)) < 1e-6 * n)   # A - B = -0.10
    # B-C is untouched by a fault in A.
    assert not oracle.compare(A, record.B, record.C, record.mask)["BC"]["mismatch"].any()


def test_case2_offset_on_c(record):
    # Blog Case 2: 0.10 nat subtracted from every frozen trainer score.
    C = synth.offset_scores(record.C, record.mask, 0.10)
    res = oracle.compare(record.A, record.B, C, record.mask)
    for p in ("BC", "AC"):
        s = res[p]
        assert np.all(s["first_div"] == 0)
        assert np.array_equal(s["mismatch"], record.resp_len)
        assert np.array_equal(s["longest_run"], record.resp_len)
        assert np.all(np.abs(s["sum_d"] + 0.10 * record.resp_len) < 1e-5)
    assert not res["AB"]["mismatch"].any()


def test_masked_positions_do_not_matter(record):
    base = oracle.compare(record.A, record.B, record.C, record.mask)
    A, B, C = record.A.copy(), record.B.copy(), record.C.copy()
    out = record.mask == 0
    A[out], B[out], C[out] = np.inf, -7.0, np.nan
    again = oracle.compare(A, B, C, record.mask)
    for p in base:
        for f in oracle.STAT_FIELDS:
            assert np.array_equal(base[p][f], again[p][f]), (p, f)


def test_additivity_of_signed_sums(record):
    # Per token A-C = (A-B) + (B-C), so the signed sums add (the MAEs do not).
    A = synth.noise_scores(record.A, record.mask, 1e-3, seed=1)
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=2)
    res = oracle.compare(A, record.B, C, record.mask)
    lhs = res["AC"]["sum_signed"]
    rhs = res["AB"]["sum_signed"] + res["BC"]["sum_signed"]
    assert np.all(np.abs(lhs - rhs) <= 1e-15 * np.maximum(1, np.abs(lhs)) * 4)
    assert np.all(res["AC"]["sum_abs"] <= res["AB"]["sum_abs"] + res["BC"]["sum_abs"] + 1e-12)


def test_signed_zero_nan_inf_and_k3_overflow():
    s = one_token(f32(0.0), f32(-0.0))
    assert s["mismatch"][0] == 1 and s["max_abs"][0] == 0.0 and s["nonfinite"][0] == 0
    nan = np.array([np.nan], f32)
    s = one_token(nan[0], nan[0])               # same NaN bits: bitwise equal
    assert s["mismatch"][0] == 0 and s["nonfinite"][0] == 1
    s = one_token(f32(np.inf), f32(-1.0))
    assert s["mismatch"][0] == 1 and s["nonfinite"][0] == 1 and s["max_abs"][0] == 0.0
    s = one_token(f32(-1000.0), f32(0.0))        # d = 1000: k3 overflows
    assert s["k3_nonfinite"][0] == 1 and s["sum_k3"][0] == 0.0
    assert s["sum_tok_tis"][0] == 2.0 and s["seq_tis"][0] == 2.0
    assert s["max_abs"][0] == 1000.0


def test_atol_mode():
    a = np.array([[-1.0, -2.0, -3.0, 0.0]], f32)
    b = np.array([[-1.0, -2.0005, -3.1, -0.0]], f32)
    m = np.ones_like(a, np.uint8)
    s = oracle.compare(a, b, b, m, atol=1e-3)["AB"]
    assert s["mismatch"][0] == 1 and s["first_div"][0] == 2
    s = oracle.compare(a, b, b, m)["AB"]
    assert s["mismatch"][0] == 3 and s["first_div"][0] == 1 and s["longest_run"][0] == 3


def _brute(left, right, mask, C, atol):
    """Token-by-token recount written directly from the definitions."""
    valid = mism = run = best = nonf = k3n = 0
    first = -1
    mx = sa = ss = sk = sd = st = 0.0
    k = 0
    for i in range(len(mask)):
        if not mask[i]:
            continue
        lv, rv = float(left[i]), float(right[i])
        bl = int(np.array(left[i], f32).view(np.uint32))
        br = int(np.array(right[i], f32).view(np.uint32))
        differ = bl != br
        if differ and atol is not None and abs(lv - rv) <= atol:
            differ = False
        if differ:
            mism += 1
            if first < 0:
                first = k
            run += 1
            best = max(best, run)
        else:
            run = 0
        if math.isfinite(lv) and math.isfinite(rv):
            dl = lv - rv
            mx = max(mx, abs(dl))
            sa += abs(dl)
            ss += dl
            d = rv - lv
            try:
                k3 = math.expm1(d) - d
            except OverflowError:
                k3 = math.inf
            if math.isfinite(k3):
                sk += k3
            else:
                k3n += 1
            sd += d
            st += C if d >= math.log(C) + 1e-12 else min(math.exp(d), C)
        else:
            nonf += 1
        valid += 1
        k += 1
    seq = C if sd > 700 else min(math.exp(sd), C)
    return dict(valid=valid, mismatch=mism, first_div=first, longest_run=best,
                nonfinite=nonf, k3_nonfinite=k3n, max_abs=mx, sum_abs=sa,
                sum_signed=ss, sum_k3=sk, sum_d=sd, seq_tis=seq, sum_tok_tis=st)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_recount(seed):
    rng = np.random.default_rng(100 + seed)
    N, L = 5, int(rng.integers(1, 40))
    B = np.log(1.0 - rng.random((N, L))).astype(f32)
    A = B.copy()
    C = B.copy()
    # sprinkle faults: value changes, +-0, NaN, inf, large d
    for arr in (A, C):
        sel = rng.random((N, L)) < 0.3
        arr[sel] = (arr[sel] + rng.normal(0, 0.05, sel.sum())).astype(f32)
    A[0, 0] = 0.0; B[0, 0] = -0.0
    if L > 2:
        C[1, 1] = np.nan; A[2, 2] = np.inf; C[3, 2] = -200.0
    mask = (rng.random((N, L)) < 0.7).astype(np.uint8)
    mask[4] = 0                                  # an empty sequence
    atol = None if seed % 2 == 0 else 0.02
    res = oracle.compare(A, B, C, mask, tis_clip=2.0, atol=atol)
    arr = {"A": A, "B": B, "C": C}
    for (l, r) in oracle.PAIRS:
        for n in range(N):
            exp = _brute(arr[l][n], arr[r][n], mask[n], 2.0, atol)
            for f, v in exp.items():
                got = res[l + r][f][n]
                if isinstance(v, int):
                    assert got == v, (l + r, n, f)
                else:
                    assert abs(got - v) <= 1e-12 * max(1.0, abs(v)), (l + r, n, f, got, v)


def test_per_token_layout(record):
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=3)
    pt = oracle.per_token(record.A, record.B, C, record.mask)
    assert pt.shape == (3, 3, record.N, record.L) and pt.dtype == np.float32
    act = record.mask != 0
    assert not pt[:, :, ~act].any()
    res = oracle.compare(record.A, record.B, C, record.mask)
    for p, name in enumerate(("AB", "BC", "AC")):
        for n in range(record.N):
            row = pt[p, 0, n][act[n]].astype(np.float64)
            assert abs(row.max(initial=0.0) - res[name]["max_abs"][n]) <= 1e-7 * max(1, res[name]["max_abs"][n])
            assert abs(row.sum() - res[name]["sum_abs"][n]) <= 1e-5 * max(1, res[name]["sum_abs"][n])


def _brute_token(left: float, right: float, clip: float):
    """One token's per-token values in Python floats, from the definitions:
    |left - right|, k3 = expm1(d) - d and min(e^d, C) with d = right - left."""
    d = right - left
    k3 = math.expm1(d) - d if d < 709.0 else math.inf
    tis = clip if d >= math.log(clip) else min(math.exp(d), clip)
    return abs(left - right), k3, tis


@pytest.mark.parametrize("seed", range(3))
def test_per_token_columns_brute_force(seed):
    # Every column of every pair against a token-by-token recount: catches a
    # flipped d, swapped columns, a missing clip or a k3 without its -d.
    rng = np.random.default_rng(40 + seed)
    N, L = 4, 33
    B = rng.uniform(-12, 0, (N, L)).astype(f32)
    A = (B + rng.normal(0, 0.3, (N, L))).astype(f32)
    C = (B + rng.normal(0, 0.8, (N, L))).astype(f32)
    A[0, 3] = B[0, 3] + 2.5                       # |d| >= ln 2: the clip decides
    C[1, 4] = np.nan
    mask = (rng.random((N, L)) < 0.75).astype(np.uint8)
    clip = 2.0 if seed != 2 else 1.25
    pt = oracle.per_token(A, B, C, mask, tis_clip=clip)
    arr = {"A": A, "B": B, "C": C}
    for p, (ln, rn) in enumerate(oracle.PAIRS):
        for n in range(N):
            for i in range(L):
                l, r = float(arr[ln][n, i]), float(arr[rn][n, i])
                got = pt[p, :, n, i]
                if not mask[n, i]:
                    assert got.tolist() == [0.0, 0.0, 0.0]
                elif not (math.isfinite(l) and math.isfinite(r)):
                    assert np.isnan(got).all()
                else:
                    want = np.array(_brute_token(l, r, clip), np.float64).astype(f32)
                    assert got.tolist() == want.tolist(), (ln + rn, n, i, got, want)


def test_per_token_ratio_example(golden_dir):
    # [AMD] "What a Logprob Difference Means": 0.10 -> 0.12 is a ratio of 1.2;
    # left = rollout, right = trainer, so k3 = r - 1 - ln r and TIS = r.
    g = json.load(open(os.path.join(golden_dir, "ratio_example.json")))
    lr = f32(math.log(g["rollout_probability"]))
    lt = f32(math.log(g["trainer_probability"]))
    a = np.array([[lr]], f32)
    b = np.array([[lt]], f32)
    pt = oracle.per_token(a, b, b, np.ones((1, 1), np.uint8))
    r = g["trainer_probability"] / g["rollout_probability"]
    assert abs(float(pt[0, 0, 0, 0]) - math.log(r)) < 1e-6
    assert abs(float(pt[0, 1, 0, 0]) - (r - 1 - math.log(r))) < 1e-7   # 0.01768, not 0.01565
    assert abs(float(pt[0, 2, 0, 0]) - r) < 1e-6
    assert round(float(pt[0, 2, 0, 0]), 2) == g["printed"]["probability_ratio"]
    # The reverse orientation gives the other k3 (1/r - 1 + ln r): not this.
    assert abs(float(pt[0, 1, 0, 0]) - (1 / r - 1 + math.log(r))) > 1e-3


def test_per_token_overflow_and_clip_closed_forms():
    # d = +100: e^d overflows fp32, k3 = e^100 - 101 -> inf in fp32, TIS = C.
    # d = -100: k3 = e^-100 + 99 -> 99.0 exactly in fp32, TIS = e^-100 (a
    # subnormal fp32). d = ln 3 > ln 2: TIS = 2 exactly, k3 = 2 - ln 3.
    left = np.array([[0.0, 0.0, 0.0]], f32)
    right = np.array([[100.0, -100.0, f32(math.log(3.0))]], f32)
    pt = oracle.per_token(left, right, right, np.ones((1, 3), np.uint8))
    k3, tis = pt[0, 1, 0], pt[0, 2, 0]
    assert np.isinf(k3[0]) and k3[0] > 0 and tis[0] == 2.0
    assert k3[1] == 99.0 and tis[1] == f32(math.exp(-100.0)) and tis[1] > 0
    d = float(f32(math.log(3.0)))
    assert tis[2] == 2.0 and abs(float(k3[2]) - (math.exp(d) - 1 - d)) < 1e-6


def test_per_token_sums_match_compare(record):
    # per_token() and compare() are written apart: their k3 and TIS agree.
    C = synth.noise_scores(record.C, record.mask, 1e-2, seed=5)
    pt = oracle.per_token(record.A, record.B, C, record.mask)
    res = oracle.compare(record.A, record.B, C, record.mask)
    act = record.mask != 0
    for p, name in enumerate(("AB", "BC", "AC")):
        for n in range(record.N):
            k3 = pt[p, 1, n][act[n]].astype(np.float64)
            tis = pt[p, 2, n][act[n]].astype(np.float64)
            assert abs(math.fsum(k3) - res[name]["sum_k3"][n]) <= 1e-6 * max(1e-9, res[name]["sum_k3"][n]) + 1e-12
            assert abs(math.fsum(tis) - res[name]["sum_tok_tis"][n]) <= 1e-6 * max(1.0, res[name]["sum_tok_tis"][n])


def test_rejects_bad_arguments():
    a = np.zeros((2, 3), f32)
    with pytest.raises(ValueError):
        oracle.compare(a, a, a[:, :2], np.ones((2, 3), np.uint8))
    with pytest.raises(ValueError):
        oracle.compare(a.astype(np.float64), a, a, np.ones((2, 3), np.uint8))
    with pytest.raises(ValueError):
        oracle.compare(a, a, a, np.ones((2, 3), np.uint8), tis_clip=0.0)
