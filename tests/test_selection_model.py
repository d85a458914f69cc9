"""A CPU model of the per-sequence quantile selection that
seq_quantile_wave_kernel performs (quantile.hip), checked against sorting.

The kernel selects the order statistics of the fp64 |left - right| keys in
three steps: a 4 096-bucket histogram of the keys' top 16 bits (the key 0, and
the keys below 1.125 * 2^-126 together, in buckets of their own), 12-bit
refinement of any range holding more than 64 keys, and counting inside the
remaining small ranges.
This model takes the same steps with the same constants and bucket bounds, so
that a flaw in the design (a bucket bound, a digit mask, a range clip, a rank
carried across a refinement) shows up here on the CPU, independently of the
GPU tests that compare the kernel itself with the oracle.
"""

import numpy as np
import pytest

NOKEY = (1 << 64) - 1
TOP_HI = (1152 << 4) | 15          # top 16 bits of the largest |delta| (< 2^130)
BINS = 4096
WLO = TOP_HI - (BINS - 3)          # top-16 value of bucket 2
GROUP = 64


def bucket(k):
    t = k >> 48
    return 0 if k == 0 else (1 if t < WLO else t - WLO + 2)


def find(hist, r):
    """Bin holding the r-th counted key (1-based), keys below it, keys in it."""
    c = np.cumsum(hist)
    b = int(np.searchsorted(c, r))
    return b, int(c[b] - hist[b]), int(hist[b])


def ranks(n, p):
    h = (n - 1) * p
    if h >= n - 1:
        return n, n
    j = int(np.floor(h))
    return j + 1, j + 2


def select(keys):
    """The six order statistics (lo / hi ranks of p50, p95, p99) as the
    kernel finds them; None when no key is counted."""
    keys = [int(k) for k in keys if int(k) != NOKEY]
    if not keys:
        return None
    hist = np.zeros(BINS, np.int64)
    for k in keys:
        hist[bucket(k)] += 1
    n = len(keys)
    tg = []
    for t in range(6):
        r = ranks(n, (0.5, 0.95, 0.99)[t >> 1])[t & 1]
        b, below, cnt = find(hist, r)
        if b == 0:
            tg.append(dict(lo=0, hi=0, sh=0, r=r - below, m=cnt))
        elif b == 1:
            tg.append(dict(lo=1, hi=WLO << 48, sh=64, r=r - below, m=cnt))
        else:
            top = b - 2 + WLO
            tg.append(dict(lo=top << 48, hi=(top + 1) << 48, sh=48, r=r - below, m=cnt))
    # Refinement: 12 bits below the range's common prefix per pass.
    for _ in range(6 * 6):
        open_big = [t for t in tg if t["sh"] and t["m"] > GROUP]
        if not open_big:
            break
        lo, hi, sh = open_big[0]["lo"], open_big[0]["hi"], open_big[0]["sh"]
        ds = sh - 12 if sh > 12 else 0
        mask = (1 << (sh - ds)) - 1
        base = 0 if sh >= 64 else (lo >> sh) << sh
        h2 = np.zeros(BINS, np.int64)
        for k in keys:
            if lo <= k < hi:
                h2[(k >> ds) & mask] += 1
        for t in tg:
            if t["sh"] and t["lo"] == lo and t["hi"] == hi:
                b, below, cnt = find(h2, t["r"])
                sub = base + (b << ds)
                t.update(lo=max(sub, lo), hi=min(sub + (1 << ds), hi), sh=ds,
                         r=t["r"] - below, m=cnt)
    else:
        raise AssertionError("refinement did not finish")
    # Counting inside each remaining range.
    out = []
    for t in tg:
        if t["sh"] == 0:
            out.append(t["lo"])
            continue
        grp = [k for k in keys if t["lo"] <= k < t["hi"]]
        assert len(grp) == t["m"] <= GROUP
        hit = [c for c in grp if sum(x < c for x in grp) < t["r"] <= sum(x <= c for x in grp)]
        out.append(hit[0])
    return n, out


def keys_of(left, right, active):
    d = left.astype(np.float64) - right.astype(np.float64)
    k = np.abs(d).view(np.uint64).copy()
    k[~(active & np.isfinite(d))] = NOKEY
    return k


def rows(kind, L, rng):
    r = rng.standard_normal(L).astype(np.float32)
    if kind == "noise":
        left = (r + rng.standard_normal(L).astype(np.float32) * np.float32(1e-3)).astype(np.float32)
    elif kind == "offset":
        left = (r + np.float32(0.01)).astype(np.float32)
    elif kind == "zeros":
        left = r.copy()
        left[rng.random(L) < 0.3] += np.float32(1e-3)
    elif kind == "ulp":
        left = (r * np.float32(1 + 1e-7)).astype(np.float32)
    elif kind == "tiny":
        r = (rng.standard_normal(L) * 1e-38).astype(np.float32)
        left = (r + np.float32(1e-44) * rng.integers(0, 50, L)).astype(np.float32)
    elif kind == "equal":
        r = np.zeros(L, np.float32)
        left = np.full(L, np.float32(0.3))
    else:
        scale = np.float32(10) ** rng.integers(-30, 3, L).astype(np.float32)
        left = (r + rng.standard_normal(L).astype(np.float32) * scale).astype(np.float32)
        left[rng.random(L) < 0.05] = np.nan
        r[rng.random(L) < 0.02] = np.inf
    return left, r


def test_bucket_bounds():
    # The smallest non-zero |delta| of two fp32 values (2^-149) and anything
    # below 1.125 * 2^-126 (top 16 bits under WLO: exponent and four mantissa
    # bits) share bucket 1; 1.125 * 2^-126 starts bucket 2; the largest
    # difference, 2 FLT_MAX < 2^129, lands in bucket 4 079 (the bound 2^130
    # leaves the top 16 buckets unused); buckets are monotone.
    as_key = lambda x: int(np.array([x], np.float64).view(np.uint64)[0])
    assert bucket(as_key(2.0 ** -149)) == 1
    assert bucket(as_key(2.0 ** -126)) == 1
    assert bucket(as_key(1.125 * 2.0 ** -126 * (1 - 2.0 ** -52))) == 1
    assert bucket(as_key(1.125 * 2.0 ** -126)) == 2
    fmax = float(np.finfo(np.float32).max)
    assert bucket(as_key(2 * fmax)) == 4079 < BINS
    xs = np.sort(np.abs(np.random.default_rng(5).standard_normal(2000)) * 10.0 ** np.arange(-40, 40, 0.04))
    bs = [bucket(as_key(x)) for x in xs]
    assert bs == sorted(bs)


KINDS = ["noise", "offset", "zeros", "ulp", "tiny", "equal", "mixed"]


@pytest.mark.parametrize("kind", KINDS)
def test_selection_model_matches_sorting(kind):
    rng = np.random.default_rng(100 + KINDS.index(kind))
    for L in (1, 7, 300, 769, 2304):
        left, right = rows(kind, L, rng)
        active = rng.random(L) < rng.uniform(0.05, 1.0)
        k = keys_of(left, right, active)
        got = select(k)
        srt = np.sort(k[k != NOKEY])
        if got is None:
            assert srt.size == 0
            continue
        n, vals = got
        assert n == srt.size
        for t in range(6):
            r = ranks(n, (0.5, 0.95, 0.99)[t >> 1])[t & 1]
            assert vals[t] == int(srt[r - 1]), (kind, L, t)
