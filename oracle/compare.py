"""Three-way comparison of generation (A), replay (B) and trainer (C) scores:
the plain per-sequence definition.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Not used by the library.

Pairs and orientation
  [AMD] §"Check Whether the Pattern Extends": differences are taken left minus
        right in the order A-B, B-C, A-C, and per token A-C = (A-B) + (B-C).
  [vLLM] §"Metric measurement basis": the k3 statistic uses
        d = lp_train - lp_rollout, i.e. right minus left in that pair order
        (the later / trainer-side score is always on the right).

Active tokens
  [vLLM] §"Compare per-token logprobs": only masked-in response tokens are
        compared; the first mismatch is reported as an index into the
        masked-in tokens of the sequence. Any non-zero mask byte is active.

Per sequence and pair, over the active tokens i_0 < i_1 < ... (k = active rank):
  valid        number of active tokens
  mismatch     [vLLM] §"Compare per-token logprobs": count of tokens whose fp32
               bit patterns differ (+0.0 vs -0.0 differ; equal NaN bits do
               not). With atol >= 0 a token whose bits differ is still counted
               equal when |left - right| <= atol.
  first_div    smallest k with a mismatch, -1 if none
  longest_run  [vLLM] §"Per-sequence observation patterns": longest run of
               consecutive active tokens that mismatch (masked positions
               neither extend nor break a run)
  nonfinite    active tokens with a non-finite left or right score; they take
               part in the mismatch count but in none of the sums below
               ([AMD] Case 1's compare() refuses such values; here they are
               counted so the caller can refuse them)
  Delta_i      fp64(left_i) - fp64(right_i), one IEEE operation
  max_abs      max |Delta_i| (0 if none)
  sum_abs      sum |Delta_i|            ([vLLM] logprob_mae numerator)
  sum_signed   sum Delta_i              ([AMD] signed mean numerator)
  d_i          right_i - left_i = -Delta_i
  sum_k3       sum (exp(d_i) - 1 - d_i) ([vLLM] Schulman k3 statistic, taken
               as expm1(d) - d); a non-finite term is counted in k3_nonfinite
               and left out, never clipped
  sum_d        sum d_i
  sum_tok_tis  sum min(exp(d_i), C)     ([VeX] §3 "How TIS takes effect":
               token TIS weight; [TII] §2.1 w_TIS = min(w, C))
  seq_tis      min(exp(sum_d), C)       ([VeX] §3: sequence TIS weight)
The sums are exactly rounded (math.fsum).
"""

from __future__ import annotations

import math

import numpy as np

PAIRS = (("A", "B"), ("B", "C"), ("A", "C"))
STAT_FIELDS = ("valid", "mismatch", "first_div", "longest_run", "nonfinite",
               "k3_nonfinite", "max_abs", "sum_abs", "sum_signed", "sum_k3",
               "sum_d", "seq_tis", "sum_tok_tis")
_INT_FIELDS = STAT_FIELDS[:6]


def _check(A, B, C, mask):
    A, B, C = (np.asarray(a) for a in (A, B, C))
    mask = np.asarray(mask)
    for a in (A, B, C):
        if a.dtype != np.float32:
            raise ValueError("scores must be float32")
    if not (A.shape == B.shape == C.shape == mask.shape) or A.ndim != 2:
        raise ValueError("A, B, C and mask must share one [N, L] shape")
    return A, B, C, mask


def _longest_true_run(flags: np.ndarray) -> int:
    best = run = 0
    for f in flags:
        run = run + 1 if f else 0
        best = max(best, run)
    return best


def _pair_stats(left: np.ndarray, right: np.ndarray, tis_clip: float,
                atol: float | None) -> dict:
    """Statistics over the active tokens of one sequence (1-D fp32 arrays)."""
    same_bits = left.view(np.uint32) == right.view(np.uint32)
    l64 = left.astype(np.float64)
    r64 = right.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        if atol is None:
            differ = ~same_bits
        else:
            differ = ~same_bits & ~(np.abs(l64 - r64) <= atol)
        finite = np.isfinite(l64) & np.isfinite(r64)
        delta = l64[finite] - r64[finite]
        d = r64[finite] - l64[finite]
        k3 = np.expm1(d) - d
        k3_ok = np.isfinite(k3)
        tok_tis = np.minimum(np.exp(d), tis_clip)
        sum_d = math.fsum(d.tolist())
        seq_tis = min(math.exp(sum_d) if sum_d < 709.0 else math.inf, tis_clip)
    nz = np.flatnonzero(differ)
    return dict(
        valid=int(left.size),
        mismatch=int(differ.sum()),
        first_div=int(nz[0]) if nz.size else -1,
        longest_run=_longest_true_run(differ.tolist()),
        nonfinite=int((~finite).sum()),
        k3_nonfinite=int((~k3_ok).sum()),
        max_abs=float(np.abs(delta).max()) if delta.size else 0.0,
        sum_abs=math.fsum(np.abs(delta).tolist()),
        sum_signed=math.fsum(delta.tolist()),
        sum_k3=math.fsum(k3[k3_ok].tolist()),
        sum_d=sum_d,
        seq_tis=float(seq_tis),
        sum_tok_tis=math.fsum(tok_tis.tolist()),
    )


def compare(A, B, C, mask, tis_clip: float = 2.0, atol: float | None = None):
    """Per-sequence statistics for the pairs (A,B), (B,C), (A,C).

    Returns {"AB"|"BC"|"AC": {field: np.ndarray [N]}} with int64 arrays for the
    integer fields and float64 arrays for the rest.
    """
    A, B, C, mask = _check(A, B, C, mask)
    if not (np.isfinite(tis_clip) and tis_clip > 0):
        raise ValueError("tis_clip must be finite and > 0")
    arrays = {"A": A, "B": B, "C": C}
    N = mask.shape[0]
    out = {}
    for lname, rname in PAIRS:
        res = {f: np.zeros(N, np.int64 if f in _INT_FIELDS else np.float64)
               for f in STAT_FIELDS}
        for n in range(N):
            act = np.flatnonzero(mask[n] != 0)
            st = _pair_stats(arrays[lname][n, act], arrays[rname][n, act],
                             float(tis_clip), atol)
            for f in STAT_FIELDS:
                res[f][n] = st[f]
        out[lname + rname] = res
    return out


def per_token(A, B, C, mask, tis_clip: float = 2.0) -> np.ndarray:
    """Per-token values [3 pairs][3: |Delta|, k3, token TIS][N][L], fp32.

    Inactive positions are 0 (a padding token carries weight 0, [VeX] §3).
    Active positions with a non-finite left or right score are NaN.
    """
    A, B, C, mask = _check(A, B, C, mask)
    arrays = {"A": A, "B": B, "C": C}
    N, L = mask.shape
    out = np.zeros((3, 3, N, L), np.float32)
    act = mask != 0
    for p, (lname, rname) in enumerate(PAIRS):
        l64 = arrays[lname].astype(np.float64)
        r64 = arrays[rname].astype(np.float64)
        with np.errstate(invalid="ignore", over="ignore"):
            finite = np.isfinite(l64) & np.isfinite(r64)
            d = r64 - l64
            vals = (np.abs(l64 - r64), np.expm1(d) - d, np.minimum(np.exp(d), tis_clip))
            for j, v in enumerate(vals):
                o = np.where(act & finite, v, np.where(act, np.nan, 0.0))
                out[p, j] = o.astype(np.float32)    # k3 beyond fp32 range -> inf
    return out


# ---------------------------------------------------------------------------
# Tail statistics of |Delta| per pair (lp_compare_tails, lp_compare_quantiles)
#
#   [AMD] "Check Whether the Pattern Extends Across the Response": p95 and p99
#          are the 95th and 99th percentiles of the absolute error over the
#          compared arrays, computed by the blog's compare() (section "Case 1:
#          A Changes; B and C Stay Close") with numpy's np.quantile at its
#          default settings; compare() takes one record's response-aligned
#          arrays, and with a single active token every percentile is that
#          token's |Delta|.
#   [vLLM] "Metric measurement basis": logprob_mae = sum(mask |lp_train -
#          lp_serve|) / sum(mask) over valid tokens, "also report p95/max and
#          position"; probability_mae = mean |exp(lp_train) - exp(lp_serve)|
#          over valid tokens.
#   [VeX] section 5, its list of practical indicators: record the p50 / p95 /
#          p99 / max of abs(delta_logprob).
#
# The tokens counted are the active ones whose two scores are finite
# (non-finite ones are reported by compare()). Quantiles follow numpy's
# default ("linear") rule, see quantile_linear(). tails() pools the whole
# batch (a run's distribution); seq_quantiles() takes each sequence alone
# (compare() applied to one record).
#   count          number of counted tokens
#   q50, q95, q99  quantile_linear of |Delta| at p = 0.5, 0.95, 0.99; 0 when
#                  count == 0
#   max_abs        max |Delta| (0 when n = 0)
#   max_seq, max_pos  sequence and position (column) of the first token, in
#                  row-major order, with |Delta| = max_abs (-1, -1 when n = 0)
#   sum_abs        sum |Delta|                  (logprob_mae numerator)
#   sum_prob_abs   sum |exp(left) - exp(right)| (probability_mae numerator)
# and per position i (column) of the rows: the sum of |Delta| over the
# sequences whose token there is counted, and how many are (pos_sum, pos_count)
# -- the error-by-position profile.
# ---------------------------------------------------------------------------

TAIL_FIELDS = ("count", "q50", "q95", "q99", "max_abs", "max_seq", "max_pos",
               "sum_abs", "sum_prob_abs")
QUANTILE_PROBS = (0.5, 0.95, 0.99)


def quantile_linear(sorted_vals: np.ndarray, p: float) -> float:
    """Quantile p of an ascending array by numpy's default ("linear") rule,
    evaluated the way numpy evaluates it (fp64, no fused multiply-add).

    With n values x_0 <= ... <= x_{n-1}: the virtual index is h = (n - 1) p
    (one fp64 product); when h >= n - 1 the result is x_{n-1}; otherwise,
    with j = floor(h) and g = h - j, it interpolates between a = x_j and
    b = x_{j+1}: a + (b - a) g when g < 0.5, else b - (b - a)(1 - g) (the
    same line taken from its nearer end). An empty array gives 0.
    """
    n = sorted_vals.size
    if n == 0:
        return 0.0
    h = float(n - 1) * float(p)
    j = math.floor(h)
    if h >= n - 1:
        return float(sorted_vals[n - 1])
    g = h - j
    a = float(sorted_vals[j])
    b = float(sorted_vals[j + 1])
    diff = b - a
    if g < 0.5:
        return a + diff * g
    return b - diff * (1.0 - g)


def tails(A, B, C, mask):
    """Per pair: dict of TAIL_FIELDS; plus pos_sum [3][L] fp64 and pos_count
    [3][L] int64. Sums are exactly rounded (math.fsum)."""
    A, B, C, mask = _check(A, B, C, mask)
    sides = {"A": A, "B": B, "C": C}
    N, L = A.shape
    out = {}
    pos_sum = np.zeros((3, L))
    pos_count = np.zeros((3, L), np.int64)
    for p, (ln, rn) in enumerate(PAIRS):
        left = sides[ln].astype(np.float64)
        right = sides[rn].astype(np.float64)
        keep = (mask != 0) & np.isfinite(left) & np.isfinite(right)
        delta = np.abs(left - right)
        vals = delta[keep]                       # row-major order
        srt = np.sort(vals)
        rec = {"count": int(vals.size)}
        for name, prob in zip(("q50", "q95", "q99"), QUANTILE_PROBS):
            rec[name] = quantile_linear(srt, prob)
        if vals.size:
            mx = float(vals.max())
            seqs, poss = np.nonzero(keep & (delta == mx))
            rec.update(max_abs=mx, max_seq=int(seqs[0]), max_pos=int(poss[0]))
        else:
            rec.update(max_abs=0.0, max_seq=-1, max_pos=-1)
        rec["sum_abs"] = math.fsum(vals.tolist())
        prob = np.abs(np.exp(left) - np.exp(right))[keep]
        rec["sum_prob_abs"] = math.fsum(prob.tolist())
        out["".join((ln, rn))] = rec
        for i in range(L):
            col = delta[:, i][keep[:, i]]
            pos_sum[p, i] = math.fsum(col.tolist())
            pos_count[p, i] = col.size
    return out, pos_sum, pos_count


def seq_quantiles(A, B, C, mask) -> dict:
    """Per pair and sequence, quantile_linear of |Delta| over the sequence's
    counted tokens at p = 0.5, 0.95, 0.99: {"AB"|"BC"|"AC": float64 [N, 3]}
    (0 for a sequence without counted tokens). [AMD] compare() applied to
    one record's arrays."""
    A, B, C, mask = _check(A, B, C, mask)
    sides = {"A": A, "B": B, "C": C}
    N = A.shape[0]
    out = {}
    for ln, rn in PAIRS:
        left = sides[ln].astype(np.float64)
        right = sides[rn].astype(np.float64)
        keep = (mask != 0) & np.isfinite(left) & np.isfinite(right)
        delta = np.abs(left - right)
        q = np.zeros((N, 3))
        for n in range(N):
            srt = np.sort(delta[n][keep[n]])
            for j, p in enumerate(QUANTILE_PROBS):
                q[n, j] = quantile_linear(srt, p)
        out[ln + rn] = q
    return out


def worst_tokens(A, B, C, mask, k: int):
    """Per pair, the k counted tokens with the largest |Delta|: a list of
    (abs_delta, seq, pos) tuples, ordered by |Delta| descending and, among
    equal |Delta|, by row-major position (sequence, then column); shorter
    than k when fewer tokens are counted.

    [vLLM] "Metric measurement basis": report the worst positions, not only
    the mean (logprob_mae with its max and where it sits); [VeX] section 5,
    practical indicators: the tail of abs(delta_logprob). The counted tokens
    and Delta are those of tails(): active, both scores finite,
    Delta = fp64(left) - fp64(right). The order is a plain stable sort.
    """
    if k < 0:
        raise ValueError("k must be >= 0")
    A, B, C, mask = _check(A, B, C, mask)
    sides = {"A": A, "B": B, "C": C}
    out = {}
    for ln, rn in PAIRS:
        left = sides[ln].astype(np.float64)
        right = sides[rn].astype(np.float64)
        keep = (mask != 0) & np.isfinite(left) & np.isfinite(right)
        delta = np.abs(left - right)
        seqs, poss = np.nonzero(keep)               # row-major order
        vals = delta[seqs, poss]
        order = np.lexsort((poss, seqs, -vals))     # last key is the primary one
        out["".join((ln, rn))] = [(float(vals[j]), int(seqs[j]), int(poss[j]))
                                  for j in order[:k]]
    return out
