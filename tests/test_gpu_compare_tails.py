"""GPU parity of lp_compare_tails (batch tail statistics of |left - right| per
pair) and lp_compare_quantiles (the same quantiles per sequence) against the
oracle: counts, quantiles (numpy's default rule, to the bit), maxima and
their positions, and the position counts exact; fp64 sums to 1e-9 relative.
Every call goes through the C ABI (liblp.so)."""

import numpy as np
import pytest

import oracle
import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import check_stats, dev

pytestmark = pytest.mark.gpu

EXACT = ("count", "q50", "q95", "q99", "max_abs", "max_seq", "max_pos")
SUMS = ("sum_abs", "sum_prob_abs")


def run_seq_quantiles(A, B, C, M):
    got = lp.compare_quantiles(dev(A), dev(B), dev(C), dev(M))
    ref = oracle.seq_quantiles(A, B, C, M)
    for p in lp.PAIRS:
        assert got[p].shape == ref[p].shape
        bad = np.argwhere(got[p] != ref[p])
        assert bad.size == 0, (p, bad[:5], got[p][tuple(bad[0])], ref[p][tuple(bad[0])])
    return got


def run(A, B, C, M, positions=True):
    run_seq_quantiles(A, B, C, M)
    got, ps, pc = lp.compare_tails(dev(A), dev(B), dev(C), dev(M), positions=True)
    ref, rps, rpc = oracle.tails(A, B, C, M)
    for p in lp.PAIRS:
        for f in EXACT:
            assert got[p][f] == ref[p][f], (p, f, got[p][f], ref[p][f])
        for f in SUMS:
            np.testing.assert_allclose(got[p][f], ref[p][f], rtol=1e-9, atol=1e-300, err_msg=f"{p} {f}")
    assert np.array_equal(pc.astype(np.int64), rpc)
    np.testing.assert_allclose(ps, rps, rtol=1e-9, atol=1e-300)
    return got, ps, pc


@pytest.fixture(scope="module")
def record():
    return synth.compare_case(N=8, max_resp=2048, prompt=256, seed=0)


def test_identical_scores(record):
    got, _, _ = run(record.A, record.B, record.C, record.mask)
    assert got["AB"]["max_abs"] == 0.0 and got["AB"]["q99"] == 0.0


@pytest.mark.parametrize("fault", ["noise", "shift", "case1", "case2", "case1_noise"])
def test_faults(record, fault):
    # After two passes a target either reads a short list of candidate keys
    # (continuous differences: noise) or, when its candidates do not fit the
    # key buffer (an offset puts every |delta| under one 16-bit prefix),
    # keeps reading the batch; identical pairs stop after one pass. The
    # faults cover each path and their mix (case1_noise: AB full, BC lists).
    c = record
    A, C = c.A, c.C
    if fault == "noise":
        C = synth.noise_scores(c.C, c.mask, 1e-3, seed=21)
    elif fault == "shift":
        C = synth.shift_scores(c.C, seq=3, k=1, fill=-5.0)
    elif fault == "case1":
        A = synth.offset_scores(c.A, c.mask, 0.10, first_pos=1)
    elif fault == "case1_noise":
        A = synth.offset_scores(c.A, c.mask, 0.10, first_pos=1)
        C = synth.noise_scores(c.C, c.mask, 1e-3, seed=22)
    else:
        C = synth.offset_scores(c.C, c.mask, 0.10)
    got, _, _ = run(A, c.B, C, c.mask)
    assert got["AC"]["count"] > 0


def test_stale_weights_rescoring():
    # B scored with W, C with W' = bf16(W + N(0, 1e-3)), both by the oracle.
    x, w, w_stale, ids = synth.stale_inputs()
    N, L = 8, 2304
    B = oracle.score(x, w, ids)[0].astype(np.float32).reshape(N, L)
    C = oracle.score(x, w_stale, ids)[0].astype(np.float32).reshape(N, L)
    rec = synth.compare_case(N=N, max_resp=2048, prompt=256, seed=5, B=B)
    Cm = rec.C.copy()
    act = rec.mask != 0
    Cm[act] = C[act]
    got, _, _ = run(rec.A, rec.B, Cm, rec.mask)
    assert got["BC"]["q50"] > 0.0


def test_masks_nonfinite_and_ties():
    rng = np.random.default_rng(3)
    N, L = 37, 301
    B = rng.standard_normal((N, L)).astype(np.float32) - 3.0
    A = B + np.round(rng.standard_normal((N, L)), 1).astype(np.float32) * np.float32(0.5)
    C = B.copy()
    C[rng.random((N, L)) < 0.3] -= np.float32(0.25)
    M = (rng.random((N, L)) < 0.8).astype(np.uint8)
    A[2, 5] = np.nan; C[7, 9] = np.inf; B[11, 300] = -np.inf
    run(A.astype(np.float32), B, C, M)


def test_seq_quantiles_one_token_long_rows_and_strides():
    # One-token and empty records (every quantile is the token's |delta|, or
    # 0); rows longer than the LDS key cache (recomputed every pass); rows
    # with a stride that is not a multiple of 4: all exact.
    rng = np.random.default_rng(17)
    N, L = 9, 5003
    B = np.log(1.0 - rng.random((N, L))).astype(np.float32)
    A = (B + rng.normal(0, 0.01, (N, L))).astype(np.float32)
    C = (B + np.round(rng.normal(0, 2, (N, L))) * np.float32(1e-3)).astype(np.float32)  # ties
    M = (rng.random((N, L)) < 0.9).astype(np.uint8)
    M[0] = 0
    M[0, 4444] = 1                                   # one token
    M[1] = 0                                         # none
    M[2, :4100] = 0                                  # short record in a long row
    C[3, 7] = np.nan
    run_seq_quantiles(A, B, C, M)
    q = lp.compare_quantiles(dev(A), dev(B), dev(C), dev(M))
    d = abs(float(A[0, 4444]) - float(B[0, 4444]))
    assert q["AB"][0].tolist() == [d, d, d] and q["AB"][1].tolist() == [0.0, 0.0, 0.0]
    for pad in (1, 3):
        big = [np.zeros((N, 700 + pad), a.dtype) for a in (A, B, C, M)]
        for b_, a_ in zip(big, (A, B, C, M)):
            b_[:, :700] = a_[:, :700]
        got = lp.compare_quantiles(*[dev(b_)[:, :700] for b_ in big])
        ref = oracle.seq_quantiles(A[:, :700], B[:, :700], C[:, :700], M[:, :700])
        for p in lp.PAIRS:
            assert np.array_equal(got[p], ref[p]), (pad, p)


def quantile_rows(kind, N, L, seed):
    """Rows whose |delta| exercise each way the per-sequence selection
    narrows a rank: continuous noise, a constant offset (every difference in
    one 16-bit bucket), mostly zeros, 1-ulp differences, differences below
    2^-126, one repeated non-zero difference, and a mix with NaN and Inf."""
    rng = np.random.default_rng(seed)
    B = rng.standard_normal((N, L)).astype(np.float32)
    if kind == "noise":
        C = (B + rng.standard_normal((N, L)) * 1e-3).astype(np.float32)
    elif kind == "offset":
        C = (B + np.float32(0.01)).astype(np.float32)
    elif kind == "zeros":
        C = B.copy()
        C[rng.random((N, L)) < 0.3] += np.float32(1e-3)
    elif kind == "ulp":
        C = (B * np.float32(1 + 1e-7)).astype(np.float32)
    elif kind == "tiny":
        B = (rng.standard_normal((N, L)) * 1e-38).astype(np.float32)
        C = (B + np.float32(1e-44) * rng.integers(0, 50, (N, L))).astype(np.float32)
    elif kind == "equal":
        B = np.zeros((N, L), np.float32)
        C = np.full((N, L), np.float32(0.3))
    else:
        C = (B + rng.standard_normal((N, L)) * np.float32(10) ** rng.integers(-30, 3, (N, L))).astype(np.float32)
        C[rng.random((N, L)) < 0.05] = np.nan
        B[rng.random((N, L)) < 0.02] = np.inf
    A = (B + rng.standard_normal((N, L)) * 1e-2).astype(np.float32)
    M = (rng.random((N, L)) < rng.uniform(0.05, 1.0, (N, 1))).astype(np.uint8)
    M[0] = 0                 # no counted token
    M[1] = 0
    M[1, L // 2] = 1         # one
    return A, B, C, M


@pytest.mark.parametrize("L", [1, 300, 768, 769, 1536, 1537, 2304, 2305, 3072, 3073, 4096, 4097])
@pytest.mark.parametrize("kind", ["noise", "offset", "zeros", "ulp", "tiny", "equal", "mixed"])
def test_seq_quantiles_every_row_length_and_kind(L, kind):
    # Row lengths on both sides of each register-held key count (3, 6, 9 or
    # 12 chunks of 256 positions; longer rows take the workgroup kernel), every
    # kind of difference, rows with 16-byte vector loads and with element
    # loads (a stride that is not a multiple of 4): all exact.
    N = 12
    A, B, C, M = quantile_rows(kind, N, L, seed=L)
    run_seq_quantiles(A, B, C, M)
    big = [np.zeros((N, L + 1), a.dtype) for a in (A, B, C, M)]
    for b_, a_ in zip(big, (A, B, C, M)):
        b_[:, :L] = a_
    got = lp.compare_quantiles(*[dev(b_)[:, :L] for b_ in big])
    ref = oracle.seq_quantiles(A, B, C, M)
    for p in lp.PAIRS:
        assert np.array_equal(got[p], ref[p]), p


@pytest.mark.parametrize("L", [1, 2, 3, 5, 767, 1535, 2303])
def test_vector_rows_with_a_partial_last_group(L):
    # Rows 16-byte aligned with a stride that is a multiple of 4 take the
    # vector loads even when L is not a multiple of 4: the last group of four
    # positions reaches past the row into its padding, which holds values
    # that must not be read as scores (NaN, huge, non-zero mask bytes).
    # Per-sequence quantiles, batch tails and the comparison: all exact.
    N = 10
    A, B, C, M = quantile_rows("mixed", N, L, seed=L)
    ld = (L + 3) // 4 * 4 + 4
    big = []
    for a_, fill in zip((A, B, C, M), (np.float32(3e38), np.float32(np.nan), np.float32(-7.5), 1)):
        b_ = np.full((N, ld), fill, a_.dtype)
        b_[:, :L] = a_
        big.append(b_)
    views = [dev(b_)[:, :L] for b_ in big]
    assert views[0].stride(0) == ld and ld % 4 == 0 and views[0].data_ptr() % 16 == 0
    got = lp.compare_quantiles(*views)
    ref = oracle.seq_quantiles(A, B, C, M)
    for p in lp.PAIRS:
        assert np.array_equal(got[p], ref[p]), p
    tg = lp.compare_tails(*views)
    tr = oracle.tails(A, B, C, M)[0]
    for p in lp.PAIRS:
        for f in EXACT:
            assert tg[p][f] == tr[p][f], (p, f)
    check_stats(lp.compare(*views, check=False), oracle.compare(A, B, C, M))


def test_seq_quantiles_random_shapes():
    # Seeded random shapes across both per-sequence kernels and every key
    # count: N in [1, 40], L in [1, 3000], row padding 0 .. 5 (so vector and
    # element loads both occur), a random kind of difference per case.
    rng = np.random.default_rng(2024)
    kinds = ["noise", "offset", "zeros", "ulp", "tiny", "equal", "mixed"]
    for case in range(24):
        N, L = int(rng.integers(1, 41)), int(rng.integers(1, 3001))
        pad = int(rng.integers(0, 6))
        kind = kinds[case % len(kinds)]
        A, B, C, M = quantile_rows(kind, N, L, seed=1000 + case) if N >= 2 else \
            tuple(x[:1] for x in quantile_rows(kind, 2, L, seed=1000 + case))
        if pad:
            big = [np.zeros((N, L + pad), a_.dtype) for a_ in (A, B, C, M)]
            for b_, a_ in zip(big, (A, B, C, M)):
                b_[:, :L] = a_
            views = [dev(b_)[:, :L] for b_ in big]
        else:
            views = [dev(x) for x in (A, B, C, M)]
        got = lp.compare_quantiles(*views)
        ref = oracle.seq_quantiles(A, B, C, M)
        for p in lp.PAIRS:
            assert np.array_equal(got[p], ref[p]), (case, N, L, pad, kind, p)


@pytest.mark.parametrize("case", ["ties_in_lists", "ties_beyond_key_buffer", "one_bucket"])
def test_selection_paths(case):
    # The selection's paths, each exact against the oracle:
    #  ties_in_lists: |delta| takes eight values k / 1024 (exact in fp32),
    #    about 18 000 tokens each. Every quantile's bucket fits its list, but
    #    more than 4 096 keys share every prefix down to the last byte: the
    #    lists are read in every pass and nothing is gathered.
    #  ties_beyond_key_buffer: two values 0.25 and 0.25 + 2^-20 in one
    #    16-bit bucket holding every token: too many for the pair's key
    #    buffer (a quarter of the positions), so the batch is read in every
    #    pass.
    #  one_bucket: |delta| continuous in [1, 1.0625), one bucket, too many
    #    for the key buffer: the batch is read until a prefix holds at most
    #    4 096 keys, which are then gathered from the batch.
    rng = np.random.default_rng({"ties_in_lists": 5, "ties_beyond_key_buffer": 6, "one_bucket": 7}[case])
    N, L = (64, 2304) if case == "ties_in_lists" else (16, 2304)
    B = -np.floor(rng.uniform(1.0, 8.0, (N, L))).astype(np.float32)   # integers: exact differences
    if case == "ties_in_lists":
        d = rng.integers(1, 9, (N, L)).astype(np.float32) / np.float32(1024.0)
    elif case == "ties_beyond_key_buffer":
        d = np.where(rng.random((N, L)) < 0.6, np.float32(0.25), np.float32(0.25 + 2.0 ** -20))
    else:
        d = (1.0 + rng.random((N, L)) / 16.0).astype(np.float32)
    A = (B - d).astype(np.float32)
    C = (B + np.float32(0.5) * d).astype(np.float32)
    M = (rng.random((N, L)) < 0.97).astype(np.uint8)
    run(A, B, C, M)
    run_worst(A, B, C, M, 64)


def random_case(seed):
    """A seeded batch whose shape, mask density and |delta| distribution are
    drawn at random: continuous noise of one of several scales, quantized
    differences (many ties), a constant offset (one bucket), identical
    scores, or a mix, with a few non-finite scores."""
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 48))
    L = int(rng.integers(1, 2600))
    B = np.log(1.0 - rng.random((N, L))).astype(np.float32)
    def delta(kind):
        if kind == "noise":
            return rng.normal(0.0, 10.0 ** rng.uniform(-6, 0), (N, L))
        if kind == "ties":
            return np.round(rng.normal(0.0, 3.0, (N, L))) * 2.0 ** -int(rng.integers(4, 12))
        if kind == "offset":
            return np.full((N, L), rng.uniform(0.01, 1.0))
        if kind == "same":
            return np.zeros((N, L))
        return np.where(rng.random((N, L)) < 0.5, rng.normal(0.0, 1e-3, (N, L)),
                        np.round(rng.normal(0.0, 2.0, (N, L))) * 2.0 ** -8)
    kinds = ("noise", "ties", "offset", "same", "mix")
    A = (B + delta(kinds[rng.integers(5)])).astype(np.float32)
    C = (B + delta(kinds[rng.integers(5)])).astype(np.float32)
    M = (rng.random((N, L)) < rng.uniform(0.05, 1.0)).astype(np.uint8)
    for arr in (A, B, C):
        if rng.random() < 0.3:
            arr[rng.integers(N), rng.integers(L)] = rng.choice([np.nan, np.inf, -np.inf])
    return A, B, C, M, int(rng.choice([0, 1, 7, 300]))


@pytest.mark.parametrize("seed", range(24))
def test_random_batches(seed):
    # Every selection path on random shapes: sources shared or split, gathers
    # after pass 0, 1 or later, lists, the batch read when a bucket does not
    # fit, ties down to the last byte; exact against the oracle.
    A, B, C, M, k = random_case(seed)
    run(A, B, C, M)
    if k:
        run_worst(A, B, C, M, k)


@pytest.mark.parametrize("N,L", [(0, 5), (3, 0), (1, 1)])
def test_degenerate_sizes(N, L):
    A = np.zeros((N, L), np.float32)
    M = np.ones((N, L), np.uint8)
    got, ps, pc = lp.compare_tails(dev(A), dev(A), dev(A), dev(M), positions=True)
    ref, rps, rpc = oracle.tails(A, A, A, M)
    for p in lp.PAIRS:
        for f in EXACT + SUMS:
            assert got[p][f] == ref[p][f], (p, f)
    assert ps.shape == (3, L) and np.array_equal(pc.astype(np.int64), rpc)
    run_seq_quantiles(A, A, A, M)


def test_sweep_size_and_repeatability():
    c = synth.compare_sweep_case(N=512)
    got, ps, pc = run(c.A, c.B, c.C, c.mask)
    again, ps2, pc2 = lp.compare_tails(dev(c.A), dev(c.B), dev(c.C), dev(c.mask), positions=True)
    for p in lp.PAIRS:
        assert got[p].tobytes() == again[p].tobytes()
    assert ps.tobytes() == ps2.tobytes() and pc.tobytes() == pc2.tobytes()


def test_vector_and_scalar_paths_agree(record):
    # Rows with a stride that is not a multiple of 4 take element loads over
    # the same positions in the same order: bitwise equal results.
    import torch
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=31)
    N, L = record.N, record.L
    vec = lp.compare_tails(dev(record.A), dev(record.B), dev(C), dev(record.mask), positions=True)
    for pad in (1, 3):
        big = [np.zeros((N, L + pad), a.dtype) for a in (record.A, record.B, C, record.mask)]
        for b, a in zip(big, (record.A, record.B, C, record.mask)):
            b[:, :L] = a
        sca = lp.compare_tails(*[dev(b)[:, :L] for b in big], positions=True)
        for p in lp.PAIRS:
            assert vec[0][p].tobytes() == sca[0][p].tobytes(), p
        assert np.array_equal(vec[1], sca[1]) and np.array_equal(vec[2], sca[2])


# ---------------------------------------------------------------------------
# Worst k tokens (lp_compare_tails_ex): every row exact against the oracle
# (|delta| bit for bit, sequence and column), the tail statistics unchanged.
# ---------------------------------------------------------------------------

def run_worst(A, B, C, M, k):
    got, worst = lp.compare_tails(dev(A), dev(B), dev(C), dev(M), worst_k=k)
    ref = oracle.worst_tokens(A, B, C, M, k)
    plain = lp.compare_tails(dev(A), dev(B), dev(C), dev(M))
    for p in lp.PAIRS:
        assert got[p].tobytes() == plain[p].tobytes(), p      # the rows cost the stats nothing
        w, r = worst[p], ref[p]
        assert w.shape == (k,)
        for j, (d, n, i) in enumerate(r):
            assert (w[j]["abs_delta"], w[j]["seq"], w[j]["pos"]) == (d, n, i), (p, j, w[j], (d, n, i))
        for j in range(len(r), k):                            # fewer counted tokens than k
            assert (w[j]["abs_delta"], w[j]["seq"], w[j]["pos"]) == (0.0, -1, -1), (p, j)
    return worst


@pytest.mark.parametrize("k", [1, 16, 300, 4096])
def test_worst_tokens_noise(record, k):
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=41)
    A = synth.offset_scores(record.A, record.mask, 0.10, first_pos=1)
    run_worst(A, record.B, C, record.mask, k)


@pytest.mark.parametrize("k", [3, 50, 2000])
def test_worst_tokens_many_ties(k):
    # Differences on a coarse grid: the k-th largest |delta| is shared by many
    # tokens, and only the first of them in row-major order are kept.
    rng = np.random.default_rng(7)
    N, L = 23, 517
    B = (rng.standard_normal((N, L)) - 4.0).astype(np.float32)
    A = (B + np.round(rng.standard_normal((N, L)), 0).astype(np.float32) * np.float32(0.25))
    C = B.copy()
    C[rng.random((N, L)) < 0.5] += np.float32(0.5)
    M = (rng.random((N, L)) < 0.9).astype(np.uint8)
    A[1, 2] = np.nan; C[4, 4] = -np.inf
    run_worst(A.astype(np.float32), B, C, M, k)


def test_worst_tokens_identical_scores_keep_row_major_order(record):
    w = run_worst(record.A, record.B, record.C, record.mask, 10)
    assert (w["AB"]["abs_delta"] == 0.0).all()


@pytest.mark.parametrize("N,L", [(0, 5), (3, 0), (1, 1), (2, 3)])
def test_worst_tokens_degenerate_sizes(N, L):
    A = np.zeros((N, L), np.float32)
    B = np.ones((N, L), np.float32)
    M = np.ones((N, L), np.uint8)
    if N * L:
        M[0, 0] = 0
    run_worst(A, B, A.copy(), M, 7)


def test_worst_tokens_sweep_size_paths_and_repeatability():
    import torch
    c = synth.compare_sweep_case(N=512)
    w1 = run_worst(c.A, c.B, c.C, c.mask, 100)
    # Strided rows take element loads: the same rows.
    N, L = c.A.shape
    big = [np.zeros((N, L + 1), a.dtype) for a in (c.A, c.B, c.C, c.mask)]
    for b, a in zip(big, (c.A, c.B, c.C, c.mask)):
        b[:, :L] = a
    _, w2 = lp.compare_tails(*[dev(b)[:, :L] for b in big], worst_k=100)
    _, w3 = lp.compare_tails(dev(c.A), dev(c.B), dev(c.C), dev(c.mask), worst_k=100)
    for p in lp.PAIRS:
        assert w1[p].tobytes() == w2[p].tobytes() == w3[p].tobytes(), p
