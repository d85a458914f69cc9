"""GPU parity of lp_compare against the oracle: integer statistics and
max_abs bit-exact, fixed-order fp64 sums to 1e-9 relative (k3 and token-TIS
sums, whose small-|d| terms are fp32, to 1e-6). Every call goes through the
C ABI (liblp.so)."""

import numpy as np
import pytest
import torch

import oracle
import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import DEV, SCORE_ATOL, check_stats, dev, dev_bf16, gpu_score

pytestmark = pytest.mark.gpu


def run(case_or_arrays, tis_clip=2.0, atol=None, per_token=False):
    if isinstance(case_or_arrays, tuple):
        A, B, C, M = case_or_arrays
    else:
        c = case_or_arrays
        A, B, C, M = c.A, c.B, c.C, c.mask
    res = lp.compare(dev(A), dev(B), dev(C), dev(M), tis_clip, atol, per_token, check=False)
    ref = oracle.compare(A, B, C, M, tis_clip, atol)
    got = res[0] if per_token else res
    check_stats(got, ref)
    return res, ref


@pytest.fixture(scope="module")
def record():
    return synth.compare_case(N=8, max_resp=2048, prompt=256, seed=0)


def with_c(c, C=None, A=None):
    return (c.A if A is None else A, c.B, c.C if C is None else C, c.mask)


def test_baseline_identical(record):
    got, _ = run(record)
    assert not got["AB"]["mismatch"].any() and (got["BC"]["first_div"] == -1).all()


def test_fault_noise(record):
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=11)
    got, _ = run(with_c(record, C))
    assert (got["BC"]["mismatch"] > 0).all()


@pytest.mark.parametrize("k", [1, -1])
def test_fault_token_shift(record, k):
    C = synth.shift_scores(record.C, seq=3, k=k, fill=-5.0)
    got, _ = run(with_c(record, C))
    assert got["BC"]["mismatch"][3] > 0
    assert not np.delete(got["BC"]["mismatch"], 3).any()


def test_fault_case1_case2_offsets(record):
    A = synth.offset_scores(record.A, record.mask, 0.10, first_pos=1)
    C = synth.offset_scores(record.C, record.mask, 0.10)
    got, _ = run(with_c(record, C, A))
    assert (got["AB"]["first_div"][record.resp_len >= 2] == 1).all()
    assert (got["BC"]["first_div"] == 0).all()


def test_fault_stale_weights():
    # Skipped weight sync: B scored with W, C with W' = bf16(W + N(0, 1e-3)),
    # both by the oracle (rounded to fp32) so the comparison inputs never come
    # from the GPU path. The GPU scorer is checked on the same rows too.
    x, w, w_stale, ids = synth.stale_inputs()
    N, L = 8, 2304
    B = oracle.score(x, w, ids)[0].astype(np.float32).reshape(N, L)
    C = oracle.score(x, w_stale, ids)[0].astype(np.float32).reshape(N, L)
    rec = synth.compare_case(N=N, max_resp=2048, prompt=256, seed=5, B=B)
    Cm = rec.C.copy()
    act = rec.mask != 0
    Cm[act] = C[act]
    got, _ = run(with_c(rec, Cm))
    assert (got["BC"]["mismatch"] > 0).all()
    rows = np.flatnonzero(act.reshape(-1))[:4096]
    g = gpu_score(x[rows], w_stale, ids[rows])
    assert np.max(np.abs(g - C.reshape(-1)[rows])) <= SCORE_ATOL


def test_fault_stale_weights_scored_on_the_gpu():
    # [AMD] "Case 3: Agreement Breaks After an Update" at the Qwen3-1.7B head:
    # every one of the 8 x 2304 positions scored by lp_score with W (B) and
    # with W' = bf16(W + N(0, 1e-3)) (C), H = 2048, V = 151 936; lp_compare on
    # those bytes against the oracle, and sampled B and C rows against the
    # fp64 oracle score.
    N, L, H = 8, 2304, 2048
    x, w, w_stale, ids = synth.stale_qwen_inputs(N, L, H)
    xd = dev_bf16(x)
    B = gpu_score(xd, w, ids).reshape(N, L)
    C = gpu_score(xd, w_stale, ids).reshape(N, L)
    rec = synth.compare_case(N=N, max_resp=2048, prompt=256, seed=5, B=B)
    act = rec.mask != 0
    Cm = rec.C.copy()
    Cm[act] = C[act]
    got, ref = run(with_c(rec, Cm))
    assert (got["BC"]["mismatch"] > 0).all() and (got["BC"]["max_abs"] > 0).all()
    assert not got["AB"]["mismatch"].any()
    # The update moves scores far more than a repeat would: B - C is the
    # weight-movement term of the blog's split, A - B (= 0 here) the rest.
    assert np.array_equal(got["AC"]["sum_signed"], got["BC"]["sum_signed"])
    rows = np.random.default_rng(55).choice(np.flatnonzero(act.reshape(-1)), 48, replace=False)
    for Wb, S in ((w, B), (w_stale, C)):
        ref_rows, _ = oracle.score(x[rows], Wb, ids[rows])
        assert np.max(np.abs(S.reshape(-1)[rows] - ref_rows)) <= SCORE_ATOL


def test_per_token_values(record):
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=12)
    C[0, 300] = np.nan
    (stats, pt), _ = run(with_c(record, C), per_token=True)
    ref = oracle.per_token(record.A, record.B, C, record.mask)
    got = pt.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[:, 0][fin[:, 0]], ref[:, 0][fin[:, 0]])        # |delta| exact
    np.testing.assert_allclose(got[:, 1:][fin[:, 1:]], ref[:, 1:][fin[:, 1:]], rtol=1e-6, atol=1e-30)


def test_per_token_k3_tis_across_the_small_range():
    # |d| < 0.5 takes the fp32 path (k3 from a fitted polynomial, e^d from the
    # same series): d swept densely over (-0.5, 0.5) on both sides of each
    # pair, also at the edges and very near 0, against the fp64 oracle; the
    # sums to the documented 1e-6 relative. TIS cap below and above e^d.
    rng = np.random.default_rng(77)
    N, L = 16, 4096
    B = -rng.uniform(0.5, 6.0, (N, L)).astype(np.float32)
    d = np.linspace(-0.4999, 0.4999, N * L).reshape(N, L)
    d[0, :64] = np.float32(2.0) ** -np.arange(1, 65)            # tiny, both signs
    d[1, :64] = -d[0, :64]
    A = (B.astype(np.float64) + d).astype(np.float32)
    C = (B.astype(np.float64) - 0.5 * d).astype(np.float32)
    M = np.ones((N, L), np.uint8)
    for clip in (2.0, 1.25, 0.875):  # fp32 caps (the C ABI takes tis_clip as float)
        (stats, pt), _ = run((A, B, C, M), per_token=True, tis_clip=clip)
        ref = oracle.per_token(A, B, C, M, tis_clip=clip)
        got = pt.cpu().numpy()
        assert np.array_equal(got[:, 0], ref[:, 0])
        np.testing.assert_allclose(got[:, 1:], ref[:, 1:], rtol=1e-6, atol=1e-30)


def test_special_values_and_atol():
    f = np.float32
    A = np.array([[0.0, -1.0, np.nan, np.inf, -1000.0, -2.0, -3.0, -4.0]], f)
    B = np.array([[-0.0, -1.0, np.nan, -1.0, 0.0, -2.0005, -3.0, -4.0]], f)
    C = np.array([[0.0, -1.5, -1.0, np.inf, -1000.0, -2.0, -3.1, np.nan]], f)
    M = np.array([[1, 1, 1, 1, 1, 1, 0, 1]], np.uint8)
    for atol in (None, 1e-3, 0.0):
        run((A, B, C, M), atol=atol)
    run((A, B, C, M), tis_clip=1.5)


@pytest.mark.parametrize("seed", range(3))
def test_random_masks_with_holes(seed):
    rng = np.random.default_rng(200 + seed)
    N, L = 37, int(rng.integers(1, 700))
    B = np.log(1.0 - rng.random((N, L))).astype(np.float32)
    A = B.copy(); C = B.copy()
    for arr in (A, C):
        sel = rng.random((N, L)) < rng.random()
        arr[sel] = (arr[sel] + rng.normal(0, 0.01, sel.sum())).astype(np.float32)
    M = (rng.random((N, L)) < 0.8).astype(np.uint8)
    M[0] = 0
    run((A, B, C, M), atol=None if seed else 0.005)


def test_strided_rows_and_degenerate_sizes(record):
    N, L = record.N, record.L
    pad = 40
    big = [np.zeros((N, L + pad), a.dtype) for a in (record.A, record.B, record.C, record.mask)]
    for b, a in zip(big, (record.A, record.B, record.C, record.mask)):
        b[:, :L] = a
    views = [dev(b)[:, :L] for b in big]
    got = lp.compare(*views, check=False)
    check_stats(got, oracle.compare(record.A, record.B, record.C, record.mask))
    # N = 0: nothing to do; L = 0: every sequence is empty.
    z = torch.zeros((0, 5), dtype=torch.float32, device=DEV)
    lp.compare(z, z, z, torch.zeros((0, 5), dtype=torch.uint8, device=DEV), check=False)
    e = torch.zeros((3, 0), dtype=torch.float32, device=DEV)
    got = lp.compare(e, e, e, torch.zeros((3, 0), dtype=torch.uint8, device=DEV), check=False)
    assert (got["AB"]["valid"] == 0).all() and (got["BC"]["first_div"] == -1).all()
    with pytest.raises(ValueError):
        lp.compare(e, e, e, torch.zeros((3, 0), dtype=torch.uint8, device=DEV))


def test_results_independent_of_batch_and_repeatable(record):
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=13)
    full = lp.compare(dev(record.A), dev(record.B), dev(C), dev(record.mask), check=False)
    again = lp.compare(dev(record.A), dev(record.B), dev(C), dev(record.mask), check=False)
    one = lp.compare(dev(record.A[5:6]), dev(record.B[5:6]), dev(C[5:6]),
                     dev(record.mask[5:6]), check=False)
    for p in lp.PAIRS:
        assert full[p].tobytes() == again[p].tobytes()
        assert full[p][5:6].tobytes() == one[p].tobytes()


def test_large_batch_sampled():
    c = synth.compare_sweep_case(N=4096)
    raw, _ = lp.compare_raw(dev(c.A), dev(c.B), dev(c.C), dev(c.mask))
    got = lp.stats_from_bytes(raw, c.N)
    seqs = np.random.default_rng(9).choice(c.N, 24, replace=False)
    ref = oracle.compare(c.A[seqs], c.B[seqs], c.C[seqs], c.mask[seqs])
    check_stats({p: got[p][seqs] for p in lp.PAIRS}, ref)
    assert np.array_equal(got["AB"]["valid"], c.mask.sum(axis=1))


def test_vector_and_scalar_paths_agree(record):
    # Rows whose stride is not a multiple of 4 take the scalar path; it visits
    # the same positions in the same order as the 16-byte path.
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=14)
    N, L = record.N, record.L
    vec = lp.compare(dev(record.A), dev(record.B), dev(C), dev(record.mask), check=False)
    big = [np.zeros((N, L + 1), a.dtype) for a in (record.A, record.B, C, record.mask)]
    for b, a in zip(big, (record.A, record.B, C, record.mask)):
        b[:, :L] = a
    sca = lp.compare(*[dev(b)[:, :L] for b in big], check=False)
    for p in lp.PAIRS:
        assert vec[p].tobytes() == sca[p].tobytes(), p


def test_large_differences_and_overflow():
    # |d| >= 0.5 takes the fp64 exponential; d = 700 stays finite, d beyond
    # the fp64 overflow threshold of e^d (about 709.78) makes k3 overflow
    # (counted, never clipped) while the TIS weight clips; d <= -745
    # underflows e^d to 0.
    rng = np.random.default_rng(321)
    N, L = 9, 1000
    B = (3.0 * np.log(1.0 - rng.random((N, L)))).astype(np.float32)
    A = B.copy()
    scale = rng.choice(np.array([0.01, 1.0, 30.0]), (N, L))
    C = (B + rng.normal(0.0, 1.0, (N, L)) * scale).astype(np.float32)
    C[0, 0] = B[0, 0] + np.float32(700.0)
    C[0, 1:40] = B[0, 1:40] + np.linspace(710.0, 720.0, 39, dtype=np.float32)
    C[1, :40] = B[1, :40] - np.linspace(700.0, 800.0, 40, dtype=np.float32)
    A[2] = (B[2] + 0.75).astype(np.float32)
    M = (rng.random((N, L)) < 0.9).astype(np.uint8)
    for clip in (2.0, 0.5):
        (stats, pt), _ = run((A, B, C, M), tis_clip=clip, per_token=True)
        assert stats["BC"]["k3_nonfinite"][0] > 0
        ref = oracle.per_token(A, B, C, M, clip)
        got = pt.cpu().numpy()
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(got[:, 0][fin[:, 0]], ref[:, 0][fin[:, 0]])
        np.testing.assert_allclose(got[:, 1:][fin[:, 1:]], ref[:, 1:][fin[:, 1:]],
                                   rtol=1e-6, atol=1e-30)


def test_records_at_an_8_byte_aligned_address(record):
    """lp_seq_stats records need only their natural 8-byte alignment: an
    output buffer 8 bytes past a 16-byte boundary gets the same bytes."""
    C = synth.noise_scores(record.C, record.mask, 1e-3, seed=31)
    A, B, M = dev(record.A), dev(record.B), dev(record.mask)
    Cd = dev(C)
    nbytes = 3 * record.A.shape[0] * lp.SEQ_STATS_DTYPE.itemsize
    aligned = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    shifted = torch.zeros(nbytes + 8, dtype=torch.uint8, device=DEV)
    lp.compare_raw(A, B, Cd, M, out=aligned)
    lp.compare_raw(A, B, Cd, M, out=shifted[8:])
    torch.cuda.synchronize()
    assert aligned.data_ptr() % 16 == 0 and shifted[8:].data_ptr() % 16 == 8
    assert torch.equal(aligned, shifted[8:])
    check_stats(lp.stats_from_bytes(aligned, record.A.shape[0]),
                oracle.compare(record.A, record.B, C, record.mask))


def test_record_layout_is_sequence_major():
    """The C ABI's output is [N][3]: record 3 n + p is pair p (AB, BC, AC) of
    sequence n. Sequences with 1 .. 5 active tokens and pairs that differ in
    a known way make every record distinguishable in the raw bytes."""
    N, L = 5, 300
    B = synth.normal_f32(40, N * L).reshape(N, L)
    A = B.copy()
    A[:, 0] += 1.0      # A differs from B (and C) at position 0 only
    C = B.copy()
    C[:, 1] -= 2.0      # C differs from B (and A) at position 1 only
    M = np.zeros((N, L), np.uint8)
    for n in range(N):
        M[n, : n + 1] = 1   # sequence n has n + 1 active tokens
    raw, _ = lp.compare_raw(dev(A), dev(B), dev(C), dev(M))
    rec = raw.cpu().numpy()[: 3 * N * lp.SEQ_STATS_DTYPE.itemsize].view(lp.SEQ_STATS_DTYPE)
    ref = oracle.compare(A, B, C, M)
    for n in range(N):
        assert rec[3 * n]["valid"] == n + 1
        assert (rec[3 * n]["mismatch"], rec[3 * n + 1]["mismatch"], rec[3 * n + 2]["mismatch"]) \
            == (1, int(n >= 1), 1 + int(n >= 1))
        for i, pair in enumerate(lp.PAIRS):
            for f in ("valid", "mismatch", "first_div", "longest_run", "max_abs"):
                assert rec[3 * n + i][f] == ref[pair][f][n], (n, pair, f)


def window_mix_rows(seed, N=24, windows=12, tail=77):
    """Rows built window by window (256 positions) from every kind of window
    the comparison kernel treats apart: empty, fully or partly active, all
    mismatching with small differences, all identical, one large |d|, one
    NaN, one 1-ulp difference, signed zeros, and mixes; plus a partial tail."""
    rng = np.random.default_rng(seed)
    L = 256 * windows + tail
    B = (-rng.exponential(2.0, (N, L))).astype(np.float32)
    A, C = B.copy(), B.copy()
    M = np.zeros((N, L), np.uint8)
    for n in range(N):
        for w0 in range(0, L, 256):
            w1 = min(L, w0 + 256)
            sl = slice(w0, w1)
            kind = rng.integers(0, 9)
            if kind == 0:
                continue
            act = np.ones(w1 - w0, bool)
            if kind in (2, 8):
                cut = sorted(rng.integers(0, w1 - w0, 2))
                act[:] = False
                act[cut[0]:cut[1] + 1] = True
                act &= rng.random(w1 - w0) < (0.5 if kind == 8 else 1.0)
            M[n, sl] = act
            noise = rng.normal(0.0, 1e-3, w1 - w0).astype(np.float32)
            if kind in (1, 2, 4, 5, 8):
                C[n, sl] = B[n, sl] + noise
            if kind == 4:
                C[n, w0 + rng.integers(0, w1 - w0)] += np.float32(0.7)
            if kind == 5:
                C[n, w0 + rng.integers(0, w1 - w0)] = np.nan
            if kind == 6:
                j = w0 + rng.integers(0, w1 - w0)
                C[n, j] = np.nextafter(B[n, j], np.float32(0.0))
            if kind == 7:
                js = w0 + rng.integers(0, w1 - w0, 3)
                B[n, js] = np.float32(0.0)
                A[n, js] = np.float32(0.0)
                C[n, js] = np.float32(-0.0)
            if kind == 8:
                same = rng.random(w1 - w0) < 0.5
                C[n, sl] = np.where(same, B[n, sl], C[n, sl])
            if rng.random() < 0.5:
                A[n, sl] = B[n, sl] + rng.normal(0.0, 1e-3, w1 - w0).astype(np.float32)
    return A, B, C, M


@pytest.mark.parametrize("seed", range(4))
def test_window_shortcuts_against_the_oracle_and_the_element_path(seed):
    A, B, C, M = window_mix_rows(seed)
    N, L = A.shape
    for clip, atol in ((2.0, None), (1.25, None), (2.0, 5e-4)):
        (stats, pt), _ = run((A, B, C, M), tis_clip=clip, atol=atol, per_token=True)
        ref = oracle.per_token(A, B, C, M, tis_clip=clip)
        got = pt.cpu().numpy()
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(got[:, 0][fin[:, 0]], ref[:, 0][fin[:, 0]])
        np.testing.assert_allclose(got[:, 1:][fin[:, 1:]], ref[:, 1:][fin[:, 1:]],
                                   rtol=1e-6, atol=1e-30)
        # Rows of stride L + 1 take element loads for every window.
        big = [np.zeros((N, L + 1), a.dtype) for a in (A, B, C, M)]
        for b, a in zip(big, (A, B, C, M)):
            b[:, :L] = a
        vec = lp.compare(dev(A), dev(B), dev(C), dev(M), clip, atol, check=False)
        sca = lp.compare(*[dev(b)[:, :L] for b in big], clip, atol, check=False)
        for p in lp.PAIRS:
            assert vec[p].tobytes() == sca[p].tobytes(), (p, clip, atol)
