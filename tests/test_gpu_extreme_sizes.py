"""Edge sizes against the oracle, through the C ABI: sequences of 300 001
positions (the 64-bit position arithmetic, a ragged last window and element
loads on a row stride that is not a multiple of 4) for lp_compare,
lp_compare_tails(_ex) and lp_correct; 70 001 scored rows (275 token tiles of
the 352 x 256 kernel, a ragged last one) and a 1 000 003-row vocabulary (2 841
vocabulary tiles, a ragged last one) for lp_score, both through the tile kernel
and through the streaming kernels; and the largest row stride lp_score
accepts (its 32-bit buffer addressing spans 255 rows of it)."""

import numpy as np
import pytest

import oracle
import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import DEV, SCORE_ATOL, check_stats, dev, dev_bf16, gpu_score
from .test_gpu_compare_tails import run as run_tails, run_worst
from .test_gpu_correct import check as check_correct

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def long_rows():
    """Three sequences of 300 001 positions: a masked prompt, holes in the
    response mask, generation noise on a third of the tokens, trainer noise
    of 1e-3, a few differences of order one (the fp64 second pass), one NaN
    and one infinity."""
    rng = np.random.default_rng(1234 + 77)
    N, L = 3, 300_001
    B = np.log(1.0 - rng.random((N, L))).astype(np.float32)
    A = B.copy()
    sel = rng.random((N, L)) < 0.3
    A[sel] = (A[sel] + rng.normal(0.0, 0.01, sel.sum())).astype(np.float32)
    C = (B + rng.normal(0.0, 1e-3, (N, L))).astype(np.float32)
    big = rng.random((N, L)) < 1e-3
    C[big] = (C[big] - rng.uniform(0.5, 3.0, big.sum())).astype(np.float32)
    M = (rng.random((N, L)) < 0.95).astype(np.uint8)
    M[:, :4096] = 0
    M[2, 250_000:] = 0
    A[0, 123_457] = np.nan
    C[1, 299_999] = np.inf
    M[0, 123_457] = M[1, 299_999] = 1
    return A, B, C, M


def test_long_sequences_compare(long_rows):
    A, B, C, M = long_rows
    got = lp.compare(dev(A), dev(B), dev(C), dev(M), check=False)
    check_stats(got, oracle.compare(A, B, C, M))
    assert got["BC"]["nonfinite"][1] == 1 and got["AB"]["nonfinite"][0] == 1


def test_long_sequences_tails_and_worst_tokens(long_rows):
    A, B, C, M = long_rows
    got, ps, pc = run_tails(A, B, C, M)
    assert ps.shape == (3, A.shape[1])
    run_worst(A, B, C, M, 64)


def test_long_sequences_correct(long_rows):
    A, _, C, M = long_rows
    for kw in (dict(tis_clip=2.0), dict(tis_clip=1.0005, mis_log_lo=-0.0015, mis_log_hi=0.002)):
        w, rec = lp.correct(dev(A), dev(C), dev(M), **kw)
        ref_w, ref = oracle.correct(A, C, M, **kw)
        check_correct(w, rec, ref_w, ref)


def test_many_rows():
    c = synth.tiny_case(T=70_001, H=64, V=1000, seed=91)
    ids = c.ids % 997
    got = gpu_score(c.x_bits, c.w_bits, ids, 0.8, 997)
    ref, _ = oracle.score(c.x_bits, c.w_bits, ids, 0.8, 997)
    assert np.max(np.abs(got - ref)) <= SCORE_ATOL


@pytest.mark.parametrize("T", [5, 40, 300])  # register streaming, LDS streaming, tiles
def test_wide_vocabulary(T):
    c = synth.tiny_case(T=T, H=64, V=1_000_003, seed=92)
    wd = dev_bf16(c.w_bits)
    got = gpu_score(c.x_bits, wd, c.ids, 1.0)
    ref, _ = oracle.score(c.x_bits, c.w_bits, c.ids, 1.0)
    assert np.max(np.abs(got - ref)) <= SCORE_ATOL
    # The same rows scored inside the 300-row batch give the same bits.
    if T < 300:
        big = synth.tiny_case(T=300, H=64, V=1_000_003, seed=93)
        x = big.x_bits.copy(); ids = big.ids.copy()
        x[100:100 + T], ids[100:100 + T] = c.x_bits, c.ids
        inside = gpu_score(x, wd, ids, 1.0)[100:100 + T]
        assert np.array_equal(inside.view(np.int32), got.view(np.int32))


def test_largest_accepted_row_stride():
    # 255 * 2 * ldh + 2 * H <= 0x7FFFFFF0 at H = 64: ldh = 4 210 744 (8.4 MB
    # per row, 2.5 GB for 300 rows). Everything past column 64 is NaN, so a
    # read outside the row's H elements would show. Rows 0..4 scored through
    # the register streaming kernel (T = 5), the LDS streaming kernel (T = 40)
    # and the tile kernel (T = 300) give the same bits and the oracle's value.
    import torch
    H, ldh, T = 64, 4_210_744, 300
    assert 255 * 2 * ldh + 2 * H <= 0x7FFFFFF0 < 255 * 2 * (ldh + 8) + 2 * H
    c = synth.tiny_case(T=T, H=H, V=1000, seed=94)
    buf = torch.full((T, ldh), 0x7FC0, dtype=torch.int16, device=DEV)   # bf16 NaN
    buf[:, :H] = dev(c.x_bits.view(np.int16))
    x = buf.view(torch.bfloat16)
    wd = dev_bf16(c.w_bits)
    ref, _ = oracle.score(c.x_bits, c.w_bits, c.ids, 1.0)
    outs = {}
    for t in (5, 40, T):
        got = gpu_score(x[:t, :H], wd, c.ids[:t], 1.0)
        assert np.max(np.abs(got - ref[:t])) <= SCORE_ATOL, t
        outs[t] = got
    for t in (5, 40):
        assert np.array_equal(outs[t].view(np.int32), outs[T][:t].view(np.int32)), t
    del buf, x
    torch.cuda.empty_cache()
