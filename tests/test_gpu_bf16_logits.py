"""GPU parity of the bf16-logit scoring mode (lp_score_ex with
LP_SCORE_BF16_LOGITS) against the oracle's bf16_logits=True, plus its bitwise
contracts: flags 0 / STATS equal lp_score / lp_score_stats, the mode is batch
invariant, and vocabulary shards merge to the same bits. Every call goes
through the C ABI (liblp.so).

Rounding a logit to bf16 is a decision taken on the kernel's fp32 sum. Its
difference from the exact sum grows like a random walk over the H products
(about 2^-24 sqrt(H) |x w|_2; the worst-case bound H 2^-24 sum|x w| would flag
nearly every row at H = 2048). A target logit within 16 times that of a bf16
rounding midpoint may round the other way on the two sides, moving the score
by one bf16 step: those rows (a few percent at most) get that step as extra
tolerance; every other row is held to 1e-3 nats."""

import math

import numpy as np
import pytest
import torch

import oracle
import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import DEV, SCORE_ATOL, dev, dev_bf16

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy()


def slack(x_bits, w_bits, ids, temperature):
    """Extra tolerance per row: one bf16 step of the target logit where its
    fp32 sum may lie on either side of a rounding midpoint, else 0."""
    x = oracle.bf16_bits_to_f64(x_bits)
    w = oracle.bf16_bits_to_f64(w_bits[ids])
    prod = x * w
    z = prod.sum(axis=1)
    err = 16 * 2.0**-24 * math.sqrt(x.shape[1]) * np.sqrt((prod ** 2).sum(axis=1)) \
        + 2.0**-24 * np.abs(z)
    step = np.array([2.0 ** (math.frexp(v)[1] - 8) if v != 0 else 0.0 for v in z])
    lo = oracle.round_to_bf16(z)
    mid = np.where(lo <= z, lo + step / 2, lo - step / 2)
    amb = np.abs(z - mid) <= err
    return np.where(amb, step / temperature, 0.0), int(amb.sum())


def check_parity(c, temperature, v_true=None, rows=None):
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    got = lp.score_ex(x, w, ids, temperature, v_true, bf16_logits=True).cpu().numpy()
    xb, idb = (c.x_bits, c.ids) if rows is None else (c.x_bits[rows], c.ids[rows])
    if rows is not None:
        got = got[rows]
    ref, _ = oracle.score(xb, c.w_bits, idb, temperature, v_true, bf16_logits=True)
    extra, n_amb = slack(xb, c.w_bits, idb, temperature)
    assert (np.abs(got - ref) <= SCORE_ATOL + extra).all()
    assert n_amb <= max(2, len(idb) // 10)
    plain, _ = oracle.score(xb, c.w_bits, idb, temperature, v_true)
    return got, ref, plain


@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_tiny_stream_path(temperature):
    c = synth.tiny_case(temperature=temperature)
    got, ref, plain = check_parity(c, temperature)
    assert np.max(np.abs(ref - plain)) > 1e-4       # the mode changes the scores


@pytest.mark.parametrize("T", [1, 300])
def test_tile_path_ragged_padded(T):
    c = synth.tiny_case(T=T, H=256, V=20000, seed=3)
    c.ids = np.minimum(c.ids, 19989)
    check_parity(c, 0.7, 19990)


def test_qwen_shaped_sampled_rows():
    c = synth.qwen_case(T=512, H=2048)
    rows = np.random.default_rng(12).choice(512, 8, replace=False)
    check_parity(c, 1.0, rows=rows)


def test_closed_form_rounding_rules():
    # x = (1, 1, 0, ...), W row v = (1, b_v, 0, ...): z_v = 1 + b_v exactly in
    # fp32; bf16 rounds 1 + 2^-8 (tie) to 1, 1 + 3 2^-9 up, 1 + 2^-10 down.
    H, V = 64, 4
    bs = [2.0**-8, 3 * 2.0**-9, 2.0**-10, 0.0]
    wf = np.zeros((V, H), np.float32)
    wf[:, 0] = 1.0
    wf[:, 1] = bs
    xf = np.zeros((4, H), np.float32)
    xf[:, :2] = 1.0
    xb, wb = synth.bf16_bits_from_f32(xf), synth.bf16_bits_from_f32(wf)
    ids = np.arange(4)
    zr = np.array([1.0, 1 + 2**-7, 1.0, 1.0])
    want = zr - math.log(np.exp(zr).sum())
    got = lp.score_ex(dev_bf16(xb), dev_bf16(wb), dev(ids), bf16_logits=True).cpu().numpy()
    assert np.max(np.abs(got - want)) < 1e-6
    plain = lp.score(dev_bf16(xb), dev_bf16(wb), dev(ids)).cpu().numpy()
    assert abs(plain[0] - got[0]) > 1e-4


def test_flags_reproduce_lp_score_and_lp_score_stats():
    c = synth.tiny_case(T=300, H=256, V=4096, seed=5)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    for temp in (1.0, 0.7):
        a = lp.score(x, w, ids, temp)
        b = lp.score_ex(x, w, ids, temp)
        assert np.array_equal(bits(a), bits(b))
        s = lp.score_stats(x, w, ids, temp)
        e = lp.score_ex(x, w, ids, temp, stats=True)
        assert np.array_equal(bits(s[0]), bits(e[0])) and np.array_equal(bits(s[1]), bits(e[1]))
        assert torch.equal(s[2], e[2])
        # Stats do not change the bf16-mode logprob either.
        f = lp.score_ex(x, w, ids, temp, bf16_logits=True)
        g = lp.score_ex(x, w, ids, temp, stats=True, bf16_logits=True)
        assert np.array_equal(bits(f), bits(g[0]))
        assert np.isfinite(g[1].cpu().numpy()).all()


def test_bf16_mode_is_batch_invariant():
    c = synth.tiny_case(T=700, H=256, V=4096, seed=6)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    full = bits(lp.score_ex(x, w, ids, bf16_logits=True))
    for lo, hi in ((0, 1), (5, 12), (10, 26), (30, 47), (40, 72), (50, 83), (100, 164),
                   (200, 600), (0, 700)):
        part = bits(lp.score_ex(x[lo:hi].contiguous(), w, ids[lo:hi].contiguous(),
                                bf16_logits=True))
        assert np.array_equal(part, full[lo:hi]), (lo, hi)


@pytest.mark.parametrize("stats", [False, True])
def test_bf16_vocabulary_shards_bitwise(stats):
    c = synth.tiny_case(T=200, H=256, V=20000, seed=7)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    ref = lp.score_ex(x, w, ids, 0.9, stats=stats, bf16_logits=True)
    for n in (3, 8):
        parts = lp.shard_partials(200, stats, DEV)
        parts.fill_(float("nan"))
        for r in range(n):
            sh = lp.vocab_shard(20000, n, r)
            lp.score_shard(x, w[sh["row_begin"]:sh["row_end"]].clone(), ids, 20000, n, r, parts,
                           0.9, stats, bf16_logits=True)
        got = lp.merge_shards(parts, ids, 20000, stats)
        if stats:
            assert np.array_equal(bits(got[0]), bits(ref[0]))
            assert np.array_equal(bits(got[1]), bits(ref[1]))
            assert torch.equal(got[2], ref[2])
        else:
            assert np.array_equal(bits(got), bits(ref))
