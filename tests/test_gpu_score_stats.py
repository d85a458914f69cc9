"""GPU parity of lp_score_stats (logprob, entropy, argmax in one fused pass)
against the fp64 oracle, closed forms, tie-breaking, and bitwise batch
invariance. Every call goes through the C ABI (liblp.so)."""

import math

import numpy as np
import pytest
import torch

import oracle
import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import DEV, SCORE_ATOL, dev, dev_bf16, gpu_score

pytestmark = pytest.mark.gpu

# Entropy is a nats quantity like the logprob: same tolerance.
ENT_ATOL = SCORE_ATOL
# The fp32 logits the kernel forms differ from the fp64 ones by far less than
# this (H <= 4096 products of bf16 values, fp32 accumulation); where the two
# largest oracle logits are closer than this, either may be the argmax.
TIE_GAP = 1e-3


def gpu_stats(x_bits, w, ids, temperature=1.0, v_true=None):
    """Run lp_score_stats; outputs pre-filled with sentinels so an unwritten
    element cannot pass. Returns numpy (logprob, entropy, argmax)."""
    w = w if isinstance(w, torch.Tensor) else dev_bf16(w)
    x = x_bits if isinstance(x_bits, torch.Tensor) else dev_bf16(x_bits)
    out, ent, am = lp.score_stats(x, w, dev(np.asarray(ids, np.int64)), temperature, v_true)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ent.cpu().numpy(), am.cpu().numpy()


def check_argmax(got, z):
    """got == the oracle's argmax where the top two logits are TIE_GAP apart;
    otherwise got must be one of the rows within TIE_GAP of the maximum."""
    ref = np.argmax(z, axis=1)
    top2 = np.sort(z, axis=1)[:, -2:] if z.shape[1] > 1 else np.stack([z[:, 0] - 1, z[:, 0]], 1)
    clear = (top2[:, 1] - top2[:, 0]) > TIE_GAP
    assert np.array_equal(got[clear], ref[clear])
    rows = np.arange(z.shape[0])
    assert np.all(z[rows, got] >= z.max(axis=1) - TIE_GAP)
    return int(clear.sum())


@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_tiny_parity(temperature):
    c = synth.tiny_case(temperature=temperature)
    got_lp, got_ent, got_am = gpu_stats(c.x_bits, c.w_bits, c.ids, temperature)
    ref_lp, _, ref_ent, _ = oracle.score_stats(c.x_bits, c.w_bits, c.ids, temperature)
    assert np.max(np.abs(got_lp - ref_lp)) <= SCORE_ATOL
    assert np.isfinite(got_ent).all()
    assert np.max(np.abs(got_ent - ref_ent)) <= ENT_ATOL
    assert check_argmax(got_am, oracle.logits(c.x_bits, c.w_bits)) >= 60


def test_logprob_bits_equal_lp_score():
    c = synth.tiny_case(T=300, H=256, V=4096, seed=3)
    a = gpu_score(c.x_bits, c.w_bits, c.ids, 0.8)
    b, _, _ = gpu_stats(c.x_bits, c.w_bits, c.ids, 0.8)
    assert np.array_equal(a.view(np.int32), b.view(np.int32))
    a1 = gpu_score(c.x_bits[:5], c.w_bits, c.ids[:5], 0.8)          # streaming kernel
    b1, _, _ = gpu_stats(c.x_bits[:5], c.w_bits, c.ids[:5], 0.8)
    assert np.array_equal(a1.view(np.int32), b1.view(np.int32))


@pytest.mark.parametrize("T", [3, 70])
def test_uniform_rows_and_lowest_index_ties(T):
    # Zero weights: every logit is 0 -- entropy ln V_true, and every index
    # ties, so the argmax must be 0 through every lane, wave, tile and merge.
    c = synth.tiny_case(T=T, H=128, V=4096)
    for v_true in (4096, 1000):
        _, ent, am = gpu_stats(c.x_bits, np.zeros_like(c.w_bits), c.ids % v_true, 0.6, v_true)
        assert np.max(np.abs(ent.astype(np.float64) - math.log(v_true))) <= 1e-5
        assert np.array_equal(am, np.zeros(T, np.int64))


@pytest.mark.parametrize("T", [3, 70])
def test_two_level_closed_form(T):
    V, H, k, target, a, b = 3000, 64, 9, 2049, 1.5, -0.25
    x = np.zeros((T, H), np.float32); x[:, k] = 1.0
    w = np.zeros((V, H), np.float32); w[:, k] = b; w[target, k] = a
    for T_ in (1.0, 0.5):
        _, ent, am = gpu_stats(synth.bf16_bits_from_f32(x), synth.bf16_bits_from_f32(w),
                               np.zeros(T, np.int64), T_)
        za, zb = a / T_, b / T_
        Z = math.exp(za) + (V - 1) * math.exp(zb)
        p1, p2 = math.exp(za) / Z, math.exp(zb) / Z
        expect = -p1 * math.log(p1) - (V - 1) * p2 * math.log(p2)
        assert np.max(np.abs(ent - expect)) <= 1e-5
        assert np.all(am == target)
    # The single logit now the smallest: 2999 tied maxima, the lowest is 0.
    w[:, k] = a; w[target, k] = b
    _, _, am = gpu_stats(synth.bf16_bits_from_f32(x), synth.bf16_bits_from_f32(w),
                         np.zeros(T, np.int64), 1.0)
    assert np.all(am == 0)


@pytest.mark.parametrize("T,H,V,v_true", [
    (1, 64, 4096, 4096), (7, 128, 1000, 1000), (255, 256, 4096, 3000),
    (257, 192, 513, 513), (300, 256, 300, 129), (520, 64, 257, 1),
])
def test_ragged_shapes_and_padding(T, H, V, v_true):
    c = synth.tiny_case(T=T, H=H, V=V, seed=T + 1)
    w = c.w_bits.copy()
    if v_true < V:
        # Padded rows past v_true get the largest logits of the head: they
        # must neither win the argmax nor enter the entropy.
        wf = synth.f32_from_bf16_bits(w).copy()
        wf[v_true:] = 4.0 * np.abs(wf[v_true:]) * np.sign(synth.f32_from_bf16_bits(c.x_bits)[0])
        w = synth.bf16_bits_from_f32(wf)
    ids = c.ids % v_true
    got_lp, got_ent, got_am = gpu_stats(c.x_bits, w, ids, 0.9, v_true)
    ref_lp, _, ref_ent, _ = oracle.score_stats(c.x_bits, w, ids, 0.9, v_true)
    assert np.max(np.abs(got_lp - ref_lp)) <= SCORE_ATOL
    assert np.max(np.abs(got_ent - ref_ent)) <= ENT_ATOL
    check_argmax(got_am, oracle.logits(c.x_bits, w, v_true))
    assert np.all((got_am >= 0) & (got_am < v_true))


@pytest.fixture(scope="module")
def qwen17b():
    c = synth.qwen_case(T=4096, H=2048)
    return c, dev_bf16(c.w_bits), dev_bf16(c.x_bits)


def test_qwen17b_shaped_sampled_rows(qwen17b):
    c, wd, xd = qwen17b
    got_lp, got_ent, got_am = gpu_stats(xd, wd, c.ids, 1.0)
    assert np.isfinite(got_ent).all() and (got_ent >= 0).all()
    assert (got_ent <= math.log(151936) + 1e-3).all()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095],
                                     np.random.default_rng(5).choice(4096, 59, replace=False)]))
    ref_lp, _, ref_ent, _ = oracle.score_stats(c.x_bits[rows], c.w_bits, c.ids[rows], 1.0)
    assert np.max(np.abs(got_lp[rows] - ref_lp)) <= SCORE_ATOL
    assert np.max(np.abs(got_ent[rows] - ref_ent)) <= ENT_ATOL
    check_argmax(got_am[rows], oracle.logits(c.x_bits[rows], c.w_bits))


def test_batch_invariance(qwen17b):
    # 48 probe rows at random positions inside batches of 1, 7, 16, 17, 32,
    # 33, 64 (streaming kernels: 16- and 32-token items in registers, 64 in
    # LDS) and 300, 4096 rows (352 x 256 tiles): bitwise equal outputs.
    c, wd, _ = qwen17b
    rng = np.random.default_rng(9)
    probes = rng.choice(c.T, 48, replace=False)
    res = {}
    for b in (1, 7, 16, 17, 32, 33, 64, 300, 4096):
        k = min(48, -(-b // 2))
        g = [np.zeros(48, np.float32), np.zeros(48, np.float32), np.zeros(48, np.int64)]
        for s in range(0, 48, k):
            sel = np.arange(s, min(s + k, 48))
            pos = rng.permutation(b)[:len(sel)]
            fill = rng.choice(c.T, b, replace=False)
            x, ids = c.x_bits[fill].copy(), c.ids[fill].copy()
            x[pos], ids[pos] = c.x_bits[probes[sel]], c.ids[probes[sel]]
            o = gpu_stats(x, wd, ids, 0.7)
            for dst, src in zip(g, o):
                dst[sel] = src[pos]
        res[b] = g
    base = res[4096]
    for b, g in res.items():
        assert np.array_equal(g[0].view(np.int32), base[0].view(np.int32)), b
        assert np.array_equal(g[1].view(np.int32), base[1].view(np.int32)), b
        assert np.array_equal(g[2], base[2]), b
