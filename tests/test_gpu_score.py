"""GPU parity of lp_score against the fp64 oracle, edge cases, and bitwise
batch invariance. Every call goes through the C ABI (liblp.so)."""

import math

import numpy as np
import pytest
import torch

import oracle
import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import DEV, SCORE_ATOL, dev, dev_bf16, gpu_score

pytestmark = pytest.mark.gpu


def oracle_f64(case, rows=None, temperature=None, v_true=None):
    x = case.x_bits if rows is None else case.x_bits[rows]
    ids = case.ids if rows is None else case.ids[rows]
    t = case.temperature if temperature is None else temperature
    return oracle.score(x, case.w_bits, ids, t, v_true)


# --------------------------------------------------------------------------
# Tiny fused logprob: T=64, H=256, V=4096, full parity.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("temperature", [1.0, 0.7, 1.3])
def test_tiny_full_parity(temperature):
    c = synth.tiny_case(temperature=temperature)
    got, got_lse = gpu_score(c.x_bits, c.w_bits, c.ids, temperature, lse=True)
    ref, ref_lse = oracle_f64(c)
    assert np.isfinite(got).all() and np.isfinite(got_lse).all()
    assert np.max(np.abs(got - ref)) <= SCORE_ATOL
    assert np.max(np.abs(got_lse - ref_lse)) <= SCORE_ATOL


@pytest.mark.parametrize("T,H,V,v_true,ldh", [
    (1, 64, 4096, 4096, 64),        # single row, minimum H
    (7, 128, 1000, 1000, 128),      # ragged vocabulary tail (1000 = 2*352 + 296, in the upper half)
    (255, 256, 4096, 3000, 256),    # true vocabulary range shorter than the head
    (257, 192, 353, 353, 200),      # two token tiles, 1-row-deep last vocab tile, strided rows
    (257, 64, 513, 513, 64),        # last vocab tile 161 rows deep: inside its lower half
    (300, 256, 300, 129, 256),      # tail inside the first vocabulary half
    (300, 128, 400, 177, 128),      # tail one row into the second half of the first tile
    (300, 128, 704, 528, 128),      # tail exactly at a half boundary (528 = 352 + 176)
    (520, 64, 257, 1, 64),          # one-token vocabulary
    (5, 128, 1000, 1000, 136),      # strided rows, register streaming kernel (16-token items)
    (29, 64, 705, 700, 72),         # strided rows, register streaming kernel (32-token items)
    (40, 192, 800, 777, 200),       # strided rows, LDS streaming kernel, tail in the upper half
])
def test_ragged_shapes(T, H, V, v_true, ldh):
    c = synth.tiny_case(T=T, H=H, V=V, seed=T)
    ids = c.ids % v_true
    buf = np.zeros((T, ldh), np.uint16)
    buf[:, :H] = c.x_bits
    xd = dev_bf16(buf)[:, :H]                       # row stride ldh
    got = gpu_score(xd, c.w_bits, ids, 0.9, v_true)
    ref, _ = oracle.score(c.x_bits, c.w_bits, ids, 0.9, v_true)
    assert np.max(np.abs(got - ref)) <= SCORE_ATOL


def test_zero_weights_give_minus_log_v():
    c = synth.tiny_case(T=70, H=128, V=4096)
    for v_true in (4096, 1000):
        got = gpu_score(c.x_bits, np.zeros_like(c.w_bits), c.ids % v_true, 0.6, v_true)
        assert np.max(np.abs(got.astype(np.float64) + math.log(v_true))) <= 1e-5


def test_probabilities_sum_to_one():
    # One row scored against every target: replicas are legitimate because
    # every row's result is independent of the batch.
    c = synth.tiny_case()
    rows = np.repeat(c.x_bits[5:6], c.V, axis=0)
    got = gpu_score(rows, c.w_bits, np.arange(c.V), 0.8)
    assert abs(math.fsum(np.exp(got.astype(np.float64))) - 1.0) < 1e-4
    ref, _ = oracle.score(c.x_bits[5:6], c.w_bits, np.arange(c.V)[:1], 0.8)
    assert abs(got[0] - ref[0]) <= SCORE_ATOL


def test_two_level_closed_form():
    V, H, k, target, a, b = 3000, 64, 9, 2049, 1.5, -0.25
    x = np.zeros((3, H), np.float32); x[:, k] = 1.0
    w = np.zeros((V, H), np.float32); w[:, k] = b; w[target, k] = a
    for T_ in (1.0, 0.5):
        got = gpu_score(synth.bf16_bits_from_f32(x), synth.bf16_bits_from_f32(w),
                        np.array([target, 0, V - 1]), T_)
        norm = math.log(math.exp(a / T_) + (V - 1) * math.exp(b / T_))
        assert abs(got[0] - (a / T_ - norm)) <= 1e-5
        assert abs(got[1] - (b / T_ - norm)) <= 1e-5 and got[1] == got[2]


def test_bad_target_ids_flagged():
    c = synth.tiny_case(T=10)
    ids = c.ids.copy()
    ids[3], ids[7] = -1, 4096
    x, w = dev_bf16(c.x_bits), dev_bf16(c.w_bits)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = lp.score(x, w, dev(ids), bad_rows=bad)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert int(bad.item()) == 2
    assert np.isnan(o[3]) and np.isnan(o[7]) and np.isfinite(np.delete(o, [3, 7])).all()
    with pytest.raises(ValueError):
        lp.score(x, w, dev(ids), check=True)
    # Valid rows are unaffected by the bad ones.
    ref, _ = oracle.score(c.x_bits, c.w_bits, np.where((ids < 0) | (ids >= 4096), 0, ids))
    good = np.array([i not in (3, 7) for i in range(10)])
    assert np.max(np.abs(o[good] - ref[good])) <= SCORE_ATOL


def test_empty_batch_is_a_noop():
    w = torch.zeros(256, 64, dtype=torch.bfloat16, device=DEV)
    out = lp.score(torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV), w,
                   torch.zeros(0, dtype=torch.int64, device=DEV))
    assert out.shape == (0,)


# --------------------------------------------------------------------------
# Qwen3-shaped scoring (vocabulary 151 936): sampled rows against the oracle.
# --------------------------------------------------------------------------

def sample_rows(T, n, seed):
    """Tile edges, one random row of every 256-row token tile (so a fault in
    any tile shows), and random rows up to n."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 255, 256, T - 257, T - 256, T - 1]
    per_tile = np.arange(0, T, 256) + rng.integers(0, 256, size=-(-T // 256))
    per_tile = per_tile[per_tile < T]
    rest = rng.choice(T, size=max(0, n - len(fixed) - len(per_tile)), replace=False)
    return np.unique(np.concatenate([fixed, per_tile, rest]))


@pytest.fixture(scope="module")
def qwen17b():
    c = synth.qwen_case(T=4096, H=2048)
    return c, dev_bf16(c.w_bits), dev_bf16(c.x_bits)


@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_qwen17b_shaped_parity(qwen17b, temperature):
    c, wd, xd = qwen17b
    got = gpu_score(xd, wd, c.ids, temperature)
    assert np.isfinite(got).all() and (got <= 0).all()
    rows = sample_rows(c.T, 256, seed=17)
    ref, _ = oracle_f64(c, rows, temperature)
    assert np.max(np.abs(got[rows] - ref)) <= SCORE_ATOL


@pytest.fixture(scope="module")
def qwen8b():
    w = synth.qwen_weight(4096)
    c = synth.qwen_case(T=8192, H=4096, w_bits=w)
    return c, dev_bf16(w), dev_bf16(c.x_bits)


def test_qwen8b_shaped_parity_and_repeatability(qwen8b):
    c, wd, xd = qwen8b
    got = gpu_score(xd, wd, c.ids)
    again = gpu_score(xd, wd, c.ids)
    assert np.array_equal(got.view(np.int32), again.view(np.int32))   # run to run
    assert np.isfinite(got).all() and (got <= 0).all()
    rows = sample_rows(c.T, 96, seed=8)          # every one of the 32 token tiles
    ref, _ = oracle_f64(c, rows)
    assert np.max(np.abs(got[rows] - ref)) <= SCORE_ATOL


def test_qwen8b_shaped_parity_every_row(qwen8b):
    """All 8192 rows of the Qwen3-8B-shaped batch against the fp64 oracle
    (in 512-row blocks of fp64 logits), so a fault confined to some token or
    vocabulary tiles cannot pass on sampled rows."""
    c, wd, xd = qwen8b
    got = gpu_score(xd, wd, c.ids)
    worst = 0.0
    for r0 in range(0, c.T, 512):
        z = oracle.logits(c.x_bits[r0:r0 + 512], c.w_bits)
        ref, _ = oracle.log_softmax_at(z, c.ids[r0:r0 + 512], c.temperature)
        worst = max(worst, float(np.max(np.abs(got[r0:r0 + 512] - ref))))
        del z
    assert worst <= SCORE_ATOL, worst


# --------------------------------------------------------------------------
# Batch invariance: 512 fixed probe rows at random positions inside batches
# of 1, 7, 64, 512 and 8192 rows, twice each; 16, 17, 32 and 33 rows sit on
# either side of the streaming kernels' item sizes (16 and 32 tokens in
# registers, 64 through LDS).
# --------------------------------------------------------------------------

def test_batch_invariance_sweep(qwen8b):
    c8, wd, _ = qwen8b
    H, V = 4096, 151936
    px, pids = synth.probe_set(H, V)
    fx, fids = synth.filler_rows(0, 8192, H, V)
    rng = np.random.default_rng(4)
    results = {}
    for b in (1, 7, 16, 17, 32, 33, 64, 512, 8192):
        k = min(512, -(-b // 2))
        for rep in range(2):
            got = np.full(512, np.nan, np.float32)
            for start in range(0, 512, k):
                probes = np.arange(start, min(start + k, 512))
                pos = rng.permutation(b)[:len(probes)]
                x = fx[rng.choice(8192, b, replace=False)].copy()
                ids = fids[rng.choice(8192, b, replace=False)].copy()
                x[pos], ids[pos] = px[probes], pids[probes]
                out = gpu_score(x, wd, ids)
                got[probes] = out[pos]
            results[(b, rep)] = got
    base = results[(8192, 0)]
    for key, got in results.items():
        assert np.array_equal(got.view(np.int32), base.view(np.int32)), key
    ref, _ = oracle.score(px, c8.w_bits, pids)
    assert np.max(np.abs(base - ref)) <= SCORE_ATOL
