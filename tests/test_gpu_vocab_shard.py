"""GPU parity of vocabulary-parallel scoring (lp_score_shard + lp_merge_shards)
with canonical chunking: for every shard count the merged results are
BITWISE equal to lp_score / lp_score_stats on the whole W (fp32 bits compared
as int32), and within 1e-3 nats of the fp64 oracle. Every shard scores its
own copy of its rows, so no shard can read another's. Every call goes through
the C ABI (liblp.so)."""

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


def sharded(x, w, ids, v_true, n, stats=False, temperature=1.0, order=None, parts=None):
    """Score every shard into one exchange buffer (what an all-gather of the
    ranks' blocks produces), then merge. Returns merge outputs + lse."""
    T = x.shape[0]
    if parts is None:
        parts = lp.shard_partials(T, stats, DEV)
    parts.fill_(float("nan"))  # sentinel: every record must be written
    for r in (order if order is not None else range(n)):
        sh = lp.vocab_shard(v_true, n, r)
        w_own = w[sh["row_begin"]:sh["row_end"]].clone()
        lp.score_shard(x, w_own, ids, v_true, n, r, parts, temperature, stats)
    lse = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    out = lp.merge_shards(parts, ids, v_true, stats, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def one_buffer(x, w, ids, v_true, stats=False, temperature=1.0):
    T = x.shape[0]
    lse = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    if stats:
        out = lp.score_stats(x, w, ids, temperature, v_true, lse=lse)
    else:
        out = lp.score(x, w, ids, temperature, v_true, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def assert_same(a, b):
    (oa, la), (ob, lb) = a, b
    if isinstance(oa, tuple):
        assert np.array_equal(bits(oa[0]), bits(ob[0])), "logprob bits"
        assert np.array_equal(bits(oa[1]), bits(ob[1])), "entropy bits"
        assert torch.equal(oa[2], ob[2]), "argmax"
    else:
        assert np.array_equal(bits(oa), bits(ob)), "logprob bits"
    assert np.array_equal(bits(la), bits(lb)), "lse bits"


SHARD_COUNTS = [1, 2, 3, 4, 5, 8, 16]


@pytest.mark.parametrize("stats", [False, True])
def test_tiny_stream_path_all_shard_counts(stats):
    # T = 64 takes the streaming kernel (half-tile partials).
    c = synth.tiny_case()
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    ref = one_buffer(x, w, ids, 4096, stats)
    for n in SHARD_COUNTS:
        assert_same(sharded(x, w, ids, 4096, n, stats), ref)
    got = ref[0][0] if stats else ref[0]
    want = oracle.score(c.x_bits, c.w_bits, c.ids)[0]
    assert np.max(np.abs(got.cpu().numpy() - want)) <= SCORE_ATOL


@pytest.mark.parametrize("T", [1, 33, 300])
@pytest.mark.parametrize("stats", [False, True])
def test_ragged_tokens_padded_vocab_temperature(T, stats):
    # T = 300: 352 x 256 tiles with a ragged token tail; V_true < V_rows, so
    # the one-buffer W has padding rows that the shards never hold.
    H, V, v_true, temp = 256, 20000, 19990, 0.7
    c = synth.tiny_case(T=T, H=H, V=V, seed=3, temperature=temp)
    ids = np.minimum(c.ids, v_true - 1)
    x, w, idd = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(ids)
    ref = one_buffer(x, w, idd, v_true, stats, temp)
    for n in (2, 5, 16):
        assert_same(sharded(x, w, idd, v_true, n, stats, temp), ref)
    want = oracle.score(c.x_bits, c.w_bits, ids, temp, v_true)[0]
    got = (ref[0][0] if stats else ref[0]).cpu().numpy()
    assert np.max(np.abs(got - want)) <= SCORE_ATOL


def test_small_vocabulary_with_empty_shards():
    # 1000 rows = 3 tiles: with 8 or 16 shards most shards own no rows and
    # still write their (empty) segment records.
    c = synth.tiny_case(T=40, H=128, V=1000, seed=4)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    for stats in (False, True):
        ref = one_buffer(x, w, ids, 1000, stats)
        for n in (3, 8, 16):
            assert_same(sharded(x, w, ids, 1000, n, stats), ref)


def test_shard_order_and_buffer_reuse():
    # The merge depends on the records only: shards scored in any order, into
    # a buffer that held another batch's records, give the same bits.
    c = synth.tiny_case(T=200, H=256, V=4096, seed=5)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    ref = one_buffer(x, w, ids, 4096)
    parts = lp.shard_partials(200, False, DEV)
    assert_same(sharded(x, w, ids, 4096, 8, order=[7, 0, 3, 5, 1, 6, 2, 4], parts=parts), ref)
    assert_same(sharded(x, w, ids, 4096, 8, order=range(7, -1, -1), parts=parts), ref)


def test_qwen_shaped_eight_shards():
    # Qwen3-1.7B-shaped head (H = 2048, V = 151 936), 512 rows, 8 shards of
    # 19 008 rows (the last 18 880): bitwise equal to the one-buffer call;
    # sampled rows against the oracle.
    c = synth.qwen_case(T=512, H=2048)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    for stats in (False, True):
        ref = one_buffer(x, w, ids, 151936, stats)
        assert_same(sharded(x, w, ids, 151936, 8, stats), ref)
    rows = np.random.default_rng(11).choice(512, 6, replace=False)
    want = oracle.score(c.x_bits[rows], c.w_bits, c.ids[rows])[0]
    got = ref[0][0].cpu().numpy()[rows]
    assert np.max(np.abs(got - want)) <= SCORE_ATOL


def test_bad_target_ids_flagged_in_the_merge():
    c = synth.tiny_case(T=50, seed=6)
    ids = c.ids.copy()
    ids[[3, 17, 40]] = [-1, 4096, 10**12]
    x, w, idd = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(ids)
    ref, _ = one_buffer(x, w, idd, 4096)
    got, _ = sharded(x, w, idd, 4096, 4)
    assert np.array_equal(bits(got), bits(ref))
    assert np.isnan(got.cpu().numpy()[[3, 17, 40]]).all()
    parts = lp.shard_partials(50, False, DEV)
    for r in range(4):
        sh = lp.vocab_shard(4096, 4, r)
        lp.score_shard(x, w[sh["row_begin"]:sh["row_end"]].clone(), idd, 4096, 4, r, parts)
    with pytest.raises(ValueError):
        lp.merge_shards(parts, idd, 4096, check=True)


def test_binding_rejects_wrong_shapes():
    c = synth.tiny_case(T=8, seed=7)
    x, w, ids = dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)
    parts = lp.shard_partials(8, False, DEV)
    rows = lp.vocab_shard(4096, 4, 0)["row_end"]   # shard 0 of 4: its rows start at 0
    with pytest.raises(ValueError):       # rows of another shard
        lp.score_shard(x, w[:rows - 24].clone(), ids, 4096, 4, 0, parts)
    with pytest.raises(ValueError):       # stats buffer expected
        lp.score_shard(x, w[:rows].clone(), ids, 4096, 4, 0, parts, stats=True)
    with pytest.raises(lp.LpError):
        lp.score_shard(x, w[:rows].clone(), ids, 4096, 4, 0, parts, temperature=0.0)
