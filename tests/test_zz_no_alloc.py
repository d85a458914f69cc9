"""lp_score_noalloc (no caller workspace: the library's own device scratch)
against lp_score, through the C ABI: the same bits on calls in a row, each
smaller than the one before (the scratch keeps the previous call's contents),
on the default and on a second stream; the oracle within 1e-3 nats on sampled
rows; a call past the scratch limit refused before anything is enqueued."""

import numpy as np
import pytest
import torch

import oracle
import rollout_logprob_consistency_amd as lp
from rollout_logprob_consistency_amd import _lib
from workloads import synth

from .gpu_helpers import DEV, SCORE_ATOL, dev, dev_bf16

pytestmark = pytest.mark.gpu


def noalloc(x, w, ids, temperature=1.0, stream=None):
    T, H = x.shape
    V = w.shape[0]
    out = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream() if stream is None else stream
    st = _lib.lib().lp_score_noalloc(x.data_ptr(), x.stride(0), w.data_ptr(), ids.data_ptr(),
                                     T, H, V, V, float(temperature), out.data_ptr(),
                                     lse.data_ptr(), None, s.cuda_stream)
    assert st == _lib.LP_OK, lp.status_string(st)
    return out, lse


def with_workspace(x, w, ids, temperature=1.0):
    T = x.shape[0]
    out = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    lp.score(x, w, ids, temperature, out=out, lse=lse)
    return out, lse


def same_bits(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_equals_lp_score_on_calls_in_a_row():
    # Call 1: the Qwen3-8B-shaped batch (T = 8192, H = 4096, V = 151 936):
    # 28.3 MB of the 32 MiB scratch. Call 2: 300 rows of a smaller head (tile
    # kernel). Call 3: 5 rows (streaming kernel), on a second stream.
    big = synth.qwen_case(T=8192, H=4096)
    xb, wb, ib = dev_bf16(big.x_bits), dev_bf16(big.w_bits), dev(big.ids)
    got, got_lse = noalloc(xb, wb, ib)
    ref, ref_lse = with_workspace(xb, wb, ib)
    torch.cuda.synchronize()
    assert same_bits(got, ref) and same_bits(got_lse, ref_lse)
    rows = np.random.default_rng(3).choice(8192, 8, replace=False)
    o, _ = oracle.score(big.x_bits[rows], big.w_bits, big.ids[rows])
    assert np.max(np.abs(got.cpu().numpy()[rows] - o)) <= SCORE_ATOL

    mid = synth.tiny_case(T=300, H=256, V=4096, seed=71)
    xm, wm, im = dev_bf16(mid.x_bits), dev_bf16(mid.w_bits), dev(mid.ids)
    got, got_lse = noalloc(xm, wm, im, 0.7)
    ref, ref_lse = with_workspace(xm, wm, im, 0.7)
    torch.cuda.synchronize()
    assert same_bits(got, ref) and same_bits(got_lse, ref_lse)
    o, _ = oracle.score(mid.x_bits, mid.w_bits, mid.ids, 0.7)
    assert np.max(np.abs(got.cpu().numpy() - o)) <= SCORE_ATOL

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got, got_lse = noalloc(xm[:5], wm, im[:5], 1.3, stream=side)
    side.synchronize()
    ref, ref_lse = with_workspace(xm[:5], wm, im[:5], 1.3)
    torch.cuda.synchronize()
    assert same_bits(got, ref) and same_bits(got_lse, ref_lse)


def test_noalloc_refuses_calls_past_the_scratch():
    # 9698 rows of a 151 936-row head need more than 32 MiB of partials: the
    # library refuses before enqueueing anything (the buffers are real and in
    # bounds all the same).
    T, H, V = 9698, 64, 151936
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((V, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(T, dtype=torch.int64, device=DEV)
    out = torch.zeros(T, dtype=torch.float32, device=DEV)
    st = _lib.lib().lp_score_noalloc(x.data_ptr(), H, w.data_ptr(), ids.data_ptr(), T, H, V, V,
                                     1.0, out.data_ptr(), None, None,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == _lib.LP_EUNSUPPORTED
    torch.cuda.synchronize()
    assert not out.any()
    # One row fewer fits: zero weights give -ln V everywhere.
    st = _lib.lib().lp_score_noalloc(x.data_ptr(), H, w.data_ptr(), ids.data_ptr(), T - 1, H, V,
                                     V, 1.0, out.data_ptr(), None, None,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == _lib.LP_OK
    torch.cuda.synchronize()
    assert torch.allclose(out[:T - 1], torch.full((T - 1,), -float(np.log(V)), device=DEV),
                          atol=1e-5)
    assert out[T - 1].item() == 0.0
