"""The library keeps no state, so calls on different streams, concurrently,
and calls captured into a HIP graph and replayed give the bits of an eager
call on the default stream. Every call goes through the C ABI (liblp.so)."""

import ctypes

import numpy as np
import pytest
import torch

import rollout_logprob_consistency_amd as lp
from workloads import synth

from .gpu_helpers import DEV, dev, dev_bf16

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy()


@pytest.fixture(scope="module")
def batch():
    c = synth.qwen_case(T=1100, H=1024, V=20000, seed=5)
    return dev_bf16(c.x_bits), dev_bf16(c.w_bits), dev(c.ids)


def test_concurrent_streams_give_the_default_stream_bits(batch):
    x, w, ids = batch
    T, H = x.shape
    V = w.shape[0]
    ref = lp.score(x, w, ids)
    small = lp.score(x[:37], w, ids[:37])        # the streaming kernel
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs, wss = [], []
    for s in streams:
        outs.append((torch.full((T,), float("nan"), device=DEV),
                     torch.full((37,), float("nan"), device=DEV)))
        wss.append((torch.empty(lp.score_workspace_bytes(T, H, V, V), dtype=torch.uint8, device=DEV),
                    torch.empty(lp.score_workspace_bytes(37, H, V, V), dtype=torch.uint8, device=DEV)))
    torch.cuda.synchronize()
    for rep in range(2):
        for s, (o, o_small), (ws, ws_small) in zip(streams, outs, wss):
            with torch.cuda.stream(s):
                lp.score(x, w, ids, out=o, workspace=ws)
                lp.score(x[:37], w, ids[:37], out=o_small, workspace=ws_small)
        torch.cuda.synchronize()
        for o, o_small in outs:
            assert np.array_equal(bits(o), bits(ref))
            assert np.array_equal(bits(o_small), bits(small))


def test_graph_capture_and_replay(batch):
    """lp_score, lp_compare and lp_compare_tails_ex captured into one graph and
    replayed three times, with other eager work and synchronisations between
    the replays; every replay gives the eager results bit for bit."""
    x, w, ids = batch
    T, H = x.shape
    V = w.shape[0]
    rec = synth.compare_case(N=6, max_resp=500, prompt=32, seed=9)
    A, B, M = dev(rec.A), dev(rec.B), dev(rec.mask)
    C = dev(synth.noise_scores(rec.C, rec.mask, 1e-3, seed=9))
    N, L = rec.A.shape
    k = 8

    out = torch.empty(T, dtype=torch.float32, device=DEV)
    lse = torch.empty(T, dtype=torch.float32, device=DEV)
    ws = torch.empty(lp.score_workspace_bytes(T, H, V, V), dtype=torch.uint8, device=DEV)
    stats = torch.empty(3 * N * lp.SEQ_STATS_DTYPE.itemsize, dtype=torch.uint8, device=DEV)
    tout = torch.empty(3 * lp.TAIL_STATS_DTYPE.itemsize, dtype=torch.uint8, device=DEV)
    worst = torch.empty(3 * k * lp.WORST_DTYPE.itemsize, dtype=torch.uint8, device=DEV)
    tws = torch.empty(lp._lib.lib().lp_compare_tails_ex_workspace_bytes(N, L, k),
                      dtype=torch.uint8, device=DEV)
    L_ = lp._lib.lib()

    def step():
        s = torch.cuda.current_stream().cuda_stream
        lp.score(x, w, ids, out=out, lse=lse, workspace=ws)
        assert L_.lp_compare(A.data_ptr(), B.data_ptr(), C.data_ptr(), M.data_ptr(), N, L, L, 2.0,
                             -1.0, stats.data_ptr(), None, s) == 0
        assert L_.lp_compare_tails_ex(A.data_ptr(), B.data_ptr(), C.data_ptr(), M.data_ptr(), N, L,
                                      L, k, tout.data_ptr(), worst.data_ptr(), None, None,
                                      tws.data_ptr(), tws.numel(), s) == 0

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (out, lse, stats, tout, worst)]

    def poison():
        for t in (out, lse):
            t.fill_(float("nan"))
        for t in (stats, tout, worst):
            t.fill_(0xAB)

    step()
    eager = snapshot()
    poison()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()                                  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        poison()
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for e, r in zip(eager, got):
            assert torch.equal(e.view(torch.uint8), r.view(torch.uint8)), rep
        del junk
