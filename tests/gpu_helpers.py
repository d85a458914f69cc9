"""Helpers shared by the GPU parity tests: move seeded numpy inputs to the
device and run the library through its binding (which calls the C ABI)."""

import numpy as np
import torch

import rollout_logprob_consistency_amd as lp

DEV = "cuda:0"
INT_FIELDS = ("valid", "mismatch", "first_div", "longest_run", "nonfinite", "k3_nonfinite")
# fp64 sums in a fixed order: compared at 1e-9 relative, except the two whose
# per-token terms are evaluated in fp32 for |d| < 0.5 (k3 by its Taylor series,
# exp(d) by exp2), compared at 1e-6 relative.
SUM_RTOL = {"sum_abs": 1e-9, "sum_signed": 1e-9, "sum_d": 1e-9, "seq_tis": 1e-9,
            "sum_k3": 1e-6, "sum_tok_tis": 1e-6}
# Score tolerance: max |GPU - fp64 oracle| in nats.
SCORE_ATOL = 1e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_score(x_bits, w_dev_or_bits, ids, temperature=1.0, v_true=None, lse=False):
    """Run lp_score; returns numpy fp32 logprob (and lse). Output buffers are
    pre-filled with a NaN sentinel so an unexercised path cannot pass."""
    w = w_dev_or_bits if isinstance(w_dev_or_bits, torch.Tensor) else dev_bf16(w_dev_or_bits)
    x = x_bits if isinstance(x_bits, torch.Tensor) else dev_bf16(x_bits)
    T = x.shape[0]
    out = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    l = torch.full((T,), float("nan"), dtype=torch.float32, device=DEV) if lse else None
    lp.score(x, w, dev(np.asarray(ids, np.int64)), temperature, v_true, out=out, lse=l)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), l.cpu().numpy()) if lse else out.cpu().numpy()


def check_stats(gpu: dict, ref: dict):
    """Integer fields and max_abs exact; sums to SUM_RTOL."""
    for p in lp.PAIRS:
        g, r = gpu[p], ref[p]
        for f in INT_FIELDS:
            assert np.array_equal(g[f].astype(np.int64), r[f]), (p, f, g[f], r[f])
        assert np.array_equal(g["max_abs"], r["max_abs"]), (p, "max_abs")
        for f, rtol in SUM_RTOL.items():
            np.testing.assert_allclose(g[f], r[f], rtol=rtol, atol=1e-12, err_msg=f"{p} {f}")
