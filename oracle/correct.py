"""Correction consumers of the rollout and trainer logprobs: per-token TIS /
MIS importance weights and sequence rejection. The plain definition.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Not used by the library.

  [TII] §2.1 "Sampling correction and proximal update control", Eq. (2): the
        sampling-correction weight is the anchor's probability of the token
        over the behaviour (rollout) policy's. After Eq. (3): truncated
        importance sampling keeps min(w, C); masked importance sampling keeps
        w where l <= w <= u and drops it (weight 0) elsewhere.
  [VeX] result 5 and the discussion of how TIS works: the correction ratio
        r_t is the old trainer probability over the rollout probability of
        the sampled token, formed from the two logprobs as exp(difference);
        token TIS clamps it at C; sequence rejection filters a whole
        trajectory by the sum over its tokens of K1(r_t) or K3(r_t); padding
        tokens weigh 0.
  K1 and K3 are Schulman's estimators of KL(rollout || train) from samples of
        the rollout policy ([vLLM] "Schulman k3"): K1(r) = -log r,
        K3(r) = r - 1 - log r.

Readings: the interval and the cap are applied in the log domain (d = log r
against log l, log u and log C), which decides exactly the same tokens as
comparing r itself except within rounding of the bounds, and keeps the
decision identical on both sides of a parity test; a sequence is accepted
when reject_lo <= stat <= reject_hi; a non-finite active token weighs 0 and
takes no part in stat; an overflowing K3 term makes stat +inf.
"""

from __future__ import annotations

import math

import numpy as np

REJECT_NONE, REJECT_K1, REJECT_K3 = 0, 1, 3
CORR_FIELDS = ("valid", "nonfinite", "kept", "capped", "accepted", "stat", "sum_weight")


def correct(rollout, train, mask, tis_clip: float = 2.0, mis_log_lo: float = -math.inf,
            mis_log_hi: float = math.inf, reject: int = REJECT_NONE,
            reject_lo: float = -math.inf, reject_hi: float = math.inf):
    """Return (weights fp32 [N, L], {field: array [N]}).

    rollout, train: fp32 [N, L] logprobs of the sampled tokens; mask: [N, L].
    """
    rollout = np.asarray(rollout, np.float32)
    train = np.asarray(train, np.float32)
    mask = np.asarray(mask)
    if rollout.shape != train.shape or rollout.shape != mask.shape or rollout.ndim != 2:
        raise ValueError("rollout, train and mask must share one [N, L] shape")
    if not tis_clip > 0 or not mis_log_lo <= mis_log_hi or not reject_lo <= reject_hi:
        raise ValueError("bad cap, interval or accepted range")
    if reject not in (REJECT_NONE, REJECT_K1, REJECT_K3):
        raise ValueError("unknown rejection estimator")
    N, L = rollout.shape
    log_cap = math.log(tis_clip)
    weights = np.zeros((N, L), np.float32)
    out = {f: np.zeros(N, np.float64 if f in ("stat", "sum_weight") else np.int64)
           for f in CORR_FIELDS}
    for n in range(N):
        r64 = rollout[n].astype(np.float64)
        t64 = train[n].astype(np.float64)
        act = mask[n] != 0
        counted = act & np.isfinite(r64) & np.isfinite(t64)
        d = np.where(counted, t64 - r64, 0.0)
        with np.errstate(over="ignore", invalid="ignore"):
            if reject == REJECT_K1:
                k = -d
            elif reject == REJECT_K3:
                k = np.expm1(d) - d
            else:
                k = np.zeros(L)
            stat = math.fsum(k[counted].tolist())
            accepted = not (stat < reject_lo) and not (stat > reject_hi)
            inside = counted & (d >= mis_log_lo) & (d <= mis_log_hi)
            capped = inside & (d >= log_cap)
            w = np.where(capped, tis_clip, np.exp(np.where(inside, d, 0.0)))
        if accepted:
            weights[n] = np.where(inside, w, 0.0).astype(np.float32)
        out["valid"][n] = int(act.sum())
        out["nonfinite"][n] = int((act & ~counted).sum())
        out["kept"][n] = int(inside.sum())
        out["capped"][n] = int(capped.sum())
        out["accepted"][n] = int(accepted)
        out["stat"][n] = stat
        out["sum_weight"][n] = math.fsum(weights[n].astype(np.float64).tolist())
    return weights, out
