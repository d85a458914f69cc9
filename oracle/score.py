"""Selected-token logprob: the plain fp64 definition.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Not used by the library.

What is computed, per scored row t (rows are independent):

  [AMD] §"What a Logprob Difference Means": the stored score of token x_t is
        the natural log of its probability given the prefix, in nats.
  [AMD] §"Case 2: A and B Stay Close; C Changes": that logprob is the target
        token's logit minus the log of the sum over the whole vocabulary of the
        exponentials of the logits, the sum taken as a stable log-sum-exp.
  [AMD] §"How this differs from a real temperature mismatch": temperature
        divides every logit before the normaliser is formed; dividing a
        finished logprob by T is a different (wrong) quantity.
  [AMD] §"Collect A/B and C": the logits are the LM-head product of the final
        hidden state; the log-softmax is taken in higher precision than the
        model's; one global normaliser spans the whole vocabulary.
  "Training and rollout stop disagreeing ..." (vime / RL-Kernel summary): the
        normaliser covers the true vocabulary range only, so padded LM-head
        rows past it take no part.

The row's entropy and argmax (score_stats):

  [AMD] §"Case 2: A and B Stay Close; C Changes": the trainer's scoring step
        computes the log probs and the entropy of the same distribution. The
        entropy here is the plain Shannon entropy of softmax(z / T) over the
        true vocabulary range, in nats: H = -sum_v p_v ln p_v.
  [vLLM] §"Metric measurement basis": the full-vocabulary argmax is reported
        separately from the token metrics; "Diagnosing Training Inference
        Mismatch ..." (result 1 and its list of practical indicators) counts a
        top-1 flip when two scorings disagree on it. The argmax is the first
        (lowest) index of the row's largest logit.

Precision: the bf16 input bits are widened exactly to fp64; every later
operation is one fp64 operation. The logit row is an fp64 matrix product
(library matmul; its rounding, at most about H * 2^-53 relative, is far below
any tolerance used against it). For memory, the product is formed in blocks of
vocabulary rows; each logit is still one full dot product over h.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64, exactly (bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def logits(x_bits: np.ndarray, w_bits: np.ndarray, v_true: int | None = None,
           block: int = 8192) -> np.ndarray:
    """z[t, v] = sum_h x[t, h] * w[v, h] in fp64, for v < v_true."""
    x = bf16_bits_to_f64(x_bits)
    V = w_bits.shape[0] if v_true is None else int(v_true)
    if x.ndim != 2 or w_bits.ndim != 2 or x.shape[1] != w_bits.shape[1]:
        raise ValueError("expected x [T, H] and w [V, H] with the same H")
    if not 1 <= V <= w_bits.shape[0]:
        raise ValueError("v_true must lie in [1, V]")
    z = np.empty((x.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, block):
        v1 = min(V, v0 + block)
        z[:, v0:v1] = x @ bf16_bits_to_f64(w_bits[v0:v1]).T
    return z


def round_to_bf16(z: np.ndarray) -> np.ndarray:
    """Logits as an LM head that stores its output in bf16 gives them: the
    exact product sum rounded to fp32 (its accumulator type), then to bf16 by
    round to nearest, ties to even (keep the top 16 bits of the fp32 pattern,
    adding half of the dropped part, the dropped part's top bit breaking ties
    toward an even kept part). Returned as fp64 values (exact).

    [AMD] §"Collect A/B and C" (notes on the trainer's extraction): the fp32
    cast applies only to the final log-softmax; the upstream computation,
    the LM head included, keeps the model's precision.
    """
    u = np.ascontiguousarray(z, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if not np.isfinite(np.asarray(z)).all():
        raise ValueError("logits must be finite")
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64).reshape(np.shape(z))


def log_softmax_at(z: np.ndarray, ids: np.ndarray, temperature: float = 1.0):
    """Return (logprob[t], lse[t]) for logit rows z [T, V], fp64.

    s = z / T;  lse = M + ln sum_v exp(s_v - M) with M = max_v s_v;
    logprob = s[ids[t]] - lse.
    """
    temperature = float(temperature)
    if not (np.isfinite(temperature) and temperature > 0.0):
        raise ValueError("temperature must be finite and > 0")
    ids = np.asarray(ids, dtype=np.int64)
    if ids.shape != (z.shape[0],):
        raise ValueError("one target id per row")
    if ids.size and (ids.min() < 0 or ids.max() >= z.shape[1]):
        raise ValueError("target id outside the true vocabulary range")
    s = z / temperature
    M = s.max(axis=1)
    S = np.exp(s - M[:, None]).sum(axis=1)
    lse = M + np.log(S)
    lp = s[np.arange(z.shape[0]), ids] - lse
    return lp, lse


def score(x_bits: np.ndarray, w_bits: np.ndarray, ids: np.ndarray,
          temperature: float = 1.0, v_true: int | None = None, bf16_logits: bool = False):
    """Selected-token logprob of every row: (logprob fp64 [T], lse fp64 [T]).
    bf16_logits: the logits are first rounded as round_to_bf16 does."""
    if x_bits.shape[0] == 0:
        return np.zeros(0), np.zeros(0)
    z = logits(x_bits, w_bits, v_true)
    if bf16_logits:
        z = round_to_bf16(z)
    return log_softmax_at(z, ids, temperature)


def sharded_log_softmax_at(z: np.ndarray, ids: np.ndarray, bounds, temperature: float = 1.0):
    """log_softmax_at with the vocabulary split into shards, as a
    vocabulary-parallel LM head computes it.

    [AMD] §"Collect A/B and C" (notes on the trainer's extraction): when the
    vocabulary is split over shards, one global normaliser must still span
    all of them; normalising each shard on its own scores a different
    distribution. The vime / RL-Kernel summary: the cross-rank LSE merge
    takes the ranks in a fixed order.

    bounds: ascending row indices 0 = b_0 <= b_1 <= ... <= b_n = V (a shard
    may be empty). Shard r holds rows [b_r, b_{r+1}) and reports
    M_r = max s_v and S_r = sum exp(s_v - M_r) over its rows (an empty shard
    reports nothing); the owner of ids[t] reports s[ids[t]]. Then, in shard
    order, M = max_r M_r and lse = M + ln sum_r S_r exp(M_r - M).
    Returns (logprob[t], lse[t]) in fp64.
    """
    temperature = float(temperature)
    if not (np.isfinite(temperature) and temperature > 0.0):
        raise ValueError("temperature must be finite and > 0")
    b = [int(v) for v in bounds]
    if b[0] != 0 or b[-1] != z.shape[1] or any(b1 < b0 for b0, b1 in zip(b, b[1:])):
        raise ValueError("bounds must rise from 0 to V")
    ids = np.asarray(ids, dtype=np.int64)
    if ids.shape != (z.shape[0],):
        raise ValueError("one target id per row")
    if ids.size and (ids.min() < 0 or ids.max() >= z.shape[1]):
        raise ValueError("target id outside the true vocabulary range")
    s = z / temperature
    parts = []
    target = np.full(z.shape[0], np.nan)
    for b0, b1 in zip(b, b[1:]):
        if b1 == b0:
            continue
        sr = s[:, b0:b1]
        Mr = sr.max(axis=1)
        parts.append((Mr, np.exp(sr - Mr[:, None]).sum(axis=1)))
        own = (ids >= b0) & (ids < b1)
        target[own] = sr[own, ids[own] - b0]
    M = np.max([Mr for Mr, _ in parts], axis=0)
    S = np.zeros(z.shape[0])
    for Mr, Sr in parts:
        S = S + Sr * np.exp(Mr - M)
    lse = M + np.log(S)
    return target - lse, lse


def entropy_argmax(z: np.ndarray, temperature: float = 1.0):
    """Return (entropy[t] in nats, argmax[t]) for logit rows z [T, V], fp64.

    p = softmax(z / T) row by row; entropy = -sum_v p_v ln p_v with
    ln p_v = s_v - lse (exact form of the log of the normalised weight);
    argmax = the lowest v with z[t, v] equal to the row's maximum.
    """
    temperature = float(temperature)
    if not (np.isfinite(temperature) and temperature > 0.0):
        raise ValueError("temperature must be finite and > 0")
    s = z / temperature
    M = s.max(axis=1)
    lse = M + np.log(np.exp(s - M[:, None]).sum(axis=1))
    logp = s - lse[:, None]
    ent = -(np.exp(logp) * logp).sum(axis=1)
    return ent, np.argmax(z, axis=1).astype(np.int64)


def score_stats(x_bits: np.ndarray, w_bits: np.ndarray, ids: np.ndarray,
                temperature: float = 1.0, v_true: int | None = None, bf16_logits: bool = False):
    """(logprob, lse, entropy, argmax) of every row: fp64, fp64, fp64, int64."""
    if x_bits.shape[0] == 0:
        return np.zeros(0), np.zeros(0), np.zeros(0), np.zeros(0, np.int64)
    z = logits(x_bits, w_bits, v_true)
    if bf16_logits:
        z = round_to_bf16(z)
    lp, lse = log_softmax_at(z, ids, temperature)
    ent, amax = entropy_argmax(z, temperature)
    return lp, lse, ent, amax
