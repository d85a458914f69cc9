"""Deterministic, batch-invariant selected-token logprobs and the three-way
logprob comparison on AMD Instinct MI355X.

Thin binding over the C ABI in include/liblp.h (liblp.so, built in-tree by
build.py). This module only checks and marshals arguments: it passes device
pointers and the current HIP stream to the library, and every arithmetic
step runs in the library's kernels. PyTorch supplies device memory and
streams.

    score(hidden, w, ids, temperature=1.0, v_true=None)   -> logprob [T] fp32
    score_stats(hidden, w, ids, ...)                      -> logprob, entropy, argmax
    score_ex(hidden, w, ids, ..., stats, bf16_logits)     -> either, optionally bf16 logits
    compare(A, B, C, mask, tis_clip=2.0, atol=None)       -> stats per pair
    compare_quantiles(A, B, C, mask)                      -> p50/p95/p99 per pair and sequence
    compare_tails(A, B, C, mask, positions=False)         -> batch tails per pair
    vocab_shard / score_shard / merge_shards              -> vocabulary-parallel scoring
    correct(rollout, train, mask, ...)                    -> TIS/MIS weights, rejection
    align(hidden, input_ids, response_mask)               -> rows, targets, mask
"""

from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from ._lib import (CORR_SEQ_DTYPE, EXPORTS, LP_OK, REJECT_K1, REJECT_K3,  # noqa: F401
                   REJECT_NONE, SEQ_STATS_DTYPE, TAIL_STATS_DTYPE, WORST_DTYPE, WORST_MAX, LpError,
                   lib, status_string)

PAIRS = ("AB", "BC", "AC")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(name: str, t: torch.Tensor, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def score_workspace_bytes(T: int, H: int, V_rows: int, V_true: int | None = None) -> int:
    return int(lib().lp_score_workspace_bytes(T, H, V_rows, V_rows if V_true is None else V_true))


def score(hidden: torch.Tensor, w: torch.Tensor, ids: torch.Tensor,
          temperature: float = 1.0, v_true: int | None = None, *,
          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
          workspace: torch.Tensor | None = None, bad_rows: torch.Tensor | None = None,
          check: bool = False) -> torch.Tensor:
    """Selected-token logprob of every row of `hidden` (fp32, nats).

    hidden [T, H] bf16 with unit column stride, w [V, H] bf16 contiguous,
    ids [T] int64. Rows must already be aligned with their targets (align()).
    With check=True the call synchronises and raises ValueError if any target
    id lies outside [0, v_true).
    """
    _need_cuda("hidden", hidden, torch.bfloat16)
    _need_cuda("w", w, torch.bfloat16)
    _need_cuda("ids", ids, torch.int64)
    if hidden.dim() != 2 or w.dim() != 2 or ids.dim() != 1:
        raise ValueError("expected hidden [T, H], w [V, H], ids [T]")
    if hidden.stride(1) != 1 or not w.is_contiguous() or not ids.is_contiguous():
        raise ValueError("hidden needs unit column stride; w and ids must be contiguous")
    T, H = hidden.shape
    V = w.shape[0]
    if w.shape[1] != H or ids.shape[0] != T:
        raise ValueError("shape mismatch between hidden, w and ids")
    vt = V if v_true is None else int(v_true)
    dev = hidden.device
    if out is None:
        out = torch.empty(T, dtype=torch.float32, device=dev)
    need = score_workspace_bytes(T, H, V, vt)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if check and bad_rows is None:
        bad_rows = torch.zeros(1, dtype=torch.int32, device=dev)
    st = lib().lp_score(_ptr(hidden), hidden.stride(0) if T else H, _ptr(w), _ptr(ids),
                        T, H, V, vt, float(temperature), _ptr(out), _ptr(lse),
                        _ptr(bad_rows), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_score")
    if check and int(bad_rows.item()) != 0:
        raise ValueError(f"{int(bad_rows.item())} row(s) have a target id outside [0, {vt})")
    return out


def score_stats_workspace_bytes(T: int, H: int, V_rows: int, V_true: int | None = None) -> int:
    return int(lib().lp_score_stats_workspace_bytes(T, H, V_rows,
                                                    V_rows if V_true is None else V_true))


def score_stats(hidden: torch.Tensor, w: torch.Tensor, ids: torch.Tensor,
                temperature: float = 1.0, v_true: int | None = None, *,
                lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                check: bool = False):
    """Selected-token logprob plus the row's entropy (nats) and argmax.

    Same arguments as score(); returns (logprob fp32 [T], entropy fp32 [T],
    argmax int64 [T]). The logprob bits equal score()'s for the same inputs.
    """
    _need_cuda("hidden", hidden, torch.bfloat16)
    _need_cuda("w", w, torch.bfloat16)
    _need_cuda("ids", ids, torch.int64)
    if hidden.dim() != 2 or w.dim() != 2 or ids.dim() != 1:
        raise ValueError("expected hidden [T, H], w [V, H], ids [T]")
    if hidden.stride(1) != 1 or not w.is_contiguous() or not ids.is_contiguous():
        raise ValueError("hidden needs unit column stride; w and ids must be contiguous")
    T, H = hidden.shape
    V = w.shape[0]
    if w.shape[1] != H or ids.shape[0] != T:
        raise ValueError("shape mismatch between hidden, w and ids")
    vt = V if v_true is None else int(v_true)
    dev = hidden.device
    out = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev)
    amax = torch.empty(T, dtype=torch.int64, device=dev)
    need = score_stats_workspace_bytes(T, H, V, vt)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    bad_rows = torch.zeros(1, dtype=torch.int32, device=dev) if check else None
    st = lib().lp_score_stats(_ptr(hidden), hidden.stride(0) if T else H, _ptr(w), _ptr(ids),
                              T, H, V, vt, float(temperature), _ptr(out), _ptr(lse), _ptr(ent),
                              _ptr(amax), _ptr(bad_rows), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_score_stats")
    if check and int(bad_rows.item()) != 0:
        raise ValueError(f"{int(bad_rows.item())} row(s) have a target id outside [0, {vt})")
    return out, ent, amax


SCORE_STATS, SCORE_BF16_LOGITS = 1, 2  # LP_SCORE_* flags


def score_ex(hidden: torch.Tensor, w: torch.Tensor, ids: torch.Tensor,
             temperature: float = 1.0, v_true: int | None = None, *, stats: bool = False,
             bf16_logits: bool = False, lse: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None, check: bool = False):
    """lp_score_ex: score() (stats=False) or score_stats() (stats=True), with
    bf16_logits=True rounding every fp32 logit to bf16 before the tempered
    log-softmax (the score of an LM head that stores bf16 logits). Returns
    logprob, or (logprob, entropy, argmax) with stats."""
    _need_cuda("hidden", hidden, torch.bfloat16)
    _need_cuda("w", w, torch.bfloat16)
    _need_cuda("ids", ids, torch.int64)
    if hidden.dim() != 2 or w.dim() != 2 or ids.dim() != 1:
        raise ValueError("expected hidden [T, H], w [V, H], ids [T]")
    if hidden.stride(1) != 1 or not w.is_contiguous() or not ids.is_contiguous():
        raise ValueError("hidden needs unit column stride; w and ids must be contiguous")
    T, H = hidden.shape
    V = w.shape[0]
    if w.shape[1] != H or ids.shape[0] != T:
        raise ValueError("shape mismatch between hidden, w and ids")
    vt = V if v_true is None else int(v_true)
    flags = (SCORE_STATS if stats else 0) | (SCORE_BF16_LOGITS if bf16_logits else 0)
    dev = hidden.device
    out = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if stats else None
    amax = torch.empty(T, dtype=torch.int64, device=dev) if stats else None
    need = int(lib().lp_score_ex_workspace_bytes(T, H, V, vt, flags))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    bad_rows = torch.zeros(1, dtype=torch.int32, device=dev) if check else None
    st = lib().lp_score_ex(_ptr(hidden), hidden.stride(0) if T else H, _ptr(w), _ptr(ids),
                           T, H, V, vt, float(temperature), flags, _ptr(out), _ptr(lse),
                           _ptr(ent), _ptr(amax), _ptr(bad_rows), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_score_ex")
    if check and int(bad_rows.item()) != 0:
        raise ValueError(f"{int(bad_rows.item())} row(s) have a target id outside [0, {vt})")
    return (out, ent, amax) if stats else out


def compare_raw(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, mask: torch.Tensor,
                tis_clip: float = 2.0, atol: float | None = None,
                per_token: bool = False, out: torch.Tensor | None = None):
    """Enqueue lp_compare; returns (stats bytes [3*N*80] uint8 device tensor,
    per-token tensor [3, 3, N, L] fp32 or None). Does not synchronise."""
    for name, t in (("A", A), ("B", B), ("C", C)):
        _need_cuda(name, t, torch.float32)
    _need_cuda("mask", mask, torch.uint8)
    if not (A.shape == B.shape == C.shape == mask.shape) or A.dim() != 2:
        raise ValueError("A, B, C and mask must share one [N, L] shape")
    N, L = A.shape
    ld = A.stride(0) if A.numel() else L
    for t in (A, B, C, mask):
        if t.numel() and (t.stride(1) != 1 or (N > 1 and t.stride(0) != ld)):
            raise ValueError("A, B, C and mask need unit column stride and one row stride")
    dev = A.device
    nbytes = 3 * N * SEQ_STATS_DTYPE.itemsize
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    pt = torch.empty((3, 3, N, L), dtype=torch.float32, device=dev) if per_token else None
    st = lib().lp_compare(_ptr(A), _ptr(B), _ptr(C), _ptr(mask), N, L, max(ld, L),
                          float(tis_clip), -1.0 if atol is None else float(atol),
                          _ptr(out), _ptr(pt), _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_compare")
    return out, pt


def stats_from_bytes(raw: torch.Tensor, N: int) -> dict:
    """Device stats bytes (lp_compare's [N][3] records) -> {"AB"|"BC"|"AC":
    numpy structured array [N]}."""
    host = raw[: 3 * N * SEQ_STATS_DTYPE.itemsize].cpu().numpy()
    rec = host.view(SEQ_STATS_DTYPE).reshape(N, 3) if N else np.zeros((0, 3), SEQ_STATS_DTYPE)
    return {p: np.ascontiguousarray(rec[:, i]) for i, p in enumerate(PAIRS)}


def compare(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, mask: torch.Tensor,
            tis_clip: float = 2.0, atol: float | None = None, per_token: bool = False,
            check: bool = True):
    """Three-way comparison; synchronises and returns per-pair statistics.

    Like the AMD blog's compare(), with check=True it raises ValueError when
    the mask holds a value other than 0 or 1, a sequence has no active token
    or an active score is non-finite. With check=False any non-zero mask
    byte is active (the library's rule).
    """
    if check and mask.numel() and bool(((mask != 0) & (mask != 1)).any()):
        raise ValueError("mask values must be 0 or 1")
    raw, pt = compare_raw(A, B, C, mask, tis_clip, atol, per_token)
    stats = stats_from_bytes(raw, A.shape[0])
    if check:
        s = stats["AB"]
        if np.any(s["valid"] == 0):
            raise ValueError("a sequence has no active token")
        for p in PAIRS:
            if np.any(stats[p]["nonfinite"] > 0):
                raise ValueError(f"non-finite score on an active token ({p})")
    return (stats, pt) if per_token else stats


def _check_compare_inputs(A, B, C, mask):
    for name, t in (("A", A), ("B", B), ("C", C)):
        _need_cuda(name, t, torch.float32)
    _need_cuda("mask", mask, torch.uint8)
    if not (A.shape == B.shape == C.shape == mask.shape) or A.dim() != 2:
        raise ValueError("A, B, C and mask must share one [N, L] shape")
    N, L = A.shape
    ld = A.stride(0) if A.numel() else L
    for t in (A, B, C, mask):
        if t.numel() and (t.stride(1) != 1 or (N > 1 and t.stride(0) != ld)):
            raise ValueError("A, B, C and mask need unit column stride and one row stride")
    return N, L, max(ld, L)


def compare_quantiles(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, mask: torch.Tensor,
                      *, out: torch.Tensor | None = None, sync: bool = True):
    """p50 / p95 / p99 of |left - right| per pair and sequence
    (lp_compare_quantiles): numpy's default quantile over each sequence's
    counted tokens, as the AMD blog's compare() returns for one record.
    Returns {"AB"|"BC"|"AC": numpy float64 [N, 3]} (sync=True), else the
    [N, 3, 3] float64 device tensor (sequence, pair, quantile) without
    synchronising."""
    N, L, ld = _check_compare_inputs(A, B, C, mask)
    dev = A.device
    if out is None:
        out = torch.empty((N, 3, 3), dtype=torch.float64, device=dev)
    elif out.dtype != torch.float64 or not out.is_contiguous() or out.numel() < 9 * N:
        raise ValueError("out must be a contiguous float64 tensor of 3 * N * 3 values")
    st = lib().lp_compare_quantiles(_ptr(A), _ptr(B), _ptr(C), _ptr(mask), N, L, ld, _ptr(out),
                                    _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_compare_quantiles")
    if not sync:
        return out
    q = out.reshape(N, 3, 3).cpu().numpy()
    return {p: np.ascontiguousarray(q[:, i]) for i, p in enumerate(PAIRS)}


def compare_tails(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, mask: torch.Tensor,
                  positions: bool = False, worst_k: int = 0):
    """Batch tail statistics of |left - right| per pair (lp_compare_tails,
    or lp_compare_tails_ex with worst_k > 0); synchronises. Returns
    {"AB"|"BC"|"AC": numpy record of TAIL_STATS_DTYPE}, then, when asked,
    (pos_sum [3, L] fp64, pos_count [3, L] int32) and the worst tokens
    {"AB"|"BC"|"AC": numpy array [worst_k] of WORST_DTYPE}."""
    for name, t in (("A", A), ("B", B), ("C", C)):
        _need_cuda(name, t, torch.float32)
    _need_cuda("mask", mask, torch.uint8)
    if not (A.shape == B.shape == C.shape == mask.shape) or A.dim() != 2:
        raise ValueError("A, B, C and mask must share one [N, L] shape")
    if not 0 <= int(worst_k) <= WORST_MAX:
        raise ValueError(f"worst_k must lie in [0, {WORST_MAX}]")
    N, L = A.shape
    ld = A.stride(0) if A.numel() else L
    for t in (A, B, C, mask):
        if t.numel() and (t.stride(1) != 1 or (N > 1 and t.stride(0) != ld)):
            raise ValueError("A, B, C and mask need unit column stride and one row stride")
    dev = A.device
    k = int(worst_k)
    out = torch.empty(3 * TAIL_STATS_DTYPE.itemsize, dtype=torch.uint8, device=dev)
    ps = torch.empty((3, L), dtype=torch.float64, device=dev) if positions else None
    pc = torch.empty((3, L), dtype=torch.int32, device=dev) if positions else None
    worst = torch.empty(max(3 * k * WORST_DTYPE.itemsize, 1), dtype=torch.uint8, device=dev)
    need = int(lib().lp_compare_tails_ex_workspace_bytes(N, L, k))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if k == 0:
        st = lib().lp_compare_tails(_ptr(A), _ptr(B), _ptr(C), _ptr(mask), N, L, max(ld, L),
                                    _ptr(out), _ptr(ps), _ptr(pc), _ptr(ws), need, _stream(dev))
    else:
        st = lib().lp_compare_tails_ex(_ptr(A), _ptr(B), _ptr(C), _ptr(mask), N, L, max(ld, L), k,
                                       _ptr(out), _ptr(worst), _ptr(ps), _ptr(pc), _ptr(ws), need,
                                       _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_compare_tails" + ("_ex" if k else ""))
    rec = out.cpu().numpy().view(TAIL_STATS_DTYPE)
    res = [{p: rec[i] for i, p in enumerate(PAIRS)}]
    if positions:
        res += [ps.cpu().numpy(), pc.cpu().numpy()]
    if k:
        wr = worst.cpu().numpy()[:3 * k * WORST_DTYPE.itemsize].view(WORST_DTYPE).reshape(3, k)
        res.append({p: wr[i] for i, p in enumerate(PAIRS)})
    return res[0] if len(res) == 1 else tuple(res)


def vocab_shard(v_true: int, n_shards: int, rank: int) -> dict:
    """Canonical vocabulary shard of rank `rank` of `n_shards` (1..16): the
    merge segments [seg_lo, seg_hi) it owns and their rows [row_begin, row_end)."""
    from ._lib import VocabShard
    out = VocabShard()
    st = lib().lp_vocab_shard_range(int(v_true), int(n_shards), int(rank), ctypes.byref(out))
    if st != LP_OK:
        raise LpError(st, "lp_vocab_shard_range")
    return {"seg_lo": out.seg_lo, "seg_hi": out.seg_hi,
            "row_begin": out.row_begin, "row_end": out.row_end}


def shard_partials(T: int, stats: bool = False, device=None) -> torch.Tensor:
    """An exchange buffer for T rows: [16, F, T] fp32 (F = 5 with stats, else 3)."""
    F = 5 if stats else 3
    assert int(lib().lp_shard_partials_bytes(T, SCORE_STATS if stats else 0)) == 16 * F * T * 4
    return torch.empty((16, F, T), dtype=torch.float32, device=device)


def score_shard(hidden: torch.Tensor, w_shard: torch.Tensor, ids: torch.Tensor, v_true: int,
                n_shards: int, rank: int, partials: torch.Tensor, temperature: float = 1.0,
                stats: bool = False, *, bf16_logits: bool = False,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Score one vocabulary shard (lp_score_shard): w_shard holds rows
    [row_begin, row_end) of W; writes this shard's segment records into
    `partials` (from shard_partials) and returns it. Does not synchronise."""
    _need_cuda("hidden", hidden, torch.bfloat16)
    _need_cuda("w_shard", w_shard, torch.bfloat16)
    _need_cuda("ids", ids, torch.int64)
    _need_cuda("partials", partials, torch.float32)
    if hidden.dim() != 2 or w_shard.dim() != 2 or ids.dim() != 1:
        raise ValueError("expected hidden [T, H], w_shard [rows, H], ids [T]")
    if hidden.stride(1) != 1 or not w_shard.is_contiguous() or not ids.is_contiguous():
        raise ValueError("hidden needs unit column stride; w_shard and ids must be contiguous")
    T, H = hidden.shape
    sh = vocab_shard(v_true, n_shards, rank)
    if w_shard.shape != (sh["row_end"] - sh["row_begin"], H) or ids.shape[0] != T:
        raise ValueError("w_shard must hold the shard's rows [row_begin, row_end) x H")
    F = 5 if stats else 3
    if not partials.is_contiguous() or partials.shape != (16, F, T):
        raise ValueError(f"partials must be a contiguous [16, {F}, T] buffer")
    flags = (SCORE_STATS if stats else 0) | (SCORE_BF16_LOGITS if bf16_logits else 0)
    need = int(lib().lp_score_shard_workspace_bytes(T, v_true, n_shards, rank, flags))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    st = lib().lp_score_shard(_ptr(hidden), hidden.stride(0) if T else H, _ptr(w_shard),
                              _ptr(ids), T, H, int(v_true), float(temperature), int(n_shards),
                              int(rank), flags, _ptr(partials), _ptr(workspace),
                              workspace.numel() * workspace.element_size(),
                              _stream(hidden.device))
    if st != LP_OK:
        raise LpError(st, "lp_score_shard")
    return partials


def merge_shards(partials: torch.Tensor, ids: torch.Tensor, v_true: int, stats: bool = False,
                 *, lse: torch.Tensor | None = None, check: bool = False):
    """Fold the gathered segment records (lp_merge_shards). Returns logprob
    fp32 [T], or (logprob, entropy, argmax) with stats; bitwise equal to
    score() / score_stats() on the whole W."""
    _need_cuda("partials", partials, torch.float32)
    _need_cuda("ids", ids, torch.int64)
    T = ids.shape[0]
    F = 5 if stats else 3
    if not partials.is_contiguous() or partials.shape != (16, F, T) or not ids.is_contiguous():
        raise ValueError(f"partials must be a contiguous [16, {F}, T] buffer and ids [T]")
    dev = ids.device
    out = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if stats else None
    amax = torch.empty(T, dtype=torch.int64, device=dev) if stats else None
    bad_rows = torch.zeros(1, dtype=torch.int32, device=dev) if check else None
    st = lib().lp_merge_shards(_ptr(partials), _ptr(ids), T, int(v_true),
                               SCORE_STATS if stats else 0, _ptr(out),
                               _ptr(lse), _ptr(ent), _ptr(amax), _ptr(bad_rows), _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_merge_shards")
    if check and int(bad_rows.item()) != 0:
        raise ValueError(f"{int(bad_rows.item())} row(s) have a target id outside [0, {v_true})")
    return (out, ent, amax) if stats else out


def correct(rollout: torch.Tensor, train: torch.Tensor, mask: torch.Tensor,
            tis_clip: float = 2.0, mis_log_lo: float = -math.inf, mis_log_hi: float = math.inf,
            reject: int = REJECT_NONE, reject_lo: float = -math.inf,
            reject_hi: float = math.inf, weights: bool = True):
    """Correction weights of r = pi_train / pi_rollout (lp_correct): TIS cap
    `tis_clip`, MIS interval [mis_log_lo, mis_log_hi] on log r, sequence
    rejection by sum K1 / K3 outside [reject_lo, reject_hi]. Returns
    (weights fp32 [N, L] device tensor or None, numpy records of
    CORR_SEQ_DTYPE [N]); synchronises."""
    for name, t in (("rollout", rollout), ("train", train)):
        _need_cuda(name, t, torch.float32)
    _need_cuda("mask", mask, torch.uint8)
    if not (rollout.shape == train.shape == mask.shape) or rollout.dim() != 2:
        raise ValueError("rollout, train and mask must share one [N, L] shape")
    N, L = rollout.shape
    ld = rollout.stride(0) if rollout.numel() else L
    for t in (rollout, train, mask):
        if t.numel() and (t.stride(1) != 1 or (N > 1 and t.stride(0) != ld)):
            raise ValueError("rollout, train and mask need unit column stride and one row stride")
    dev = rollout.device
    w = torch.empty((N, L), dtype=torch.float32, device=dev) if weights else None
    out = torch.empty(max(N * CORR_SEQ_DTYPE.itemsize, 1), dtype=torch.uint8, device=dev)
    st = lib().lp_correct(_ptr(rollout), _ptr(train), _ptr(mask), N, L, max(ld, L),
                          float(tis_clip), float(mis_log_lo), float(mis_log_hi), int(reject),
                          float(reject_lo), float(reject_hi), _ptr(w), _ptr(out), _stream(dev))
    if st != LP_OK:
        raise LpError(st, "lp_correct")
    rec = out[:N * CORR_SEQ_DTYPE.itemsize].cpu().numpy().view(CORR_SEQ_DTYPE)
    return w, rec


def align(hidden: torch.Tensor, input_ids: torch.Tensor, response_mask: torch.Tensor):
    """Pair every prediction row with the token it predicts.

    The output after position j scores token j + 1, so the first response
    token is scored by the last prompt position and the mask moves with its
    target (AMD blog, "Align Each Score With the Token It Predicts").
    hidden [B, S, H], input_ids [B, S], response_mask [B, S] (0/1) ->
    rows [B*S, H] (a view), targets [B*S] int64, mask [B*S] uint8, where
    position j of each sequence targets input_ids[:, j + 1] and the last
    position has target 0 with mask 0. Every position is scored; apply the
    mask afterwards to A, B and C alike.
    """
    if hidden.dim() != 3 or input_ids.shape != hidden.shape[:2] or \
            response_mask.shape != input_ids.shape:
        raise ValueError("expected hidden [B, S, H], input_ids and response_mask [B, S]")
    if bool(((response_mask != 0) & (response_mask != 1)).any()):
        raise ValueError("response_mask values must be 0 or 1")
    if bool((response_mask[:, 0] != 0).any()):
        raise ValueError("response_mask[:, 0] must be 0: nothing before the first "
                         "position predicts it")
    B, S, H = hidden.shape
    targets = torch.zeros_like(input_ids, dtype=torch.int64)
    targets[:, :-1] = input_ids[:, 1:]
    mask = torch.zeros((B, S), dtype=torch.uint8, device=response_mask.device)
    mask[:, :-1] = response_mask[:, 1:] != 0
    return hidden.reshape(B * S, H), targets.reshape(-1), mask.reshape(-1)
