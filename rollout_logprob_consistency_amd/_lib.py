"""ctypes declarations of the liblp C ABI (include/liblp.h).

The shared library must have been built in-tree (build.py); importing the
package without it raises, there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblp.so")

LP_OK, LP_EINVAL, LP_EUNSUPPORTED, LP_EHIP = 0, 1, 2, 3

# Names of every function include/liblp.h declares.
EXPORTS = ("lp_status_string", "lp_score_workspace_bytes", "lp_score",
           "lp_score_stats_workspace_bytes", "lp_score_stats", "lp_compare",
           "lp_compare_tails_workspace_bytes", "lp_compare_tails",
           "lp_vocab_shard_range", "lp_shard_partials_bytes",
           "lp_score_shard_workspace_bytes", "lp_score_shard", "lp_merge_shards",
           "lp_correct", "lp_score_ex_workspace_bytes", "lp_score_ex",
           "lp_compare_tails_ex_workspace_bytes", "lp_compare_tails_ex",
           "lp_compare_quantiles", "lp_score_noalloc")

REJECT_NONE, REJECT_K1, REJECT_K3 = 0, 1, 3  # LP_REJECT_*

# numpy mirror of `lp_corr_seq` (6 int32 then 2 double).
CORR_SEQ_DTYPE = np.dtype([
    ("valid", "<i4"), ("nonfinite", "<i4"), ("kept", "<i4"), ("capped", "<i4"),
    ("accepted", "<i4"), ("reserved", "<i4"), ("stat", "<f8"), ("sum_weight", "<f8"),
], align=True)
assert CORR_SEQ_DTYPE.itemsize == 40

MERGE_SEGMENTS = 16  # LP_MERGE_SEGMENTS
VOCAB_TILE_ROWS = 352  # LP_VOCAB_TILE_ROWS


class VocabShard(ctypes.Structure):
    """Mirror of `lp_vocab_shard`."""
    _fields_ = [("seg_lo", ctypes.c_int32), ("seg_hi", ctypes.c_int32),
                ("row_begin", ctypes.c_int64), ("row_end", ctypes.c_int64)]

# numpy mirror of `lp_seq_stats` (natural C alignment: 6 int32 then 7 double).
SEQ_STATS_DTYPE = np.dtype([
    ("valid", "<i4"), ("mismatch", "<i4"), ("first_div", "<i4"),
    ("longest_run", "<i4"), ("nonfinite", "<i4"), ("k3_nonfinite", "<i4"),
    ("max_abs", "<f8"), ("sum_abs", "<f8"), ("sum_signed", "<f8"),
    ("sum_k3", "<f8"), ("sum_d", "<f8"), ("seq_tis", "<f8"), ("sum_tok_tis", "<f8"),
], align=True)
assert SEQ_STATS_DTYPE.itemsize == 80

# numpy mirror of `lp_tail_stats`.
TAIL_STATS_DTYPE = np.dtype([
    ("count", "<i8"), ("q50", "<f8"), ("q95", "<f8"), ("q99", "<f8"),
    ("max_abs", "<f8"), ("max_seq", "<i4"), ("max_pos", "<i4"),
    ("sum_abs", "<f8"), ("sum_prob_abs", "<f8"),
], align=True)
assert TAIL_STATS_DTYPE.itemsize == 64

# numpy mirror of `lp_worst_token`.
WORST_DTYPE = np.dtype([("abs_delta", "<f8"), ("seq", "<i4"), ("pos", "<i4")], align=True)
assert WORST_DTYPE.itemsize == 16
WORST_MAX = 4096  # LP_WORST_MAX
NOALLOC_SCRATCH_BYTES = 32 << 20  # LP_NOALLOC_SCRATCH_BYTES


class LpError(RuntimeError):
    """A non-OK lp_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m rollout_logprob_consistency_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    L.lp_status_string.restype = ctypes.c_char_p
    L.lp_status_string.argtypes = [ctypes.c_int]
    L.lp_score_workspace_bytes.restype = ctypes.c_size_t
    L.lp_score_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.lp_score.restype = ctypes.c_int
    L.lp_score.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, f32,
                           vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.lp_score_stats_workspace_bytes.restype = ctypes.c_size_t
    L.lp_score_stats_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.lp_score_stats.restype = ctypes.c_int
    L.lp_score_stats.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, f32,
                                 vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.lp_compare.restype = ctypes.c_int
    L.lp_compare.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, f32, vp, vp, vp]
    L.lp_compare_tails_workspace_bytes.restype = ctypes.c_size_t
    L.lp_compare_tails_workspace_bytes.argtypes = [i64, i64]
    L.lp_compare_tails.restype = ctypes.c_int
    L.lp_compare_tails.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    L.lp_compare_tails_ex_workspace_bytes.restype = ctypes.c_size_t
    L.lp_compare_tails_ex_workspace_bytes.argtypes = [i64, i64, ctypes.c_int32]
    L.lp_compare_tails_ex.restype = ctypes.c_int
    L.lp_compare_tails_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int32, vp, vp, vp,
                                      vp, vp, ctypes.c_size_t, vp]
    L.lp_score_noalloc.restype = ctypes.c_int
    L.lp_score_noalloc.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, f32, vp, vp, vp, vp]
    L.lp_compare_quantiles.restype = ctypes.c_int
    L.lp_compare_quantiles.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp]
    i32 = ctypes.c_int32
    u32 = ctypes.c_uint32
    L.lp_score_ex_workspace_bytes.restype = ctypes.c_size_t
    L.lp_score_ex_workspace_bytes.argtypes = [i64, i64, i64, i64, u32]
    L.lp_score_ex.restype = ctypes.c_int
    L.lp_score_ex.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, f32, u32, vp, vp, vp, vp, vp,
                              vp, ctypes.c_size_t, vp]
    L.lp_vocab_shard_range.restype = ctypes.c_int
    L.lp_vocab_shard_range.argtypes = [i64, i32, i32, ctypes.POINTER(VocabShard)]
    L.lp_shard_partials_bytes.restype = ctypes.c_size_t
    L.lp_shard_partials_bytes.argtypes = [i64, u32]
    L.lp_score_shard_workspace_bytes.restype = ctypes.c_size_t
    L.lp_score_shard_workspace_bytes.argtypes = [i64, i64, i32, i32, u32]
    L.lp_score_shard.restype = ctypes.c_int
    L.lp_score_shard.argtypes = [vp, i64, vp, vp, i64, i64, i64, f32, i32, i32, u32,
                                 vp, vp, ctypes.c_size_t, vp]
    L.lp_merge_shards.restype = ctypes.c_int
    L.lp_merge_shards.argtypes = [vp, vp, i64, i64, u32, vp, vp, vp, vp, vp, vp]
    f64 = ctypes.c_double
    L.lp_correct.restype = ctypes.c_int
    L.lp_correct.argtypes = [vp, vp, vp, i64, i64, i64, f64, f64, f64, i32, f64, f64, vp, vp, vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().lp_status_string(int(status)).decode()
