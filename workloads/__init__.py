"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module only draws random numbers and lays them out. It contains none of
the scored method's arithmetic (no matrix product, no log-sum-exp, no
comparison statistic), so the oracle and the GPU path can both consume its
bytes without sharing any of the computation they are checked on.
"""

from .synth import (  # noqa: F401
    BASE_SEED,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    normal_f32,
    uniform_ids,
    zipf_ids,
    rmsnorm_rows_f32,
    ScoreCase,
    tiny_case,
    qwen_case,
    probe_set,
    filler_rows,
    CompareCase,
    compare_case,
    compare_sweep_case,
)
