"""fp64 CPU oracle for the selected-token logprob and the three-way comparison.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow definition that the
GPU library is checked against. Only tests/, the smoke check in
__graft_entry__.py and bench.py's CPU-baseline leg may import it; the library
in rollout_logprob_consistency_amd/ never does, and the two share no code.

Every function cites the passage of the source pages it writes out:
  [AMD]  "Debugging Logprob Mismatches in LLM Reinforcement Learning"
  [vLLM] "Fault localization and mismatch bisect" (train-inference-consistency
         guide)
  [TII]  "Rollout-Training Mismatch in LLM RL"
  [VeX]  "Diagnosing Training Inference Mismatch in LLM Reinforcement Learning"
"""

from .score import (bf16_bits_to_f64, score, score_stats, entropy_argmax, logits,  # noqa: F401
                    log_softmax_at, sharded_log_softmax_at, round_to_bf16)
from .compare import (compare, per_token, tails, worst_tokens, quantile_linear, seq_quantiles,  # noqa: F401
                      QUANTILE_PROBS, PAIRS,
                      STAT_FIELDS, TAIL_FIELDS)
from .correct import correct, CORR_FIELDS, REJECT_NONE, REJECT_K1, REJECT_K3  # noqa: F401
