"""CPU oracle for packed draft-token verification.

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline import this package. The HIP library never does, and this package
imports nothing from it.
"""
from .philox import philox4x32_10, row_uniform
from .verify import (BF16, F32, PreconditionError, bf16_bits_to_f64,
                     draft_confidence, filtered_support, greedy_token,
                     logsumexp, rank_of, rank_order, relaxed_accepts, row_f64,
                     sample_from_u, sampled_row_margins, verify_greedy,
                     verify_greedy_relaxed, verify_sampled)
