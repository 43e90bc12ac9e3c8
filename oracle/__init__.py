"""fp64 CPU oracle for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the entry module's smoke
check and the benchmark's CPU-baseline leg, never by the product path.
"""
from .attention import (allowed_mask, attention_backward_fp64, attention_backward_sampled_fp64, attention_fp64,
                        attention_lse_fp64, multi_head_attention_fp64, softmax_rows_fp64)

__all__ = ["allowed_mask", "attention_backward_fp64", "attention_backward_sampled_fp64", "attention_fp64",
           "attention_lse_fp64", "multi_head_attention_fp64", "softmax_rows_fp64"]
