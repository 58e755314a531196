"""Float64 CPU oracle for the attention forward and backward.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU baseline. The product path never imports it.
"""
from .attention import attention_ref, attention_rows, attention_ref_pool, attention_varlen_ref, head_ref
from .attention_bwd import attention_bwd_ref, attention_varlen_bwd_ref, head_bwd_ref, dq_rows

__all__ = ["attention_ref", "attention_rows", "attention_ref_pool", "attention_varlen_ref", "head_ref",
           "attention_bwd_ref", "attention_varlen_bwd_ref", "head_bwd_ref", "dq_rows"]
