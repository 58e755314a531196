"""Float64 CPU oracle for the attention forward.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU baseline. The product path never imports it.
"""
from .attention import attention_ref, attention_rows, attention_ref_pool, head_ref

__all__ = ["attention_ref", "attention_rows", "attention_ref_pool", "head_ref"]
