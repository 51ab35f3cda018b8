"""CPU oracle (float64) for exact attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and has no fallback to it.
"""
from .core import (attention, attention_bwd_flops, attention_flops, attention_grad, attention_probs, decode,
                   gather_pages, naive_workspace_bytes, online_attention, paged_decode, split_decode)

__all__ = ["attention", "attention_probs", "online_attention", "decode", "split_decode", "paged_decode",
           "gather_pages", "attention_grad",
           "naive_workspace_bytes", "attention_flops", "attention_bwd_flops"]
