"""CPU oracle (float64) for exact attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and has no fallback to it.
"""
from .core import (attention, attention_flops, attention_grad, decode, gather_pages, naive_workspace_bytes,
                   online_attention, paged_decode, split_decode)

__all__ = ["attention", "online_attention", "decode", "split_decode", "paged_decode", "gather_pages",
           "attention_grad", "naive_workspace_bytes", "attention_flops"]
