"""Whole-tensor oracle references for the full-size workloads, one head per task in
worker processes.

Test infrastructure only. Each task regenerates its head's inputs from the seeded
generator (nothing large crosses a process boundary) and applies the plain
oracle to that head alone, exactly as a serial loop over heads would: the pool
only runs independent heads side by side so that the 16K workload's 32 heads
(a 16384 x 16384 float64 score matrix each) finish in well under a minute on a
many-core host. No torch and no GPU in the workers.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor, as_completed

import numpy as np

import oracle
import seeded_inputs as si


def _limit_blas_threads(n: int):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(n)
    except Exception:    # threadpoolctl missing: the BLAS keeps its default
        pass


def forward_head(name: str, b: int, h: int):
    """Oracle O [N, d] and LSE [N] of head (b, h) of a prefill workload."""
    w = si.WORKLOADS[name]
    q, k, v = (si.as_float64(si.tensor_slice(w, t, b, h), w.dtype)[None, None] for t in ("q", "k", "v"))
    O, L = oracle.attention(q, k, v, w.causal, w.scale)
    return b, h, O[0, 0], L[0, 0]


def fp8_forward_head(key, q8, k8, v8, descales, causal: bool, scale: float):
    """Oracle O and LSE of one head of FP8 inputs: the plain definition on the dequantised values
    (descale x e4m3 value, exact in float64). q8, k8, v8: that head's [N, d] e4m3 codes."""
    q, k, v = (si.fp8_as_float64(x, ds)[None, None] for x, ds in zip((q8, k8, v8), descales))
    O, L = oracle.attention(q, k, v, causal, scale)
    return key, O[0, 0], L[0, 0], float(np.abs(v).max())


def decode_heads(name: str, b: int, hs):
    """Oracle o [d] and lse of heads (b, h) for h in hs of the decode workload."""
    w = si.WORKLOADS[name]
    out = []
    for h in hs:
        q, k, v = (si.as_float64(si.tensor_slice(w, t, b, h), w.dtype)[None, None] for t in ("q", "k", "v"))
        o, lse = oracle.decode(q, k, v)
        out.append((b, h, o[0, 0], lse[0, 0]))
    return out


def default_workers(mem_per_task_gib: float) -> int:
    """Half the usable cores (each task's BLAS calls get two threads), at most 8, and no more
    tasks at once than a quarter of the host's memory holds."""
    cores = len(os.sched_getaffinity(0))
    try:
        mem_gib = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES") / 2**30
    except (ValueError, OSError):
        mem_gib = 32.0
    return max(1, min(8, cores // 2, int(mem_gib / 4 / mem_per_task_gib)))


def run(fn, tasks, workers: int):
    """Yields fn(*task) for every task, in completion order, from a pool of spawned workers."""
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(workers, mp_context=ctx, initializer=_limit_blas_threads, initargs=(2,)) as ex:
        futs = [ex.submit(fn, *t) for t in tasks]
        for f in as_completed(futs):
            yield f.result()
