"""Shared helpers of the GPU tests: moving seeded inputs to the device and the
parity metrics with their bounds."""
from __future__ import annotations

import numpy as np
import torch

import seeded_inputs as si

# Tolerances of the parity bar.
BF16_REL_L2 = 5e-3
BF16_MAX_ABS = 2e-2
BF16_LSE_ABS = 1e-3
F32_REL_L2 = 1e-5
F32_MAX_ABS = 1e-4
F32_LSE_ABS = 1e-5


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Kernel inputs (bf16 bit patterns or float32) to a device tensor, bit-exact."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device output to float64 (bf16 and float32 widen exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def metrics(out: np.ndarray, ref: np.ndarray):
    diff = out - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.max(np.abs(diff))) if diff.size else 0.0


def assert_close(out, ref, dtype: str, what: str = "O"):
    rel, mx = metrics(out, ref)
    if dtype == "bf16":
        assert np.isfinite(out).all(), f"{what}: non-finite values"
        assert rel <= BF16_REL_L2, f"{what}: relative L2 {rel:.3e} > {BF16_REL_L2}"
        assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx:.3e} > {BF16_MAX_ABS}"
    else:
        assert np.isfinite(out).all(), f"{what}: non-finite values"
        assert rel <= F32_REL_L2, f"{what}: relative L2 {rel:.3e} > {F32_REL_L2}"
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3e} > {F32_MAX_ABS}"
    return rel, mx


def assert_lse_close(out, ref, dtype: str):
    bound = BF16_LSE_ABS if dtype == "bf16" else F32_LSE_ABS
    mx = float(np.max(np.abs(out - ref))) if out.size else 0.0
    assert np.isfinite(out).all(), "LSE: non-finite values"
    assert mx <= bound, f"LSE: max abs {mx:.3e} > {bound}"
    return mx


def workload_inputs(w: si.Workload):
    """Full q, k, v of a workload as kernel inputs (numpy)."""
    return tuple(si.tensor_full(w, t) for t in ("q", "k", "v"))


def sample_rows(N: int, count: int, seed: int, tile: int = 128):
    """Query rows for sampled checks: tile edges, the ends, and random rows."""
    fixed = {0, 1, N - 1, N - 2}
    for t in range(tile, N, tile * max(1, (N // tile) // 8)):
        fixed.update({t - 1, t})
    rng = np.random.default_rng(seed)
    rest = rng.choice(N, size=min(N, count), replace=False)
    return sorted(r for r in fixed.union(rest.tolist()) if 0 <= r < N)
