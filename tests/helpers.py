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
# Per output row (the last axis, d values): relative L2 of each row on its own. The whole-tensor bound above is
# dominated by the rows of largest norm (in a causal pass the early rows, which see few keys), so an error
# confined to the small late rows could hide under it. Bound: the output's rounding to bf16 moves each element
# by at most 2^-8 of itself, and the probabilities' rounding moves a row by at most 2^-8 where one key dominates
# it (spread over many keys the errors average out), so a row's relative error stays below 2^-7 ~ 7.8e-3;
# measured worst rows are 4.7e-3 (forward, logit spread up to 2.5) and 2.0e-3 (decode). A row whose norm is
# below ROW_FLOOR * sqrt(d) is held to that absolute level instead.
BF16_ROW_REL = 1e-2
F32_ROW_REL = 1e-4
ROW_FLOOR = 1e-3


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


def worst_row(out: np.ndarray, ref: np.ndarray):
    """Largest per-row relative L2 (rows along the last axis) and its flat row index."""
    d = out.shape[-1]
    o2, r2 = out.reshape(-1, d), ref.reshape(-1, d)
    if o2.shape[0] == 0:
        return 0.0, -1
    ratio = np.linalg.norm(o2 - r2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), ROW_FLOOR * np.sqrt(d))
    i = int(np.argmax(ratio))
    return float(ratio[i]), i


def assert_close(out, ref, dtype: str, what: str = "O"):
    rel, mx = metrics(out, ref)
    row, at = worst_row(out, ref)
    if dtype == "bf16":
        assert np.isfinite(out).all(), f"{what}: non-finite values"
        assert rel <= BF16_REL_L2, f"{what}: relative L2 {rel:.3e} > {BF16_REL_L2}"
        assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx:.3e} > {BF16_MAX_ABS}"
        assert row <= BF16_ROW_REL, f"{what}: row {at} relative L2 {row:.3e} > {BF16_ROW_REL}"
    else:
        assert np.isfinite(out).all(), f"{what}: non-finite values"
        assert rel <= F32_REL_L2, f"{what}: relative L2 {rel:.3e} > {F32_REL_L2}"
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3e} > {F32_MAX_ABS}"
        assert row <= F32_ROW_REL, f"{what}: row {at} relative L2 {row:.3e} > {F32_ROW_REL}"
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


class WholeTensorCheck:
    """Parity over a whole output tensor, accumulated head by head: relative L2 over every
    element (sqrt of the summed squared errors over the summed squared reference), the
    largest absolute error, the largest LSE error, and the worst head's relative L2."""

    def __init__(self, dtype: str):
        self.dtype = dtype
        self.err2 = 0.0
        self.ref2 = 0.0
        self.max_abs = 0.0
        self.lse_abs = 0.0
        self.worst_head = (0.0, None)
        self.worst_row = (0.0, None)
        self.heads = 0
        self.finite = True

    def add(self, key, got, ref, got_lse=None, ref_lse=None):
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        self.finite = self.finite and bool(np.isfinite(got).all())
        diff = got - ref
        e2, r2 = float(np.sum(diff * diff)), float(np.sum(ref * ref))
        self.err2 += e2
        self.ref2 += r2
        self.max_abs = max(self.max_abs, float(np.max(np.abs(diff))) if diff.size else 0.0)
        head_rel = (e2 / r2) ** 0.5 if r2 > 0 else 0.0
        if head_rel >= self.worst_head[0]:
            self.worst_head = (head_rel, key)
        row, at = worst_row(got, ref)
        if row >= self.worst_row[0]:
            self.worst_row = (row, (key, at))
        if got_lse is not None:
            gl = np.asarray(got_lse, np.float64)
            self.finite = self.finite and bool(np.isfinite(gl).all())
            self.lse_abs = max(self.lse_abs, float(np.max(np.abs(gl - np.asarray(ref_lse, np.float64)))))
        self.heads += 1

    @property
    def rel_l2(self) -> float:
        return (self.err2 / self.ref2) ** 0.5 if self.ref2 > 0 else 0.0

    def summary(self) -> dict:
        return {"heads": self.heads, "rel_l2": self.rel_l2, "max_abs": self.max_abs, "lse_max_abs": self.lse_abs,
                "worst_head_rel_l2": self.worst_head[0], "worst_head": self.worst_head[1],
                "worst_row_rel_l2": self.worst_row[0], "worst_row": self.worst_row[1]}

    def assert_bounds(self, with_lse: bool = True):
        rel_b, abs_b, lse_b = ((BF16_REL_L2, BF16_MAX_ABS, BF16_LSE_ABS) if self.dtype == "bf16"
                               else (F32_REL_L2, F32_MAX_ABS, F32_LSE_ABS))
        s = self.summary()
        assert self.finite, f"non-finite outputs: {s}"
        assert self.rel_l2 <= rel_b, f"whole-tensor relative L2 {self.rel_l2:.3e} > {rel_b}: {s}"
        assert self.max_abs <= abs_b, f"max abs {self.max_abs:.3e} > {abs_b}: {s}"
        row_b = BF16_ROW_REL if self.dtype == "bf16" else F32_ROW_REL
        assert self.worst_row[0] <= row_b, f"row relative L2 {self.worst_row[0]:.3e} > {row_b}: {s}"
        if with_lse:
            assert self.lse_abs <= lse_b, f"LSE max abs {self.lse_abs:.3e} > {lse_b}: {s}"
        return s
