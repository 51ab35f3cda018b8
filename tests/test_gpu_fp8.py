"""Parity of the FP8 forward (fa_fwd_fp8) with the oracle's plain definition on
the dequantised inputs (descale * e4m3 value, exact in float64), through the
C ABI.

Tolerance. The pages fix no FP8 arithmetic, so the bound is derived from what
the kernel rounds: the probabilities enter the P V product as e4m3 (3
mantissa bits, relative rounding error at most 2^-4, after an exact
power-of-two scaling that keeps them normal down to 2^-12 of the row
reference), the row sums use the unrounded fp32 probabilities, and O is
rounded once to bf16. Every output element therefore satisfies
|O - exact| <= (2^-4 + 2^-8) * max|V| (the fp32 accumulation adds far less):
the max-abs bound below is 0.07 * max|V|. With random-sign rounding errors
the normwise error is about 2^-4 / sqrt(3) times a factor below 1; a numpy
emulation of these roundings gives relative L2 errors of 0.5 % (peaked rows)
to 2.6 % (flat rows) on these shapes, and the bound is 4e-2. The LSE uses the
fp32 probabilities and keeps the bf16 path's bound (1e-3). Cases whose
probabilities are exact powers of two (scale 0, a single key) are checked to
the bf16 bounds.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from exact_io_aware_74_amd import binding as fa
import oracle_pool
from helpers import assert_close, assert_lse_close, to_f64

pytestmark = pytest.mark.gpu

FP8_REL_L2 = 4e-2
FP8_MAX_ABS_OF_VMAX = 0.07


def dev8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def assert_fp8_close(got, ref, vmax, what="O"):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.abs(got - ref).max())
    assert rel <= FP8_REL_L2, f"{what}: relative L2 {rel:.3e} > {FP8_REL_L2}"
    assert mx <= FP8_MAX_ABS_OF_VMAX * vmax, f"{what}: max abs {mx:.3e} > {FP8_MAX_ABS_OF_VMAX} * {vmax:.3f}"
    return rel, mx / vmax


def fp8_case_run(q8, k8, v8, ds, causal, scale, rows=None, heads=None):
    o, lse = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds, causal=causal, scale=scale)
    torch.cuda.synchronize()
    B, H = q8.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    sel = slice(None) if rows is None else rows
    got_o, got_l, ref_o, ref_l, vmax = [], [], [], [], 0.0
    for b, h in pairs:
        one = [si.fp8_as_float64(x[b:b + 1, h:h + 1], d) for x, d in zip((q8, k8, v8), ds)]
        O, L = oracle.attention(*one, causal, scale, rows=rows)
        ref_o.append(O[0, 0])
        ref_l.append(L[0, 0])
        got_o.append(to_f64(o[b, h])[sel])
        got_l.append(to_f64(lse[b, h])[sel])
        vmax = max(vmax, float(np.abs(one[2]).max()))
    return np.stack(got_o), np.stack(ref_o), np.stack(got_l), np.stack(ref_l), vmax


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000])
def test_ragged_shapes(causal, N, d):
    B, H = (2, 3) if N <= 257 else (1, 2)
    q8, k8, v8, ds = si.fp8_case(N + 7 * causal + d, B, H, N, d)
    go, ro, gl, rl, vmax = fp8_case_run(q8, k8, v8, ds, causal, fa.default_scale(d))
    assert_fp8_close(go, ro, vmax)
    assert_lse_close(gl, rl, "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("std", [0.25, 1.0, 3.0])
def test_logit_ranges(std, d):
    q8, k8, v8, ds = si.fp8_case(int(100 * std) + d, 1, 4, 600, d, std=std)
    go, ro, gl, rl, vmax = fp8_case_run(q8, k8, v8, ds, True, fa.default_scale(d))
    print("fp8 std", std, assert_fp8_close(go, ro, vmax))
    assert_lse_close(gl, rl, "bf16")


@pytest.mark.timeout(900)
def test_workload_8k_causal_whole_tensor():
    """The 8K causal prefill workload's draws (K doubled), quantised per tensor to e4m3: every element
    of all 32 heads against the oracle on the dequantised inputs (worker processes, one head each)."""
    w = si.WORKLOADS["bf16_h32_n8192_d128_causal_k2"]
    q8, k8, v8, ds = si.fp8_workload(w)
    o, lse = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    O, L = o.float().cpu().numpy(), lse.cpu().numpy()
    err2 = ref2 = mx = lmx = vmax = 0.0
    tasks = [((0, h), q8[0, h], k8[0, h], v8[0, h], ds, True, w.scale) for h in range(w.H)]
    for (b, h), Oref, Lref, vm in oracle_pool.run(oracle_pool.fp8_forward_head, tasks,
                                                  oracle_pool.default_workers(2.0)):
        diff = O[b, h].astype(np.float64) - Oref
        err2, ref2 = err2 + float(np.sum(diff * diff)), ref2 + float(np.sum(Oref * Oref))
        mx = max(mx, float(np.abs(diff).max()))
        lmx = max(lmx, float(np.abs(L[b, h].astype(np.float64) - Lref).max()))
        vmax = max(vmax, vm)
    rel = (err2 / ref2) ** 0.5
    assert np.isfinite(O).all() and np.isfinite(L).all()
    assert rel <= FP8_REL_L2, f"whole-tensor relative L2 {rel:.3e} > {FP8_REL_L2}"
    assert mx <= FP8_MAX_ABS_OF_VMAX * vmax, f"max abs {mx:.3e} > {FP8_MAX_ABS_OF_VMAX} * {vmax:.3f}"
    assert lmx <= 1e-3, f"LSE max abs {lmx:.3e}"
    print("fp8 8K whole tensor", rel, mx / vmax, lmx)


def test_scale_zero_closed_form():
    """scale 0: every probability is exactly 2^6, so O is the prefix mean of the dequantised V
    (bf16 bounds) and LSE = ln(i + 1)."""
    N = 300
    q8, k8, v8, ds = si.fp8_case(5, 1, 2, N, 128)
    o, lse = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds, causal=True, scale=0.0)
    v64 = si.fp8_as_float64(v8, ds[2])
    ref = np.cumsum(v64, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert_close(to_f64(o), ref, "bf16")
    assert_lse_close(to_f64(lse), np.broadcast_to(np.log(np.arange(1, N + 1)), (1, 2, N)), "bf16")


def test_single_key_returns_v():
    q8, k8, v8, ds = si.fp8_case(6, 2, 2, 1, 128)
    o, lse = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds, causal=True)
    v64 = si.fp8_as_float64(v8, ds[2])
    assert_close(to_f64(o), v64, "bf16")
    s = fa.default_scale(128)
    qk = np.einsum("bhnd,bhnd->bhn", si.fp8_as_float64(q8, ds[0]), si.fp8_as_float64(k8, ds[1]))
    assert_lse_close(to_f64(lse), float(np.float32(s)) * qk, "bf16")


def test_descales_act_on_the_logical_inputs():
    """Halving every V code's value (exact: all values are normal e4m3 numbers of magnitude
    >= 2^-4) and doubling v_descale leaves the logical V, and the output, unchanged bit for bit."""
    q8, k8, _, ds = si.fp8_case(9, 1, 2, 200, 128)
    rng = np.random.default_rng(9)
    vals = (rng.choice([-1.0, 1.0], size=q8.shape) * np.exp2(rng.integers(-4, 7, size=q8.shape))
            * rng.choice([1.0, 1.25, 1.5, 1.75], size=q8.shape)).astype(np.float32)
    v8, v8h = si.f32_to_e4m3_bits(vals), si.f32_to_e4m3_bits(vals / 2)
    assert np.array_equal(si.e4m3_bits_to_f32(v8h) * 2, si.e4m3_bits_to_f32(v8))
    vd = float(np.float32(0.01))
    a, _ = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), (ds[0], ds[1], vd), causal=False)
    b, _ = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8h), (ds[0], ds[1], 2 * vd), causal=False)
    assert torch.equal(a, b)


def test_deterministic_and_fully_written():
    q8, k8, v8, ds = si.fp8_case(10, 2, 3, 777, 128)
    o1 = torch.full((2, 3, 777, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((2, 3, 777), float("nan"), device="cuda")
    fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds, causal=True, out=o1, lse=l1)
    o2, l2 = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds, causal=True)
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_float8_dtype_accepted():
    q8, k8, v8, ds = si.fp8_case(11, 1, 1, 64, 128)
    a, _ = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), ds)
    b, _ = fa.fwd_fp8(*(dev8(x).view(torch.float8_e4m3fn) for x in (q8, k8, v8)), ds)
    assert torch.equal(a, b)


def test_head_grouped_order():
    """B=2 H=32 N=4096 causal: 64 heads of 16 query tiles take the workgroup order in groups of 16 heads.
    Whole heads from both groups and several XCD positions against the oracle."""
    q8, k8, v8, ds = si.fp8_case(4244, 2, 32, 4096, 128)
    go, ro, gl, rl, vmax = fp8_case_run(q8, k8, v8, ds, True, fa.default_scale(128),
                                        heads=[(0, 0), (0, 9), (0, 23), (1, 6), (1, 31)])
    print("fp8 grouped", assert_fp8_close(go, ro, vmax))
    assert_lse_close(gl, rl, "bf16")
