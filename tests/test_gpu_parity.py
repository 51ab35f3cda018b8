"""Parity of the HIP path with the CPU oracle, element by element, on seeded
inputs; at full workload sizes on sampled rows/heads the oracle computes one
by one. All calls go through the C ABI (via the ctypes binding)."""
import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from exact_io_aware_74_amd import binding as fa
import oracle_pool
from helpers import (WholeTensorCheck, assert_close, assert_lse_close, sample_rows, to_device, to_f64,
                     workload_inputs)

pytestmark = pytest.mark.gpu

W = si.WORKLOADS


def _fwd_case(q, k, v, dtype, causal, scale, rows=None, heads=None):
    """Run the GPU forward on full tensors and compare (sampled) rows/heads with the oracle."""
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    O, L = to_f64(o), to_f64(lse)
    q64, k64, v64 = (si.as_float64(x, dtype) for x in (q, k, v))
    B, H = q.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    Oref, Lref = oracle.attention(q64, k64, v64, causal, scale, rows=rows, heads=pairs)
    sel = slice(None) if rows is None else rows
    got_o = np.stack([O[b, h][sel] for b, h in pairs])
    got_l = np.stack([L[b, h][sel] for b, h in pairs])
    ref_o = np.stack([Oref[b, h] for b, h in pairs])
    ref_l = np.stack([Lref[b, h] for b, h in pairs])
    rel, mx = assert_close(got_o, ref_o, dtype)
    lmx = assert_lse_close(got_l, ref_l, dtype)
    return rel, mx, lmx


def test_workload_f32_n256_d64():
    w = W["f32_n256_d64"]
    q, k, v = workload_inputs(w)
    print("f32 256x64", _fwd_case(q, k, v, "f32", w.causal, w.scale))


def test_workload_bf16_b4h16_n1024_d64_causal():
    w = W["bf16_b4h16_n1024_d64_causal"]
    q, k, v = workload_inputs(w)
    print("bf16 4x16x1024x64 causal", _fwd_case(q, k, v, "bf16", w.causal, w.scale))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["bf16_h32_n8192_d128_causal_k2", "bf16_h32_n16384_d128_causal"])
def test_workload_whole_tensor(name):
    """The 8K (K x2) and 16K causal prefills against the oracle on every element of O and LSE,
    all 32 heads: whole-tensor relative L2, max abs and LSE bounds. The oracle runs head by head
    in worker processes, each regenerating its head from the seed."""
    w = W[name]
    q, k, v = workload_inputs(w)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    del q, k, v
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    O = o.float().cpu().numpy()
    L = lse.cpu().numpy()
    del qd, kd, vd, o, lse
    chk = WholeTensorCheck("bf16")
    tasks = [(name, b, h) for b in range(w.B) for h in range(w.H)]
    gib = 3.2 * w.N * w.N * 8 / 2**30          # about 3.2 score-sized float64 arrays live per task
    for b, h, Oref, Lref in oracle_pool.run(oracle_pool.forward_head, tasks, oracle_pool.default_workers(gib)):
        chk.add((b, h), O[b, h], Oref, L[b, h], Lref)
    assert chk.heads == w.B * w.H
    print(name, chk.assert_bounds())


def test_workload_128k_prefill_sampled():
    """128K-token causal prefill, B=4 x H=32: each tensor holds 2^31 elements, so element offsets
    of the later heads pass 2^31. Sampled rows of heads at both ends against the oracle; only those
    rows leave the device."""
    w = W["bf16_b4h32_n131072_d128_causal"]
    q, k, v = workload_inputs(w)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o, lse = fa.fwd(qd, kd, vd, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, 48, seed=w.wid, tile=256)
    ridx = torch.tensor(rows, device="cuda")
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, h in [(0, 0), (1, 17), (3, 30), (3, 31)]:
        got_o.append(to_f64(o[b, h].index_select(0, ridx)))
        got_l.append(to_f64(lse[b, h].index_select(0, ridx)))
        one = lambda x: si.as_float64(x[b:b + 1, h:h + 1], "bf16")
        O, L = oracle.attention(one(q), one(k), one(v), True, w.scale, rows=rows)
        ref_o.append(O[0, 0])
        ref_l.append(L[0, 0])
    print("128K", assert_close(np.stack(got_o), np.stack(ref_o), "bf16"),
          assert_lse_close(np.stack(got_l), np.stack(ref_l), "bf16"))
    assert torch.isfinite(o[3, 31]).all().item()


@pytest.mark.parametrize("name", ["bf16_h32_n8192_d128_causal_k2", "bf16_h32_n16384_d128_causal",
                                  "bf16_b4h32_n131072_d128_causal"])
def test_fused_pass_allocates_nothing(name):
    """The fused pass needs no workspace: device memory is unchanged across the
    call (an N x N score buffer would be 1 GiB per head at N = 16384)."""
    w = W[name]
    shape = (w.B, w.H, w.N, w.d)
    q, k, v = (torch.randn(shape, device="cuda").to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(shape[:3], device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert free0 - torch.cuda.mem_get_info()[0] <= (2 << 20)
    assert torch.isfinite(o.float()).all().item()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 383, 1000])
def test_ragged_shapes(dtype, d, causal, N):
    B, H = (2, 3) if N <= 200 else (1, 2)
    q, k, v = si.random_case(N * 7 + d, B, H, N, d, dtype)
    _fwd_case(q, k, v, dtype, causal, fa.default_scale(d))


@pytest.mark.parametrize("std", [0.25, 3.0, 6.0])
def test_logit_ranges(std):
    """Flat and very peaked softmax rows (large logits stress the running-max rescale)."""
    q, k, v = si.random_case(int(std * 100), 1, 4, 300, 128, "bf16", std=std)
    _fwd_case(q, k, v, "bf16", True, fa.default_scale(128))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_zero_closed_form(dtype):
    """scale 0: row i of causal attention is the mean of V rows 0..i; LSE = ln(i+1)."""
    N, d = 300, 64
    q, k, v = si.random_case(5, 1, 2, N, d, dtype)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    o, lse = fa.fwd(qd, kd, vd, causal=True, scale=0.0)
    v64 = si.as_float64(v, dtype)
    ref = np.cumsum(v64, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert_close(to_f64(o), ref, dtype)
    assert_lse_close(to_f64(lse), np.broadcast_to(np.log(np.arange(1, N + 1)), (1, 2, N)), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_key_returns_v(dtype):
    q, k, v = si.random_case(6, 2, 2, 1, 128, dtype)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    o, lse = fa.fwd(qd, kd, vd, causal=True)
    assert torch.equal(o, vd)
    s = fa.default_scale(128)
    ref = s * np.einsum("bhnd,bhnd->bhn", si.as_float64(q, dtype), si.as_float64(k, dtype))
    assert_lse_close(to_f64(lse), ref, dtype)


def test_deterministic_and_fully_written():
    q, k, v = si.random_case(7, 2, 4, 777, 128, "bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o1 = torch.full_like(qd, float("nan"))
    l1 = torch.full((2, 4, 777), float("nan"), device="cuda")
    fa.fwd(qd, kd, vd, causal=True, out=o1, lse=l1)
    o2, l2 = fa.fwd(qd, kd, vd, causal=True)
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_guard_bands_untouched():
    """Writes stay inside O and LSE: canaries around both survive."""
    B, H, N, d = 1, 3, 200, 64
    q, k, v = si.random_case(8, B, H, N, d, "bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    n = B * H * N * d
    buf = torch.full((n + 2 * 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    o = buf[4096:4096 + n].view(B, H, N, d)
    lbuf = torch.full((B * H * N + 2 * 1024,), 7.0, device="cuda")
    lse = lbuf[1024:1024 + B * H * N].view(B, H, N)
    fa.fwd(qd, kd, vd, causal=False, out=o, lse=lse)
    assert (buf[:4096] == 7).all() and (buf[4096 + n:] == 7).all()
    assert (lbuf[:1024] == 7).all() and (lbuf[1024 + B * H * N:] == 7).all()


def test_lse_optional():
    q, k, v = si.random_case(9, 1, 2, 150, 64, "bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o1, _ = fa.fwd(qd, kd, vd, causal=True)
    o2, l2 = fa.fwd(qd, kd, vd, causal=True, return_lse=False)
    assert l2 is None and torch.equal(o1, o2)


def test_misaligned_pointer_rejected():
    base = torch.zeros(4 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    t = base[1:1 + 4 * 64].view(1, 1, 4, 64)   # contiguous, but 2 bytes past a 16-byte boundary
    with pytest.raises(fa.FaError) as ei:
        fa.fwd(t, t, t)
    assert ei.value.status == -1


def test_forward_replays_from_a_captured_graph():
    """The fused pass allocates nothing and never synchronises, so it can be captured in a HIP graph.
    Replays, with other eager work and host synchronisations between them, match the eager result
    bit for bit; the inputs are rewritten between replays to show each replay really recomputes."""
    q, k, v = si.random_case(31, 2, 4, 700, 128, "bf16")
    q2, k2, v2 = si.random_case(32, 2, 4, 700, 128, "bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((2, 4, 700), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up outside capture
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=lse)
    for src in ((q, k, v), (q2, k2, v2), (q, k, v)):
        for dst, x in zip((qd, kd, vd), src):
            dst.copy_(to_device(x, "bf16"))
        ref_o, ref_l = fa.fwd(qd, kd, vd, causal=True)       # eager, on the current stream
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


def test_extreme_logits():
    """Logits spanning hundreds of exp2 units (q, k ~ 4 N(0,1), d = 64, scale 1): most rows are
    dominated by one key, most probabilities underflow to 0, and the running maximum is raised
    many times along a row."""
    q, k, v = si.random_case(41, 1, 2, 500, 64, "bf16", std=4.0)
    print("extreme", _fwd_case(q, k, v, "bf16", True, 1.0))


@pytest.mark.parametrize("causal", [True, False])
def test_rising_row_maxima(causal):
    """Every row's logits climb along the keys (Q shifted along a unit direction u, K rows moved along u by a
    ramp up to 100), so the reference maximum must be raised in many sub-tiles after the first, each time
    rescaling an output that already holds earlier keys. A float64 model of the kernel's rule predicts the
    exact update on about a third of all sub-tiles here (one 777-row head, d = 128); N is ragged."""
    q, k, v = si.random_case(77, 1, 2, 777, 128, "bf16")
    u = np.random.Generator(np.random.PCG64([0, 77])).standard_normal(128)
    u /= np.linalg.norm(u)
    ramp = np.linspace(0.0, 100.0, k.shape[2])[None, None, :, None]
    q2 = si.f32_to_bf16_bits((si.as_float64(q, "bf16") + 3.0 * u).astype(np.float32))
    k2 = si.f32_to_bf16_bits((si.as_float64(k, "bf16") + ramp * u).astype(np.float32))
    print("rising", causal, _fwd_case(q2, k2, v, "bf16", causal, fa.default_scale(128)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_common_key_offset_shifts_only_lse(causal, d):
    """Adding one vector u to every key row adds scale * q_i . u to every logit of row i: the softmax,
    so O, is unchanged and the LSE moves by exactly that amount ("flashattention-memory-bound"
    (appliedaiprep.com), "Exact or approximate? Exact"). K and u sit on a 1/16 grid with |K + u| < 8,
    so K + u is exact in bf16 and the kernel sees precisely the shifted keys. Both runs are compared
    with the oracle on the unshifted keys."""
    B, H, N = 1, 3, 333
    rng = np.random.Generator(np.random.PCG64([0, 9100, d, int(causal)]))
    q = si.f32_to_bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))
    kq = np.clip(np.round(rng.standard_normal((B, H, N, d)) * 16), -64, 64) / 16          # |K| <= 4
    u = np.clip(np.round(rng.standard_normal((B, H, 1, d)) * 24), -48, 48) / 16            # |u| <= 3
    k = si.f32_to_bf16_bits(kq.astype(np.float32))
    k_shift = si.f32_to_bf16_bits((kq + u).astype(np.float32))
    assert np.array_equal(si.as_float64(k_shift, "bf16"), kq + u)                          # exact in bf16
    v = si.f32_to_bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))
    scale = fa.default_scale(d)
    q64, v64 = si.as_float64(q, "bf16"), si.as_float64(v, "bf16")
    Oref, Lref = oracle.attention(q64, kq, v64, causal, scale)
    shift = float(np.float32(scale)) * np.einsum("bhnd,bhd->bhn", q64, u[:, :, 0, :])
    qd, vd = to_device(q, "bf16"), to_device(v, "bf16")
    o0, l0 = fa.fwd(qd, to_device(k, "bf16"), vd, causal=causal, scale=scale)
    o1, l1 = fa.fwd(qd, to_device(k_shift, "bf16"), vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert_close(to_f64(o0), Oref, "bf16")
    assert_lse_close(to_f64(l0), Lref, "bf16")
    rel, mx = assert_close(to_f64(o1), Oref, "bf16", what="O with shifted keys")
    lmx = assert_lse_close(to_f64(l1), Lref + shift, "bf16")
    print("key offset", causal, d, rel, mx, lmx, float(np.abs(shift).max()))


@pytest.mark.parametrize("d", [64, 128])
def test_joint_key_value_permutation_and_query_permutation(d):
    """Non-causal: permuting the K and V rows together leaves O and LSE unchanged, and permuting the
    Q rows permutes them ("flashattention-memory-bound" (appliedaiprep.com), "Exact or approximate?
    Exact"). The kernel's key order and wave membership change, so only rounding may differ:
    every run is checked against the oracle on the original order."""
    B, H, N = 2, 2, 450
    q, k, v = si.random_case(9200 + d, B, H, N, d, "bf16", std=1.5)
    scale = fa.default_scale(d)
    Oref, Lref = oracle.attention(*(si.as_float64(x, "bf16") for x in (q, k, v)), False, scale)
    pk = np.random.default_rng(d).permutation(N)
    pq = np.random.default_rng(d + 1).permutation(N)
    o1, l1 = fa.fwd(*(to_device(np.ascontiguousarray(x), "bf16") for x in (q, k[:, :, pk], v[:, :, pk])),
                    causal=False, scale=scale)
    o2, l2 = fa.fwd(*(to_device(np.ascontiguousarray(x), "bf16") for x in (q[:, :, pq], k, v)), causal=False,
                    scale=scale)
    torch.cuda.synchronize()
    assert_close(to_f64(o1), Oref, "bf16", what="O with K/V rows permuted")
    assert_lse_close(to_f64(l1), Lref, "bf16")
    assert_close(to_f64(o2), Oref[:, :, pq], "bf16", what="O with Q rows permuted")
    assert_lse_close(to_f64(l2), Lref[:, :, pq], "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_d64_large_grid_takes_the_eight_wave_path(causal):
    """At d = 64 the launcher takes 128-row workgroups only when 256-row tiles would give fewer than two
    workgroups per CU (512 tiles); B=1 H=32 N=4096 has exactly 512, so this runs the 256-row, eight-wave
    kernel (N ragged by one key past a tile in the second case). Every element against the oracle."""
    N = 4096 if causal else 4095
    q, k, v = si.random_case(9300 + N, 1, 32, N, 64, "bf16", std=1.5)
    print("d64 eight-wave", causal, _fwd_case(q, k, v, "bf16", causal, fa.default_scale(64)))


@pytest.mark.parametrize("B,H,N,causal", [(2, 32, 4096, True), (3, 24, 4000, False)])
def test_head_grouped_workgroup_order(B, H, N, causal):
    """With 64 or more heads of 16 or more 256-row query tiles the launcher orders the workgroups in
    groups of 16 heads (two per XCD at a time); B*H = 72 leaves a short last group of 8 heads. Every
    element of O and the LSE against the oracle."""
    q, k, v = si.random_case(9400 + N + B, B, H, N, 128, "bf16", std=1.0)
    print("grouped order", B, H, N, causal, _fwd_case(q, k, v, "bf16", causal, fa.default_scale(128)))
