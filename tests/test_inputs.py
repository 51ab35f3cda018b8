"""The seeded input generator: determinism, slice independence and the bf16 cast."""
import numpy as np
import torch

import seeded_inputs as si


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(123)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # add exact ties (low 16 bits == 0x8000) with both even and odd kept bits
    u = rng.integers(0, 2**32, size=4096, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0x3FFF0000)) | np.uint32(0x8000)
    ties = u.view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-40, 65504.0, 3.4e38])])
    ours = si.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = si.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    np.testing.assert_array_equal(si.f32_to_bf16_bits(f[finite]), bits[finite])


def test_deterministic_and_independent_slices():
    w = si.WORKLOADS["bf16_b4h16_n1024_d64_causal"]
    a = si.tensor_slice(w, "q", 1, 3)
    b = si.tensor_slice(w, "q", 1, 3)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (1024, 64) and a.dtype == np.uint16
    assert not np.array_equal(si.tensor_slice(w, "q", 1, 4), a)
    assert not np.array_equal(si.tensor_slice(w, "k", 1, 3), a)
    full = si.tensor_full(w, "q")
    np.testing.assert_array_equal(full[1, 3], a)
    part = si.tensor_full(w, "q", heads=[(1, 3)])
    np.testing.assert_array_equal(part[1, 3], a)
    assert not part[0, 0].any()


def test_k_multiplier_exact():
    w = si.WORKLOADS["bf16_h32_n8192_d128_causal_k2"]
    k = si.bf16_bits_to_f32(si.tensor_slice(w, "k", 0, 5)[:64])
    raw = si.normal_f32(w.wid, "k", 0, 5, (w.N, w.d))[:64]
    np.testing.assert_array_equal(k, 2.0 * si.bf16_bits_to_f32(si.f32_to_bf16_bits(raw)))


def test_workload_table():
    w = si.WORKLOADS["f32_n256_d64"]
    assert w.dtype == "f32" and w.scale == np.float32(0.125) and not w.causal
    d = si.WORKLOADS["decode_b16h32_l32768_d128"]
    assert d.decode and d.nk == 32768 and d.nsplit == 64
    assert si.tensor_slice(d, "q", 0, 0).shape == (1, 128)
    x = si.tensor_slice(w, "q", 0, 0)
    assert x.dtype == np.float32 and abs(float(x.std()) - 1.0) < 0.05
