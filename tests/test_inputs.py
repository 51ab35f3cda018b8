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


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * 60,
                        np.float32(2.0) ** rng.uniform(-14, 8.8, 100_000).astype(np.float32),
                        np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6])])
    x = np.clip(x, -448, 448).astype(np.float32)
    # exact ties between neighbouring codes, both signs
    codes = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = ((codes[:-1] + codes[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = si.f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_decoder_exact_on_every_code():
    bits = np.arange(256, dtype=np.uint8)
    ours = si.e4m3_bits_to_f32(bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(ours, ref)                 # NaN positions compare equal here
    finite = np.isfinite(ours)
    np.testing.assert_array_equal(si.f32_to_e4m3_bits(ours[finite]), bits[finite])


def test_fp8_quantisation_recipe():
    q8, k8, v8, (dq, dk, dv) = si.fp8_case(3, 1, 2, 100, 128, std=2.0)
    assert q8.dtype == np.uint8 and q8.shape == (1, 2, 100, 128)
    for codes, ds in ((q8, dq), (k8, dk), (v8, dv)):
        vals = si.fp8_as_float64(codes, ds)
        assert np.isclose(np.abs(vals).max(), 448 * ds, rtol=2 ** -4)   # the largest element maps to ~448
        assert ds == float(np.float32(ds))
    a = si.fp8_case(3, 1, 2, 100, 128, std=2.0)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], (q8, k8, v8)))
