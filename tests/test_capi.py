"""The C ABI without a GPU: every declared symbol is exported, and argument
validation rejects bad calls before anything reaches the device."""
import ctypes
import json
import os
import re

import pytest

from exact_io_aware_74_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, INVALID, UNSUPPORTED = 0, -1, -2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|void|const\s+char\s*\*)\s*\**\s*(fa_\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_f32", "fa_decode", "fa_naive_fwd", "fa_naive_workspace_bytes", "fa_status_str",
              "fa_last_hip_error", "fa_shutdown", "fa_decode_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes",
              "fa_decode_paged", "fa_fwd_fp8", "fa_decode_noalloc"):
        assert n in names
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES, f"binding lacks {name}"


# Fake, 16-byte aligned, never dereferenced "device" addresses: validation must
# fail (or the problem be empty) before any of them is used.
A = 0x100000
Bp = 0x200000
C = 0x300000
Dp = 0x400000
L = 0x500000


def fwd(lib, *, q=A, k=Bp, v=C, o=Dp, lse=L, B=1, H=1, N=16, d=64, causal=0, scale=0.125, f32=False):
    fn = lib.fa_fwd_f32 if f32 else lib.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_validation(lib, f32):
    assert fwd(lib, d=96, f32=f32) == UNSUPPORTED
    assert fwd(lib, d=32, f32=f32) == UNSUPPORTED
    assert fwd(lib, d=0, f32=f32) == INVALID
    assert fwd(lib, q=0, f32=f32) == INVALID
    assert fwd(lib, o=0, f32=f32) == INVALID
    assert fwd(lib, k=A + 8, f32=f32) == INVALID                    # misaligned
    assert fwd(lib, lse=L + 2, f32=f32) == INVALID                  # misaligned lse
    assert fwd(lib, N=-1, f32=f32) == INVALID
    assert fwd(lib, B=-3, f32=f32) == INVALID
    assert fwd(lib, scale=float("nan"), f32=f32) == INVALID
    assert fwd(lib, scale=float("inf"), f32=f32) == INVALID
    assert fwd(lib, scale=-0.5, f32=f32) == INVALID
    assert fwd(lib, o=A, f32=f32) == INVALID                        # output aliases q
    assert fwd(lib, o=A + 256, f32=f32) == INVALID                  # output overlaps q
    assert fwd(lib, lse=Bp + 64, f32=f32) == INVALID                # lse inside k
    assert fwd(lib, lse=Dp, f32=f32) == INVALID                     # lse on the output
    assert fwd(lib, B=1 << 20, H=1 << 12, N=1 << 12, f32=f32) == INVALID   # grid overflow
    # empty problems succeed without touching anything (null pointers allowed)
    assert fwd(lib, B=0, q=0, k=0, v=0, o=0, lse=0, f32=f32) == FA_OK
    assert fwd(lib, N=0, q=0, k=0, v=0, o=0, lse=0, f32=f32) == FA_OK
    assert fwd(lib, H=0, f32=f32) == FA_OK


def test_fwd_fp8_validation(lib):
    def f8(**kw):
        return lib.fa_fwd_fp8(kw.get("q", A), kw.get("k", Bp), kw.get("v", C), kw.get("o", Dp), kw.get("lse", L),
                              kw.get("B", 1), kw.get("H", 1), kw.get("N", 16), kw.get("d", 128), kw.get("causal", 1),
                              kw.get("scale", 0.088), kw.get("qd", 0.01), kw.get("kd", 0.01), kw.get("vd", 0.01), None)
    assert f8(d=96) == UNSUPPORTED                                   # FP8 path: d = 64 or 128
    assert f8(d=32) == UNSUPPORTED
    assert f8(d=0) == INVALID
    for bad in (float("nan"), float("inf"), -1.0):
        assert f8(scale=bad) == INVALID
        assert f8(qd=bad) == INVALID
        assert f8(vd=bad) == INVALID
    assert f8(q=0) == INVALID
    assert f8(v=C + 4) == INVALID
    assert f8(lse=L + 1) == INVALID
    assert f8(o=A) == INVALID                                        # output over q
    assert f8(o=Bp - 16 * 128) == INVALID                            # bf16 output (4 KiB) running into k
    assert f8(lse=A + 8 * 128) == INVALID                            # lse inside q
    assert f8(N=0, q=0, k=0, v=0, o=0, lse=0) == FA_OK


def test_decode_validation(lib):
    dec = lambda **kw: lib.fa_decode(kw.get("q", A), kw.get("k", Bp), kw.get("v", C), kw.get("o", Dp),
                                     kw.get("B", 2), kw.get("H", 2), kw.get("Lkv", 100), kw.get("d", 128),
                                     kw.get("nsplit", 4), None)
    assert dec(d=80) == UNSUPPORTED
    assert dec(Lkv=0) == INVALID
    assert dec(nsplit=0) == INVALID
    assert dec(nsplit=-2) == INVALID
    assert dec(q=0) == INVALID
    assert dec(v=C + 4) == INVALID
    assert dec(o=Bp) == INVALID                                      # output inside the K cache
    assert dec(B=0, q=0, k=0, v=0, o=0) == FA_OK


T = 0x600000
S = 0x700000


def test_decode_paged_validation(lib):
    def dec(**kw):
        return lib.fa_decode_paged(kw.get("q", A), kw.get("k", Bp), kw.get("v", C), kw.get("table", T),
                                   kw.get("lens", S), kw.get("o", Dp), kw.get("B", 2), kw.get("H", 2),
                                   kw.get("d", 128), kw.get("page_size", 16), kw.get("num_pages", 8),
                                   kw.get("max_pages", 4), kw.get("nsplit", 4), None)
    assert dec(d=80) == UNSUPPORTED
    for bad in (0, -16, 12, 3, 1 << 17):                            # not a power of two in 1 .. 65536
        assert dec(page_size=bad) == INVALID
    assert dec(num_pages=0) == INVALID
    assert dec(max_pages=0) == INVALID
    assert dec(nsplit=0) == INVALID
    assert dec(max_pages=1 << 16, page_size=1 << 15) == INVALID      # more than 2^30 keys per sequence
    assert dec(table=0) == INVALID
    assert dec(lens=0) == INVALID
    assert dec(table=T + 2) == INVALID                               # misaligned int32 table
    assert dec(lens=S + 1) == INVALID
    assert dec(k=Bp + 8) == INVALID
    assert dec(o=T) == INVALID                                       # output over the block table
    assert dec(o=Bp + 64) == INVALID                                 # output inside the K pool
    assert dec(o=S) == INVALID                                       # output over the lengths
    assert dec(B=0, q=0, k=0, v=0, table=0, lens=0, o=0) == FA_OK
    assert dec(H=0) == FA_OK


def test_decode_workspace_size(lib):
    # 16 x 32 heads, 64 splits of 512 keys, (d + 2) floats per split
    assert lib.fa_decode_workspace_bytes(16, 32, 32768, 128, 64) == 17_039_360
    # nsplit is clamped to Lkv and empty chunks are dropped: Lkv=10, nsplit=6 -> chunk 2 -> 5 splits
    assert lib.fa_decode_workspace_bytes(1, 1, 10, 64, 6) == 5 * 66 * 4
    assert lib.fa_decode_workspace_bytes(1, 1, 10, 64, 1000) == 10 * 66 * 4
    assert lib.fa_decode_workspace_bytes(1, 1, 0, 64, 4) == 0


def test_naive_workspace_matches_pages(lib, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pages_figures.json")))
    for key in ("score_matrix_t8192", "score_matrix_t16384"):
        e = g[key]
        # the ablation keeps S/P in float32: twice the pages' fp16 figure
        per_head = lib.fa_naive_workspace_bytes(1, 1, e["T"])
        assert per_head == 2 * e["T"] * e["T"] * e["elem_bytes"]
        assert lib.fa_naive_workspace_bytes(1, e["heads"], e["T"]) == e["heads"] * per_head
    assert lib.fa_naive_workspace_bytes(1, 32, 8192) == 8_589_934_592
    assert lib.fa_naive_workspace_bytes(-1, 1, 4) == 0


def test_naive_validation(lib):
    far = 1 << 36   # tensors far apart so that large N does not make them overlap
    nv = lambda ws=6 * far, nbytes=1 << 40, N=16, **kw: lib.fa_naive_fwd(
        far, 2 * far, 3 * far, 4 * far, 5 * far, kw.get("B", 1), kw.get("H", 1), N, kw.get("d", 64), 1, 0.125,
        ws, nbytes, None)
    assert nv(ws=0) == INVALID
    assert nv(nbytes=16 * 16 * 4 - 1) == INVALID
    assert nv(N=40000) == UNSUPPORTED
    assert nv(d=256) == UNSUPPORTED


def test_status_strings(lib):
    assert lib.fa_status_str(0) == b"FA_OK"
    assert lib.fa_status_str(-1) == b"FA_ERR_INVALID_ARG"
    assert lib.fa_status_str(-2) == b"FA_ERR_UNSUPPORTED"
    assert lib.fa_status_str(-3) == b"FA_ERR_HIP"
    assert lib.fa_status_str(-4) == b"FA_ERR_NOMEM"
    assert lib.fa_status_str(-5) == b"FA_ERR_TOO_LARGE"
    assert lib.fa_status_str(7) == b"FA_ERR_UNKNOWN"
    assert lib.fa_last_hip_error() == 0


def test_fwd_f32_rejects_a_grid_past_int(lib):
    """B*H*ceil(N/64) fits an int, but the fp32 kernel's one workgroup per four rows would need 2^31
    workgroups: rejected before any launch (fake tensors 2^42 bytes apart, so nothing overlaps)."""
    g = 1 << 42
    assert fwd(lib, q=g, k=2 * g, v=3 * g, o=4 * g, lse=5 * g, B=1, H=1 << 12, N=1 << 21, d=64, f32=True) == INVALID


def test_binding_errors_are_raised(lib):
    with pytest.raises(binding.FaError) as ei:
        binding._check("fa_fwd", UNSUPPORTED)
    assert "FA_ERR_UNSUPPORTED" in str(ei.value)


def test_product_path_does_not_touch_the_oracle():
    """The package and its C sources never import, call or link the oracle."""
    pkg = os.path.join(ROOT, "exact_io_aware_74_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
    assert "oracle" not in open(HEADER).read().lower()


def bwd(lib, *, q=A, k=Bp, v=C, o=Dp, do=0x600000, lse=L, dq=0x700000, dk=0x800000, dv=0x900000, B=1, H=1, N=16,
        d=64, causal=0, scale=0.125, ws=0xA00000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(B, H, N)
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, causal, scale, ws, ws_bytes, None)


def test_bwd_workspace_bytes(lib):
    # two float32 statistics per query row, rows padded to a multiple of 64 per head
    assert lib.fa_bwd_workspace_bytes(1, 1, 1) == 2 * 64 * 4
    assert lib.fa_bwd_workspace_bytes(2, 3, 65) == 2 * 6 * 128 * 4
    assert lib.fa_bwd_workspace_bytes(1, 32, 8192) == 2 * 32 * 8192 * 4
    assert lib.fa_bwd_workspace_bytes(0, 1, 16) == 0 and lib.fa_bwd_workspace_bytes(1, 1, -1) == 0


def test_bwd_validation(lib):
    assert bwd(lib, d=96) == UNSUPPORTED
    assert bwd(lib, scale=-1.0) == INVALID
    assert bwd(lib, scale=float("nan")) == INVALID
    assert bwd(lib, N=-1) == INVALID
    assert bwd(lib, do=0) == INVALID and bwd(lib, lse=0) == INVALID
    assert bwd(lib, dq=0) == INVALID and bwd(lib, dk=0) == INVALID and bwd(lib, dv=0) == INVALID
    assert bwd(lib, ws=0) == INVALID
    assert bwd(lib, ws_bytes=lib.fa_bwd_workspace_bytes(1, 1, 16) - 4) == INVALID  # too small
    assert bwd(lib, do=0x600002) == INVALID and bwd(lib, dk=0x800008) == INVALID   # misaligned
    assert bwd(lib, ws=0xA00004) == INVALID
    assert bwd(lib, dq=A) == INVALID            # output aliases q
    assert bwd(lib, dv=0x700000) == INVALID      # dv aliases dq
    assert bwd(lib, dk=0x600000) == INVALID      # dk aliases dout
    assert bwd(lib, ws=0x900000) == INVALID      # workspace aliases dv
    assert bwd(lib, B=0) == FA_OK and bwd(lib, N=0, ws=0, ws_bytes=0) == FA_OK   # empty problem: nothing enqueued


def test_bwd_rejects_a_statistics_grid_past_int(lib):
    """B*H*ceil(N/64) fits an int, but the row-statistics kernel's d/8 lanes per padded row would need
    2^31 workgroups: rejected before any launch. The fake tensors sit 2^43 bytes apart, so nothing
    overlaps and the grid check is what fails."""
    H, N, d = 1 << 16, 1 << 20, 64
    g = 1 << 43
    ptr = [g * (i + 1) for i in range(10)]
    ws_bytes = lib_ws = 2 * H * N * 4
    assert bwd(lib, q=ptr[0], k=ptr[1], v=ptr[2], o=ptr[3], do=ptr[4], lse=ptr[5], dq=ptr[6], dk=ptr[7],
               dv=ptr[8], ws=ptr[9], B=1, H=H, N=N, d=d, ws_bytes=ws_bytes) == INVALID
    assert lib.fa_bwd_workspace_bytes(1, H, N) == lib_ws
    assert lib.fa_bwd_workspace_bytes(1, 1, 2**31 - 1) == 0      # padding N to 64 rows would overflow


def test_decode_noalloc_validation(lib):
    """fa_decode's checks, then the fixed 32 MiB partials array's limit, all before any HIP call."""
    g = 1 << 40   # fake tensors far apart: large caches do not overlap

    def call(B=2, H=2, L=100, d=128, ns=4, q=g, k=2 * g, v=3 * g, o=4 * g):
        return lib.fa_decode_noalloc(q, k, v, o, B, H, L, d, ns, None)
    assert call(d=80) == UNSUPPORTED
    assert call(L=0) == INVALID and call(ns=0) == INVALID and call(B=-1) == INVALID
    assert call(q=0) == INVALID and call(v=3 * g + 4) == INVALID and call(o=2 * g) == INVALID
    assert call(B=0, q=0, k=0, v=0, o=0) == FA_OK
    assert lib.fa_decode_workspace_bytes(64, 32, 64, 128, 64) == 68157440 > 32 << 20
    assert call(B=64, H=32, L=64, ns=64) == -5                         # FA_ERR_TOO_LARGE
    assert lib.fa_decode_workspace_bytes(16, 32, 32768, 128, 64) <= 32 << 20   # the decode workload fits
