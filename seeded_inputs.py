"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds random draws and the fp32 -> bf16 input cast only; it holds
none of the attention arithmetic. Both the CPU oracle's tests and the GPU
tests/bench draw their Q, K, V here, so the two sides see identical values.

Recipe (same for every workload):
  * one numpy PCG64 stream per (workload id, tensor, batch index, head index),
    seeded with the sequence [0, workload id, tensor id, b, h], so any single
    head can be regenerated alone;
  * values i.i.d. standard normal drawn in float32;
  * an optional exact multiplier (the 8K workload doubles K, which is exact in
    bf16 because it only moves the exponent);
  * for bf16 workloads, round-to-nearest-even to bf16. The bf16 bit patterns
    are what the GPU receives and what the oracle decodes to float64.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BASE_SEED = 0
TENSOR_ID = {"q": 0, "k": 1, "v": 2}


@dataclass(frozen=True)
class Workload:
    wid: int            # workload id, part of every seed
    name: str
    B: int
    H: int
    N: int              # query rows per head (1 for decode)
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    decode: bool = False
    Lkv: int = 0        # decode cache length
    nsplit: int = 0     # decode split count
    k_mult: float = 1.0

    @property
    def scale(self) -> float:
        """1/sqrt(d), rounded to float32 (the value the kernels receive)."""
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def nk(self) -> int:
        """Number of key rows per head."""
        return self.Lkv if self.decode else self.N


# The workloads of this library's test and benchmark plan.
WORKLOADS = {
    "f32_n256_d64": Workload(1, "f32_n256_d64", 1, 1, 256, 64, "f32", False),
    "bf16_b4h16_n1024_d64_causal": Workload(2, "bf16_b4h16_n1024_d64_causal", 4, 16, 1024, 64, "bf16", True),
    "bf16_h32_n8192_d128_causal_k2": Workload(3, "bf16_h32_n8192_d128_causal_k2", 1, 32, 8192, 128, "bf16", True,
                                              k_mult=2.0),
    "bf16_h32_n16384_d128_causal": Workload(4, "bf16_h32_n16384_d128_causal", 1, 32, 16384, 128, "bf16", True),
    "decode_b16h32_l32768_d128": Workload(5, "decode_b16h32_l32768_d128", 16, 32, 1, 128, "bf16", False,
                                          decode=True, Lkv=32768, nsplit=64),
    "bf16_b4h32_n131072_d128_causal": Workload(6, "bf16_b4h32_n131072_d128_causal", 4, 32, 131072, 128, "bf16",
                                               True),
}


def normal_f32(wid: int, tensor: str, b: int, h: int, shape) -> np.ndarray:
    """i.i.d. N(0,1) float32 draws for one (workload, tensor, b, h) slice."""
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, wid, TENSOR_ID[tensor], b, h]))
    return rng.standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bit patterns.

    Inputs here are finite normal draws, so NaN handling is not needed; a NaN
    input is rejected rather than silently rounded.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("f32_to_bf16_bits expects finite inputs")
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _slice_values(w: Workload, tensor: str, b: int, h: int, rows: int) -> np.ndarray:
    x = normal_f32(w.wid, tensor, b, h, (rows, w.d))
    if tensor == "k" and w.k_mult != 1.0:
        x = (x * np.float32(w.k_mult)).astype(np.float32)
    return x


def tensor_slice(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One head of one tensor, as the kernels receive it.

    Returns uint16 bf16 bit patterns for bf16 workloads, float32 otherwise.
    Shape [rows, d], rows = N for q (1 for decode) and nk for k/v.
    """
    rows = (1 if w.decode else w.N) if tensor == "q" else w.nk
    x = _slice_values(w, tensor, b, h, rows)
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else x


def tensor_full(w: Workload, tensor: str, heads=None, threads: int | None = None) -> np.ndarray:
    """Whole [B, H, rows, d] tensor (or only the (b, h) pairs in ``heads``, others zero).

    Slices are generated in parallel threads; numpy releases the GIL while it
    fills them.
    """
    rows = (1 if w.decode else w.N) if tensor == "q" else w.nk
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    out = np.zeros((w.B, w.H, rows, w.d), dtype=dt)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)] if heads is None else list(heads)

    def fill(bh):
        b, h = bh
        out[b, h] = tensor_slice(w, tensor, b, h)

    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    if len(pairs) <= 1 or nthreads <= 1:
        for bh in pairs:
            fill(bh)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, pairs))
    return out


def as_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode kernel-input values (bf16 bits or float32) to float64, exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def random_case(seed: int, B: int, H: int, N: int, d: int, dtype: str, nk: int | None = None, std: float = 1.0):
    """Small ad-hoc case for ragged-shape tests: returns (q, k, v) kernel inputs.

    q is [B,H,N,d]; k, v are [B,H,nk,d] (nk defaults to N). q and k are
    std * N(0,1) (std sets how peaked the softmax rows are), v is N(0,1);
    all cast to bf16 (RNE) for bf16 cases.
    """
    nk = N if nk is None else nk
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, 1000 + seed, B, H, N, d, nk]))
    outs = []
    for rows, sd in ((N, std), (nk, std), (nk, 1.0)):
        x = (rng.standard_normal((B, H, rows, d), dtype=np.float32) * np.float32(sd)).astype(np.float32)
        outs.append(f32_to_bf16_bits(x) if dtype == "bf16" else x)
    return tuple(outs)


def upstream_grad(seed: int, B: int, H: int, N: int, d: int, dtype: str) -> np.ndarray:
    """Seeded upstream gradient dL/dO for backward tests: N(0,1), [B,H,N,d], cast like the inputs."""
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, 5000 + seed, B, H, N, d]))
    x = rng.standard_normal((B, H, N, d), dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


BF16_NAN_BITS = 0x7FC0


def seq_lengths(seed: int, B: int, Lmax: int, page_size: int) -> np.ndarray:
    """Seeded ragged cache lengths in [1, Lmax] for paged-decode tests.

    The first entries take edge values that cut pages at every place (one key,
    one page minus one key, one full page, one page plus one key, Lmax), the
    rest are uniform draws; values above Lmax are clipped.
    """
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, 6000 + seed, B, Lmax, page_size]))
    lens = rng.integers(1, Lmax + 1, size=B)
    edges = [1, page_size - 1, page_size, page_size + 1, Lmax]
    for i, e in enumerate(edges[:B]):
        lens[i] = e
    return np.clip(lens, 1, Lmax).astype(np.int32)


def page_table(seed: int, B: int, H: int, Lmax: int, d: int, seq_lens, page_size: int, spare_pages: int = 3):
    """The block table of ``page_cache`` alone: (table int32 [B, ceil(Lmax / page_size)], num_pages).

    Sequence b takes ceil(seq_lens[b] / page_size) pool pages, handed out in a
    seeded random order; entries past its last page are -1.
    """
    lens = np.asarray(seq_lens, dtype=np.int32)
    if lens.shape != (B,) or lens.min(initial=0) < 0 or lens.max(initial=0) > Lmax:
        raise ValueError("seq_lens must be [B] values in [0, Lmax]")
    max_pages = -(-Lmax // page_size)
    used = [-(-int(n) // page_size) for n in lens]
    num_pages = sum(used) + spare_pages
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, 7000 + seed, B, H, Lmax, d, page_size]))
    order = rng.permutation(num_pages)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        table[b, :used[b]] = order[cursor:cursor + used[b]]
        cursor += used[b]
    return table, num_pages


def page_cache(seed: int, kc: np.ndarray, vc: np.ndarray, seq_lens, page_size: int, spare_pages: int = 3):
    """Scatter contiguous caches into a shuffled page pool (layout only, no arithmetic).

    kc, vc: [B, H, Lmax, d] kernel inputs. Returns (k_pages, v_pages,
    block_table, seq_lens): pools [num_pages, H, page_size, d] of the same
    dtype, block_table int32 [B, ceil(Lmax / page_size)] and seq_lens int32.
    Sequence b's key j (j < seq_lens[b]) is row j % page_size of pool page
    block_table[b, j // page_size]. Pool pages are handed out in a seeded
    random order; every pool row that holds no key (the tail of a partly
    filled page, spare pages) is NaN, and block-table entries past a
    sequence's last page are -1, so reading either shows up.
    """
    B, H, Lmax, d = kc.shape
    lens = np.asarray(seq_lens, dtype=np.int32)
    table, num_pages = page_table(seed, B, H, Lmax, d, lens, page_size, spare_pages)
    filler = np.uint16(BF16_NAN_BITS) if kc.dtype == np.uint16 else np.float32(np.nan)
    pools = [np.full((num_pages, H, page_size, d), filler, dtype=kc.dtype) for _ in range(2)]
    for b in range(B):
        n = int(lens[b])
        pages = table[b, :-(-n // page_size)]
        full = n // page_size
        for pool, src in zip(pools, (kc, vc)):
            if full:
                pool[pages[:full]] = src[b, :, :full * page_size].reshape(H, full, page_size, d).transpose(1, 0, 2, 3)
            if n % page_size:
                pool[pages[full], :, :n % page_size] = src[b, :, full * page_size:n]
    return pools[0], pools[1], table, lens


# ---- FP8 (OCP e4m3, "fn": no infinities, 0x7F / 0xFF are NaN, largest finite 448) ----
E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to e4m3 with round-to-nearest-even; returns uint8 codes.

    Values beyond the largest finite code after rounding are rejected (the
    inputs are scaled into range first); subnormals (steps of 2^-9 below
    2^-6) are rounded like normals.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("f32_to_e4m3_bits expects finite inputs")
    a = np.abs(x).astype(np.float64)
    _, ef = np.frexp(a)                                   # a = f * 2^ef, f in [0.5, 1)
    e = np.maximum(ef.astype(np.int64) - 1, -6)           # exponent of the leading bit; subnormals share -6
    q = np.rint(a * np.exp2(3 - e))                       # 3 mantissa bits: exact scaling, ties to even
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q).astype(np.int64)
    code = np.where(q < 8, q, ((e + 7) << 3) | (q - 8))
    if (code > 0x7E).any():
        raise ValueError("value out of the e4m3 range")
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decoding of e4m3 codes (NaN for 0x7F and 0xFF)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    ef, m = (b >> 3) & 15, b & 7
    val = np.where(ef == 0, m * 2.0 ** -9, (8 + m) * np.exp2(ef - 10.0))
    val = np.where((ef == 15) & (m == 7), np.nan, val)
    return np.where(b >> 7, -val, val).astype(np.float32)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor FP8 quantisation: descale = max|x| / 448 (float32), codes = e4m3(x / descale).

    The logical tensor is descale * decode(codes)."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    scaled = np.clip(x / descale, -E4M3_MAX, E4M3_MAX)    # division rounding may step past 448
    return f32_to_e4m3_bits(scaled), float(descale)


def fp8_as_float64(codes: np.ndarray, descale: float) -> np.ndarray:
    """The logical values of an FP8 tensor, exactly, in float64."""
    return e4m3_bits_to_f32(codes).astype(np.float64) * np.float64(np.float32(descale))


def fp8_case(seed: int, B: int, H: int, N: int, d: int, std: float = 1.0):
    """Seeded FP8 inputs: q, k ~ std * N(0,1), v ~ N(0,1), each quantised per tensor.

    Returns (q8, k8, v8, (q_descale, k_descale, v_descale))."""
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, 8000 + seed, B, H, N, d]))
    outs, scales = [], []
    for sd in (std, std, 1.0):
        x = (rng.standard_normal((B, H, N, d), dtype=np.float32) * np.float32(sd)).astype(np.float32)
        codes, ds = quantize_e4m3(x)
        outs.append(codes)
        scales.append(ds)
    return outs[0], outs[1], outs[2], tuple(scales)


def fp8_workload(w: Workload):
    """A workload's Q, K, V draws (the same float32 values as its bf16 inputs before the
    bf16 cast), quantised to FP8 per tensor. Returns (q8, k8, v8, descales)."""
    outs, scales = [], []
    for t in ("q", "k", "v"):
        x = np.empty((w.B, w.H, w.N, w.d), dtype=np.float32)
        for b in range(w.B):
            for h in range(w.H):
                x[b, h] = _slice_values(w, t, b, h, w.N)
        codes, ds = quantize_e4m3(x)
        outs.append(codes)
        scales.append(ds)
    return outs[0], outs[1], outs[2], tuple(scales)
