// Attention backward with recompute, bf16 in/out, fp32 accumulation, gfx950.
//
// The backward pass does not read a stored probability matrix: it recomputes
// the score tiles from Q, K and V and the forward's per-row log-sum-exp, as
// "Describe Flash Attention at a high level" (mantramindai.in), section "The
// two ideas", item 3, and "How FlashAttention Speeds Up the Attention Layer"
// (hassanahmed.net), the paragraph on training, describe. The gradients are
// the chain rule of the plain definition (the pages only state that they match
// standard attention):
//   P = exp(scale Q K^T - LSE)        (masked entries 0)
//   dV = P^T dO,   dP = dO V^T,   D = rowsum(dO * O),   dS = P * (dP - D),
//   dQ = scale dS K,   dK = scale dS^T Q.
//
// Three kernels:
//  * bwd_prep: -D (fp32) and LSE * log2(e) per query row, into the caller's
//    workspace (rows padded to a multiple of 64 with zeros). The other two
//    kernels start each dP accumulation from -D, so the MFMA result is
//    already dP - D and dS = P * (dP - D) costs one multiply per element;
//  * bwd_dkdv: one workgroup per 128 keys of a head, eight waves, two per
//    SIMD. The two waves of a SIMD own the same 32 keys and take the first
//    and the second 32-query block of each 64-row Q / dO tile; K and V of the
//    workgroup's keys stay in LDS as MFMA B operands. Per block a wave
//    recomputes S = Q K^T and dP = dO V^T (lane l holds key l % 32 and 16
//    queries), forms P and dS in registers and accumulates dV += P^T dO and
//    dK += dS^T Q, the P^T / dS^T operands coming straight from those
//    registers and dO / Q through the transposing LDS read. The step is laid
//    out as a chain in which each stretch of arithmetic sits under MFMAs that
//    do not need it: S, then dP with P formed between its MFMAs, then dV with
//    dS formed between them, then dK. The second wave
//    of each pair adds its sums into the first's through LDS at the end;
//  * bwd_dq: one workgroup per 256 queries (8 waves x 32 rows), laid out like
//    the forward: S^T = K Q^T and dP^T = V dO^T with Q / dO in VGPRs, then
//    dQ^T += K^T dS^T with K^T from the transposing read. No atomics: dQ is
//    owned by one wave, so results are deterministic.
// Tiles are copied HBM -> LDS with global_load_lds_dwordx4 into a two-slot
// ring (one barrier per tile), row-major by 64-dim octets with the 16-byte
// chunks XOR-swizzled per row by one function that keeps both the
// row-fragment reads (16 rows, one chunk) and the transposing reads (4 rows x
// 4 chunks) free of bank conflicts.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int BT = 64;  // rows per LDS tile


__device__ __forceinline__ int bswz(int row) { return 4 * ((row >> 1) & 1) + ((row >> 2) & 3); }

template <int D>
struct BwdTile {
  static constexpr int NC = D / 16;             // 16-deep k-chunks over the head dim
  static constexpr int NDB = D / 32;            // 32-wide head-dim blocks
  static constexpr int BYTES = BT * D * 2;      // one tile
  static constexpr int NCOPY = BYTES / 1024;    // copy instructions per tile
};

// Copy instruction v of the tile holding rows r0 .. r0 + 63 of a [rows, D]
// bf16 matrix: octet v / 8 of rows r0 + 8*(v % 8) .. + 7. Rows past the end
// repeat the last row (masked by the caller).
template <int D>
__device__ __forceinline__ void copy_part(const uint16_t* base, int r0, int rows, uint32_t dst, int v, int l) {
  const int o = v >> 3, b = v & 7;
  const int rr = 8 * b + (l >> 3);
  const int row = min(r0 + rr, rows - 1);
  global_load_lds16(base + (size_t)row * D + 64 * o + 8 * ((l & 7) ^ bswz(rr)), dst + o * (BT * 128) + b * 1024);
}
// The same copy for a tile that lies inside the matrix: a scalar tile base
// plus lane l's byte offset for instruction v (copy_off), which is the same
// for every tile, so no vector address math is spent per copy.
template <int D>
__device__ __forceinline__ uint32_t copy_off(int v, int l) {
  const int o = v >> 3, b = v & 7;
  const int rr = 8 * b + (l >> 3);
  return 2u * (uint32_t)(rr * D + 64 * o + 8 * ((l & 7) ^ bswz(rr)));
}
__device__ __forceinline__ void copy_part_s(const uint16_t* tile_base, uint32_t off, uint32_t dst, int v) {
  global_load_lds16_s(tile_base, off, dst + (v >> 3) * (BT * 128) + (v & 7) * 1024);
}

// Per-lane byte offsets into a tile. Row fragment (MFMA A or B operand taken
// along a row): row 32*h + lq, logical chunk 2c + hf -> row_lane[c % 4] +
// (c / 4) * 8192 + h * 4096. Transposing read for 16-row chunk kc and 32-col
// block db: lane (g, s) addresses row 4*(g/2) + s/4 (+8 for the second read)
// and cols 16*(g%2) + 4*(s%4) -> tr_lane[db % 2][second] + (db / 2) * 8192 +
// (32*h + 16*kc) * 128.
struct TileLanes {
  int row[4];
  int tr[2][2];
  __device__ __forceinline__ explicit TileLanes(int l) {
    const int hf = l >> 5, lq = l & 31, g = l >> 4, s = l & 15;
#pragma unroll
    for (int c = 0; c < 4; ++c) row[c] = lq * 128 + 16 * ((2 * c + hf) ^ bswz(lq));
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * (g >> 1) + (s >> 2) + 8 * hi;
        const int chunk = 4 * a + 2 * (g & 1) + ((s & 3) >> 1);
        tr[a][hi] = r * 128 + 16 * (chunk ^ bswz(r)) + 8 * (s & 1);
      }
  }
};

__device__ __forceinline__ bf16x8 row_frag(const uint8_t* lds, int tile, const TileLanes& tl, int h, int c) {
  return *(const bf16x8*)(lds + (tile + tl.row[c & 3]) + ((c >> 2) * (BT * 128) + h * 32 * 128));
}
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* lds, int tile, const TileLanes& tl, int h, int kc, int db) {
  const int imm = (db >> 1) * (BT * 128) + (32 * h + 16 * kc) * 128;
  const s16x4 lo = lds_read_tr16(lds + (tile + tl.tr[db & 1][0]) + imm);
  const s16x4 hi = lds_read_tr16(lds + (tile + tl.tr[db & 1][1]) + imm);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---- -D = -rowsum(dO * O) and LSE in exp2 units, per query row ----
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ LSE, float* __restrict__ lse2,
                                                       float* __restrict__ Dsum, int BH, int N, int Npad) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  // 64-bit: BH * Npad * LPR threads may pass 2^31
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t prow = gid / LPR;  // padded row index over BH * Npad
  const int part = (int)(gid % LPR);
  const size_t bh = prow / (size_t)Npad;
  const int i = (int)(prow % (size_t)Npad);
  const bool valid = bh < (size_t)BH && i < N;
  float acc = 0.f;
  if (valid) {
    const size_t off = ((size_t)bh * N + i) * D + 8 * part;
    const u32x4 a = *(const u32x4*)(O + off), b = *(const u32x4*)(dO + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(b[e]) + bf16_hi(a[e]) * bf16_hi(b[e]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (part == 0 && bh < (size_t)BH) {
    lse2[prow] = valid ? LSE[(size_t)bh * N + i] * kLog2e : 0.f;
    Dsum[prow] = valid ? -acc : 0.f;  // stored negated: the dP accumulations start from it
  }
}

// ---- dK, dV: one workgroup per 128 keys of one head ----
// Eight waves, two per SIMD: waves w and w + 4 share a SIMD and the 32 keys
// k0 + 32 (w % 4) .. + 31, wave w taking the first and wave w + 4 the second
// 32-query block of every 64-row Q / dO tile. K and V of the workgroup's keys
// stay in LDS for its lifetime and feed the score MFMAs as B operands, so a
// wave holds only its dK / dV sums and one block's scores; the two waves of a
// SIMD hide each other's LDS waits and arithmetic. At the end the second wave
// of each pair hands its sums to the first through LDS. Causality is a
// run-time flag here (uniform branches): the causal and non-causal cases then
// share one register allocation.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ lse2, const float* __restrict__ Dsum,
                                                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N,
                                                          int Npad, float scale, float c2, int BH, int causal_flag,
                                                          int GH) {
  const bool CAUSAL = causal_flag != 0;
  using T = BwdTile<D>;
  constexpr int SLOT = 2 * T::BYTES + 512;  // Q tile, dO tile, 64 x (LSE2, D) floats
  constexpr int KVB = 4 * T::BYTES;         // K rows k0 .., k0 + 64 .., then V rows k0 .., k0 + 64 ..
  constexpr int IPW = 2 * T::NCOPY / 8;     // Q / dO copy instructions per wave per tile
  constexpr int KV_IPW = 4 * T::NCOPY / 8;  // K / V copy instructions per wave
  constexpr int MERGE = 4 * 2 * T::NDB * 16 * 64 * 4;  // hand-over: 4 key blocks x (dK, dV) x 64 lanes
  static_assert(MERGE <= KVB + 2 * SLOT, "hand-over buffer");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[KVB + 2 * SLOT];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, hf = l >> 5, lq = l & 31;
  const int kb = w & 3, par = w >> 2;  // key block, query block within each tile
  // heads in groups of GH (see head_group), each group's key tiles in order:
  // heaviest first
  const int n_kt = (N + 127) / 128;
  const int grp = blockIdx.x / (GH * n_kt);
  const int gh = min(GH, BH - grp * GH);
  const int rr = blockIdx.x - grp * GH * n_kt;
  const int bh = grp * GH + rr % gh, kt = rr / gh;
  const int k0 = kt * 128, kw0 = k0 + 32 * kb;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t *Qh = Q + head, *Kh = K + head, *Vh = V + head, *dOh = dO + head;
  const float* L2h = lse2 + (size_t)bh * Npad;
  const float* Dh = Dsum + (size_t)bh * Npad;

  f32x16 dv[T::NDB], dk[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) {
    dv[db] = (f32x16){};
    dk[db] = (f32x16){};
  }

  const TileLanes tl(l);
  const int n_qt = (N + BT - 1) / BT;
  const int qt0 = CAUSAL ? k0 / BT : 0;         // earlier query tiles see none of these keys
  const int n_t = n_qt > qt0 ? n_qt - qt0 : 0;  // query tiles this workgroup visits (>= 1)
  uint32_t coff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) coff[i] = copy_off<D>((w * IPW + i) % T::NCOPY, l);
  // tile t (counted from qt0) into ring slot `slot` (t % 2)
  auto copy = [&](int t, int slot) __attribute__((always_inline)) {
    const int qt = qt0 + t;
    const uint32_t base = lds_addr(lds) + KVB + slot * SLOT;
    if (qt * BT + BT <= N) {
      const uint16_t* qtile = Qh + (size_t)qt * (BT * D);
      const uint16_t* dotile = dOh + (size_t)qt * (BT * D);
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int v = w * IPW + i;  // 0 .. 2 NCOPY - 1: Q, then dO
        if (v < T::NCOPY)
          copy_part_s(qtile, coff[i], base, v);
        else
          copy_part_s(dotile, coff[i], base + T::BYTES, v - T::NCOPY);
      }
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int v = w * IPW + i;
        if (v < T::NCOPY)
          copy_part<D>(Qh, qt * BT, N, base, v, l);
        else
          copy_part<D>(dOh, qt * BT, N, base + T::BYTES, v - T::NCOPY, l);
      }
    }
    if (w == 0 && l < 32) {  // LSE2 then D of the tile's 64 rows (the workspace is padded)
      const float* src = (l < 16 ? L2h : Dh) + qt * BT + 4 * (l & 15);
      global_load_lds16(src, base + 2 * T::BYTES);
    }
  };
  // the workgroup's K and V rows; rows past N repeat the last row, which only
  // feeds the scores of those keys, whose dK / dV are not written
#pragma unroll
  for (int i = 0; i < KV_IPW; ++i) {
    const int v = w * KV_IPW + i, tile = v / T::NCOPY, part = v % T::NCOPY;
    copy_part<D>(tile < 2 ? Kh : Vh, k0 + 64 * (tile & 1), N, lds_addr(lds) + tile * T::BYTES, part, l);
  }
  copy(0, 0);
  wait_vmcnt<0>();
  __syncthreads();
  if (n_t > 1) copy(1, 1);

  // this wave's keys: rows 32 (kb % 2) .. of K / V tile kb / 2
  const int tK = (kb >> 1) * T::BYTES, tV = 2 * T::BYTES + tK, hk = kb & 1;
  for (int t = 0; t < n_t; ++t) {
    const int tQ = KVB + (t & 1) * SLOT, tdO = tQ + T::BYTES;
    // Block: queries qb0 .. qb0 + 31. Lane: key kw0 + lq; accumulator element
    // r: query qb0 + (r%4) + 8(r/4) + 4hf. A block wholly before this wave's
    // keys (causal) or past the last row adds exactly zero and is skipped.
    const int qb0 = (qt0 + t) * BT + 32 * par;
    if (qb0 < N && !(CAUSAL && qb0 + 31 < kw0)) {
      // -D of the block's queries in accumulator order: the starting value of
      // dP, so the MFMA result is already dP - D
      f32x16 dp;
      {
        const float* st = (const float*)(lds + tQ + 2 * T::BYTES) + BT + 32 * par + 4 * hf;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 x = *(const f32x4*)(st + 8 * rb);
#pragma unroll
          for (int i = 0; i < 4; ++i) dp[4 * rb + i] = x[i];
        }
      }
      // S = Q K^T over the head dim; then dP - D = dO V^T - D with the
      // probabilities P = exp2(S c2 - LSE2) formed between those MFMAs; then
      // dV += P^T dO with dS = P (dP - D) formed between them; then dK += dS^T Q
      f32x16 sc = (f32x16){};
#pragma unroll
      for (int c = 0; c < T::NC; ++c) sc = mfma32x32x16(row_frag(lds, tQ, tl, par, c), row_frag(lds, tK, tl, hk, c), sc);
      const bool edge = (qb0 + 32 > N) || (CAUSAL && qb0 < kw0 + 31);
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb0 + 8 * (r >> 2) + 4 * hf + (r & 3), key = kw0 + lq;
          if (!(q < N && (!CAUSAL || key <= q))) sc[r] = -INFINITY;  // P = 0
        }
      }
      const float* stats = (const float*)(lds + tQ + 2 * T::BYTES);  // [LSE2 x 64][-D x 64]
      float pr[16];
      bf16x8 pb[2], sb[2];
      constexpr int PPM = 8 / T::NC;  // probability pairs per dP MFMA
#pragma unroll
      for (int c = 0; c < T::NC; ++c) {
        dp = mfma32x32x16(row_frag(lds, tdO, tl, par, c), row_frag(lds, tV, tl, hk, c), dp);
#pragma unroll
        for (int j = 0; j < PPM; ++j) {
          const int r = 2 * (PPM * c + j), rb = r >> 2, e = r & 3;
          const f32x4 L = *(const f32x4*)(stats + 32 * par + 8 * rb + 4 * hf);
          pr[r] = fast_exp2(fmaf(sc[r], c2, -L[e]));
          pr[r + 1] = fast_exp2(fmaf(sc[r + 1], c2, -L[e + 1]));
          const bf16x2 pp = to_bf16x2(pr[r], pr[r + 1]);
          pb[r >> 3][r & 7] = pp[0];
          pb[r >> 3][(r & 7) + 1] = pp[1];
        }
      }
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb0 + 8 * (r >> 2) + 4 * hf + (r & 3), key = kw0 + lq;
          if (!(q < N && (!CAUSAL || key <= q))) dp[r] = 0.f;  // dS = 0 * 0 = 0 whatever the row data holds
        }
      }
      // dV += P^T dO (dO through the transposing read), dS between them
      constexpr int SPM = 8 / (2 * T::NDB);  // dS pairs per dV MFMA
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          dv[db] = mfma32x32x16(pb[kc], tr_frag(lds, tdO, tl, par, kc, db), dv[db]);
#pragma unroll
          for (int j = 0; j < SPM; ++j) {
            const int r = 2 * (SPM * (kc * T::NDB + db) + j);
            const bf16x2 ss = to_bf16x2(pr[r] * dp[r], pr[r + 1] * dp[r + 1]);
            sb[r >> 3][r & 7] = ss[0];
            sb[r >> 3][(r & 7) + 1] = ss[1];
          }
        }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) dk[db] = mfma32x32x16(sb[kc], tr_frag(lds, tQ, tl, par, kc, db), dk[db]);
    }
    // end of tile t: tile t + 1 has landed for every wave and every wave is
    // done with tile t, whose slot then receives tile t + 2
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 2 < n_t) copy(t + 2, t & 1);
  }

  // the second wave of each pair hands its sums to the first (the last
  // barrier above ended every read of the ring and of K / V)
  float* hand = (float*)lds;
  auto at = [&](int which, int db, int r) { return (((kb * 2 + which) * T::NDB + db) * 16 + r) * 64 + l; };
  if (par == 1) {
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hand[at(0, db, r)] = dk[db][r];
        hand[at(1, db, r)] = dv[db][r];
      }
  }
  __syncthreads();
  if (par == 0) {
    // lane l holds head dim 32*db + lq of keys kw0 + (r%4) + 8(r/4) + 4hf
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw0 + (r & 3) + 8 * (r >> 2) + 4 * hf;
        if (key < N) {
          const size_t off = head + (size_t)key * D + 32 * db + lq;
          dV[off] = to_bf16_bits(dv[db][r] + hand[at(1, db, r)]);
          dK[off] = to_bf16_bits((dk[db][r] + hand[at(0, db, r)]) * scale);
        }
      }
  }
}

// ---- dQ: one workgroup per 256 queries of one head ----
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ lse2, const float* __restrict__ Dsum,
                                                        uint16_t* __restrict__ dQ, int N, int Npad, float scale, float c2,
                                                        int n_qt, int BH, int GH) {
  using T = BwdTile<D>;
  constexpr int SLOT = 2 * T::BYTES;      // K tile, V tile
  constexpr int IPW = 2 * T::NCOPY / 8;   // copy instructions per wave per tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * SLOT];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, hf = l >> 5, lq = l & 31;
  const int grp = blockIdx.x / (GH * n_qt);  // heads in groups of GH (see head_group)
  const int gh = min(GH, BH - grp * GH);
  const int rr = blockIdx.x - grp * GH * n_qt;
  const int bh = grp * GH + rr % gh, rank = rr / gh;
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;  // heaviest causal query tiles first
  const int q0 = qt * 256, wq0 = q0 + 32 * w;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t *Qh = Q + head, *Kh = K + head, *Vh = V + head, *dOh = dO + head;

  // Q and dO rows as B operands: lane (query wq0 + lq, half hf), dims 16c + 8hf .. + 7
  const int qrow = wq0 + lq;
  bf16x8 qT[T::NC], doT[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    if (qrow < N) {
      qT[c] = *(const bf16x8*)(Qh + (size_t)qrow * D + 16 * c + 8 * hf);
      doT[c] = *(const bf16x8*)(dOh + (size_t)qrow * D + 16 * c + 8 * hf);
    } else {
      qT[c] = (bf16x8){};
      doT[c] = (bf16x8){};
    }
  }
  const float lq2 = qrow < N ? lse2[(size_t)bh * Npad + qrow] : 0.f;
  // -D of this lane's query, the starting value of every dP^T accumulation
  // (so the MFMA result is dP - D)
  const float nd = qrow < N ? Dsum[(size_t)bh * Npad + qrow] : 0.f;
  f32x16 nd16;
#pragma unroll
  for (int r = 0; r < 16; ++r) nd16[r] = nd;
  f32x16 dqT[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) dqT[db] = (f32x16){};

  const TileLanes tl(l);
  const int kv_end = CAUSAL ? min(N, q0 + 256) : N;
  const int n_kt = (kv_end + BT - 1) / BT;
  const int wv_end = CAUSAL ? min(N, wq0 + 32) : N;
  const int n_st = wq0 < N ? (wv_end + 31) / 32 : 0;  // 32-key sub-tiles this wave needs
  uint32_t coff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) coff[i] = copy_off<D>((w * IPW + i) % T::NCOPY, l);
  auto copy = [&](int j, int slot) __attribute__((always_inline)) {
    const uint32_t base = lds_addr(lds) + slot * SLOT;
    if (j * BT + BT <= N) {
      const uint16_t* ktile = Kh + (size_t)j * (BT * D);
      const uint16_t* vtile = Vh + (size_t)j * (BT * D);
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int v = w * IPW + i;
        if (v < T::NCOPY)
          copy_part_s(ktile, coff[i], base, v);
        else
          copy_part_s(vtile, coff[i], base + T::BYTES, v - T::NCOPY);
      }
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int v = w * IPW + i;
        if (v < T::NCOPY)
          copy_part<D>(Kh, j * BT, N, base, v, l);
        else
          copy_part<D>(Vh, j * BT, N, base + T::BYTES, v - T::NCOPY, l);
      }
    }
  };

  if (n_kt > 0) copy(0, 0);
  wait_vmcnt<0>();
  __syncthreads();
  // key tile j in ring slot `slot` (= j % 2)
  auto tile = [&](int j, int slot) __attribute__((always_inline)) {
    if (j + 1 < n_kt) copy(j + 1, slot ^ 1);
    const int tK = slot * SLOT, tV = tK + T::BYTES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 2 * j + h;
      if (t >= n_st) continue;
      f32x16 sT = (f32x16){}, dpT = nd16;
#pragma unroll
      for (int c = 0; c < T::NC; ++c) {
        sT = mfma32x32x16(row_frag(lds, tK, tl, h, c), qT[c], sT);
        dpT = mfma32x32x16(row_frag(lds, tV, tl, h, c), doT[c], dpT);
      }
      // lane: query qrow; element r: key 32t + (r%4) + 8(r/4) + 4hf. Hidden
      // scores become -inf (P = 0) and their dP 0 (dS = 0) in one uniform
      // branch, so the probability code below is straight-line.
      if ((32 * t + 32 > N) || (CAUSAL && 32 * t + 31 > wq0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * hf;
          if (!(key < N && (!CAUSAL || key <= qrow))) {
            sT[r] = -INFINITY;
            dpT[r] = 0.f;
          }
        }
      }
      bf16x8 sb[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(sT[r], c2, -lq2));
        const float p1 = fast_exp2(fmaf(sT[r + 1], c2, -lq2));
        const bf16x2 ss = to_bf16x2(p0 * dpT[r], p1 * dpT[r + 1]);  // dpT holds dP - D
        sb[r >> 3][r & 7] = ss[0];
        sb[r >> 3][(r & 7) + 1] = ss[1];
      }
      // dQ^T += K^T dS^T: A = K^T (transposing read), B = dS^T from the registers
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) dqT[db] = mfma32x32x16(tr_frag(lds, tK, tl, h, kc, db), sb[kc], dqT[db]);
    }
    wait_vmcnt<0>();
    __syncthreads();
  };
  // unrolled over the two ring slots (j is even at the top), so the slot
  // offsets are compile-time constants
  int j = 0;
  for (; j + 2 <= n_kt; j += 2) {
    tile(j, 0);
    tile(j + 1, 1);
  }
  if (j < n_kt) tile(j, 0);

  // lane l holds query qrow, head dims 32*db + (r%4) + 8(r/4) + 4hf
  if (qrow < N) {
    uint16_t* out = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x2 a = to_bf16x2(dqT[db][4 * rb] * scale, dqT[db][4 * rb + 1] * scale);
        const bf16x2 b = to_bf16x2(dqT[db][4 * rb + 2] * scale, dqT[db][4 * rb + 3] * scale);
        *(bf16x4*)(out + 32 * db + 8 * rb + 4 * hf) = __builtin_shufflevector(a, b, 0, 1, 2, 3);
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                        void* dq, void* dk, void* dv, float* ws, int B, int H, int N, float scale, hipStream_t s) {
  const int BH = B * H;
  int Npad = bwd_rows_padded(N);
  float* lse2 = ws;
  float* dsum = ws + (size_t)BH * Npad;
  float c2 = scale * kLog2e;  // a positive floor keeps masked scores at 0 when scale is 0
  if (!(c2 >= FLT_MIN)) c2 = FLT_MIN;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v,
                 *op = (const uint16_t*)o, *dop = (const uint16_t*)dout;
  uint16_t *dqp = (uint16_t*)dq, *dkp = (uint16_t*)dk, *dvp = (uint16_t*)dv;

  const long long prep_threads = (long long)BH * Npad * (D / 8);
  dim3 g0((unsigned)((prep_threads + 255) / 256)), b0(256);
  void* a0[] = {&op, &dop, (void*)&lse, &lse2, &dsum, (void*)&BH, &N, &Npad};
  hipError_t e = hipLaunchKernel((const void*)&bwd_prep_kernel<D>, g0, b0, a0, 0, s);
  if (e != hipSuccess) return e;

  dim3 g1((unsigned)(((N + 127) / 128) * BH)), b1(512);
  int causal_flag = CAUSAL ? 1 : 0;
  int n_qt = (N + 255) / 256;
  int GH = head_group(8, BH, n_qt);  // the same sequence-length thresholds as the forward's 256-row tiles
  void* a1[] = {&qp, &kp, &vp, &dop, &lse2, &dsum, &dkp, &dvp, &N, &Npad, &scale, &c2, (void*)&BH, &causal_flag, &GH};
  e = hipLaunchKernel((const void*)&bwd_dkdv_kernel<D>, g1, b1, a1, 0, s);
  if (e != hipSuccess) return e;

  dim3 g2((unsigned)(n_qt * BH)), b2(512);
  void* a2[] = {&qp, &kp, &vp, &dop, &lse2, &dsum, &dqp, &N, &Npad, &scale, &c2, &n_qt, (void*)&BH, &GH};
  return hipLaunchKernel((const void*)&bwd_dq_kernel<D, CAUSAL>, g2, b2, a2, 0, s);
}

}  // namespace

int bwd_rows_padded(int N) { return (N + BT - 1) / BT * BT; }

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* ws, int B, int H, int N, int d, bool causal, float scale,
                      hipStream_t s) {
  if (d == 64)
    return causal ? launch_bwd_t<64, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s)
                  : launch_bwd_t<64, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s);
  return causal ? launch_bwd_t<128, true>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s)
                : launch_bwd_t<128, false>(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, scale, s);
}

}  // namespace fa
