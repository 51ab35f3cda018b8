// Fused exact attention forward with FP8 inputs (OCP e4m3), bf16 output,
// fp32 accumulation, gfx950.
//
// The method is the one-pass tiled online softmax of "Describe Flash Attention
// at a high level" (mantramindai.in), section "The two ideas", with both
// products on the FP8 matrix cores, as the FlashAttention-3 FP8 mode the pages
// mention ("How FlashAttention Speeds Up the Attention Layer", hassanahmed.net,
// the section on later versions; the mantramindai.in page, the paragraph on
// FA-3). The pages give no scaling convention; this kernel takes one float
// descale factor per tensor, so the logical inputs are q_descale * Q8, etc.
//
// Mapping (d = 128; d = 64 is the same with half the chunks per key row, one
// score MFMA per 32 keys and two 32-dim blocks of O^T):
//  * eight waves x 32 query rows per workgroup; S^T = K Q^T and O^T += V^T P^T
//    on v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales), 64 contraction slots
//    per instruction: lane l holds row l % 32 and k-slots 32*(l/32) .. +31 of
//    A, column l % 32 and the same k-slots of B (measured layout). Two MFMAs
//    score 32 keys; four accumulate one 64-key unit of P V;
//  * K/V tiles of 128 keys (128 bytes per key) are copied HBM -> LDS with
//    global_load_lds_dwordx4 into a 4-slot ring; the 16-byte chunks of a key
//    are XOR-swizzled by key bits (K and V differently), which keeps both the
//    K row reads and the transposing V reads free of bank conflicts;
//  * P^T for a 64-key unit comes from the two 32-key score accumulators: lane
//    l's k-slot 16*st + r holds the probability of accumulator st's element r,
//    so V^T's k-slots are gathered to match with ds_read_b64_tr_b8 (within a
//    16-lane group, lane t takes byte t % 8 of the chunk addressed by lane
//    2e + t / 8 as its element e);
//  * probabilities are scaled by 2^6 before the e4m3 rounding (exact), and the
//    running reference maximum is raised when a unit exceeds it by more than
//    2 in exp2 units, so every probability is at most 2^8 (e4m3 holds 448) and
//    those down to 2^-12 of the reference stay normal numbers. The row sum
//    takes the unrounded fp32 probabilities;
//  * software pipeline over 64-key units: the score MFMAs of unit u + 1 run
//    with unit u's probabilities between them (unit u's V^T reads in flight
//    meanwhile), then the P V MFMAs of unit u with the K reads of unit u + 2
//    in flight and unit u + 1's row maximum and reference update after them,
//    so every unit's reference is settled before its probabilities are taken;
//  * as in the bf16 kernel: each SIMD holds one low and one high row block,
//    the last tiles run without barriers once every copy is in, the score
//    MFMA stretch runs at raised wave priority, and workgroups take heads in
//    groups (head_group) with the heaviest causal query tiles first.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

template <int HD>
struct Fp8Tile {
  static constexpr int D = HD;         // head dimension = bytes per key row (64 or 128)
  static constexpr int NCH = D / 16;   // 16-byte chunks per key row
  static constexpr int KPI = 1024 / D; // keys per 1 KB copy instruction
  static constexpr int NQ = D / 64;    // score MFMAs per 32-key sub-tile (64 contraction slots each)
  static constexpr int NDB = D / 32;   // 32-dim blocks of O^T
  static constexpr int NW = 8;         // waves per workgroup
  static constexpr int BR = 32 * NW;   // query rows per workgroup
  static constexpr int BC = 128;       // keys per LDS tile (two 64-key units)
  static constexpr int NBUF = 4;       // ring depth
  static constexpr int KT = BC * D;    // bytes of one K (or V) tile
  static constexpr int VREG = NBUF * KT;
  static constexpr int IPW = KT / 1024 / NW;  // copy instructions per wave per tensor per tile
  static_assert(IPW * NW * 1024 == KT, "copy split");
  static_assert(2 * NBUF * KT <= 163840, "LDS budget");
};

constexpr int kP8Shift = 6;             // exponent offset of the stored probabilities
constexpr float kP8Threshold = 2.f;     // reference raise threshold, exp2 units

// Swizzles of the 16-byte chunks of a key row in LDS (logical chunk ^ swz).
// K rows are read 16 keys at one logical chunk. d = 128 (128-byte rows):
// bits 1..3 of the key spread them over all eight positions, the key's parity
// picks the other half of the 64 banks. d = 64 (64-byte rows, four keys per
// bank sweep): bits 2..3 spread the four keys that share bank groups over the
// four positions.
template <int D>
__device__ __forceinline__ int swz8(int key) {
  if constexpr (D == 128)
    return (key >> 1) & 7;
  else
    return (key >> 2) & 3;
}
// A transposing V read of a half-wave touches keys {0..3, 8..11} (+4) at two
// adjacent chunks. d = 128: bits 1 and 3 of the key move each key to its own
// pair of positions, so the 8 keys x 2 chunks cover all 16 bank groups. d = 64:
// keys k and k + 8 share bank groups; bit 3 moves k + 8 to the other pair of
// positions, so the 8 keys x 2 chunks x 2 halves cover all 64 banks.
template <int D>
__device__ __forceinline__ int swz8v(int key) {
  if constexpr (D == 128)
    return 2 * ((key >> 1) & 1) + 4 * ((key >> 3) & 1);
  else
    return 2 * ((key >> 3) & 1);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(p));
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                       const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                                                       float* __restrict__ LSE, int N, float lse_scale, float c2,
                                                       float v_descale, int n_qt, int BH, int GH) {
  using T = Fp8Tile<HD>;
  constexpr int D = T::D;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * T::NBUF * T::KT];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, hf = l >> 5, lq = l & 31;
  // heads in groups of GH, each group's query tiles in rank order (see head_group)
  const int grp = blockIdx.x / (GH * n_qt);
  const int gh = min(GH, BH - grp * GH);
  const int r = blockIdx.x - grp * GH * n_qt;
  const int bh = grp * GH + r % gh;
  const int rank = r / gh;
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;
  const int q0 = qt * T::BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* Qh = Q + head;
  const uint8_t* Kh = K + head;
  const uint8_t* Vh = V + head;
  // Waves w and w + 4 share a SIMD. Row block w goes to wave w for w < 4 and
  // to wave 11 - w otherwise, so each SIMD holds one low and one high row
  // block and carries the same work in the causal diagonal.
  const int rb = w < T::NW / 2 ? w : (3 * T::NW / 2 - 1 - w);
  const int wq0 = q0 + 32 * rb;

  // copy instruction v of a tile moves keys KPI*v .. + KPI - 1 (1 KB); lane l
  // fetches the logical chunk that its LDS position holds
  auto dma = [&](int j, int slot) __attribute__((always_inline)) {
    const uint32_t kb = lds_addr(lds) + slot * T::KT;
    const uint32_t vb = kb + T::VREG;
#pragma unroll
    for (int i = 0; i < T::IPW; ++i) {
      const int v = w * T::IPW + i;
      const int kr = T::KPI * v + l / T::NCH;
      const int pos = l % T::NCH;
      const size_t key = (size_t)min(j * T::BC + kr, N - 1);  // keys past N: any valid row, masked later
      global_load_lds16(Kh + key * D + 16 * (pos ^ swz8<D>(kr)), kb + v * 1024);
      global_load_lds16(Vh + key * D + 16 * (pos ^ swz8v<D>(kr)), vb + v * 1024);
    }
  };

  const int kv_end = CAUSAL ? min(N, q0 + T::BR) : N;
  const int n_kt = (kv_end + T::BC - 1) / T::BC;
  const int wv_end = CAUSAL ? min(N, wq0 + 32) : N;
  const int n_u = wq0 < N ? (wv_end + 63) / 64 : 0;  // 64-key units this wave computes

  dma(0, 0);
  if (n_kt > 1) dma(1, 1);
  // Q^T as the B operand: for MFMA c, lane (query lq, half hf) holds dims
  // 64c + 32hf .. + 31 (the same k-slots as the K rows of the A operand)
  i32x8 qop[T::NQ];
  {
    const int row = wq0 + lq;
#pragma unroll
    for (int c = 0; c < T::NQ; ++c) {
      if (row < N) {
        const u32x4 a = *(const u32x4*)(Qh + (size_t)row * D + 64 * c + 32 * hf);
        const u32x4 b = *(const u32x4*)(Qh + (size_t)row * D + 64 * c + 32 * hf + 16);
        qop[c] = __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        qop[c] = (i32x8){};
      }
    }
  }

  // Per-lane LDS offsets. K rows (A operand of S^T): key lq of a 32-key
  // sub-tile, 16-byte chunk 4c + 2hf + i -> k_lane[2c + i]. V^T (transposing
  // reads) for 32-dim block db: lane (group g, t) addresses key
  // 8*(e/4) + e%4 + 4*hf (e = t/2) of a 16-key group, chunk 2db + g%2, bytes
  // 8*(t%2) .. + 7 -> v_lane[db]; the key-group offsets are immediates.
  int k_lane[2 * T::NQ], v_lane[T::NDB];
#pragma unroll
  for (int i4 = 0; i4 < 2 * T::NQ; ++i4)
    k_lane[i4] = lq * D + 16 * ((4 * (i4 >> 1) + 2 * hf + (i4 & 1)) ^ swz8<D>(lq));
  {
    const int t = l & 15, g = l >> 4, e = t >> 1;
    const int key = 8 * (e >> 2) + (e & 3) + 4 * hf;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
      v_lane[db] = T::VREG + key * D + 16 * ((2 * db + (g & 1)) ^ swz8v<D>(key)) + 8 * (t & 1);
  }

  // 64-key unit u lives in tile u / 2, keys 64 * (u % 2) .. of its slot;
  // read_k and read_v take that byte offset (base)
  auto unit_base = [](int u) { return ((u >> 1) & 3) * T::KT + (u & 1) * 64 * T::D; };
  auto read_k = [&](i32x8(&kf)[2][T::NQ], int base) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int c = 0; c < T::NQ; ++c) {
        const u32x4 a = *(const u32x4*)(lds + (k_lane[2 * c] + base) + st * 32 * D);
        const u32x4 b = *(const u32x4*)(lds + (k_lane[2 * c + 1] + base) + st * 32 * D);
        kf[st][c] = __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  auto read_v = [&](i32x8(&vf)[T::NDB], int base) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) {
      i32x2 part[4];
#pragma unroll
      for (int rho = 0; rho < 4; ++rho) part[rho] = lds_read_tr8(lds + (v_lane[db] + base) + (16 * rho) * D);
      const auto lo = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3);
      const auto hi = __builtin_shufflevector(part[2], part[3], 0, 1, 2, 3);
      vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto qk = [&](f32x16(&s)[2], const i32x8(&kf)[2][T::NQ]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = mfma_fp8(kf[st][0], qop[0], (f32x16){});
#pragma unroll
      for (int c = 1; c < T::NQ; ++c) s[st] = mfma_fp8(kf[st][c], qop[c], s[st]);
    }
  };

  f32x16 sA[2], sB[2];
  f32x16 oacc[T::NDB];
  i32x8 kf[2][T::NQ], pb = {};
  float m = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) oacc[db] = (f32x16){};

  auto needs_mask = [&](int u) __attribute__((always_inline)) {
    return (64 * u + 64 > N) || (CAUSAL && 64 * u + 63 > wq0);
  };
  auto mask_unit = [&](f32x16(&s)[2], int u) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 64 * u + 32 * st + (r & 3) + 8 * (r >> 2) + 4 * hf;
        if (!(key < N && (!CAUSAL || key <= wq0 + lq))) s[st][r] = -INFINITY;
      }
  };
  // The reference update for a unit whose in-lane maximum is x: raised (O and
  // the running sum rescaled) only when the unit exceeds it by more than the
  // threshold.
  auto update_ref = [&](float x) __attribute__((always_inline)) {
    const float mt = halves_max(x);
    if (__builtin_amdgcn_ballot_w64((mt - m) * c2 > kP8Threshold) != 0) {
      const float m_new = fmaxf(m, mt);
      const float alpha = fast_exp2((m - m_new) * c2);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < T::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  };
  auto unit_max = [&](const f32x16(&s)[2]) __attribute__((always_inline)) {
    float x0 = fmaxf(s[0][0], s[0][1]), x1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) {
      x0 = fmaxf(x0, s[0][r]);
      x1 = fmaxf(x1, s[1][r]);
    }
    return fmaxf(x0, x1);
  };
  // Probabilities of word wd (four scores) of a unit, converted to e4m3 into pb.
  auto probs = [&](const f32x16(&cur)[2], float mc, float& ps, int wd) __attribute__((always_inline)) {
    const int st = wd >> 2, r0 = 4 * (wd & 3);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(cur[st][r0 + i], c2, -mc));
    ps += (p[0] + p[1]) + (p[2] + p[3]);
    // the conversion writes one half of the word and keeps the other; the
    // previous word stands in for it (overwritten next), so no zero is set
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pb[wd], false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
    pb[wd] = word;
  };
  // One unit u (u < n_u): `cur` holds its masked scores and the reference
  // already covers them; kf holds the K rows of unit u + 1. The score MFMAs of
  // unit u + 1 run with this unit's probabilities between them; then the P V
  // MFMAs of unit u, then the mask, row maximum and reference update of unit
  // u + 1. The score MFMAs and the K read of unit u + 2 are unconditional:
  // past the last unit they read an in-range ring slot into registers nobody
  // uses (a conditional read costs a 32-register copy per unit). The
  // scheduling barriers keep the V and K reads where they are issued, ahead
  // of the arithmetic that hides their latency.
  auto step = [&](f32x16(&cur)[2], f32x16(&nxt)[2], int u, int vb_u, int kb_u2, bool clean)
                  __attribute__((always_inline)) {
    if (u >= n_u) return;
    const bool has_next = clean || u + 1 < n_u;
    const float mc = m * c2 - (float)kP8Shift;
    float ps0 = 0.f, ps1 = 0.f;
    constexpr int NS = 2 * T::NQ;
    i32x8 vf[T::NDB];
    // the score MFMA stretch runs at raised wave priority: when both waves of
    // a SIMD can issue, the one feeding the matrix core goes first
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int st = i & 1, c = i >> 1;
      nxt[st] = mfma_fp8(kf[st][c], qop[c], c == 0 ? (f32x16){} : nxt[st]);
      if (i == 0) {
        read_v(vf, vb_u);  // V reads in flight under the probabilities
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int wd = 8 * i / NS; wd < 8 * (i + 1) / NS; ++wd) probs(cur, mc, wd < 4 ? ps0 : ps1, wd);
    }
    __builtin_amdgcn_s_setprio(0);
    lsum += ps0 + ps1;
    if (!clean && has_next && needs_mask(u + 1)) mask_unit(nxt, u + 1);
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) {
      oacc[db] = mfma_fp8(vf[db], pb, oacc[db]);
      if (db == 0) {
        read_k(kf, kb_u2);  // K reads of unit u + 2 in flight under the P V MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (has_next) update_ref(unit_max(nxt));
  };
  // End of tile j: tile j + 2 resident for every wave (its K rows are read
  // from the next tile's steps on) and every wave done with tile j, whose
  // slot then receives tile j + 4. A wave's copies complete in issue order, so
  // with tile j + 3 also in flight it waits until only that tile's copies
  // remain. Once the last copy has been issued, one wait for all copies and
  // one barrier end the synchronisation: no slot is written again, and each
  // wave finishes the last tiles at its own pace.
  auto end_tile = [&](int j, int slot) __attribute__((always_inline)) {
    if (j + 4 < n_kt) {
      wait_vmcnt<2 * T::IPW>();
      __syncthreads();
      dma(j + 4, slot);
    } else if (j == max(0, n_kt - 4)) {
      wait_vmcnt<0>();
      __syncthreads();
    }
  };

  wait_vmcnt<0>();  // Q, tiles 0 and 1
  __syncthreads();
  if (n_kt > 2) dma(2, 2);
  if (n_kt > 3) dma(3, 3);
  if (n_u > 0) {
    read_k(kf, unit_base(0));
    qk(sA, kf);
    read_k(kf, unit_base(1));  // unit 1 is in tile 0 (in range even when unused)
    if (needs_mask(0)) mask_unit(sA, 0);
    update_ref(unit_max(sA));  // from m = -inf: alpha = 0
  }
  // Leading units whose successor needs no mask: tiles whose two steps both
  // satisfy that run the straight-line step. Unrolled over the 4-slot ring
  // (j is a multiple of 4 at its top), so every ring offset is a compile-time
  // constant folded into the LDS instructions.
  static_assert(T::NBUF == 4, "the unrolled loop walks a 4-slot ring");
  const int n_clean = min(CAUSAL ? (wq0 + 1) / 64 : N / 64, N / 64);
  const int j_clean = max(0, (n_clean - 1) / 2);
  int j = 0;
  for (; j + 4 <= j_clean; j += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      step(sA, sB, 2 * (j + r), unit_base(2 * r), unit_base(2 * r + 2), true);
      step(sB, sA, 2 * (j + r) + 1, unit_base(2 * r + 1), unit_base(2 * r + 3), true);
      end_tile(j + r, r);
    }
  }
  for (; j < n_kt; ++j) {
    step(sA, sB, 2 * j, unit_base(2 * j), unit_base(2 * j + 2), false);
    step(sB, sA, 2 * j + 1, unit_base(2 * j + 1), unit_base(2 * j + 3), false);
    end_tile(j, j & 3);
  }

  // ---- epilogue: O = v_descale * acc / l, one rounding to bf16; LSE in natural log ----
  const float ltot = halves_sum(lsum);
  const int qrow = wq0 + lq;
  if (qrow < N) {
    const float f = v_descale / ltot;
    uint16_t* orow = O + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x2 a = to_bf16x2(oacc[db][4 * rb] * f, oacc[db][4 * rb + 1] * f);
        const bf16x2 b = to_bf16x2(oacc[db][4 * rb + 2] * f, oacc[db][4 * rb + 3] * f);
        *(bf16x4*)(orow + 32 * db + 8 * rb + 4 * hf) = __builtin_shufflevector(a, b, 0, 1, 2, 3);
      }
    if (LSE != nullptr && hf == 0) LSE[(size_t)bh * N + qrow] = m * lse_scale + __logf(ltot) - kP8Shift * kLn2;
  }
}

template <int D>
static hipError_t launch_fwd_fp8_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                   int N, bool causal, float scale, float q_descale, float k_descale,
                                   float v_descale, hipStream_t s) {
  using T = Fp8Tile<D>;
  int n_qt = (N + T::BR - 1) / T::BR;
  int BH = B * H;
  float lse_scale = scale * q_descale * k_descale;  // logit = lse_scale * (Q8 . K8)
  float c2 = lse_scale * kLog2e;
  if (!(c2 >= FLT_MIN)) c2 = FLT_MIN;  // as in the bf16 kernel: masked scores stay at probability 0
  const uint8_t *qp = (const uint8_t*)q, *kp = (const uint8_t*)k, *vp = (const uint8_t*)v;
  uint16_t* op = (uint16_t*)o;
  int GH = head_group(T::NW, BH, n_qt);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, &lse_scale, &c2, &v_descale, &n_qt, &BH, &GH};
  const void* kern = causal ? (const void*)&fwd_fp8_kernel<D, true> : (const void*)&fwd_fp8_kernel<D, false>;
  return hipLaunchKernel(kern, dim3((unsigned)(n_qt * BH)), dim3(64 * T::NW), args, 0, s);
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                          int d, bool causal, float scale, float q_descale, float k_descale, float v_descale,
                          hipStream_t s) {
  if (d == 64)
    return launch_fwd_fp8_t<64>(q, k, v, o, lse, B, H, N, causal, scale, q_descale, k_descale, v_descale, s);
  return launch_fwd_fp8_t<128>(q, k, v, o, lse, B, H, N, causal, scale, q_descale, k_descale, v_descale, s);
}

}  // namespace fa
