// Fused exact attention forward, bf16 in/out, fp32 accumulation, gfx950.
//
// The method is the tiling + online-softmax pass of "Describe Flash Attention
// at a high level" (mantramindai.in), section "The two ideas", and of "How
// FlashAttention Speeds Up the Attention Layer" (hassanahmed.net), sections on
// tiling and on the online softmax: each workgroup owns a block of query rows,
// streams the key/value tiles of its head through on-chip memory once, keeps
// the scores in registers, and rescales its running sum and output whenever the
// running row maximum is raised. The N x N score matrix never leaves the chip.
//
// Mapping onto CDNA4 (lane layouts in fa_device.h):
//  * one workgroup = 8 waves (two per SIMD) x 32 query rows = 256 rows of one
//    (b, h) head (the code also builds a 4-wave variant with 64 rows per
//    wave, see kFwdQB);
//  * scores are computed transposed, S^T = K Q^T, with K rows as the A operand
//    (LDS) and the wave's queries as the B operand (VGPRs, loaded once). In the
//    accumulator lane l owns query l % 32 and 16 keys of a 32-key block, so row
//    max and row sum are in-lane reductions plus one v_permlane32_swap. S is
//    accumulated in VGPRs, where the softmax reads it;
//  * the same registers, rounded to bf16, are the B operand of O^T += V^T P^T;
//    V^T comes from the V tile through the transposing LDS read;
//  * K/V tiles of 64 keys are copied HBM -> LDS by global_load_lds_dwordx4
//    (no VGPR staging) into a 4-deep ring, up to three tiles ahead, one
//    barrier per tile. Tiles are row-major by 64-dim octets (one copy
//    instruction moves 8 keys x 128 contiguous bytes) with the 16-byte chunks
//    XOR-swizzled per key, so K fragment reads and transposing V reads are
//    free of bank conflicts and every read address is one of a few per-lane
//    bases plus an immediate;
//  * software pipeline over 32-key sub-tiles: the wave turns sub-tile t's
//    scores into probabilities while the MFMAs for S(t+1) run, then
//    accumulates P V for t; with two waves per SIMD the hardware also
//    overlaps one wave's softmax with the other's MFMAs;
//  * probabilities are taken against a reference maximum that is raised only
//    when needed: a sub-tile is accepted against the current reference if
//    every lane's sum of its probabilities is at most 256 (so each of them
//    is: exact in fp32 range, representable in bf16). Otherwise the wave
//    takes the exact update (reference raised to the row maximum, O and the
//    running sum rescaled) and recomputes the sub-tile's probabilities. Any
//    reference leaves O and the log-sum-exp unchanged mathematically, so no
//    per-sub-tile row maximum is computed, and the rare update sits on a
//    wave-uniform branch, as does the causal / ragged-tail mask;
//  * causal: key tiles past the workgroup's last query are never loaded and
//    sub-tiles past a wave's last query are skipped by that wave;
//  * heaviest causal query tiles are dispatched first, and consecutive
//    workgroups take consecutive heads so a head's K/V stays in one XCD's L2.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, int QB>
struct FwdTile {
  static constexpr int NW = 8 / QB;             // waves per workgroup
  static constexpr int WR = 32 * QB;            // query rows per wave (QB MFMA blocks of 32)
  static constexpr int BR = NW * WR;            // query rows per workgroup
  static constexpr int BC = 64;                 // keys per LDS tile (two 32-key sub-tiles)
  static constexpr int NBUF = 4;                // LDS ring depth
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int NC = D / 16;             // 16-deep k-chunks of the QK product
  static constexpr int NDB = D / 32;            // 32-wide head-dim blocks of O
  static constexpr int NO = D / 64;             // 64-dim octets (8 chunks, 128 B) per row
  static constexpr int KT = BC * D * 2;         // bytes of one K (or V) tile: [octet][key][128 B]
  static constexpr int VREG = NBUF * KT;        // the V ring follows the K ring
  static constexpr int IPW = CH / NW;           // DMA instructions per wave per tensor per tile
  static_assert(IPW * NW == CH, "DMA split");
  static_assert(2 * NBUF * KT <= 163840, "LDS budget");
};

// O^T += V^T P^T for one 32x32 block. With one query block per wave O^T
// (64 registers at d = 128) lives in VGPRs next to everything else and the
// compiler's MFMA is used; with two blocks O^T needs 128 registers and is
// pinned in AGPRs through asm (the scores stay in VGPRs for the softmax).
template <int QB>
__device__ __forceinline__ void pv_mfma(f32x16& acc, const bf16x8& v, const bf16x8& p) {
  if constexpr (QB == 1)
    acc = mfma32x32x16(v, p, acc);
  else
    mfma32x32x16_agpr(acc, v, p);
}
// Makes the O^T accumulators safe to touch with VALU instructions (only the
// AGPR variant needs the explicit wait states).
template <int QB, int NDB>
__device__ __forceinline__ void o_fence(f32x16 (&oacc)[QB][NDB]) {
  if constexpr (QB > 1) {
    agpr_fence<true>(oacc[0][0]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        if (qb + db > 0) agpr_fence<false>(oacc[qb][db]);
  }
}

// Largest in-lane sum of a sub-tile's probabilities accepted against the
// current reference maximum. Probabilities are non-negative, so the sum bounds
// each of them: every probability that enters O and the row sum is at most
// 256, exact in fp32 range and representable in bf16. A larger sum (or an
// overflow to inf) sends the wave through the exact update instead.
constexpr float kPsumLimit = 256.f;

// A tile is stored row-major by 64-dim octets: octet o of key k is 128 bytes
// at o*64*128 + k*128, so one copy instruction moves 8 keys x 128 contiguous
// bytes. Inside the octet the eight 16-byte chunks are XOR-swizzled per key
// (K and V differently) so that the fragment reads are free of bank
// conflicts: 16 keys at one logical chunk (K) and 4 keys x 4 chunks (the
// transposing V read) land in distinct 16-byte bank groups.
__device__ __forceinline__ int swz_k(int key) { return (key >> 1) & 7; }
__device__ __forceinline__ int swz_v(int key) { return 4 * ((key >> 1) & 1); }

template <int D, int QB, bool CAUSAL>
__global__ __launch_bounds__(64 * (8 / QB), 1) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                          int N, float scale, float c2, int n_qt, int BH) {
  using T = FwdTile<D, QB>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * T::NBUF * T::KT];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform: scalar branches below
  const int l = tid & 63, hf = l >> 5, lq = l & 31;
  const int bh = blockIdx.x % BH;
  const int rank = blockIdx.x / BH;
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;
  const int q0 = qt * T::BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const int wq0 = q0 + T::WR * w;  // first query row of this wave

  // ---- DMA of one K/V tile into a ring slot: instruction v of the tile
  // (wave w issues v = w*IPW .. w*IPW + IPW - 1 for each tensor) copies octet
  // v / 8 of keys k0 + 8*(v % 8) .. + 7; lane l fetches the logical chunk that
  // its LDS position holds. A tile that lies inside [0, N) is addressed as a
  // scalar tile base plus a per-lane byte offset that is the same for every
  // tile (no vector address math per copy); the tile that crosses N clamps
  // each key to N - 1 (any valid row: those keys are masked later) ----
  uint32_t k_off[T::IPW], v_off[T::IPW];
#pragma unroll
  for (int i = 0; i < T::IPW; ++i) {
    const int v = w * T::IPW + i, o = v >> 3, b = v & 7;
    const int kr = 8 * b + (l >> 3);  // key within the tile
    k_off[i] = 2u * (uint32_t)(kr * D + 64 * o + 8 * ((l & 7) ^ swz_k(kr)));
    v_off[i] = 2u * (uint32_t)(kr * D + 64 * o + 8 * ((l & 7) ^ swz_v(kr)));
  }
  auto dma = [&](int j, int slot) __attribute__((always_inline)) {
    const uint32_t kb = lds_addr(lds) + slot * T::KT;
    const uint32_t vb = kb + T::VREG;
    if (j * T::BC + T::BC <= N) {
      const uint16_t* kt = Kh + (size_t)j * (T::BC * D);
      const uint16_t* vt = Vh + (size_t)j * (T::BC * D);
#pragma unroll
      for (int i = 0; i < T::IPW; ++i) {
        const int v = w * T::IPW + i, o = v >> 3, b = v & 7;
        global_load_lds16_s(kt, k_off[i], kb + o * (T::BC * 128) + b * 1024);
        global_load_lds16_s(vt, v_off[i], vb + o * (T::BC * 128) + b * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::IPW; ++i) {
        const int v = w * T::IPW + i, o = v >> 3, b = v & 7;
        const int kr = 8 * b + (l >> 3);
        const int key = min(j * T::BC + kr, N - 1);
        const uint16_t* src = Kh + (size_t)key * D + 64 * o;
        global_load_lds16(src + 8 * ((l & 7) ^ swz_k(kr)), kb + o * (T::BC * 128) + b * 1024);
        const uint16_t* vsrc = Vh + (size_t)key * D + 64 * o;
        global_load_lds16(vsrc + 8 * ((l & 7) ^ swz_v(kr)), vb + o * (T::BC * 128) + b * 1024);
      }
    }
  };

  const int kv_end = CAUSAL ? min(N, q0 + T::BR) : N;
  const int n_kt = (kv_end + T::BC - 1) / T::BC;
  // 32-key sub-tiles this wave computes (0 for a wave entirely past N)
  const int wv_end = CAUSAL ? min(N, wq0 + T::WR) : N;
  const int n_st = wq0 < N ? (wv_end + 31) / 32 : 0;

  dma(0, 0);
  if (n_kt > 1) dma(1, 1);

  // ---- Q^T as the B operand: k-slots of chunk c are head dims 16c + 8*hf + (0..7) ----
  bf16x8 qop[QB][T::NC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wq0 + 32 * qb + lq;
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
      if (row < N)
        qop[qb][c] = *(const bf16x8*)(Qh + (size_t)row * D + 16 * c + 8 * hf);
      else
        qop[qb][c] = (bf16x8){};
    }
  }

  // Per-lane LDS byte offsets within a ring slot. K fragment (A operand of
  // S^T): key lq of the sub-tile, logical chunk 2c + hf; the swizzle makes the
  // offset depend on c % 4 (k_lane[c % 4]), the octet c / 4 is an immediate.
  // V^T fragment (transposing read): lane (g, s) of 16-lane group g addresses
  // key 4*(g/2) + s/4 (+8 for the second read) and head dims 16*(g%2) +
  // 4*(s%4) of 32-dim block db; the offset depends on db % 2 (v_lane[db % 2]),
  // the octet db / 2 and the key offsets are immediates.
  const int g16 = l >> 4, s16 = l & 15;
  int k_lane[4], v_lane[2];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_lane[c] = lq * 128 + 16 * ((2 * c + hf) ^ swz_k(lq));
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int key = 4 * (g16 >> 1) + (s16 >> 2);
    const int chunk = 4 * a + 2 * (g16 & 1) + ((s16 & 3) >> 1);
    v_lane[a] = T::VREG + key * 128 + 16 * (chunk ^ swz_v(key)) + 8 * (s16 & 1);
  }

  f32x16 sA[QB], sB[QB];    // S^T of one 32-key sub-tile per query block (VGPRs)
  f32x16 oacc[QB][T::NDB];  // O^T (AGPRs): lane l owns query l % 32 of each block
  float m[QB];              // reference maximum of the raw scores q.k
  float lsum[QB];           // this half-wave's share of the running sum
  float mt[QB];             // maximum of a sub-tile (exact update only)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) oacc[qb][db] = (f32x16){};
    m[qb] = -INFINITY;
    lsum[qb] = 0.f;
  }

  // K fragment c (A operand of S^T) of 32-key half h of the tile in the ring
  // slot at byte offset k_slot
  auto k_frag = [&](int k_slot, int h, int c) __attribute__((always_inline)) {
    return *(const bf16x8*)(lds + (k_lane[c & 3] + k_slot) + ((c >> 2) * (T::BC * 128) + h * 32 * 128));
  };
  // S^T for the 32-key half h of the tile in the slot at k_slot
  auto qk = [&](f32x16(&s)[QB], int k_slot, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
      const bf16x8 a = k_frag(k_slot, h, c);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = mfma32x32x16(a, qop[qb][c], c == 0 ? (f32x16){} : s[qb]);
    }
  };
  auto tile_max = [&](const f32x16(&s)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x = s[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, s[qb][r]);
      mt[qb] = halves_max(x);
    }
  };
  // keys past N and (causal) keys after the query row get -inf
  auto needs_mask = [&](int t) __attribute__((always_inline)) {
    return (32 * t + 32 > N) || (CAUSAL && 32 * t + 31 > wq0);
  };
  auto mask = [&](f32x16(&s)[QB], int t) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = wq0 + 32 * qb + lq;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * hf;
        const bool vis = key < N && (!CAUSAL || key <= qrow);
        if (!vis) s[qb][r] = -INFINITY;
      }
    }
  };
  // The exact online-softmax update for sub-tile s: the reference maximum
  // of every row becomes max(m, rowmax s) and O and the running sum are
  // rescaled by alpha = exp2((m_old - m_new) c2) (alpha = 1 where the
  // maximum did not move). Returns alpha per query block.
  auto raise_ref = [&](const f32x16(&s)[QB], float(&alpha)[QB]) __attribute__((always_inline)) {
    tile_max(s);
    o_fence(oacc);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = fmaxf(m[qb], mt[qb]);
      alpha[qb] = fast_exp2((m[qb] - m_new) * c2);
      m[qb] = m_new;
      lsum[qb] *= alpha[qb];
#pragma unroll
      for (int db = 0; db < T::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha[qb];
    }
  };
  // True (wave-uniform) when some lane's probability sum is above the limit
  // or not finite.
  auto over_limit = [&](const float(&x)[QB]) __attribute__((always_inline)) {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bad = bad || !(x[qb] <= kPsumLimit);
    return __builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0);
  };
  // Probabilities of a sub-tile against the reference maximum: bf16 B operand
  // of P V and this half-wave's fp32 row sums. One call handles elements r,
  // r + 1 of query block qb (mc = reference maximum in exp2 units).
  // The sum goes to ps0 for the first 16-key chunk (elements 0-7) and to ps1
  // for the second: two independent add chains.
  auto prob_pair = [&](const f32x16(&s)[QB], bf16x8(&pb)[QB][2], float(&ps0)[QB], float(&ps1)[QB],
                       const float(&mc)[QB], int qb, int r) __attribute__((always_inline)) {
    const float p0 = fast_exp2(fmaf(s[qb][r], c2, -mc[qb]));
    const float p1 = fast_exp2(fmaf(s[qb][r + 1], c2, -mc[qb]));
    if (r < 8)
      ps0[qb] += p0 + p1;
    else
      ps1[qb] += p0 + p1;
    const bf16x2 two = to_bf16x2(p0, p1);
    pb[qb][r >> 3][r & 7] = two[0];
    pb[qb][r >> 3][(r & 7) + 1] = two[1];
  };
  // element pairs in the order P V consumes them: 16-key chunk, block, element
  constexpr int NPAIR = 8 * QB;
  auto pair_qb = [](int i) { return (i >> 2) % QB; };
  auto pair_r = [](int i) { return 8 * (i / (4 * QB)) + 2 * (i & 3); };
  // V^T fragment (A operand of O^T) for 16-key chunk kc and head-dim block db
  // of 32-key half h of the tile in the slot at v_slot
  auto load_v = [&](int v_slot, int h, int kc, int db) __attribute__((always_inline)) {
    const int imm = (db >> 1) * (T::BC * 128) + (32 * h + 16 * kc) * 128;
    const s16x4 lo = lds_read_tr16(lds + (v_lane[db & 1] + v_slot) + imm);
    const s16x4 hi = lds_read_tr16(lds + (v_lane[db & 1] + v_slot) + (imm + 8 * 128));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  bf16x8 kf[T::NC];  // K fragments of the next sub-tile to score

  // One pipeline step: finish sub-tile t (its V in the slot at v_slot, half
  // t % 2), score sub-tile t + 1 (needs t + 1 < n_st; its first two K
  // fragments are already in kf, the others are read two k-chunks ahead) and
  // fetch the first K fragments of sub-tile t + 2 (half t % 2 of the slot at
  // kp_slot). The source order is the intended issue order: the score MFMAs
  // of t + 1 with the probabilities of t and the first V^T reads between
  // them, then the P V MFMAs of t with the other V^T reads and the next K
  // fragments. With two waves per SIMD the hardware interleaves the waves.
  //
  // Probabilities are taken against the current reference maximum. Before
  // P V reads them the wave checks their in-lane sums: if one is above
  // kPsumLimit (or not finite), the wave takes the exact update for sub-tile
  // t and recomputes its probabilities. No row maximum is computed otherwise.
  // (Checking each 16-key half just before its P V products, so that part of
  // the probabilities could still be computed under the P V MFMAs, keeps the
  // sub-tile's scores live across more code and spills at d = 128.)
  auto step_body = [&](f32x16(&cur)[QB], f32x16(&nxt)[QB], int t, int v_slot, int kp_slot)
                       __attribute__((always_inline)) {
    const int h = t & 1;
    const int kp_slot_cur = h ? kp_slot : v_slot;  // slot of sub-tile t + 1 (rest of its K fragments)
    bf16x8 vf[2][T::NDB], pb[QB][2];
    float ps0[QB], ps1[QB], mc[QB], alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ps0[qb] = -0.f;  // x + (-0) = x exactly, so the first add folds away
      ps1[qb] = -0.f;
      mc[qb] = m[qb] * c2;
    }
    constexpr int EARLY = NPAIR;  // every pair is computed under the score MFMAs
    // The score MFMAs run at raised wave priority: when both waves of a SIMD
    // can issue, the one feeding the matrix core goes first (measured 1-2%).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) nxt[qb] = mfma32x32x16(kf[c], qop[qb][c], c == 0 ? (f32x16){} : nxt[qb]);
      if (c + 2 < T::NC) kf[c + 2] = k_frag(kp_slot_cur, (t + 1) & 1, c + 2);
#pragma unroll
      for (int i = EARLY * c / T::NC; i < EARLY * (c + 1) / T::NC; ++i)
        prob_pair(cur, pb, ps0, ps1, mc, pair_qb(i), pair_r(i));
      if (c < T::NDB) vf[0][c] = load_v(v_slot, h, 0, c);  // the 16-key chunk kc = 1 follows below
    }
    __builtin_amdgcn_s_setprio(0);
    {
      float chk[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) chk[qb] = ps0[qb] + ps1[qb];
      if (over_limit(chk)) {
        raise_ref(cur, alpha);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          ps0[qb] = -0.f;
          ps1[qb] = -0.f;
          mc[qb] = m[qb] * c2;
        }
#pragma unroll
        for (int i = 0; i < NPAIR; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_qb(i), pair_r(i));
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * T::NDB; ++i) {
      const int kc = i / T::NDB, db = i % T::NDB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) pv_mfma<QB>(oacc[qb][db], vf[kc][db], pb[qb][kc]);
      if (i < T::NDB) vf[1][i] = load_v(v_slot, h, 1, i);
      if (i >= 2 * T::NDB - 2) kf[i - (2 * T::NDB - 2)] = k_frag(kp_slot, h, i - (2 * T::NDB - 2));
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb] += ps0[qb] + ps1[qb];
  };
  // the same when sub-tile t + 1 is known to be fully visible
  auto clean_step = [&](f32x16(&cur)[QB], f32x16(&nxt)[QB], int t, int v_slot, int kp_slot)
                        __attribute__((always_inline)) { step_body(cur, nxt, t, v_slot, kp_slot); };
  auto full_step = [&](f32x16(&cur)[QB], f32x16(&nxt)[QB], int t, int v_slot, int kp_slot)
                       __attribute__((always_inline)) {
    step_body(cur, nxt, t, v_slot, kp_slot);
    if (needs_mask(t + 1)) mask(nxt, t + 1);
  };
  // the wave's last sub-tile: probabilities and P V only
  auto last_step = [&](f32x16(&cur)[QB], int t, int v_slot) __attribute__((always_inline)) {
    bf16x8 pb[QB][2];
    float ps0[QB], ps1[QB], mc[QB], alpha[QB], chk[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ps0[qb] = -0.f;
      ps1[qb] = -0.f;
      mc[qb] = m[qb] * c2;
    }
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_qb(i), pair_r(i));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) chk[qb] = ps0[qb] + ps1[qb];
    if (over_limit(chk)) {
      raise_ref(cur, alpha);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        ps0[qb] = -0.f;
        ps1[qb] = -0.f;
        mc[qb] = m[qb] * c2;
      }
#pragma unroll
      for (int i = 0; i < NPAIR; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_qb(i), pair_r(i));
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) {
        const bf16x8 a = load_v(v_slot, t & 1, kc, db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) pv_mfma<QB>(oacc[qb][db], a, pb[qb][kc]);
      }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb] += ps0[qb] + ps1[qb];
  };
  auto tail_step = [&](f32x16(&cur)[QB], f32x16(&nxt)[QB], int t, int v_slot, int kp_slot)
                       __attribute__((always_inline)) {
    if (t + 1 < n_st)
      full_step(cur, nxt, t, v_slot, kp_slot);
    else if (t < n_st)
      last_step(cur, t, v_slot);
  };
  // End of tile j: tile j + 2 resident for every wave (its K is fetched from
  // the next step on) and every wave done with tile j, whose ring slot then
  // receives tile j + 4. A wave's copies complete in issue order, so with
  // tile j + 3 also in flight it waits until only that tile's copies remain.
  auto end_tile = [&](int j, int slot) __attribute__((always_inline)) {
    if (j + 3 < n_kt)
      wait_vmcnt<2 * T::IPW>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (j + 4 < n_kt) dma(j + 4, slot);
  };

  wait_vmcnt<0>();  // Q, tiles 0 and 1
  __syncthreads();
  if (n_kt > 2) dma(2, 2);
  if (n_kt > 3) dma(3, 3);
  if (n_st > 0) {
    // sub-tile 0 sets the first reference (from m = -inf: alpha = 0)
    float alpha0[QB];
    qk(sA, 0, 0);
    if (needs_mask(0)) mask(sA, 0);
    raise_ref(sA, alpha0);
  }
  kf[0] = k_frag(0, 1, 0);  // sub-tile 1 (tile 0, second half)
  kf[1] = k_frag(0, 1, 1);
  // Leading sub-tiles that need no mask: the steady-state loop runs the tiles
  // whose both steps start such a sub-tile, with no branch but the rare
  // exact update; the remaining tiles (diagonal, ragged end, or waves that are
  // done and only help with the copies) go through the general step. Tile j
  // sits in ring slot j % 4. Steps past a wave's last sub-tile fetch unused
  // (in-range) K fragments.
  const int n_clean = min(CAUSAL ? (wq0 + 1) / 32 : N / 32, N / 32);
  const int j_clean = max(0, (n_clean - 1) / 2);
  // The steady-state loop is unrolled over the ring depth, so every ring
  // slot offset is a compile-time constant that folds into the LDS
  // instructions' immediate offsets (j is a multiple of 4 at its top).
  static_assert(T::NBUF == 4, "the unrolled loop walks a 4-slot ring");
  int j = 0;
  for (; j + 4 <= j_clean; j += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s0 = r * T::KT, s1 = ((r + 1) & 3) * T::KT;
      clean_step(sA, sB, 2 * (j + r), s0, s1);
      clean_step(sB, sA, 2 * (j + r) + 1, s0, s1);
      end_tile(j + r, r);
    }
  }
  for (; j < j_clean; ++j) {
    const int s0 = (j & 3) * T::KT, s1 = ((j + 1) & 3) * T::KT;
    clean_step(sA, sB, 2 * j, s0, s1);
    clean_step(sB, sA, 2 * j + 1, s0, s1);
    end_tile(j, j & 3);
  }
  for (; j < n_kt; ++j) {
    const int s0 = (j & 3) * T::KT, s1 = ((j + 1) & 3) * T::KT;
    tail_step(sA, sB, 2 * j, s0, s1);
    tail_step(sB, sA, 2 * j + 1, s0, s1);
    end_tile(j, j & 3);
  }

  // ---- epilogue: O = acc / l, one rounding to bf16; LSE in natural log ----
  o_fence(oacc);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = halves_sum(lsum[qb]);
    const int qrow = wq0 + 32 * qb + lq;
    if (qrow < N) {
      const float inv = 1.f / ltot;
      uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < T::NDB; ++db)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const bf16x2 a = to_bf16x2(oacc[qb][db][4 * rb] * inv, oacc[qb][db][4 * rb + 1] * inv);
          const bf16x2 b = to_bf16x2(oacc[qb][db][4 * rb + 2] * inv, oacc[qb][db][4 * rb + 3] * inv);
          const bf16x4 four = __builtin_shufflevector(a, b, 0, 1, 2, 3);
          *(bf16x4*)(orow + 32 * db + 8 * rb + 4 * hf) = four;
        }
      if (LSE != nullptr && hf == 0) LSE[(size_t)bh * N + qrow] = m[qb] * scale + __logf(ltot);
    }
  }
}

#ifndef FA_FWD_QB
#define FA_FWD_QB 1
#endif
// query blocks of 32 rows per wave: 1 = eight waves (two per SIMD, the
// hardware interleaves them), 2 = four waves with every LDS fragment feeding
// two MFMAs (with every probability computed under the score MFMAs, that
// variant keeps both blocks' probabilities live and spills at d = 128)
constexpr int kFwdQB = FA_FWD_QB;

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int N, float scale, hipStream_t s) {
  using T = FwdTile<D, kFwdQB>;
  const int n_qt = (N + T::BR - 1) / T::BR;
  const int BH = B * H;
  // exp2 units; a positive floor keeps masked (-inf) scores at probability 0
  // when scale is 0 (every visible probability is then exp2(~0) = 1)
  float c2 = scale * kLog2e;
  if (!(c2 >= FLT_MIN)) c2 = FLT_MIN;
  dim3 grid((unsigned)(n_qt * BH)), block(64 * T::NW);
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)o;
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, &scale, &c2, (void*)&n_qt, (void*)&BH};
  return hipLaunchKernel((const void*)&fwd_bf16_kernel<D, kFwdQB, CAUSAL>, grid, block, args, 0, s);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, bool causal, float scale, hipStream_t s) {
  if (d == 64)
    return causal ? launch_fwd_bf16_t<64, true>(q, k, v, o, lse, B, H, N, scale, s)
                  : launch_fwd_bf16_t<64, false>(q, k, v, o, lse, B, H, N, scale, s);
  return causal ? launch_fwd_bf16_t<128, true>(q, k, v, o, lse, B, H, N, scale, s)
                : launch_fwd_bf16_t<128, false>(q, k, v, o, lse, B, H, N, scale, s);
}

}  // namespace fa
