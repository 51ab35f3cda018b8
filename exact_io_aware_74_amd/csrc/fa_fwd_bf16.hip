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
//  * one workgroup = NW waves x 32 query rows of one (b, h) head: 8 waves (256
//    rows, two waves per SIMD) normally; 4 waves (128 rows, two workgroups per
//    CU) at d = 64 when 256-row tiles would leave the chip short of
//    workgroups, so the heaviest causal tile is half as long;
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
//    sub-tiles past a wave's last query are skipped by that wave. The two
//    waves of a SIMD hold one low and one high row block, so the diagonal's
//    growing work is the same on every SIMD, and the last three tiles (all
//    copies in, no slot rewritten) run without barriers;
//  * heaviest causal query tiles are dispatched first, and consecutive
//    workgroups take consecutive heads, all heads interleaved or, where each
//    XCD would otherwise stream many heads' K/V at once, in groups of 16
//    heads so that an XCD's workgroups share K/V tiles in its L2.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, int NW>
struct FwdTile {
  static constexpr int WR = 32;                 // query rows per wave (one MFMA block)
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
  static constexpr int WG_PER_CU = 8 / NW;      // workgroups per CU for two waves per SIMD
  static_assert(IPW * NW == CH, "DMA split");
  static_assert(WG_PER_CU * 2 * NBUF * KT <= 163840, "LDS budget");
};

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

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                                   const uint16_t* __restrict__ K,
                                                                   const uint16_t* __restrict__ V,
                                                                   uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                                   int N, float scale, float c2, int n_qt, int BH,
                                                                   int GH) {
  using T = FwdTile<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * T::NBUF * T::KT];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform: scalar branches below
  const int l = tid & 63, hf = l >> 5, lq = l & 31;
  // Workgroup -> (head, query tile): heads in groups of GH, each group's
  // query tiles in rank order (heaviest causal tiles first, the group's heads
  // interleaved). Workgroup i runs on XCD i % 8, so with GH a multiple of 8
  // each XCD works on GH / 8 heads of a group at a time; GH = BH is one group.
  const int grp = blockIdx.x / (GH * n_qt);
  const int gh = min(GH, BH - grp * GH);  // heads in this group (the last may be short)
  const int r = blockIdx.x - grp * GH * n_qt;
  const int bh = grp * GH + r % gh;
  const int rank = r / gh;
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;
  const int q0 = qt * T::BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  // Waves w and w + NW/2 share a SIMD. Row block w goes to wave w in the
  // first half and to wave NW/2 + (NW - 1 - w) in the second, so each SIMD
  // holds one low and one high row block: in the causal diagonal, where a row
  // block's work grows with its index, every SIMD then carries the same load.
  const int rb = w < NW / 2 ? w : (3 * NW / 2 - 1 - w);
  const int wq0 = q0 + T::WR * rb;  // first query row of this wave
  const int qrow = wq0 + lq;       // the query row this lane's scores and output belong to

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
  bf16x8 qop[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
    if (qrow < N)
      qop[c] = *(const bf16x8*)(Qh + (size_t)qrow * D + 16 * c + 8 * hf);
    else
      qop[c] = (bf16x8){};
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

  f32x16 sA, sB;            // S^T of one 32-key sub-tile (VGPRs)
  f32x16 oacc[T::NDB];      // O^T: lane l owns query l % 32
  float m = -INFINITY;      // reference maximum of the raw scores q.k
  float lsum = 0.f;         // this half-wave's share of the running sum
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) oacc[db] = (f32x16){};

  // K fragment c (A operand of S^T) of 32-key half h of the tile in the ring
  // slot at byte offset k_slot
  auto k_frag = [&](int k_slot, int h, int c) __attribute__((always_inline)) {
    return *(const bf16x8*)(lds + (k_lane[c & 3] + k_slot) + ((c >> 2) * (T::BC * 128) + h * 32 * 128));
  };
  // S^T for the 32-key half h of the tile in the slot at k_slot
  auto qk = [&](f32x16& s, int k_slot, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < T::NC; ++c) s = mfma32x32x16(k_frag(k_slot, h, c), qop[c], c == 0 ? (f32x16){} : s);
  };
  // keys past N and (causal) keys after the query row get -inf
  auto needs_mask = [&](int t) __attribute__((always_inline)) {
    return (32 * t + 32 > N) || (CAUSAL && 32 * t + 31 > wq0);
  };
  auto mask = [&](f32x16& s, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * t + (r & 3) + 8 * (r >> 2) + 4 * hf;
      const bool vis = key < N && (!CAUSAL || key <= qrow);
      if (!vis) s[r] = -INFINITY;
    }
  };
  // The exact online-softmax update for sub-tile s: the reference maximum
  // of every row becomes max(m, rowmax s) and O and the running sum are
  // rescaled by alpha = exp2((m_old - m_new) c2) (alpha = 1 where the
  // maximum did not move).
  auto raise_ref = [&](const f32x16& s) __attribute__((always_inline)) {
    float x = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) x = fmaxf(x, s[r]);
    const float m_new = fmaxf(m, halves_max(x));
    const float alpha = fast_exp2((m - m_new) * c2);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
  };
  // True (wave-uniform) when some lane's probability sum is above the limit
  // or not finite.
  auto over_limit = [&](float x) __attribute__((always_inline)) {
    return __builtin_expect(__builtin_amdgcn_ballot_w64(!(x <= kPsumLimit)) != 0, 0);
  };
  // Probabilities of a sub-tile against the reference maximum: bf16 B operand
  // of P V and this half-wave's fp32 row sums. One call handles elements r,
  // r + 1 (mc = reference maximum in exp2 units). The sum goes to ps0 for the
  // first 16-key chunk (elements 0-7) and to ps1 for the second: two
  // independent add chains.
  auto prob_pair = [&](const f32x16& s, bf16x8(&pb)[2], float& ps0, float& ps1, float mc, int r)
                       __attribute__((always_inline)) {
    const float p0 = fast_exp2(fmaf(s[r], c2, -mc));
    const float p1 = fast_exp2(fmaf(s[r + 1], c2, -mc));
    if (r < 8)
      ps0 += p0 + p1;
    else
      ps1 += p0 + p1;
    const bf16x2 two = to_bf16x2(p0, p1);
    pb[r >> 3][r & 7] = two[0];
    pb[r >> 3][(r & 7) + 1] = two[1];
  };
  // the eight element pairs in the order P V consumes them: 16-key chunk, element
  constexpr int NPAIR = 8;
  auto pair_r = [](int i) { return 8 * (i / 4) + 2 * (i & 3); };
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
  auto step_body = [&](f32x16& cur, f32x16& nxt, int t, int v_slot, int kp_slot) __attribute__((always_inline)) {
    const int h = t & 1;
    const int kp_slot_cur = h ? kp_slot : v_slot;  // slot of sub-tile t + 1 (rest of its K fragments)
    bf16x8 vf[2][T::NDB], pb[2];
    float ps0 = -0.f, ps1 = -0.f;  // x + (-0) = x exactly, so the first add folds away
    float mc = m * c2;
    // Every probability pair is computed under the score MFMAs, which run at
    // raised wave priority: when both waves of a SIMD can issue, the one
    // feeding the matrix core goes first (measured 1-2%).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
      nxt = mfma32x32x16(kf[c], qop[c], c == 0 ? (f32x16){} : nxt);
      if (c + 2 < T::NC) kf[c + 2] = k_frag(kp_slot_cur, (t + 1) & 1, c + 2);
#pragma unroll
      for (int i = NPAIR * c / T::NC; i < NPAIR * (c + 1) / T::NC; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_r(i));
      if constexpr (D == 64) {
        // d = 64 (bound by VALU issue): all of the sub-tile's V^T is read under
        // the score MFMAs, and the issue order per k-chunk is pinned: its MFMA,
        // then its LDS reads, then its probability pairs (measured 1-3% faster
        // at d = 64; at d = 128 the compiler's own order is as fast)
        if (c < T::NDB)
          vf[0][c] = load_v(v_slot, h, 0, c);
        else if (c < 2 * T::NDB)
          vf[1][c - T::NDB] = load_v(v_slot, h, 1, c - T::NDB);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // one MFMA
        if (c + 2 < T::NC)                                                       // K and V^T reads
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        else                                                                     // V^T reads
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8 * NPAIR / T::NC, 0);      // the probability pairs
      } else {
        if (c < T::NDB) vf[0][c] = load_v(v_slot, h, 0, c);  // the 16-key chunk kc = 1 follows below
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (over_limit(ps0 + ps1)) {
      raise_ref(cur);
      ps0 = -0.f;
      ps1 = -0.f;
      mc = m * c2;
#pragma unroll
      for (int i = 0; i < NPAIR; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_r(i));
    }
#pragma unroll
    for (int i = 0; i < 2 * T::NDB; ++i) {
      const int kc = i / T::NDB, db = i % T::NDB;
      oacc[db] = mfma32x32x16(vf[kc][db], pb[kc], oacc[db]);
      if constexpr (D != 64) {
        if (i < T::NDB) vf[1][i] = load_v(v_slot, h, 1, i);
      }
      if (i >= 2 * T::NDB - 2) kf[i - (2 * T::NDB - 2)] = k_frag(kp_slot, h, i - (2 * T::NDB - 2));
    }
    lsum += ps0 + ps1;
  };
  // the same when sub-tile t + 1 is known to be fully visible
  auto clean_step = [&](f32x16& cur, f32x16& nxt, int t, int v_slot, int kp_slot) __attribute__((always_inline)) {
    step_body(cur, nxt, t, v_slot, kp_slot);
  };
  auto full_step = [&](f32x16& cur, f32x16& nxt, int t, int v_slot, int kp_slot) __attribute__((always_inline)) {
    step_body(cur, nxt, t, v_slot, kp_slot);
    if (needs_mask(t + 1)) mask(nxt, t + 1);
  };
  // the wave's last sub-tile: probabilities and P V only
  auto last_step = [&](f32x16& cur, int t, int v_slot) __attribute__((always_inline)) {
    bf16x8 pb[2];
    float ps0 = -0.f, ps1 = -0.f;
    float mc = m * c2;
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_r(i));
    if (over_limit(ps0 + ps1)) {
      raise_ref(cur);
      ps0 = -0.f;
      ps1 = -0.f;
      mc = m * c2;
#pragma unroll
      for (int i = 0; i < NPAIR; ++i) prob_pair(cur, pb, ps0, ps1, mc, pair_r(i));
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) oacc[db] = mfma32x32x16(load_v(v_slot, t & 1, kc, db), pb[kc], oacc[db]);
    lsum += ps0 + ps1;
  };
  auto tail_step = [&](f32x16& cur, f32x16& nxt, int t, int v_slot, int kp_slot) __attribute__((always_inline)) {
    if (t + 1 < n_st)
      full_step(cur, nxt, t, v_slot, kp_slot);
    else if (t < n_st)
      last_step(cur, t, v_slot);
  };
  // End of tile j: tile j + 2 resident for every wave (its K is fetched from
  // the next step on) and every wave done with tile j, whose ring slot then
  // receives tile j + 4. A wave's copies complete in issue order, so with
  // tile j + 3 also in flight it waits until only that tile's copies remain.
  // After the last copy has been issued, one wait for all copies and one
  // barrier end the synchronisation.
  auto end_tile = [&](int j, int slot) __attribute__((always_inline)) {
    if (j + 4 < n_kt) {
      wait_vmcnt<2 * T::IPW>();  // tile j + 3 may still be in flight
      __syncthreads();
      dma(j + 4, slot);
    } else if (j == max(0, n_kt - 4)) {
      // every tile has been issued: once all copies are in, no slot is
      // written again, so the last tiles need no barrier and each wave
      // finishes them at its own pace
      wait_vmcnt<0>();
      __syncthreads();
    }
  };

  wait_vmcnt<0>();  // Q, tiles 0 and 1
  __syncthreads();
  if (n_kt > 2) dma(2, 2);
  if (n_kt > 3) dma(3, 3);
  if (n_st > 0) {
    // sub-tile 0 sets the first reference (from m = -inf: alpha = 0)
    qk(sA, 0, 0);
    if (needs_mask(0)) mask(sA, 0);
    raise_ref(sA);
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
  const float ltot = halves_sum(lsum);
  if (qrow < N) {
    const float inv = 1.f / ltot;
    uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x2 a = to_bf16x2(oacc[db][4 * rb] * inv, oacc[db][4 * rb + 1] * inv);
        const bf16x2 b = to_bf16x2(oacc[db][4 * rb + 2] * inv, oacc[db][4 * rb + 3] * inv);
        const bf16x4 four = __builtin_shufflevector(a, b, 0, 1, 2, 3);
        *(bf16x4*)(orow + 32 * db + 8 * rb + 4 * hf) = four;
      }
    if (LSE != nullptr && hf == 0) LSE[(size_t)bh * N + qrow] = m * scale + __logf(ltot);
  }
}

// A launch with fewer workgroups than this per CU takes 128-row tiles at
// d = 64 (two 4-wave workgroups per CU instead of one 8-wave one): the grid
// doubles and the heaviest causal tile, which sets the time of a short
// launch, halves.
constexpr int kSmallGridPerCU = 2;
constexpr int kNumCU = 256;

template <int D, int NW, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int N, float scale, hipStream_t s) {
  using T = FwdTile<D, NW>;
  const int n_qt = (N + T::BR - 1) / T::BR;
  const int BH = B * H;
  // exp2 units; a positive floor keeps masked (-inf) scores at probability 0
  // when scale is 0 (every visible probability is then exp2(~0) = 1)
  float c2 = scale * kLog2e;
  if (!(c2 >= FLT_MIN)) c2 = FLT_MIN;
  dim3 grid((unsigned)(n_qt * BH)), block(64 * NW);
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)o;
  int GH = head_group(NW, BH, n_qt);
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, &scale, &c2, (void*)&n_qt, (void*)&BH, &GH};
  return hipLaunchKernel((const void*)&fwd_bf16_kernel<D, NW, CAUSAL>, grid, block, args, 0, s);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, bool causal, float scale, hipStream_t s) {
  if (d == 64) {
    const long long big_tiles = (long long)B * H * ((N + 255) / 256);
    if (big_tiles < (long long)kSmallGridPerCU * kNumCU)
      return causal ? launch_fwd_bf16_t<64, 4, true>(q, k, v, o, lse, B, H, N, scale, s)
                    : launch_fwd_bf16_t<64, 4, false>(q, k, v, o, lse, B, H, N, scale, s);
    return causal ? launch_fwd_bf16_t<64, 8, true>(q, k, v, o, lse, B, H, N, scale, s)
                  : launch_fwd_bf16_t<64, 8, false>(q, k, v, o, lse, B, H, N, scale, s);
  }
  return causal ? launch_fwd_bf16_t<128, 8, true>(q, k, v, o, lse, B, H, N, scale, s)
                : launch_fwd_bf16_t<128, 8, false>(q, k, v, o, lse, B, H, N, scale, s);
}

}  // namespace fa
