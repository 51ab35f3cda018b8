// Fused exact attention forward, bf16 in/out, fp32 accumulation, gfx950.
//
// One workgroup owns BR = 128 query rows of one (b, h) head (4 waves x 32
// rows) and walks the key/value tiles of BC = 64 rows once, keeping the
// scores on chip: the tiling and online-softmax method of "Describe Flash
// Attention at a high level" (mantramindai.in), section "The two ideas", and
// of "How FlashAttention Speeds Up the Attention Layer" (hassanahmed.net),
// sections on tiling and on the online softmax.
//
// Register plumbing (lane layouts in fa_device.h):
//  * each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, K tile
//    rows as the A operand (from LDS), its 32 query rows as the B operand
//    (held in VGPRs for the whole pass). In the S^T accumulator lane l holds
//    query (l % 32) and 16 keys per 32-key block, so the row max and row sum
//    are in-lane reductions plus one exchange with lane l ^ 32;
//  * the same registers, rounded to bf16, are directly the B operand of
//    O^T += V^T P^T: accumulator element r of lane l is key
//    (r%4) + 8*(r/4) + 4*(l/32) of its block, and the V^T A operand is read
//    from the row-major V tile with the transposing LDS read so that its
//    k-slots hold exactly those keys;
//  * O^T stays in 4 x 16 accumulators per lane (d = 128), lane l owning query
//    (l % 32), so the per-row rescale by exp(m_old - m_new) is a per-lane
//    scalar multiply.
// Causal: key tiles past the workgroup's last query are never loaded, tiles
// past a wave's last query are skipped by that wave, and only tiles that
// straddle the diagonal (or the ragged end of N) evaluate the mask.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdTile {
  static constexpr int NW = 4;                 // waves per workgroup
  static constexpr int BR = 32 * NW;           // query rows per workgroup
  static constexpr int BC = 64;                // keys per tile
  static constexpr int KP = D + 8;             // LDS pitch of a K row, bf16 elements (16 B pad)
  static constexpr int VP = D + 32;            // LDS pitch of a V row (64 B pad)
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int LOADS = BC * CH / (64 * NW);  // chunks per thread per tensor per tile
  static_assert(LOADS * 64 * NW == BC * CH, "tile must split evenly over the threads");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                          int N, float scale, int n_qt, int BH) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[T::BC * T::KP];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[T::BC * T::VP];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, hf = l >> 5, lq = l & 31;
  // Consecutive workgroups take consecutive heads of the same query-tile rank,
  // so with B*H a multiple of 8 every head stays on one XCD (workgroups are
  // dealt round-robin over the 8 XCDs) and its K/V tiles are shared in that
  // XCD's L2. Causal: the heaviest query tiles are dispatched first.
  const int bh = blockIdx.x % BH;
  const int rank = blockIdx.x / BH;
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;
  const int q0 = qt * T::BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const int wq0 = q0 + 32 * w;          // first query row of this wave
  const int qrow = wq0 + lq;            // the query row this lane owns

  // Q^T as the B operand: k-slots of chunk c are head dims 16c + 8*hf + (0..7).
  bf16x8 qop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (qrow < N)
      qop[c] = *(const bf16x8*)(Qh + (size_t)qrow * D + 16 * c + 8 * hf);
    else
      qop[c] = (bf16x8){};
  }

  const float c2 = scale * kLog2e;      // logits in base-2 units: exp(scale*x) = exp2(c2*x)
  float m = -FLT_MAX;                   // running max of the raw scores q.k
  float lsum = 0.f;                     // this half-wave's share of the running sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = (f32x16){};

  const int kv_end = CAUSAL ? min(N, q0 + T::BR) : N;
  const int n_kt = (kv_end + T::BC - 1) / T::BC;

  u32x4 kst[T::LOADS], vst[T::LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int idx = tid + 64 * T::NW * i;
      const int row = idx / T::CH, ch = idx % T::CH;
      const int key = kt * T::BC + row;
      if (key < N) {
        kst[i] = *(const u32x4*)(Kh + (size_t)key * D + ch * 8);
        vst[i] = *(const u32x4*)(Vh + (size_t)key * D + ch * 8);
      } else {  // rows past N are zero so that 0 * V stays finite
        kst[i] = (u32x4){};
        vst[i] = (u32x4){};
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int idx = tid + 64 * T::NW * i;
      const int row = idx / T::CH, ch = idx % T::CH;
      *(u32x4*)(k_lds + row * T::KP + ch * 8) = kst[i];
      *(u32x4*)(v_lds + row * T::VP + ch * 8) = vst[i];
    }
  };

  // Source address of this lane in the transposing V reads: lane (g, s) of
  // 16-lane group g serves key 4*(g/2) + s/4 (+16*kc, +8 for the second read)
  // and head dims 16*(g%2) + 4*(s%4) .. +3 (+32*db).
  const int g16 = l >> 4, s16 = l & 15;
  const int v_src = (4 * (g16 >> 1) + (s16 >> 2)) * T::VP + 16 * (g16 & 1) + 4 * (s16 & 3);

  const bool wave_has_rows = wq0 < N;
  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) gload(kt + 1);   // next tile's loads fly while this one is used
    const int k0 = kt * T::BC;
    const bool active = wave_has_rows && (!CAUSAL || k0 <= wq0 + 31);
    if (active) {
      // ---- S^T = K Q^T for BC keys x 32 queries ----
      f32x16 sacc[T::BC / 32];
#pragma unroll
      for (int kb = 0; kb < T::BC / 32; ++kb) {
        sacc[kb] = (f32x16){};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8 a = *(const bf16x8*)(k_lds + (32 * kb + lq) * T::KP + 16 * c + 8 * hf);
          sacc[kb] = mfma32x32x16(a, qop[c], sacc[kb]);
        }
      }
      // ---- mask (only tiles that reach past N or cross the diagonal) ----
      const bool need_mask = (k0 + T::BC > N) || (CAUSAL && k0 + T::BC - 1 > wq0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < T::BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + (r & 3) + 8 * (r >> 2) + 4 * hf;
            const bool vis = key < N && (!CAUSAL || key <= qrow);
            if (!vis) sacc[kb][r] = -INFINITY;
          }
      }
      // ---- online softmax update ----
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < T::BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = halves_max(mt);
      const float m_new = fmaxf(m, mt);
      const float alpha = fast_exp2((m - m_new) * c2);
      const float mc = m_new * c2;
      m = m_new;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(sacc[kb][r], c2, -mc));
          if (need_mask && sacc[kb][r] == -INFINITY) p = 0.f;  // also right when scale == 0
          sacc[kb][r] = p;
          ps += p;
        }
      lsum = alpha * lsum + ps;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int kc = 0; kc < T::BC / 16; ++kc) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 two = to_bf16x2(sacc[kc >> 1][8 * (kc & 1) + e], sacc[kc >> 1][8 * (kc & 1) + e + 1]);
          pb[e] = two[0];
          pb[e + 1] = two[1];
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint16_t* src = v_lds + v_src + 16 * kc * T::VP + 32 * db;
          const s16x4 lo = lds_read_tr16(src);
          const s16x4 hi = lds_read_tr16(src + 8 * T::VP);
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, both), pb, oacc[db]);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < n_kt) {
      lstore();
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / l, one rounding to bf16; LSE in natural log ----
  const float ltot = halves_sum(lsum);
  if (qrow < N) {
    const float inv = 1.f / ltot;
    uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
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

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int N, float scale, hipStream_t s) {
  using T = FwdTile<D>;
  const int n_qt = (N + T::BR - 1) / T::BR;
  const int BH = B * H;
  dim3 grid((unsigned)(n_qt * BH)), block(64 * T::NW);
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)o;
  void* args[] = {&qp, &kp, &vp, &op, &lse, &N, &scale, (void*)&n_qt, (void*)&BH};
  return hipLaunchKernel((const void*)&fwd_bf16_kernel<D, CAUSAL>, grid, block, args, 0, s);
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
