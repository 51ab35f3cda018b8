// Split-KV decode (Flash-Decoding) for one query row per (b, h), gfx950.
//
// With a single query row there is no query tile to spread over the chip, so
// the key/value cache is cut into chunks that run in separate workgroups; each
// yields a partial (max, sum of exponentials, unnormalised output) and a
// second kernel merges the partials with the max-and-sum rule of the online
// softmax: "Describe Flash Attention at a high level" (mantramindai.in),
// section "Follow-up questions to expect", the question on decode.
//
// The split kernel is HBM-bound (every cached byte is read once). Each key
// row (d bf16 = 128 or 256 B) is read by TPK = d/8 adjacent lanes, 16 B each,
// so a wave reads whole rows with 16-byte loads; a workgroup's G = 256/TPK
// lane groups walk the chunk's rows in an interleaved order, UNR rows per
// group per batch so that 2*UNR loads per lane are in flight. A row's score
// is a DPP butterfly sum over its TPK lanes; each group keeps its own running
// (max, sum, output slice), and the groups are merged in LDS at the end.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct DecTile {
  static constexpr int TPK = D / 8;            // lanes per key row
  static constexpr int THREADS = 256;
  static constexpr int G = THREADS / TPK;      // key groups per workgroup
  static constexpr int UNR = 8;                // rows per group per batch
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of TPK (8 or 16) lanes; every lane of the group
// gets the bit-identical result (each step adds the same two values).
template <int TPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <-> 7-i within 8
  if constexpr (TPK == 16) x += dpp_mov<0x140>(x);  // row_mirror: lane i <-> 15-i within 16
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ Kc,
                                                           const uint16_t* __restrict__ Vc, float* __restrict__ ws,
                                                           int Lkv, int nsplit, int chunk, int BH, float c2) {
  using T = DecTile<D>;
  __shared__ float sm_m[T::G], sm_l[T::G];
  __shared__ float sm_o[T::G * D];

  const int split = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;  // a head's splits are adjacent
  const int tid = threadIdx.x, g = tid / T::TPK, sub = tid % T::TPK;
  const int kbeg = split * chunk;
  const int kend = min(Lkv, kbeg + chunk);
  const size_t head = (size_t)bh * (size_t)Lkv * D;
  const uint16_t* Kh = Kc + head + 8 * sub;
  const uint16_t* Vh = Vc + head + 8 * sub;

  const u32x4 qw = *(const u32x4*)(Q + (size_t)bh * D + 8 * sub);
  float qf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qf[2 * i] = bf16_lo(qw[i]);
    qf[2 * i + 1] = bf16_hi(qw[i]);
  }
  float m = -FLT_MAX, lsum = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  const int n_it = (kend - kbeg + T::G * T::UNR - 1) / (T::G * T::UNR);  // same for every lane
  for (int it = 0; it < n_it; ++it) {
    const int base = kbeg + it * T::G * T::UNR + g;
    u32x4 kk[T::UNR], vv[T::UNR];
#pragma unroll
    for (int u = 0; u < T::UNR; ++u) {
      const int key = base + T::G * u;
      if (key < kend) {
        kk[u] = *(const u32x4*)(Kh + (size_t)key * D);
        vv[u] = *(const u32x4*)(Vh + (size_t)key * D);
      } else {
        kk[u] = (u32x4){};
        vv[u] = (u32x4){};
      }
    }
    float s[T::UNR];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < T::UNR; ++u) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part = fmaf(qf[2 * i], bf16_lo(kk[u][i]), part);
        part = fmaf(qf[2 * i + 1], bf16_hi(kk[u][i]), part);
      }
      part = group_sum<T::TPK>(part);
      s[u] = (base + T::G * u < kend) ? part : -INFINITY;
      mt = fmaxf(mt, s[u]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = fast_exp2((m - m_new) * c2);
    const float mc = m_new * c2;
    m = m_new;
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < T::UNR; ++u) {
      const float p = (s[u] == -INFINITY) ? 0.f : fast_exp2(fmaf(s[u], c2, -mc));
      s[u] = p;
      ps += p;
    }
    lsum = alpha * lsum + ps;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a0 = o[2 * i] * alpha, a1 = o[2 * i + 1] * alpha;
#pragma unroll
      for (int u = 0; u < T::UNR; ++u) {
        a0 = fmaf(s[u], bf16_lo(vv[u][i]), a0);
        a1 = fmaf(s[u], bf16_hi(vv[u][i]), a1);
      }
      o[2 * i] = a0;
      o[2 * i + 1] = a1;
    }
  }

  // merge the G groups of this workgroup
  if (sub == 0) {
    sm_m[g] = m;
    sm_l[g] = lsum;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sm_o[g * D + 8 * sub + i] = o[i];
  __syncthreads();
  if (tid < D) {
    float M = -FLT_MAX;
    for (int j = 0; j < T::G; ++j) M = fmaxf(M, sm_m[j]);
    float L = 0.f, acc = 0.f;
    for (int j = 0; j < T::G; ++j) {
      const float wgt = fast_exp2((sm_m[j] - M) * c2);
      L = fmaf(wgt, sm_l[j], L);
      acc = fmaf(wgt, sm_o[j * D + tid], acc);
    }
    const size_t part = (size_t)bh * nsplit + split;
    ws[(size_t)BH * nsplit * 2 + part * D + tid] = acc;
    if (tid == 0) {
      ws[2 * part] = M;
      ws[2 * part + 1] = L;
    }
  }
}

// Merge nsplit partials of one (b, h): M = max m_s, w_s = exp(m_s - M),
// o = sum w_s o_s / sum w_s l_s, rounded once to bf16.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws, uint16_t* __restrict__ O,
                                                           int nsplit, int BH, float c2) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* ml = ws + (size_t)bh * nsplit * 2;
  const float* os = ws + (size_t)BH * nsplit * 2 + (size_t)bh * nsplit * D;
  float M = -FLT_MAX;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = fast_exp2((ml[2 * s] - M) * c2);
    L = fmaf(wgt, ml[2 * s + 1], L);
    acc = fmaf(wgt, os[(size_t)s * D + t], acc);
  }
  const __bf16 r = (__bf16)(acc / L);  // round to nearest even
  O[(size_t)bh * D + t] = __builtin_bit_cast(uint16_t, r);
}

template <int D>
static hipError_t launch_decode_t(const void* q, const void* kc, const void* vc, void* o, float* ws, int B, int H,
                                  int Lkv, int nsplit, int chunk, hipStream_t s) {
  int BH = B * H;
  const float scale = (float)(1.0 / sqrt((double)D));  // 1/sqrt(d) rounded once to float32
  float c2 = scale * kLog2e;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)kc, *vp = (const uint16_t*)vc;
  uint16_t* op = (uint16_t*)o;
  void* a1[] = {&qp, &kp, &vp, &ws, &Lkv, &nsplit, &chunk, &BH, &c2};
  hipError_t e = hipLaunchKernel((const void*)&decode_split_kernel<D>, dim3((unsigned)(nsplit * BH)),
                                 dim3(DecTile<D>::THREADS), a1, 0, s);
  if (e != hipSuccess) return e;
  const float* wsc = ws;
  void* a2[] = {&wsc, &op, &nsplit, &BH, &c2};
  return hipLaunchKernel((const void*)&decode_combine_kernel<D>, dim3((unsigned)BH), dim3(D), a2, 0, s);
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* o, float* ws, int B, int H, int Lkv,
                         int d, int nsplit, int chunk, hipStream_t s) {
  if (d == 64) return launch_decode_t<64>(q, kc, vc, o, ws, B, H, Lkv, nsplit, chunk, s);
  return launch_decode_t<128>(q, kc, vc, o, ws, B, H, Lkv, nsplit, chunk, s);
}

}  // namespace fa
