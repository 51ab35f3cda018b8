// Fused exact attention forward in float32 throughout (no bf16 anywhere).
//
// Same tiled, single-pass online-softmax method as the bf16 kernel
// ("Describe Flash Attention at a high level" (mantramindai.in), section
// "The two ideas"), written for full fp32 precision on the vector ALUs: each
// query row is owned by TPR = d/32 adjacent lanes, every lane holding 32 of
// the row's head dims of q and of the running output. Key/value tiles of 32
// rows are staged in LDS; a tile's scores are reduced across the TPR lanes,
// the running max and sum are updated once per tile, and the old output is
// rescaled by exp(m_old - m_new) before the tile's weighted V rows are added.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct F32Tile {
  static constexpr int TPR = D / 32;           // lanes per query row
  static constexpr int THREADS = 256;
  static constexpr int BR = THREADS / TPR;     // query rows per workgroup
  static constexpr int BK = 32;                // keys per tile
  static constexpr int P = D + 4;              // LDS pitch (floats)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int N, float scale, int n_qt) {
  using T = F32Tile<D>;
  __shared__ float k_lds[T::BK * T::P];
  __shared__ float v_lds[T::BK * T::P];

  const int tid = threadIdx.x;
  const int sub = tid % T::TPR;
  const int qt = blockIdx.x % n_qt;
  const int bh = blockIdx.x / n_qt;
  const int q0 = qt * T::BR;
  const int qrow = q0 + tid / T::TPR;
  const size_t head = (size_t)bh * (size_t)N * D;

  float q[32], o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    q[i] = qrow < N ? Q[head + (size_t)qrow * D + 32 * sub + i] : 0.f;
    o[i] = 0.f;
  }
  float m = -FLT_MAX, lsum = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + T::BR) : N;
  for (int k0 = 0; k0 < kv_end; k0 += T::BK) {
    __syncthreads();
    for (int idx = tid; idx < T::BK * D; idx += T::THREADS) {
      const int r = idx / D, c = idx % D;
      const int key = k0 + r;
      k_lds[r * T::P + c] = key < N ? K[head + (size_t)key * D + c] : 0.f;
      v_lds[r * T::P + c] = key < N ? V[head + (size_t)key * D + c] : 0.f;
    }
    __syncthreads();
    float s[T::BK];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < T::BK; ++j) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) part = fmaf(q[i], k_lds[j * T::P + 32 * sub + i], part);
#pragma unroll
      for (int x = 1; x < T::TPR; x <<= 1) part += __shfl_xor(part, x);
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= qrow);
      s[j] = vis ? part * scale : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);
    m = m_new;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < T::BK; ++j) {
      s[j] = s[j] == -INFINITY ? 0.f : expf(s[j] - m_new);
      ps += s[j];
    }
    lsum = alpha * lsum + ps;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float acc = o[i] * alpha;
#pragma unroll
      for (int j = 0; j < T::BK; ++j) acc = fmaf(s[j], v_lds[j * T::P + 32 * sub + i], acc);
      o[i] = acc;
    }
  }
  if (qrow < N) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < 32; ++i) O[head + (size_t)qrow * D + 32 * sub + i] = o[i] * inv;
    if (LSE != nullptr && sub == 0) LSE[(size_t)bh * N + qrow] = m + logf(lsum);
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_f32_t(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                               int N, float scale, hipStream_t s) {
  using T = F32Tile<D>;
  int n_qt = (N + T::BR - 1) / T::BR;
  dim3 grid((unsigned)(n_qt * B * H)), block(T::THREADS);
  void* args[] = {&q, &k, &v, &o, &lse, &N, &scale, &n_qt};
  return hipLaunchKernel((const void*)&fwd_f32_kernel<D, CAUSAL>, grid, block, args, 0, s);
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                          int d, bool causal, float scale, hipStream_t s) {
  if (d == 64)
    return causal ? launch_f32_t<64, true>(q, k, v, o, lse, B, H, N, scale, s)
                  : launch_f32_t<64, false>(q, k, v, o, lse, B, H, N, scale, s);
  return causal ? launch_f32_t<128, true>(q, k, v, o, lse, B, H, N, scale, s)
                : launch_f32_t<128, false>(q, k, v, o, lse, B, H, N, scale, s);
}

}  // namespace fa
