// Naive three-step attention, kept only as an ablation of the fused kernel.
//
// Exactly the formulation the pages contrast FlashAttention with ("Describe
// Flash Attention at a high level" (mantramindai.in), section "What naive
// attention does"; "How FlashAttention Speeds Up the Attention Layer"
// (hassanahmed.net), the three-step formulation): the full N x N score matrix
// goes to HBM, is read back for the softmax, written again as probabilities
// and read once more for the product with V. Per head that is four N^2 fp32
// passes over HBM, which is what the byte counters are meant to show next to
// the fused kernel's O(N d).
//   1. naive_scores:  S = scale * Q K^T, -inf where causally masked (fp32)
//   2. naive_softmax: P = softmax(S) row by row, in place; LSE per row
//   3. naive_pv:      O = P V, rounded to bf16
// All arithmetic is fp32 on the vector ALUs.
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

// 64x64 score tile per workgroup; each of 256 threads computes 4x4 scores.
template <int D>
__global__ __launch_bounds__(256) void naive_scores_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K, float* __restrict__ S,
                                                           int N, float scale, int causal) {
  __shared__ float q_lds[64 * (D + 1)];
  __shared__ float k_lds[64 * (D + 1)];
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64, bh = blockIdx.z;
  const size_t head = (size_t)bh * (size_t)N * D;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    q_lds[r * (D + 1) + c] = (i0 + r < N) ? bf16_at(Q + head + (size_t)(i0 + r) * D + c) : 0.f;
    k_lds[r * (D + 1) + c] = (j0 + r < N) ? bf16_at(K + head + (size_t)(j0 + r) * D + c) : 0.f;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int c = 0; c < D; ++c) {
    float a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = q_lds[(ty + 16 * u) * (D + 1) + c];
      b[u] = k_lds[(tx + 16 * u) * (D + 1) + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty + 16 * u;
    if (i >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + tx + 16 * v;
      if (j >= N) continue;
      S[((size_t)bh * N + i) * N + j] = (causal && j > i) ? -INFINITY : acc[u][v] * scale;
    }
  }
}

__device__ __forceinline__ float block_max(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return x;
}
__device__ __forceinline__ float block_sum(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return x;
}

// One workgroup per row: the row is read once into LDS, then written back as
// probabilities.
__global__ __launch_bounds__(256) void naive_softmax_kernel(float* __restrict__ S, float* __restrict__ LSE, int N) {
  extern __shared__ float row[];
  __shared__ float red[4];
  const size_t r = (size_t)blockIdx.y * N + blockIdx.x;
  float* srow = S + r * N;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < N; j += 256) {
    row[j] = srow[j];
    mx = fmaxf(mx, row[j]);
  }
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < N; j += 256) {
    const float e = expf(row[j] - mx);
    row[j] = e;
    sum += e;
  }
  sum = block_sum(sum, red);
  const float inv = 1.f / sum;
  for (int j = threadIdx.x; j < N; j += 256) srow[j] = row[j] * inv;
  if (LSE != nullptr && threadIdx.x == 0) LSE[r] = mx + logf(sum);
}

// 64 output rows per workgroup; each thread computes 4 rows x D/16 columns.
template <int D>
__global__ __launch_bounds__(256) void naive_pv_kernel(const float* __restrict__ P, const uint16_t* __restrict__ V,
                                                       uint16_t* __restrict__ O, int N) {
  __shared__ float p_lds[64 * 33];
  __shared__ float v_lds[32 * D];
  const int i0 = blockIdx.x * 64, bh = blockIdx.y;
  const size_t head = (size_t)bh * (size_t)N * D;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][D / 16] = {};
  for (int j0 = 0; j0 < N; j0 += 32) {
    __syncthreads();
    for (int idx = tid; idx < 64 * 32; idx += 256) {
      const int r = idx / 32, c = idx % 32;
      p_lds[r * 33 + c] = (i0 + r < N && j0 + c < N) ? P[((size_t)bh * N + i0 + r) * N + j0 + c] : 0.f;
    }
    for (int idx = tid; idx < 32 * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      v_lds[r * D + c] = (j0 + r < N) ? bf16_at(V + head + (size_t)(j0 + r) * D + c) : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < 32; ++j) {
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = p_lds[(ty + 16 * u) * 33 + j];
#pragma unroll
      for (int v = 0; v < D / 16; ++v) {
        const float b = v_lds[j * D + tx + 16 * v];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u][v] = fmaf(a[u], b, acc[u][v]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty + 16 * u;
    if (i >= N) continue;
#pragma unroll
    for (int v = 0; v < D / 16; ++v) {
      const __bf16 r = (__bf16)acc[u][v];
      O[head + (size_t)i * D + tx + 16 * v] = __builtin_bit_cast(uint16_t, r);
    }
  }
}

template <int D>
static hipError_t launch_naive_t(const void* q, const void* k, const void* v, void* o, float* lse, float* S, int B,
                                 int H, int N, bool causal, float scale, hipStream_t s) {
  int BH = B * H, caus = causal ? 1 : 0;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)o;
  const unsigned nt = (unsigned)((N + 63) / 64);
  void* a1[] = {&qp, &kp, &S, &N, &scale, &caus};
  hipError_t e = hipLaunchKernel((const void*)&naive_scores_kernel<D>, dim3(nt, nt, (unsigned)BH), dim3(256), a1, 0, s);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)N * sizeof(float);
  e = hipFuncSetAttribute((const void*)&naive_softmax_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  void* a2[] = {&S, &lse, &N};
  e = hipLaunchKernel((const void*)&naive_softmax_kernel, dim3((unsigned)N, (unsigned)BH), dim3(256), a2, lds, s);
  if (e != hipSuccess) return e;
  const float* Pc = S;
  void* a3[] = {&Pc, &vp, &op, &N};
  return hipLaunchKernel((const void*)&naive_pv_kernel<D>, dim3(nt, (unsigned)BH), dim3(256), a3, 0, s);
}

hipError_t launch_naive(const void* q, const void* k, const void* v, void* o, float* lse, float* S, int B, int H,
                        int N, int d, bool causal, float scale, hipStream_t s) {
  if (d == 64) return launch_naive_t<64>(q, k, v, o, lse, S, B, H, N, causal, scale, s);
  return launch_naive_t<128>(q, k, v, o, lse, S, B, H, N, causal, scale, s);
}

}  // namespace fa
