// Fused exact attention forward in float32 throughout (no bf16 anywhere).
//
// Same tiled, single-pass online-softmax method as the bf16 kernel
// ("Describe Flash Attention at a high level" (mantramindai.in), section
// "The two ideas"), written for full fp32 precision on the vector ALUs.
//
// Mapping: one wave per query row, four rows per workgroup, so even a single
// 256-row head spreads over 64 workgroups. Key/value tiles of 64 rows are
// staged in LDS (the next tile is fetched into registers while the current
// one is used). For the scores each lane takes one key of the tile and forms
// its dot product with the wave's query row (held in registers); the tile's
// maximum and sum are wave reductions; the running output is then owned by
// head dimension (lane l holds dims l, l + 64, ...), and each lane adds the
// tile's probability-weighted V values of its dims, the probabilities being
// broadcast through LDS. The running maximum and sum are updated once per
// tile, with the old output rescaled by exp(m_old - m_new).
#include <float.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct F32Tile {
  static constexpr int ROWS = 4;               // query rows per workgroup (one per wave)
  static constexpr int THREADS = 64 * ROWS;
  static constexpr int BK = 64;                // keys per tile (one per lane)
  static constexpr int KP = D + 4;             // K row pitch in LDS (floats): 16-byte row offsets mod 128 B
  static constexpr int DPL = D / 64;           // output dims per lane
  static constexpr int F4 = D / 4;             // float4 per row
  static constexpr int LPT = BK * F4 / THREADS;  // float4 per thread per tensor per tile
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) x = fmaxf(x, __shfl_xor(x, k, 64));
  return x;
}
// Butterfly sum: lanes l and l ^ k add the same two values, so every lane
// ends with the identical total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) x += __shfl_xor(x, k, 64);
  return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int N, float scale, int n_qt) {
  using T = F32Tile<D>;
  __shared__ float4 k_lds[T::BK * T::KP / 4];
  __shared__ float4 v_lds[T::BK * T::F4];
  __shared__ float4 p_lds[T::ROWS][T::BK / 4];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int qt = blockIdx.x % n_qt;
  const int bh = blockIdx.x / n_qt;
  const int q0 = qt * T::ROWS;
  const int row = q0 + w;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float4* K4 = (const float4*)(K + head);
  const float4* V4 = (const float4*)(V + head);

  float4 q4[T::F4];
#pragma unroll
  for (int i = 0; i < T::F4; ++i)
    q4[i] = row < N ? ((const float4*)(Q + head + (size_t)row * D))[i] : make_float4(0.f, 0.f, 0.f, 0.f);

  const int kv_end = CAUSAL ? min(N, q0 + T::ROWS) : N;
  const int n_tiles = (kv_end + T::BK - 1) / T::BK;

  // this thread's share of a tile copy: float4 `idx` of the tile's rows
  float4 kr[T::LPT], vr[T::LPT];
  auto fetch = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::LPT; ++i) {
      const int idx = tid + T::THREADS * i, r = idx / T::F4, c = idx % T::F4;
      const int key = t * T::BK + r;
      const size_t off = (size_t)key * T::F4 + c;
      kr[i] = key < N ? K4[off] : make_float4(0.f, 0.f, 0.f, 0.f);
      vr[i] = key < N ? V4[off] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  float m = -FLT_MAX, lsum = 0.f, acc[T::DPL];
#pragma unroll
  for (int dd = 0; dd < T::DPL; ++dd) acc[dd] = 0.f;

  if (n_tiles > 0) fetch(0);
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < T::LPT; ++i) {
      const int idx = tid + T::THREADS * i, r = idx / T::F4, c = idx % T::F4;
      k_lds[r * (T::KP / 4) + c] = kr[i];
      v_lds[idx] = vr[i];
    }
    __syncthreads();
    if (t + 1 < n_tiles) fetch(t + 1);

    // score of key t*BK + l against this wave's row: four partial sums
    const int key = t * T::BK + l;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < T::F4; ++i) {
      const float4 kk = k_lds[l * (T::KP / 4) + i];
      part[i & 3] = fmaf(q4[i].x, kk.x, part[i & 3]);
      part[i & 3] = fmaf(q4[i].y, kk.y, part[i & 3]);
      part[i & 3] = fmaf(q4[i].z, kk.z, part[i & 3]);
      part[i & 3] = fmaf(q4[i].w, kk.w, part[i & 3]);
    }
    const bool vis = key < N && (!CAUSAL || key <= row);
    const float s = vis ? ((part[0] + part[1]) + (part[2] + part[3])) * scale : -INFINITY;
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = expf(m - m_new);
    m = m_new;
    const float p = vis ? expf(s - m_new) : 0.f;
    lsum = alpha * lsum + wave_sum(p);
    ((float*)p_lds[w])[l] = p;
    __builtin_amdgcn_wave_barrier();

    // output dims l + 64 dd: add the tile's probability-weighted V values
#pragma unroll
    for (int dd = 0; dd < T::DPL; ++dd) {
      float a = acc[dd] * alpha;
#pragma unroll
      for (int j4 = 0; j4 < T::BK / 4; ++j4) {
        const float4 pj = p_lds[w][j4];
        const float* vrow = (const float*)v_lds + (4 * j4) * D + 64 * dd + l;
        a = fmaf(pj.x, vrow[0], a);
        a = fmaf(pj.y, vrow[D], a);
        a = fmaf(pj.z, vrow[2 * D], a);
        a = fmaf(pj.w, vrow[3 * D], a);
      }
      acc[dd] = a;
    }
    __builtin_amdgcn_wave_barrier();  // p_lds is rewritten by the next tile
  }
  if (row < N) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int dd = 0; dd < T::DPL; ++dd) O[head + (size_t)row * D + 64 * dd + l] = acc[dd] * inv;
    if (LSE != nullptr && l == 0) LSE[(size_t)bh * N + row] = m + logf(lsum);
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_f32_t(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                               int N, float scale, hipStream_t s) {
  using T = F32Tile<D>;
  int n_qt = (N + T::ROWS - 1) / T::ROWS;
  dim3 grid((unsigned)((long long)n_qt * B * H)), block(T::THREADS);
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
