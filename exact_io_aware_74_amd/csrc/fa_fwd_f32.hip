// Fused exact attention forward in float32 throughout (no bf16 anywhere).
//
// Same tiled, single-pass online-softmax method as the bf16 kernel
// ("Describe Flash Attention at a high level" (mantramindai.in), section
// "The two ideas"), written for full fp32 precision on the vector ALUs.
//
// Mapping: one wave per query row, four rows per workgroup, so even a single
// 256-row head spreads over 64 workgroups (problems of at most 512 rows in
// all take fwd_f32_split_kernel below instead: one row per workgroup, the
// keys split over its four waves). Key/value tiles of 64 rows are
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


// Small problems: one workgroup per query row, its four waves splitting the
// keys (wave w takes 64-key tiles w, w + 4, ...). Each lane reads its key's
// row and, for the output, column l + 64 dd of the tile's V rows straight
// from global memory (no LDS staging, no workgroup barrier in the loop); the
// waves' (maximum, sum, output) are merged through LDS at the end.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_split_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                            const float* __restrict__ V, float* __restrict__ O,
                                                            float* __restrict__ LSE, int N, float scale) {
  using T = F32Tile<D>;
  constexpr int W = 4;  // waves per workgroup
  __shared__ float p_lds[W][T::BK];
  __shared__ float m_lds[W], l_lds[W];
  __shared__ float o_lds[W][D];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int row = blockIdx.x % N;
  const int bh = blockIdx.x / N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float4* q4p = (const float4*)(Q + head + (size_t)row * D);
  float4 q4[T::F4];
#pragma unroll
  for (int i = 0; i < T::F4; ++i) q4[i] = q4p[i];

  const int kv_end = CAUSAL ? row + 1 : N;
  const int n_tiles = (kv_end + T::BK - 1) / T::BK;
  float m = -FLT_MAX, lsum = 0.f, acc[T::DPL];
#pragma unroll
  for (int dd = 0; dd < T::DPL; ++dd) acc[dd] = 0.f;

  for (int t = w; t < n_tiles; t += W) {
    const int key = t * T::BK + l;
    const bool vis = key < kv_end;
    const float4* k4 = (const float4*)(K + head + (size_t)(vis ? key : 0) * D);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < T::F4; ++i) {
      const float4 kk = k4[i];
      part[i & 3] = fmaf(q4[i].x, kk.x, part[i & 3]);
      part[i & 3] = fmaf(q4[i].y, kk.y, part[i & 3]);
      part[i & 3] = fmaf(q4[i].z, kk.z, part[i & 3]);
      part[i & 3] = fmaf(q4[i].w, kk.w, part[i & 3]);
    }
    const float s = vis ? ((part[0] + part[1]) + (part[2] + part[3])) * scale : -INFINITY;
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = expf(m - m_new);
    m = m_new;
    const float p = vis ? expf(s - m_new) : 0.f;
    lsum = alpha * lsum + wave_sum(p);
    p_lds[w][l] = p;
    __builtin_amdgcn_wave_barrier();
    const int nk = min(T::BK, kv_end - t * T::BK);  // keys of this tile (uniform)
#pragma unroll
    for (int dd = 0; dd < T::DPL; ++dd) {
      const float* vcol = V + head + (size_t)(t * T::BK) * D + 64 * dd + l;
      float a[4] = {acc[dd] * alpha, 0.f, 0.f, 0.f};
      for (int j = 0; j < nk; ++j) a[j & 3] = fmaf(p_lds[w][j], vcol[(size_t)j * D], a[j & 3]);
      acc[dd] = (a[0] + a[1]) + (a[2] + a[3]);
    }
    __builtin_amdgcn_wave_barrier();  // p_lds is rewritten by the next tile
  }
  // merge the waves' partial (maximum, sum, output); wave 0 holds tile 0, so
  // the merged maximum is finite
  if (l == 0) {
    m_lds[w] = m;
    l_lds[w] = lsum;
  }
#pragma unroll
  for (int dd = 0; dd < T::DPL; ++dd) o_lds[w][64 * dd + l] = acc[dd];
  __syncthreads();
  if (w == 0) {
    float M = m_lds[0];
#pragma unroll
    for (int i = 1; i < W; ++i) M = fmaxf(M, m_lds[i]);
    float L = 0.f, wt[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      wt[i] = expf(m_lds[i] - M);
      L = fmaf(wt[i], l_lds[i], L);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int dd = 0; dd < T::DPL; ++dd) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < W; ++i) a = fmaf(wt[i], o_lds[i][64 * dd + l], a);
      O[head + (size_t)row * D + 64 * dd + l] = a * inv;
    }
    if (LSE != nullptr && l == 0) LSE[(size_t)bh * N + row] = M + logf(L);
  }
}

// Up to this many query rows in all (two workgroups per CU), one workgroup
// per row with the keys split over its waves: such a launch is bound by each
// wave's chain of tiles, which the split shortens fourfold. Larger problems
// share each K/V tile across four rows (measured: the split is faster up to
// 512 rows and 1.3-2x slower from 1024 rows, where every row re-reading its
// keys costs more than the shorter chains save).
constexpr long long kSplitRows = 512;

template <int D, bool CAUSAL>
static hipError_t launch_f32_t(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                               int N, float scale, hipStream_t s) {
  using T = F32Tile<D>;
  if ((long long)B * H * N <= kSplitRows) {
    dim3 grid((unsigned)((long long)B * H * N)), block(256);
    void* args[] = {&q, &k, &v, &o, &lse, &N, &scale};
    return hipLaunchKernel((const void*)&fwd_f32_split_kernel<D, CAUSAL>, grid, block, args, 0, s);
  }
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
