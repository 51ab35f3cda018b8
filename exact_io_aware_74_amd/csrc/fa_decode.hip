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

#include <mutex>

#include "fa.h"
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

// Where the key/value rows of one (b, h) live. offset(u, key) is the element
// offset of row `key` from the lane's base pointer; prime(base, kend) makes the
// offsets of keys base + G*u (u < UNR) available to the next offset() calls.

// A contiguous [Lkv, D] cache per head.
template <int D>
struct ContigRows {
  __device__ __forceinline__ void prime(int, int) {}
  __device__ __forceinline__ size_t offset(int, int key) { return (size_t)key * D; }
  __device__ __forceinline__ bool poisoned() const { return false; }
};

// A paged cache: key j of the sequence is row j % page_size of pool page
// table[j / page_size], each pool page holding [H, page_size, D] (the lane's
// base pointer already points at this head's rows of page 0). prime() loads
// the page ids of the next keys one iteration ahead of their use, clamped to
// the last key so the table is never read past the sequence. A page id
// outside the pool is replaced by page 0 (no access leaves the pool) and
// poisons the partial, which turns the output row into NaN.
template <int D, int G, int UNR>
struct PagedRows {
  const int* __restrict__ table;
  size_t page_stride;  // H * page_size * D elements
  int lps;             // log2(page_size)
  int num_pages;
  int pg[UNR];
  bool bad = false;

  __device__ __forceinline__ void prime(int base, int kend) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) pg[u] = table[min(base + G * u, kend - 1) >> lps];
  }
  __device__ __forceinline__ size_t offset(int u, int key) {
    int p = pg[u];
    if ((unsigned)p >= (unsigned)num_pages) {
      bad = true;
      p = 0;
    }
    return (size_t)p * page_stride + (size_t)(key & ((1 << lps) - 1)) * D;
  }
  __device__ __forceinline__ bool poisoned() const { return bad; }
};

// One split: keys [kbeg, kend) of one (b, h) against query row q. Writes the
// partial (max m, sum l of exp(s - m), unnormalised output) of this split to
// partial `part` of the workspace (n_parts partials in all). An empty split
// writes (-FLT_MAX, 0, 0); `poison` (or a poisoned row source) writes l = NaN.
template <int D, class Rows>
__device__ __forceinline__ void split_partial(const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kh,
                                              const uint16_t* __restrict__ Vh, Rows& rows, float* __restrict__ ws,
                                              int kbeg, int kend, bool poison, size_t part, size_t n_parts,
                                              float c2) {
  using T = DecTile<D>;
  __shared__ float sm_m[T::G], sm_l[T::G];
  __shared__ float sm_o[T::G * D];
  constexpr int STEP = T::G * T::UNR;

  const int tid = threadIdx.x, g = tid / T::TPK, sub = tid % T::TPK;
  const u32x4 qw = *(const u32x4*)(q + 8 * sub);
  float qf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qf[2 * i] = bf16_lo(qw[i]);
    qf[2 * i + 1] = bf16_hi(qw[i]);
  }
  float m = -FLT_MAX, lsum = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  const int n_it = kend > kbeg ? (kend - kbeg + STEP - 1) / STEP : 0;  // same for every lane
  if (n_it > 0) rows.prime(kbeg + g, kend);
  for (int it = 0; it < n_it; ++it) {
    const int base = kbeg + it * STEP + g;
    u32x4 kk[T::UNR], vv[T::UNR];
#pragma unroll
    for (int u = 0; u < T::UNR; ++u) {
      const int key = base + T::G * u;
      if (key < kend) {
        const size_t off = rows.offset(u, key);
        // non-temporal: every cached key is read once, so the stream is not
        // kept in L2 or the Infinity Cache (measured 6.14 -> 6.59 TB/s)
        kk[u] = __builtin_nontemporal_load((const u32x4*)(Kh + off));
        vv[u] = __builtin_nontemporal_load((const u32x4*)(Vh + off));
      } else {
        kk[u] = (u32x4){};
        vv[u] = (u32x4){};
      }
    }
    rows.prime(base + STEP, kend);
    float s[T::UNR];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < T::UNR; ++u) {
      float part_s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part_s = fmaf(qf[2 * i], bf16_lo(kk[u][i]), part_s);
        part_s = fmaf(qf[2 * i + 1], bf16_hi(kk[u][i]), part_s);
      }
      part_s = group_sum<T::TPK>(part_s);
      s[u] = (base + T::G * u < kend) ? part_s : -INFINITY;
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
  if (poison || rows.poisoned()) lsum = __builtin_nanf("");

  // merge the G groups of this workgroup (all lanes of a group hold the same m, l)
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
    ws[n_parts * 2 + part * D + tid] = acc;
    if (tid == 0) {
      ws[2 * part] = M;
      ws[2 * part + 1] = L;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ Kc,
                                                           const uint16_t* __restrict__ Vc, float* __restrict__ ws,
                                                           int Lkv, int nsplit, int chunk, int BH, float c2) {
  const int split = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;  // a head's splits are adjacent
  const int sub = threadIdx.x % DecTile<D>::TPK;
  const int kbeg = split * chunk;
  const int kend = min(Lkv, kbeg + chunk);
  const size_t head = (size_t)bh * (size_t)Lkv * D + 8 * sub;
  ContigRows<D> rows;
  split_partial<D>(Q + (size_t)bh * D, Kc + head, Vc + head, rows, ws, kbeg, kend, false,
                   (size_t)bh * nsplit + split, (size_t)BH * nsplit, c2);
}

// Paged cache: pools [num_pages, H, page_size, D], table [B, max_pages],
// lengths [B]. A length outside [0, max_pages * page_size] is clamped into
// that range and poisons the row.
template <int D>
__global__ __launch_bounds__(256) void decode_split_paged_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kp, const uint16_t* __restrict__ Vp,
    const int* __restrict__ table, const int* __restrict__ lens, float* __restrict__ ws, int H, int lps,
    int num_pages, int max_pages, int nsplit, int chunk, int BH, float c2) {
  using T = DecTile<D>;
  const int split = blockIdx.x % nsplit, bh = blockIdx.x / nsplit;
  const int b = bh / H, h = bh - b * H;
  const int sub = threadIdx.x % T::TPK;
  const int lmax = max_pages << lps;
  const int len_raw = lens[b];
  const bool bad_len = len_raw < 0 || len_raw > lmax;
  const int len = min(max(len_raw, 0), lmax);
  const int kbeg = split * chunk;
  const int kend = min(len, kbeg + chunk);
  PagedRows<D, T::G, T::UNR> rows;
  rows.table = table + (size_t)b * max_pages;
  rows.page_stride = ((size_t)H << lps) * D;
  rows.lps = lps;
  rows.num_pages = num_pages;
  const size_t head = ((size_t)h << lps) * D + 8 * sub;
  split_partial<D>(Q + (size_t)bh * D, Kp + head, Vp + head, rows, ws, kbeg, kend, bad_len,
                   (size_t)bh * nsplit + split, (size_t)BH * nsplit, c2);
}

// Merge nsplit partials of one (b, h): M = max m_s, w_s = exp(m_s - M),
// o = sum w_s o_s / sum w_s l_s, rounded once to bf16. Empty splits carry
// l_s = 0 and add nothing; a head with no keys at all gives 0, and a NaN
// l_s (a poisoned split) gives NaN.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws, uint16_t* __restrict__ O,
                                                           int nsplit, int BH, float c2) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* ml = ws + (size_t)bh * nsplit * 2;
  const float* os = ws + (size_t)BH * nsplit * 2 + (size_t)bh * nsplit * D;
  // unrolled so that a batch of independent loads is in flight at a time
  // (one load per iteration would pay the memory latency nsplit times)
  float M = -FLT_MAX;
#pragma unroll 16
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, acc = 0.f;
#pragma unroll 16
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = fast_exp2((ml[2 * s] - M) * c2);
    L = fmaf(wgt, ml[2 * s + 1], L);
    acc = fmaf(wgt, os[(size_t)s * D + t], acc);
  }
  const __bf16 r = (__bf16)(L == 0.f ? 0.f : acc / L);  // round to nearest even; no keys -> 0
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

// Decode partials in a fixed device array, for the entry point that allocates
// nothing. Every GPU that loads the library holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, so its
// device address is looked up once per device (with that device current) and
// only that address is handed to kernels.
static __device__ __align__(256) float scratch[FA_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = (float*)g_scratch_ptr[dev];
  return hipSuccess;
}

template <int D>
static hipError_t launch_decode_paged_t(const void* q, const void* kpool, const void* vpool, const int* table,
                                        const int* lens, void* o, float* ws, int B, int H, int lps, int num_pages,
                                        int max_pages, int nsplit, int chunk, hipStream_t s) {
  int BH = B * H;
  const float scale = (float)(1.0 / sqrt((double)D));  // 1/sqrt(d) rounded once to float32
  float c2 = scale * kLog2e;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)kpool, *vp = (const uint16_t*)vpool;
  uint16_t* op = (uint16_t*)o;
  void* a1[] = {&qp, &kp, &vp, &table, &lens, &ws, &H, &lps, &num_pages, &max_pages, &nsplit, &chunk, &BH, &c2};
  hipError_t e = hipLaunchKernel((const void*)&decode_split_paged_kernel<D>, dim3((unsigned)(nsplit * BH)),
                                 dim3(DecTile<D>::THREADS), a1, 0, s);
  if (e != hipSuccess) return e;
  const float* wsc = ws;
  void* a2[] = {&wsc, &op, &nsplit, &BH, &c2};
  return hipLaunchKernel((const void*)&decode_combine_kernel<D>, dim3((unsigned)BH), dim3(D), a2, 0, s);
}

hipError_t launch_decode_paged(const void* q, const void* kpool, const void* vpool, const int* table, const int* lens,
                               void* o, float* ws, int B, int H, int d, int log2_page, int num_pages, int max_pages,
                               int nsplit, int chunk, hipStream_t s) {
  if (d == 64)
    return launch_decode_paged_t<64>(q, kpool, vpool, table, lens, o, ws, B, H, log2_page, num_pages, max_pages,
                                     nsplit, chunk, s);
  return launch_decode_paged_t<128>(q, kpool, vpool, table, lens, o, ws, B, H, log2_page, num_pages, max_pages,
                                    nsplit, chunk, s);
}

}  // namespace fa
