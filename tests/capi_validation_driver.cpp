// Host-only driver for the C ABI's argument validation, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer (see test_capi_sanitized.py).
// Every call passes fake, never-dereferenced "device" addresses and at least
// one invalid argument, or an empty problem, so validation must return before
// any HIP call; the launchers are stubs that abort if reached.
//
// The few HIP runtime functions the C ABI calls are defined here too (the
// driver links no HIP library), so the decode workspace's allocation can be
// made to fail on demand: that path must return FA_ERR_NOMEM with nothing
// launched, and a later growth must release the old buffer exactly once.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "fa.h"
#include "fa_launch.h"

// ---- stand-ins for the HIP runtime calls of the C ABI ----
static bool g_malloc_fails = false;
static int g_mallocs = 0, g_frees = 0, g_syncs = 0;
static uintptr_t g_next_fake = (uintptr_t)1 << 44;
extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) {
  ++g_syncs;
  return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t bytes) {
  if (g_malloc_fails) return hipErrorOutOfMemory;
  ++g_mallocs;
  *p = (void*)g_next_fake;
  g_next_fake += (bytes + 0xFFFFF) & ~(uintptr_t)0xFFFFF;
  return hipSuccess;
}
hipError_t hipFree(void* p) {
  if (p) ++g_frees;
  return hipSuccess;
}
}

namespace fa {
static bool g_decode_may_launch = false;
static int g_decode_launches = 0;
static float* g_last_ws = nullptr;
static float* const kFakeScratch = (float*)((uintptr_t)1 << 45);
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "launcher %s reached from a call that should have failed validation\n", what);
  std::abort();
}
hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, float*, int, int, int, int, bool, float,
                           hipStream_t) { reached("fwd_bf16"); }
hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, int, int, int, int, bool, float,
                          hipStream_t) { reached("fwd_f32"); }
hipError_t launch_fwd_fp8(const void*, const void*, const void*, void*, float*, int, int, int, int, bool, float,
                          float, float, float, hipStream_t) { reached("fwd_fp8"); }
hipError_t launch_decode(const void*, const void*, const void*, void*, float* ws, int, int, int, int, int, int,
                         hipStream_t) {
  if (!g_decode_may_launch) reached("decode");
  ++g_decode_launches;
  g_last_ws = ws;
  return hipSuccess;
}
hipError_t decode_scratch(float** ptr) {
  if (!g_decode_may_launch) reached("decode_scratch");
  *ptr = kFakeScratch;
  return hipSuccess;
}
hipError_t launch_decode_paged(const void*, const void*, const void*, const int*, const int*, void*, float*, int, int,
                               int, int, int, int, int, int, hipStream_t) { reached("decode_paged"); }
// the backward workspace rows: N rounded up to a multiple of 64 (the documented size)
int bwd_rows_padded(int N) { return (N + 63) / 64 * 64; }
hipError_t launch_bwd(const void*, const void*, const void*, const void*, const void*, const float*, void*, void*,
                      void*, float*, int, int, int, int, bool, float, hipStream_t) { reached("bwd"); }
hipError_t launch_naive(const void*, const void*, const void*, void*, float*, float*, int, int, int, int, bool, float,
                        hipStream_t) { reached("naive"); }
}  // namespace fa

static int failures = 0;
#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const int got_ = (call);                                                                            \
    if (got_ != (want)) {                                                                               \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                                       \
    }                                                                                                   \
  } while (0)

int main() {
  // fake, 16-byte aligned, never dereferenced addresses (1 MiB apart)
  const uintptr_t base = (uintptr_t)1 << 40;
  void* A = (void*)(base + 0x000000);
  void* Bp = (void*)(base + 0x100000);
  void* C = (void*)(base + 0x200000);
  void* Dp = (void*)(base + 0x300000);
  float* L = (float*)(base + 0x400000);
  void* W = (void*)(base + 0x500000);
  void* T = (void*)(base + 0x600000);
  void* S = (void*)(base + 0x700000);
  auto off = [](void* p, int b) { return (void*)((uintptr_t)p + b); };
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
  const int INV = FA_ERR_INVALID_ARG, UNS = FA_ERR_UNSUPPORTED;

  for (int f32 = 0; f32 < 2; ++f32) {
    auto fwd = [&](const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale) {
      return f32 ? fa_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, B, H, N, d, 1, scale,
                              nullptr)
                 : fa_fwd(q, k, v, o, lse, B, H, N, d, 1, scale, nullptr);
    };
    EXPECT(fwd(A, Bp, C, Dp, L, 1, 1, 16, 96, 0.1f), UNS);
    EXPECT(fwd(A, Bp, C, Dp, L, 1, 1, 16, 0, 0.1f), INV);
    EXPECT(fwd(nullptr, Bp, C, Dp, L, 1, 1, 16, 64, 0.1f), INV);
    EXPECT(fwd(off(A, 8), Bp, C, Dp, L, 1, 1, 16, 64, 0.1f), INV);
    EXPECT(fwd(A, Bp, C, Dp, (float*)off(L, 2), 1, 1, 16, 64, 0.1f), INV);
    EXPECT(fwd(A, Bp, C, Dp, L, -1, 1, 16, 64, 0.1f), INV);
    EXPECT(fwd(A, Bp, C, Dp, L, 1, -1, 16, 64, 0.1f), INV);
    EXPECT(fwd(A, Bp, C, Dp, L, 1, 1, -16, 64, 0.1f), INV);
    EXPECT(fwd(A, Bp, C, Dp, L, 1, 1, 16, 64, nan), INV);
    EXPECT(fwd(A, Bp, C, Dp, L, 1, 1, 16, 64, inf), INV);
    EXPECT(fwd(A, Bp, C, Dp, L, 1, 1, 16, 64, -1.f), INV);
    EXPECT(fwd(A, Bp, C, A, L, 1, 1, 16, 64, 0.1f), INV);                 // output aliases q
    EXPECT(fwd(A, Bp, C, Dp, (float*)Dp, 1, 1, 16, 64, 0.1f), INV);       // lse over the output
    EXPECT(fwd(A, Bp, C, Dp, L, 1 << 20, 1 << 12, 1 << 12, 64, 0.1f), INV);  // grid overflow
    EXPECT(fwd(A, Bp, C, Dp, L, 65536, 65536, 16, 64, 0.1f), INV);        // B * H overflows int
    EXPECT(fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 16, 64, 0.1f), FA_OK);
    EXPECT(fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 0, 64, 0.1f), FA_OK);
  }

  auto f8 = [&](const void* q, void* o, float* lse, int N, int d, float s, float qd) {
    return fa_fwd_fp8(q, Bp, C, o, lse, 1, 1, N, d, 1, s, qd, 1.f, 1.f, nullptr);
  };
  EXPECT(f8(A, Dp, L, 16, 96, 0.1f, 1.f), UNS);
  EXPECT(f8(A, Dp, L, 16, 32, 0.1f, 1.f), UNS);
  EXPECT(f8(A, Dp, L, 16, 128, nan, 1.f), INV);
  EXPECT(f8(A, Dp, L, 16, 128, 0.1f, -1.f), INV);
  EXPECT(f8(A, Dp, L, 16, 128, 0.1f, inf), INV);
  EXPECT(f8(nullptr, Dp, L, 16, 128, 0.1f, 1.f), INV);
  EXPECT(f8(A, A, L, 16, 128, 0.1f, 1.f), INV);
  EXPECT(f8(A, Dp, (float*)A, 16, 128, 0.1f, 1.f), INV);
  EXPECT(f8(A, Dp, L, -3, 128, 0.1f, 1.f), INV);
  EXPECT(fa_fwd_fp8(nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 0, 128, 1, 0.1f, 1.f, 1.f, 1.f, nullptr),
         FA_OK);

  EXPECT(fa_decode(A, Bp, C, Dp, 2, 2, 100, 80, 4, nullptr), UNS);
  EXPECT(fa_decode(A, Bp, C, Dp, 2, 2, 0, 128, 4, nullptr), INV);
  EXPECT(fa_decode(A, Bp, C, Dp, 2, 2, 100, 128, 0, nullptr), INV);
  EXPECT(fa_decode(A, Bp, C, Dp, 2, 2, 100, 128, -5, nullptr), INV);
  EXPECT(fa_decode(nullptr, Bp, C, Dp, 2, 2, 100, 128, 4, nullptr), INV);
  EXPECT(fa_decode(A, Bp, off(C, 4), Dp, 2, 2, 100, 128, 4, nullptr), INV);
  EXPECT(fa_decode(A, Bp, C, Bp, 2, 2, 100, 128, 4, nullptr), INV);
  EXPECT(fa_decode(nullptr, nullptr, nullptr, nullptr, 0, 2, 100, 128, 4, nullptr), FA_OK);

  auto pg = [&](void* o, const void* table, const void* lens, int page, int num_pages, int max_pages, int nsplit) {
    return fa_decode_paged(A, Bp, C, (const int32_t*)table, (const int32_t*)lens, o, 2, 2, 128, page, num_pages,
                           max_pages, nsplit, nullptr);
  };
  for (int bad_page : {0, -16, 12, 3, 1 << 17}) EXPECT(pg(Dp, T, S, bad_page, 8, 4, 4), INV);
  EXPECT(pg(Dp, T, S, 16, 0, 4, 4), INV);
  EXPECT(pg(Dp, T, S, 16, 8, 0, 4), INV);
  EXPECT(pg(Dp, T, S, 16, 8, 4, 0), INV);
  EXPECT(pg(Dp, T, S, 1 << 15, 8, 1 << 16, 4), INV);
  EXPECT(pg(Dp, nullptr, S, 16, 8, 4, 4), INV);
  EXPECT(pg(Dp, off(T, 2), S, 16, 8, 4, 4), INV);
  EXPECT(pg(T, T, S, 16, 8, 4, 4), INV);
  EXPECT(pg(off(Bp, 64), T, S, 16, 8, 4, 4), INV);
  EXPECT(fa_decode_paged(A, Bp, C, (const int32_t*)T, (const int32_t*)S, Dp, 2, 2, 64 + 16, 16, 8, 4, 4, nullptr),
         UNS);

  auto bw = [&](void* dq, void* ws, size_t wsb, int N) {
    return fa_bwd(A, Bp, C, Dp, W, L, dq, T, S, 1, 2, N, 128, 1, 0.1f, ws, wsb, nullptr);
  };
  const size_t need = fa_bwd_workspace_bytes(1, 2, 100);
  void* WS = (void*)(base + 0x900000);
  void* DQ = (void*)(base + 0x800000);
  EXPECT(bw(DQ, nullptr, need, 100), INV);
  EXPECT(bw(DQ, WS, need - 4, 100), INV);
  EXPECT(bw(nullptr, WS, need, 100), INV);
  EXPECT(bw(A, WS, need, 100), INV);                                      // dq over q
  EXPECT(bw(DQ, L, need, 100), INV);                                     // workspace over lse
  EXPECT(bw(off(DQ, 2), WS, need, 100), INV);
  EXPECT(fa_bwd(A, Bp, C, Dp, W, L, DQ, T, S, 1, 2, 100, 96, 1, 0.1f, WS, need, nullptr), UNS);
  EXPECT(fa_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 2, 100, 128, 1,
                0.1f, nullptr, 0, nullptr),
         FA_OK);

  // the backward's row-statistics grid (d/8 lanes per padded row) past 2^31 - 1 workgroups, with
  // B*H*ceil(N/64) still inside an int; tensors 2^43 bytes apart so that nothing overlaps
  {
    const uintptr_t g = (uintptr_t)1 << 43;
    auto P = [&](int i) { return (void*)(g * (uintptr_t)(i + 1)); };
    const int Hb = 1 << 16, Nb = 1 << 20;
    EXPECT(fa_bwd(P(0), P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), 1, Hb, Nb, 64, 1, 0.1f, P(9),
                  fa_bwd_workspace_bytes(1, Hb, Nb), nullptr),
           INV);
    EXPECT((int)(fa_bwd_workspace_bytes(1, 1, 2147483647) == 0), 1);
  }

  // fa_decode_noalloc: fa_decode's validation, then the fixed array's limit
  EXPECT(fa_decode_noalloc(A, Bp, C, Dp, 2, 2, 100, 80, 4, nullptr), UNS);
  EXPECT(fa_decode_noalloc(A, Bp, C, Dp, 2, 2, 0, 128, 4, nullptr), INV);
  EXPECT(fa_decode_noalloc(nullptr, Bp, C, Dp, 2, 2, 100, 128, 4, nullptr), INV);
  EXPECT(fa_decode_noalloc(A, Bp, off(C, 4), Dp, 2, 2, 100, 128, 4, nullptr), INV);
  EXPECT(fa_decode_noalloc(A, Bp, C, Bp, 2, 2, 100, 128, 4, nullptr), INV);
  EXPECT(fa_decode_noalloc(nullptr, nullptr, nullptr, nullptr, 0, 2, 100, 128, 4, nullptr), FA_OK);
  {
    // 64*32 heads, 64 splits, d = 128: 68,157,440 bytes of partials > 32 MiB (caches 2^40 bytes apart)
    const uintptr_t g = (uintptr_t)1 << 40;
    EXPECT(fa_decode_noalloc((void*)g, (void*)(2 * g), (void*)(3 * g), (void*)(4 * g), 64, 32, 64, 128, 64, nullptr),
           (int)FA_ERR_TOO_LARGE);
  }

  // forced allocation failure of the decode workspace: FA_ERR_NOMEM, nothing launched
  // (q, caches and o 2^40 bytes apart, so that larger caches do not overlap)
  void* QF = (void*)((uintptr_t)1 << 40);
  void* KF = (void*)((uintptr_t)2 << 40);
  void* VF = (void*)((uintptr_t)3 << 40);
  void* OF = (void*)((uintptr_t)4 << 40);
  fa::g_decode_may_launch = true;
  g_malloc_fails = true;
  EXPECT(fa_decode(QF, KF, VF, OF, 2, 2, 100, 128, 4, nullptr), (int)FA_ERR_NOMEM);
  EXPECT(fa_decode_paged(A, Bp, C, (const int32_t*)T, (const int32_t*)S, Dp, 2, 2, 128, 16, 8, 4, 4, nullptr),
         (int)FA_ERR_NOMEM);
  EXPECT(fa::g_decode_launches, 0);
  EXPECT(g_mallocs, 0);
  // a first buffer, then a growth whose allocation fails: the old buffer is released once (after
  // the stream is synchronised) and nothing is launched; the next call allocates afresh
  g_malloc_fails = false;
  EXPECT(fa_decode(QF, KF, VF, OF, 2, 2, 100, 128, 4, nullptr), FA_OK);
  EXPECT(fa::g_decode_launches, 1);
  EXPECT(g_mallocs, 1);
  g_malloc_fails = true;
  EXPECT(fa_decode(QF, KF, VF, OF, 2, 2, 4000, 128, 64, nullptr), (int)FA_ERR_NOMEM);
  EXPECT(fa::g_decode_launches, 1);
  EXPECT(g_syncs, 1);
  EXPECT(g_frees, 1);
  EXPECT(fa_decode(QF, KF, VF, OF, 2, 2, 100, 128, 4, nullptr), (int)FA_ERR_NOMEM);  // nothing left to reuse
  g_malloc_fails = false;
  EXPECT(fa_decode(QF, KF, VF, OF, 2, 2, 100, 128, 4, nullptr), FA_OK);
  EXPECT(fa::g_decode_launches, 2);
  EXPECT(g_mallocs, 2);
  // the no-allocation entry point takes the fixed array and never allocates
  EXPECT(fa_decode_noalloc(QF, KF, VF, OF, 16, 32, 32768, 128, 64, nullptr), FA_OK);
  EXPECT(fa::g_decode_launches, 3);
  EXPECT((int)(fa::g_last_ws == fa::kFakeScratch), 1);
  EXPECT(g_mallocs, 2);
  fa_shutdown();
  EXPECT(g_frees, 2);
  fa_shutdown();  // twice: nothing left to free
  EXPECT(g_frees, 2);
  fa::g_decode_may_launch = false;

  const size_t nw = fa_naive_workspace_bytes(1, 1, 16);
  EXPECT(fa_naive_fwd(A, Bp, C, Dp, L, 1, 1, 16, 64, 0, 0.1f, W, nw - 4, nullptr), INV);
  EXPECT(fa_naive_fwd(A, Bp, C, Dp, L, 1, 1, 16, 64, 0, 0.1f, nullptr, nw, nullptr), INV);
  EXPECT(fa_naive_fwd(A, Bp, C, Dp, L, 1, 1, 16, 96, 0, 0.1f, W, nw, nullptr), UNS);

  // sizes: zero on bad arguments, exact values otherwise, no overflow on large ones
  EXPECT((int)(fa_decode_workspace_bytes(0, 1, 10, 64, 2) == 0), 1);
  EXPECT((int)(fa_decode_workspace_bytes(16, 32, 32768, 128, 64) == 17039360), 1);
  EXPECT((int)(fa_bwd_workspace_bytes(1, 1, -1) == 0), 1);
  EXPECT((int)(fa_bwd_workspace_bytes(1, 32, 8192) == 2u * 32 * 8192 * 4), 1);
  EXPECT((int)(fa_naive_workspace_bytes(1, 1, 0) == 0), 1);
  EXPECT((int)(fa_naive_workspace_bytes(4, 32, 131072) == (size_t)4 * 32 * 131072 * 131072 * 4), 1);
  for (int st : {(int)FA_OK, INV, UNS, (int)FA_ERR_HIP, (int)FA_ERR_NOMEM, (int)FA_ERR_TOO_LARGE, -99})
    if (fa_status_str(st) == nullptr) ++failures;

  if (failures) {
    std::fprintf(stderr, "%d validation checks failed\n", failures);
    return 1;
  }
  std::printf("all validation paths returned the expected status\n");
  return 0;
}
