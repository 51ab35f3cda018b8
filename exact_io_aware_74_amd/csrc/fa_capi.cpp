// C ABI of the attention library (declared in include/fa.h): argument
// validation, kernel dispatch and the decode workspace. Every check runs
// before anything is enqueued, so a call that fails has no device effects.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "fa.h"
#include "fa_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Shared checks of the forward entry points. Returns FA_OK, an error, or 1
// for "empty problem, nothing to do".
int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int N,
              int d, float scale, size_t elem) {
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) return 1;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_INVALID_ARG;
  // grid size: (B*H) * ceil(N/64) workgroups must fit an int
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX || bh * (((int64_t)N + 63) / 64) > INT_MAX) return FA_ERR_INVALID_ARG;
  const size_t bytes = (size_t)bh * (size_t)N * (size_t)d * elem;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
    return FA_ERR_INVALID_ARG;
  if (lse) {
    const size_t lbytes = (size_t)bh * N * 4;
    if (overlaps(lse, lbytes, o, bytes) || overlaps(lse, lbytes, q, bytes) || overlaps(lse, lbytes, k, bytes) ||
        overlaps(lse, lbytes, v, bytes))
      return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

// Decode partials: one buffer per (device, stream).
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
           float scale, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 2);
  if (st != FA_OK) return st == 1 ? FA_OK : st;
  const hipError_t e = fa::launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal != 0, scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 4);
  if (st != FA_OK) return st == 1 ? FA_OK : st;
  // the fp32 kernel runs one workgroup per four query rows: its grid must fit an int
  if ((int64_t)B * H * (((int64_t)N + 3) / 4) > INT_MAX) return FA_ERR_INVALID_ARG;
  const hipError_t e = fa::launch_fwd_f32(q, k, v, o, lse, B, H, N, d, causal != 0, scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, float q_descale, float k_descale, float v_descale, void* stream) {
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  for (float x : {scale, q_descale, k_descale, v_descale})
    if (!std::isfinite(x) || x < 0.f) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return FA_ERR_INVALID_ARG;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT_MAX || bh * (((int64_t)N + 255) / 256) > INT_MAX) return FA_ERR_INVALID_ARG;
  const size_t in_bytes = (size_t)bh * (size_t)N * (size_t)d, out_bytes = 2 * in_bytes;
  if (overlaps(o, out_bytes, q, in_bytes) || overlaps(o, out_bytes, k, in_bytes) || overlaps(o, out_bytes, v, in_bytes))
    return FA_ERR_INVALID_ARG;
  if (lse && (overlaps(lse, (size_t)bh * N * 4, o, out_bytes) || overlaps(lse, (size_t)bh * N * 4, q, in_bytes) ||
              overlaps(lse, (size_t)bh * N * 4, k, in_bytes) || overlaps(lse, (size_t)bh * N * 4, v, in_bytes)))
    return FA_ERR_INVALID_ARG;
  const hipError_t e = fa::launch_fwd_fp8(q, k, v, o, lse, B, H, N, d, causal != 0, scale, q_descale, k_descale,
                                          v_descale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

// The decode partials buffer of (current device, stream), grown to `need`
// bytes if smaller. Growing synchronises the stream first: earlier decodes on
// it may still read the old buffer.
static int decode_workspace(void* stream, size_t need, float** ws) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, (hipStream_t)stream}];
  if (w.bytes < need) {
    if (w.ptr) {
      e = hipStreamSynchronize((hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e);
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, need) != hipSuccess) {
      (void)hipGetLastError();
      w.ptr = nullptr;
      return FA_ERR_NOMEM;
    }
    w.bytes = need;
  }
  *ws = (float*)w.ptr;
  return FA_OK;
}

static void decode_split_shape(int Lkv, int nsplit, int* chunk, int* nsplit_eff) {
  const int n = nsplit < Lkv ? nsplit : Lkv;
  *chunk = (Lkv + n - 1) / n;
  *nsplit_eff = (Lkv + *chunk - 1) / *chunk;  // no empty chunk
}

size_t fa_decode_workspace_bytes(int B, int H, int Lkv, int d, int nsplit) {
  if (B <= 0 || H <= 0 || Lkv <= 0 || d <= 0 || nsplit <= 0) return 0;
  int chunk, ns;
  decode_split_shape(Lkv, nsplit, &chunk, &ns);
  return (size_t)B * (size_t)H * (size_t)ns * (size_t)(d + 2) * sizeof(float);
}

int fa_decode(const void* q, const void* kcache, const void* vcache, void* o, int B, int H, int Lkv, int d, int nsplit,
              void* stream) {
  if (B < 0 || H < 0 || Lkv <= 0 || d <= 0 || nsplit <= 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return FA_OK;
  if (!q || !kcache || !vcache || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  int chunk, ns;
  decode_split_shape(Lkv, nsplit, &chunk, &ns);
  const int64_t bh = (int64_t)B * H;
  if (bh * ns > INT_MAX) return FA_ERR_INVALID_ARG;
  const size_t qbytes = (size_t)bh * d * 2, cbytes = (size_t)bh * Lkv * d * 2;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, kcache, cbytes) || overlaps(o, qbytes, vcache, cbytes))
    return FA_ERR_INVALID_ARG;

  float* ws = nullptr;
  const int st = decode_workspace(stream, fa_decode_workspace_bytes(B, H, Lkv, d, nsplit), &ws);
  if (st != FA_OK) return st;
  const hipError_t e = fa::launch_decode(q, kcache, vcache, o, ws, B, H, Lkv, d, ns, chunk, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, void* o, int B, int H, int Lkv, int d,
                      int nsplit, void* stream) {
  if (B < 0 || H < 0 || Lkv <= 0 || d <= 0 || nsplit <= 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return FA_OK;
  if (!q || !kcache || !vcache || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  int chunk, ns;
  decode_split_shape(Lkv, nsplit, &chunk, &ns);
  const int64_t bh = (int64_t)B * H;
  if (bh * ns > INT_MAX) return FA_ERR_INVALID_ARG;
  const size_t qbytes = (size_t)bh * d * 2, cbytes = (size_t)bh * Lkv * d * 2;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, kcache, cbytes) || overlaps(o, qbytes, vcache, cbytes))
    return FA_ERR_INVALID_ARG;
  if (fa_decode_workspace_bytes(B, H, Lkv, d, nsplit) > FA_DECODE_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;

  float* ws = nullptr;
  hipError_t e = fa::decode_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e);
  e = fa::launch_decode(q, kcache, vcache, o, ws, B, H, Lkv, d, ns, chunk, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                    const int32_t* seq_lens, void* o, int B, int H, int d, int page_size, int num_pages,
                    int max_pages, int nsplit, void* stream) {
  if (B < 0 || H < 0 || d <= 0 || num_pages <= 0 || max_pages <= 0 || nsplit <= 0) return FA_ERR_INVALID_ARG;
  if (page_size <= 0 || page_size > 65536 || (page_size & (page_size - 1))) return FA_ERR_INVALID_ARG;
  if ((int64_t)max_pages * page_size > (int64_t)1 << 30) return FA_ERR_INVALID_ARG;  // key indices stay far from INT_MAX
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return FA_OK;
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)block_table & 3u) || ((uintptr_t)seq_lens & 3u)) return FA_ERR_INVALID_ARG;
  const int lmax = max_pages * page_size;
  int chunk, ns;
  decode_split_shape(lmax, nsplit, &chunk, &ns);
  const int64_t bh = (int64_t)B * H;
  if (bh * ns > INT_MAX) return FA_ERR_INVALID_ARG;
  const size_t qbytes = (size_t)bh * d * 2;
  const size_t pbytes = (size_t)num_pages * (size_t)H * (size_t)page_size * (size_t)d * 2;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k_pages, pbytes) || overlaps(o, qbytes, v_pages, pbytes) ||
      overlaps(o, qbytes, block_table, (size_t)B * max_pages * 4) || overlaps(o, qbytes, seq_lens, (size_t)B * 4))
    return FA_ERR_INVALID_ARG;
  int lps = 0;
  while ((1 << lps) < page_size) ++lps;
  float* ws = nullptr;
  const int st = decode_workspace(stream, fa_decode_workspace_bytes(B, H, lmax, d, nsplit), &ws);
  if (st != FA_OK) return st;
  const hipError_t e = fa::launch_decode_paged(q, k_pages, v_pages, block_table, seq_lens, o, ws, B, H, d, lps,
                                               num_pages, max_pages, ns, chunk, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0 || N > INT_MAX - 64) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)fa::bwd_rows_padded(N) * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 2);
  if (st != FA_OK) return st == 1 ? FA_OK : st;
  if (!dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_workspace_bytes(B, H, N);
  if (need == 0 || workspace_bytes < need) return FA_ERR_INVALID_ARG;
  // the statistics kernel runs d/8 lanes per padded row: its grid must fit
  const int64_t prep_blocks = ((int64_t)B * H * fa::bwd_rows_padded(N) * (d / 8) + 255) / 256;
  if (prep_blocks > INT_MAX) return FA_ERR_INVALID_ARG;
  const size_t bytes = (size_t)B * H * (size_t)N * (size_t)d * 2, lbytes = (size_t)B * H * (size_t)N * 4;
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (void* out : outs) {
    for (const void* in : ins)
      if (overlaps(out, bytes, in, bytes)) return FA_ERR_INVALID_ARG;
    if (overlaps(out, bytes, lse, lbytes) || overlaps(out, bytes, workspace, need)) return FA_ERR_INVALID_ARG;
  }
  if (overlaps(dq, bytes, dk, bytes) || overlaps(dq, bytes, dv, bytes) || overlaps(dk, bytes, dv, bytes))
    return FA_ERR_INVALID_ARG;
  for (const void* in : ins)
    if (overlaps(workspace, need, in, bytes)) return FA_ERR_INVALID_ARG;
  if (overlaps(workspace, need, lse, lbytes)) return FA_ERR_INVALID_ARG;
  const hipError_t e = fa::launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, d, causal != 0,
                                      scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

size_t fa_naive_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return 0;
  const unsigned __int128 b = (unsigned __int128)B * H * N * N * 4u;
  return b > (unsigned __int128)SIZE_MAX ? 0 : (size_t)b;
}

int fa_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                 int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 2);
  if (st != FA_OK) return st == 1 ? FA_OK : st;
  // one row of S is staged in LDS by the softmax kernel; grid y/z carry B*H
  if (N > 32768 || (int64_t)B * H > 65535) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_naive_workspace_bytes(B, H, N);
  if (!workspace || need == 0 || workspace_bytes < need || ((uintptr_t)workspace & 3u)) return FA_ERR_INVALID_ARG;
  const hipError_t e = fa::launch_naive(q, k, v, o, lse, (float*)workspace, B, H, N, d, causal != 0, scale,
                                        (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_NOMEM: return "FA_ERR_NOMEM";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE";
    default: return "FA_ERR_UNKNOWN";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

void fa_shutdown(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      if (hipSetDevice(kv.first.first) == hipSuccess) (void)hipFree(kv.second.ptr);
    }
  }
  g_ws.clear();
  if (have_cur) (void)hipSetDevice(cur);
}

}  // extern "C"
