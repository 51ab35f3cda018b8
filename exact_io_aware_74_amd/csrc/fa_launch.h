// Host-side launchers of the attention kernels (internal to the library; the
// public surface is the C ABI in fa.h). Arguments are assumed validated.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

// Heads per group of the forward kernels' workgroup order, for workgroups of
// `waves` waves x 32 query rows (n_qt query tiles per head). One group (all
// heads interleaved) keeps the heaviest causal tiles of every head first,
// which packs the workgroups best, but each XCD then streams the K/V of BH / 8
// heads at once. Where that is 8 heads or more (and heads have 16 or more
// query tiles), or a head's K/V alone is far beyond an XCD's L2 (128 or more
// query tiles), groups of 16 heads (two per XCD at a time) let the workgroups
// of an XCD share K/V tiles in its L2. Four-wave workgroups (the small-grid
// path) keep one group: all of them are resident at once, two per CU.
inline int head_group(int waves, int BH, int n_qt) {
  if (waves == 8 && ((BH >= 64 && n_qt >= 16) || n_qt >= 128)) return 16 < BH ? 16 : BH;
  return BH;
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, bool causal, float scale, hipStream_t s);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int N, int d, bool causal, float scale, hipStream_t s);

// FP8 (e4m3) forward, d = 128: the logical inputs are descale * tensor.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                          int d, bool causal, float scale, float q_descale, float k_descale, float v_descale,
                          hipStream_t s);

// Decode: `chunk` keys per split, `nsplit` splits (every split non-empty).
// `ws` holds B*H*nsplit*(d+2) floats.
hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* o, float* ws,
                         int B, int H, int Lkv, int d, int nsplit, int chunk, hipStream_t s);

// The device address of this device's fixed decode-partials array
// (FA_DECODE_SCRATCH_BYTES bytes), looked up on the first call per device.
hipError_t decode_scratch(float** ptr);

// Paged decode: pools [num_pages, H, 2^log2_page, d], table [B, max_pages],
// lens [B] (device). Splits cover `chunk` keys of max_pages * 2^log2_page;
// splits past a sequence's length are empty. `ws` as for launch_decode.
hipError_t launch_decode_paged(const void* q, const void* kpool, const void* vpool, const int* table, const int* lens,
                               void* o, float* ws, int B, int H, int d, int log2_page, int num_pages, int max_pages,
                               int nsplit, int chunk, hipStream_t s);

// Backward with recompute: dq, dk, dv from q, k, v, o, dout and the forward's
// lse. `ws` holds 2 * B*H*bwd_rows_padded(N) floats.
int bwd_rows_padded(int N);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* ws, int B, int H, int N, int d, bool causal, float scale,
                      hipStream_t s);

// Naive three-kernel ablation; `S` holds B*H*N*N floats.
hipError_t launch_naive(const void* q, const void* k, const void* v, void* o, float* lse, float* S,
                        int B, int H, int N, int d, bool causal, float scale, hipStream_t s);

}  // namespace fa
