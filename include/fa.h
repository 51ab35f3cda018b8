/*
 * fa.h -- C ABI of an MI355X (gfx950) library for exact scaled-dot-product
 * attention: a fused, tiled forward pass with online softmax (prefill), a
 * split-KV decode with a max-and-sum merge, and a deliberately naive
 * three-kernel path kept for comparison.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major and contiguous. Q, K, V and O are [B, H, N, d]
 *   with d contiguous; LSE is [B, H, N] float32. Decode Q and O are [B, H, d],
 *   the caches [B, H, Lkv, d].
 * - All tensor pointers are DEVICE pointers owned by the caller. The library
 *   never frees them and never keeps them past the call. Every tensor pointer
 *   must be 16-byte aligned.
 * - `stream` is a hipStream_t (NULL = the legacy default stream) on the current
 *   device. Calls only enqueue work and return; results are ready once the
 *   caller synchronises with that stream. Errors raised while the kernels run
 *   surface at that synchronisation, not in the return value.
 * - Arguments are fully validated before anything is enqueued: a call that
 *   returns an error has had no device side effects.
 * - Sizes are int; every element offset is computed in 64-bit.
 * - A size of zero (B, H or N equal to 0) is an empty problem: the call returns
 *   FA_OK and enqueues nothing (pointers may then be NULL).
 * - Return value: FA_OK (0) or a negative FA_ERR_* code; fa_status_str()
 *   names it. After FA_ERR_HIP, fa_last_hip_error() returns the hipError_t.
 *
 * The method is described on "Describe Flash Attention at a high level"
 * (mantramindai.in) and "How FlashAttention Speeds Up the Attention Layer"
 * (hassanahmed.net). The pages give no programming interface; they only say
 * the kernel is normally reached through a framework.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null or misaligned pointer, negative size, bad scale or nsplit */
  FA_ERR_UNSUPPORTED = -2, /* head dimension d other than 64 or 128 */
  FA_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  FA_ERR_NOMEM = -4,       /* the library could not allocate its decode workspace */
  FA_ERR_TOO_LARGE = -5    /* the problem needs more than the fixed FA_DECODE_SCRATCH_BYTES */
};

/*
 * fa_fwd -- fused exact attention forward, bf16 inputs and output.
 *
 * O = softmax(scale * Q K^T [+ causal mask]) V, computed per query tile in one
 * pass over the key tiles with the online-softmax recurrence (running row max,
 * running sum, output rescaled by exp(m_old - m_new) when the max rises), so
 * the N x N score matrix is never written to memory. Sources: mantramindai.in,
 * section "The two ideas" (tiling, online softmax); hassanahmed.net, the
 * sections on tiling and on the online softmax.
 *
 *   q, k, v  const bf16 [B,H,N,d]; o: bf16 [B,H,N,d] (may not alias q, k, v)
 *   lse      float32 [B,H,N], natural-log log-sum-exp of each row's scaled
 *            logits over its visible keys; NULL = not written; may not
 *            overlap q, k, v or o
 *   causal   nonzero: key j is visible to query i iff j <= i
 *   scale    multiplier of the logits; must be finite and >= 0
 *   d        64 or 128 (else FA_ERR_UNSUPPORTED)
 * Arithmetic: bf16 MFMA products with fp32 accumulation; softmax in fp32; the
 * probabilities are rounded to bf16 (round to nearest even) for the P V
 * product; O is divided by the row sum in fp32 and rounded once to bf16.
 * The dot products and the scaled logits are fp32 values: a row whose logits
 * (scale * q.k, in base-2 units) leave the fp32 range gets non-finite outputs.
 * Uses no workspace and allocates nothing.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_fwd_f32 -- the same operation as fa_fwd with float32 Q, K, V and O, and
 * float32 arithmetic throughout (no bf16 rounding anywhere). Same arguments,
 * layouts and errors as fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_fwd_fp8 -- the fused forward with FP8 inputs on the FP8 matrix cores, the
 * FlashAttention-3 FP8 mode that hassanahmed.net (the section on later
 * versions) and mantramindai.in (the paragraph on FA-3) mention. The pages fix
 * no scaling convention; here each input tensor carries one float descale
 * factor, so the logical inputs are q_descale * Q, k_descale * K and
 * v_descale * V, and the output is attention of those (same mask and LSE
 * definition as fa_fwd).
 *
 *   q, k, v     const FP8 e4m3 (OCP "fn" encoding, 1 byte) [B,H,N,d]
 *   o           bf16 [B,H,N,d]
 *   lse         float32 [B,H,N] or NULL: natural-log LSE of the scaled logits
 *   d           64 or 128 (FA_ERR_UNSUPPORTED otherwise)
 *   scale, q_descale, k_descale, v_descale: finite and >= 0
 * Arithmetic: Q K^T on FP8 MFMAs with fp32 accumulation; the probabilities
 * are rounded to e4m3 (nearest even, after an exact power-of-two scaling that
 * keeps them in e4m3's normal range) for the P V product; the row sums use
 * the fp32 probabilities; O is rounded once to bf16. Each probability carries
 * a relative error of at most 2^-4, so |O - exact| <= (2^-4 + 2^-8) max|V|.
 * Errors and alignment as fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale,
               float q_descale, float k_descale, float v_descale, void* stream);

/*
 * fa_decode -- attention of one new query row per (b, h) over a whole KV cache,
 * split across workgroups (Flash-Decoding): the cache is cut into nsplit chunks
 * of ceil(Lkv/nsplit) keys; each chunk yields its max, its sum of exponentials
 * and its unnormalised output; a second kernel merges the chunks with the same
 * max-and-sum rule as the online softmax. Source: mantramindai.in, section
 * "Follow-up questions to expect", the question on decode.
 *
 *   q               const bf16 [B,H,d]
 *   kcache, vcache  const bf16 [B,H,Lkv,d]
 *   o               bf16 [B,H,d]
 *   Lkv             >= 1 (no mask: every cached key is visible)
 *   nsplit          >= 1; clamped so that no chunk is empty
 *   d               64 or 128
 * The logit scale is 1/sqrt(d) (rounded to float32).
 * Workspace: the library owns one float32 partials buffer per (device, stream),
 * grown on demand (hipMalloc) and freed by fa_shutdown(); growing it first
 * synchronises `stream`. Calls on one stream are ordered; calls on different
 * streams use different buffers. FA_ERR_NOMEM if the buffer cannot be grown.
 */
int fa_decode(const void* q, const void* kcache, const void* vcache, void* o,
              int B, int H, int Lkv, int d, int nsplit, void* stream);

/* Bytes of decode partials for this shape (the buffer fa_decode keeps). */
size_t fa_decode_workspace_bytes(int B, int H, int Lkv, int d, int nsplit);

/* Size of the fixed per-device decode-partials array of fa_decode_noalloc. */
#define FA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. Same operation, arguments, layouts, kernels and
 * results as fa_decode (bit for bit), but the partials live in a fixed
 * device array of FA_DECODE_SCRATCH_BYTES bytes that the library holds on
 * every GPU it runs on until the process ends. The call never allocates,
 * frees or synchronises; on its first call on a device it looks up that
 * device's array address (no allocation).
 *
 * Limit: fa_decode_workspace_bytes(B, H, Lkv, d, nsplit) must not exceed
 * FA_DECODE_SCRATCH_BYTES (32 MiB: e.g. B*H = 1024 heads at d = 128 with 64
 * splits need 17,039,360 bytes), else FA_ERR_TOO_LARGE before anything is
 * enqueued. Every call on one GPU shares that GPU's array, so calls that may
 * overlap in time on one GPU (different streams without ordering between
 * them) race: order them, or use fa_decode. Nothing in the array needs
 * clearing: each split writes its whole partial before the merge reads it.
 * Other errors as fa_decode (never FA_ERR_NOMEM).
 */
int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, void* o,
                      int B, int H, int Lkv, int d, int nsplit, void* stream);

/*
 * fa_decode_paged -- fa_decode over a paged KV cache: the keys of each
 * sequence live in fixed-size pages of a shared pool, found through a block
 * table, as the decode kernels of serving engines keep them. Sources:
 * mantramindai.in, the paragraph on how the kernel is reached through
 * frameworks (paged variants for decode); appliedaiprep.com, the follow-up on
 * long-context serving. The pages give no layout; this one keeps each
 * (page, head) contiguous.
 *
 *   q               const bf16 [B,H,d]
 *   k_pages,
 *   v_pages         const bf16 [num_pages, H, page_size, d] (the pools)
 *   block_table     const int32 [B, max_pages], device memory: key j of
 *                   sequence b is row j % page_size of pool page
 *                   block_table[b][j / page_size]; entries past a sequence's
 *                   last page are never read
 *   seq_lens        const int32 [B], device memory: keys per sequence, in
 *                   [0, max_pages * page_size]
 *   o               bf16 [B,H,d]
 *   page_size       a power of two, 1 .. 65536
 *   num_pages, max_pages, nsplit >= 1; max_pages * page_size <= 2^30
 *   d               64 or 128
 * The cache is split as fa_decode splits a cache of Lkv = max_pages *
 * page_size keys; splits past a sequence's length contribute nothing. The
 * logit scale is 1/sqrt(d) (rounded to float32). Values that live in device
 * memory are checked by the kernels, which never read outside the pool or the
 * table: a sequence of length 0 gives o = 0; a length outside the range, or a
 * page id outside [0, num_pages) among a sequence's pages, gives NaN in that
 * sequence's rows of o. Host-side arguments are checked as in fa_decode;
 * overlap of o with any input is FA_ERR_INVALID_ARG. Workspace: the same
 * library-owned buffer as fa_decode, fa_decode_workspace_bytes(B, H,
 * max_pages * page_size, d, nsplit) bytes.
 */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                    const int32_t* seq_lens, void* o, int B, int H, int d, int page_size, int num_pages,
                    int max_pages, int nsplit, void* stream);

/*
 * fa_bwd -- gradients of fa_fwd with respect to Q, K and V, computed with the
 * recompute method: the score tiles are rebuilt from Q, K and the forward's
 * LSE instead of being stored. Sources: mantramindai.in, section "The two
 * ideas", item 3 (recompute in backward); hassanahmed.net, the paragraph on
 * training. The gradient is the chain rule of the definition (P = softmax of
 * the scaled, masked logits): dV = P^T dO; dS = P * (dO V^T - rowsum(dO * O));
 * dQ = scale dS K; dK = scale dS^T Q.
 *
 *   q, k, v, o  const bf16 [B,H,N,d]: the forward's inputs and output
 *   dout        const bf16 [B,H,N,d]: dL/dO
 *   lse         const float32 [B,H,N]: the LSE fa_fwd wrote for the same call
 *   dq, dk, dv  bf16 [B,H,N,d] outputs; may not alias any input or each other
 *   B, H, N, d, causal, scale: as passed to fa_fwd
 *   workspace   caller-owned device buffer of at least
 *               fa_bwd_workspace_bytes(B,H,N) bytes (float32 row statistics;
 *               contents on entry are ignored), 16-byte aligned
 * Arithmetic: bf16 MFMA products, fp32 accumulation; P and dS are rounded to
 * bf16 (nearest even) as MFMA operands; dq, dk, dv are rounded once to bf16.
 * The result is deterministic (no atomics). Errors as fa_fwd; a workspace that
 * is NULL, misaligned or too small gives FA_ERR_INVALID_ARG.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of backward workspace: 2 * B*H*ceil(N/64)*64 * 4 (0 on bad sizes). */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_naive_fwd -- the three-step attention of the pages, kept as an ablation:
 * kernel 1 writes S = scale * Q K^T (masked entries -inf) to `workspace` as
 * float32 [B,H,N,N]; kernel 2 turns each row into softmax probabilities in
 * place and writes LSE; kernel 3 reads P back and writes O = P V. The N x N
 * matrix makes every step an HBM round trip. Sources: mantramindai.in,
 * section "What naive attention does"; hassanahmed.net, the three-step
 * formulation.
 *
 * Same q, k, v, o, lse, B, H, N, d, causal, scale as fa_fwd (bf16 inputs and
 * output; S, P and the products in float32). `workspace` is a caller-owned
 * device buffer of at least fa_naive_workspace_bytes(B,H,N) bytes, passed in
 * `workspace_bytes` (too small: FA_ERR_INVALID_ARG).
 */
int fa_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale,
                 void* workspace, size_t workspace_bytes, void* stream);

/* B*H*N*N*4 bytes: one float32 score matrix per head. 0 on overflow or bad sizes. */
size_t fa_naive_workspace_bytes(int B, int H, int N);

/* Static, NUL-terminated name of a status code ("FA_OK", ...). */
const char* fa_status_str(int status);

/* The hipError_t behind the most recent FA_ERR_HIP on this thread (0 if none). */
int fa_last_hip_error(void);

/* Frees every decode workspace the library owns (on all devices). Safe to call
 * more than once; later fa_decode calls allocate again. */
void fa_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
