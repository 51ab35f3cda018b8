// Device-side building blocks for the gfx950 attention kernels: vector types,
// bf16 conversions, the bf16 MFMA and the LDS transposing read.
//
// Lane layouts used throughout (measured on gfx950 with a layout probe):
//  * v_mfma_f32_32x32x16_bf16, D = A*B with A 32x16, B 16x32:
//      A: lane l holds row (l % 32), 8 consecutive k-slots of half (l / 32);
//      B: lane l holds column (l % 32), the same 8 k-slots of half (l / 32);
//      D: lane l, accumulator r holds row (r%4) + 8*(r/4) + 4*(l/32),
//         column l % 32.
//    A's k-slot (half h, element e) multiplies B's k-slot (h, e), so any
//    assignment of real contraction indices to slots is valid as long as A
//    and B use the same one.
//  * ds_read_b64_tr_b16, within each group of 16 lanes: lane t receives,
//    as its element e (e = 0..3), the 16-bit value at position (t % 4) of the
//    8-byte chunk addressed by lane 4*e + t/4 of its group.
//  * global_load_lds_dwordx4: lane l's 16 bytes land at the (wave-uniform)
//    LDS destination + 16*l, whatever global address the lane supplied.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

#define FA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round two floats to bf16 (round to nearest even) and pack them.
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  return __builtin_convertvector((f32x2){a, b}, bf16x2);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Transposing 8-byte LDS read (see the layout note above).
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p));
}

// 16-byte copy global -> LDS without a VGPR round trip: lane l's 16 bytes
// land at LDS byte address `lds_addr` + 16*l (`lds_addr` wave-uniform). Issued
// through asm so the compiler does not tie later LDS reads to its completion
// (it cannot tell the ring slots apart and would wait for every copy): the
// caller must wait for them (wait_vmcnt) before a barrier that publishes the
// data.
__device__ __forceinline__ void global_load_lds16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds_addr) : "memory", "m0");
}
// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset: the address math stays on the scalar unit.
__device__ __forceinline__ void global_load_lds16_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave remain
// outstanding (loads complete in issue order). Issued through the builtin so
// the compiler accounts for it in its own waits.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}
// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(FA_LDS const void*)p; }

// Reductions over the lane pair (l, l ^ 32). v_permlane32_swap on (x, x)
// returns, in lanes 0..31, (x[l], x[l+32]) and in lanes 32..63,
// (x[l-32], x[l]): both lanes of a pair see the two values in the same
// order, so both get bit-identical results.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace fa
