// Device-side building blocks shared by the gfx950 kernels: vector types, the
// direct global -> LDS loads with the waits and barriers that order them, and
// small wavefront helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace fa2 {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr_t;
typedef __attribute__((address_space(1))) const void* global_ptr_t;


constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Word 3 of a raw buffer resource on this GPU family (stride 0, 32-bit data).
constexpr int kBufferFlags = 0x00020000;

// Value of x combined with the one held 32 lanes away (the two lane halves of
// a 32x32 MFMA tile hold different keys of the same query row).
// v_permlane32_swap swaps the upper 32 lanes of its first operand with the
// lower 32 lanes of its second; with x in both, lane l < 32 ends with (x[l],
// x[l+32]) and lane l >= 32 with (x[l-32], x[l]), so every lane holds its own
// value and its partner's, and max or sum of the two is the same in both
// halves.  Inline assembly with both registers read and written: the compiler
// builtin, given the same value twice, has its two results taken for one
// register (r0 - r1 compiles to v - v).  The s_nop gives the two wait states a
// VALU write needs before the swap reads its operands.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float halves_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_halves(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float halves_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_halves(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Direct global -> LDS loads of 16 bytes per lane (lane i fills LDS bytes
// lds + 16i .. +16), and the waits and barriers that order them.  They are
// inline assembly on purpose: the compiler treats every LDS read that follows
// a direct load it knows about as a possible reader of that load and waits for
// all of them, which would cut the prefetch distance to a fraction of a block.
// The kernel orders these loads itself (vmcnt waits, then a barrier), and the
// memory clobbers keep the compiler from moving LDS accesses across them.
__device__ __forceinline__ void lds_dma(const void* base, uint32_t voff, uint32_t lds) {
  // address = base (scalar) + voff (per lane)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               : : "s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma(const void* addr, uint32_t lds) {
  // address = addr (per lane)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               : : "s"(lds), "v"(addr) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}
// Wait until at most N vector-memory operations of this wavefront are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// The lane index, recomputed where it is used: values derived from it that
// only the masked or ragged-tail paths need are then not kept in registers
// across the whole KV loop.
__device__ __forceinline__ int fresh_lane() {
  int l = (int)threadIdx.x;
  asm volatile("" : "+v"(l));
  return l & 63;
}
// Workgroup barrier after this wavefront's own LDS accesses have completed.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// The two 16-bit input types: their 8- and 4-element vectors and the 32x32x16
// MFMA that multiplies them (fp32 accumulation for both).
template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
  typedef bf16x8_t x8;
  typedef bf16x4_t x4;
};
template <> struct Vec16<_Float16> {
  typedef f16x8_t x8;
  typedef f16x4_t x4;
};
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32x32x16(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
}  // namespace dev
}  // namespace fa2
