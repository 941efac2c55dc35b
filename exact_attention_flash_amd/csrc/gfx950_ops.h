// Device building blocks for the gfx950 attention kernels: vector types, the
// 32x32x16 MFMA, 16-bit packing, LDS reads (plain and transposing), buffer
// descriptors and loads (to registers and straight to LDS), the 16-byte chunk
// swizzle shared by every tile kept in LDS, and the vector-memory wait.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace ops {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kBufferConfig = 0x00020000u;  // raw buffer descriptor word 3 (gfx9 family)

// XOR swizzle of the 16-byte chunk index within a row of a row-major tile of
// D-element rows: row-major 16-row reads of 16 bytes per lane (the MFMA A/B
// operand pattern) and the transposing reads of 4 rows each hit every LDS bank
// once.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <bool FP16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (FP16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
}

template <bool FP16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (FP16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 lds_read16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kBufferConfig);
}

// Buffer descriptor from a wave-uniform base address and range, forced into scalar
// registers as the descriptor operand of a load requires (free when they already
// are; needed where the compiler cannot prove a value built under a branch on the
// wave index uniform).
// A wave-uniform copy of an address in scalar registers. readfirstlane yields an
// int: each half goes through uint32_t before the halves are joined, because a
// signed low half would be sign-extended over the high half whenever its bit 31 is
// set (an unmapped address for every buffer placed there).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  return buffer_rsrc(uniform_ptr(base), __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// 16 bytes per lane from the buffer straight into LDS at lds_base + 16 * lane
// (buffer_load_dwordx4 ... lds; M0 holds the wave-uniform LDS base). Written as
// inline assembly so that the compiler does not treat every later LDS read as
// possibly aliasing the in-flight copy (it would then wait for all outstanding
// loads, tiles prefetched for later iterations included); completion is instead
// awaited explicitly with wait_vmcnt before the barrier that publishes a tile.
// M0 takes the LDS byte address, the low 32 bits of a generic pointer into LDS
// (the cast to the LDS address space would add a null-pointer select). The load
// reads scalar registers that the VALU may have just written: the descriptor and
// M0 come from v_readfirstlane. A vector-memory instruction needs five wait states
// after a VALU write of an SGPR it reads (and one after a write of M0); the
// compiler inserts them for its own loads (s_nop 2 after a readfirstlane-built
// descriptor and two other instructions) but cannot see the reads inside this asm,
// so the s_nop 4 supplies all five. Without it, a wave issuing eight of these loads
// in a row fetched wrong data for some of them.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, char* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(m0) : "memory");
}

// The same load with the LDS byte address given as a wave-uniform 32-bit value that
// the scalar unit computed (the caller keeps its parts in scalar registers). A load
// to LDS may follow a scalar write of M0 after one wait state (s_nop 0); neither the
// descriptor nor M0 may have been written by a VALU instruction within five wait
// states, which the build audit checks on the generated code.
__device__ __forceinline__ void buffer_load16_lds_s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr) : "memory");
}

// 4 bytes per lane from the buffer straight into LDS at lds_base + 4 * lane
// (buffer_load_dword ... lds); completion awaited with wait_vmcnt like the 16-byte form.
__device__ __forceinline__ void buffer_load4_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, char* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(m0) : "memory");
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: expcnt and lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace ops
}  // namespace fa
