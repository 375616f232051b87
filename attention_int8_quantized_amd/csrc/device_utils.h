// Device helpers for the gfx950 (CDNA4, wave64) attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq8 {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// A raw (unswizzled, stride 0) buffer resource over [base, base + bytes):
// loads at offsets >= bytes return zero and access no memory.  The third
// descriptor word is the gfx9 data-format setting for raw 32-bit access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Exact int8 -> fp16 of four codes (the trick described in "hip: gfx12 (RDNA4)
// WMMA kernel for the int8-KV QSA prompt attention", How, in a gfx9 form): xor
// 0x80 turns each signed code c into the byte c + 128; v_perm_b32 places two
// such bytes under an exponent byte 0x64, so each 16-bit half reads
// 1024 + (c + 128) as fp16; one packed subtraction of 1152 leaves c.  Every
// step is exact for all 256 byte values.
__device__ __forceinline__ half4_t dword_codes_to_f16(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // [c0, c1]
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // [c2, c3]
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  const half2_t a = __builtin_bit_cast(half2_t, lo) - bias;
  const half2_t b = __builtin_bit_cast(half2_t, hi) - bias;
  return (half4_t){a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ half8_t codes8_to_f16(uint32_t w0, uint32_t w1) {
  const half4_t a = dword_codes_to_f16(w0);
  const half4_t b = dword_codes_to_f16(w1);
  return (half8_t){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Direct-to-LDS loads.  `lds_addr` (wave-uniform) receives 16 (or 4) bytes per
// lane at lds_addr + 16 * lane (4 * lane) from the lane's buffer offset; an
// offset past the resource's range stores zeros.  They are issued through
// inline assembly so that the compiler does not serialise later LDS reads
// behind them: completion is tracked by the caller with wait_vmcnt<N>().
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ half_t f16_from_bits(uint16_t b) {
  return __builtin_bit_cast(half_t, b);
}

__device__ __forceinline__ float wave_max_groups(float x) {
  // max across the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
  // gfx950 lane swaps: a swap of a register with itself returns, per lane,
  // the lane's own value and its partner's (l^16, then l^32), in some order
  uint32_t u = __float_as_uint(x);
  auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  u = __float_as_uint(x);
  auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// max over all 64 lanes: DPP within rows of 16 (lane ^ 1, lane ^ 2, the
// half-row mirror i <-> 7 - i, the row mirror i <-> 15 - i), then the row
// swaps of wave_max_groups; every lane returns the same value
__device__ __forceinline__ float wave_max_all(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
  return wave_max_groups(x);
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

}  // namespace attnq8
