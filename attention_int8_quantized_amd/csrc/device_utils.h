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

// Exact int8 -> fp16 for two codes (the trick described in "hip: gfx12 (RDNA4)
// WMMA kernel for the int8-KV QSA prompt attention", How): v_perm_b32 places
// two code bytes in the low byte of each 16-bit half with zero high bytes; xor
// with 0x64806480 flips each code's sign bit and sets the fp16 exponent field
// of 1024, so each half reads 1024 + (code + 128); one packed subtraction of
// 1152 leaves the code.  Every step is exact for all 256 byte values.
//
// `sel` is a v_perm_b32 selector whose bytes 1 and 3 are 0x0c (zero) and whose
// bytes 0 and 2 pick code bytes from the 8-byte value {src_hi : src_lo}.
__device__ __forceinline__ half2_t codes_to_f16(uint32_t src_hi, uint32_t src_lo, uint32_t sel) {
  const uint32_t x = __builtin_amdgcn_perm(src_hi, src_lo, sel) ^ 0x64806480u;
  const half2_t h = __builtin_bit_cast(half2_t, x);
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  return h - bias;
}

// Four codes of one dword -> four fp16 values, in byte order.
__device__ __forceinline__ half4_t dword_codes_to_f16(uint32_t w) {
  const half2_t a = codes_to_f16(0u, w, 0x0c010c00u);
  const half2_t b = codes_to_f16(0u, w, 0x0c030c02u);
  return (half4_t){a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ half_t f16_from_bits(uint16_t b) {
  return __builtin_bit_cast(half_t, b);
}

__device__ __forceinline__ float wave_max_groups(float x) {
  // max across the four 16-lane groups (lanes l, l^16, l^32, l^48)
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float wave_sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

}  // namespace attnq8
