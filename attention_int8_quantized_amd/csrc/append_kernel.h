// Block-32 int8 quantisation of new K/V rows into the attention's cache.
//
// The cache format is the pages' Q8 KV: int8 codes in blocks of 32 consecutive
// head_dim elements with one fp16 scale per block ("perf(gfx1100): share Q8 KV
// scans across verifier rows", Summary; the Q8_0 block of "[Engine] perf(hip):
// optimize MTP draft, shared expert, and verify/sampler head kernels on RDNA4",
// Problem and result item 2, Summary item 4).  Per block:
//   scale = fp16_rne(amax / 127)              (fp32 divide, then fp16)
//   code  = clamp(round_half_away(x / scale), -127, 127)   (fp32 divide)
//   scale == 0  ->  every code 0
// The scale's divide is an IEEE fp32 divide (HIP's default division is
// correctly rounded).  The code's fp32 quotient never lands on a rounding
// boundary it did not reach exactly (an fp16 scale times k + 1/2 has at most 19
// significant bits, so any other fp32 x lies at least one of its ulps away), so
// the code is the exactly rounded |x| / scale: it is taken as
// k = floor(|x| * rcp(scale)) -- within 3e-5 of |x| / scale, so k is the floor
// of the exact quotient or one off across an integer -- plus 1 when
// |x| - (k + 1/2) * scale >= 0, a difference one fma computes with the exact
// sign ((k + 1/2) * scale is exact in fp32; equality is the tie, which goes
// away from zero); then the clamp and x's sign.  This replaces eight divides
// per lane with a reciprocal and a few multiply-adds.
//
// Mapping: a lane owns 8 consecutive elements (one 32-byte or 16-byte load), a
// quad of lanes owns a block; the block maximum is two DPP quad permutes.  The
// kernel is a pure stream (4 or 2 bytes read and 1 + 1/16 bytes written per
// element), so it is a grid-stride loop over 8-element units with coalesced
// loads and 8-byte code stores.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnq8 {

constexpr int kAppendThreads = 256;

struct AppendArgs {
  const void* x[2];      // K rows, V rows: [n_tokens][n_kv_heads][head_dim]
  int8_t* codes[2];      // [n_kv_heads][kv_stride][head_dim]
  uint16_t* scales[2];   // [n_kv_heads][kv_stride][head_dim / 32]
  long long units;       // n_tokens * row_units (8-element units per tensor)
  int row_units;         // n_kv_heads * head_dim / 8
  int step_tokens;       // (gridDim.x * threads) / row_units
  int step_in_row;       // (gridDim.x * threads) % row_units
  int head_units;        // head_dim / 8
  int head_dim;
  int kv_stride;
  int pos0;
};

// max over the 4 lanes of a quad (non-negative floats compare as integers)
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  return v > o ? v : o;
}

__device__ __forceinline__ uint32_t pack_codes4(const float* y) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= ((uint32_t)(int)y[i] & 0xFFu) << (8 * i);
  return w;
}

template <bool F32>
__global__ __launch_bounds__(kAppendThreads) void kv_append_q8_kernel(AppendArgs a) {
  const int tensor = blockIdx.y;
  const char* xbase = static_cast<const char*>(a.x[tensor]);
  int8_t* codes = a.codes[tensor];
  uint16_t* scales = a.scales[tensor];
  const long long step = (long long)gridDim.x * kAppendThreads;
  // unit u = t * row_units + in_row; (t, in_row) advance with u without a divide
  const int u0 = blockIdx.x * kAppendThreads + threadIdx.x;
  long long t = u0 / a.row_units;
  int in_row = u0 - (int)t * a.row_units;
  // units is a multiple of 4 and every quad starts on a multiple of 4, so the
  // four lanes of a block are active together
  for (long long u = u0; u < a.units; u += step) {
    float x[8];
    if constexpr (F32) {
      const float4* p = reinterpret_cast<const float4*>(xbase) + 2 * u;
      const float4 lo = p[0];
      const float4 hi = p[1];
      x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
      x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    } else {
      const uint4 w = reinterpret_cast<const uint4*>(xbase)[u];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __half2float(__ushort_as_half((unsigned short)(ws[i] & 0xFFFFu)));
        x[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(ws[i] >> 16)));
      }
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = __float_as_uint(x[i]) & 0x7FFFFFFFu;
      m = m > b ? m : b;
    }
    const float amax = __uint_as_float(quad_max_u32(m));
    const __half s16 = __float2half_rn(amax / 127.0f);
    const float d = __half2float(s16);
    // a zero scale (an all-zero block) and an infinite one (a block beyond
    // fp16's range) both give code 0: with the divisor taken as +inf the
    // reciprocal is 0 and the rounding test below never passes
    const float dv = d == 0.0f ? __builtin_inff() : d;
    const float rinv = __builtin_amdgcn_rcpf(dv);  // v_rcp_f32, about 1 ulp

    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ax = fabsf(x[i]);
      float k = floorf(ax * rinv);
      k = fmaf(-(k + 0.5f), dv, ax) >= 0.0f ? k + 1.0f : k;  // |x| >= (k + 1/2) scale, exactly
      y[i] = __builtin_copysignf(fminf(k, 127.0f), x[i]);
    }

    const int h = in_row / a.head_units;
    const int j = (in_row - h * a.head_units) * 8;
    const long long row = (long long)h * a.kv_stride + a.pos0 + t;
    uint2 packed;
    packed.x = pack_codes4(y);
    packed.y = pack_codes4(y + 4);
    *reinterpret_cast<uint2*>(codes + row * a.head_dim + j) = packed;
    if ((threadIdx.x & 3) == 0) scales[row * (a.head_dim / 32) + j / 32] = __half_as_ushort(s16);
    t += a.step_tokens;
    in_row += a.step_in_row;
    if (in_row >= a.row_units) {
      in_row -= a.row_units;
      ++t;
    }
  }
}

}  // namespace attnq8
