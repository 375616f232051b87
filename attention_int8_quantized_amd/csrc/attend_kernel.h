// The int8-KV attention tile kernel shared by the verify and prompt paths.
//
// One workgroup owns the query vectors (row, Q head) of a group of consecutive
// rows that read one KV head -- the "one owner of several query rows shares
// every K/V scan" organisation of "perf(gfx1100): share Q8 KV scans across
// verifier rows" (Summary) -- and scans one range of that head's keys, 32 keys
// at a time:
//
//   1. cooperative staging: the workgroup reads the tile's int8 K/V codes and
//      fp16 scales with coalesced loads, converts K codes exactly to fp16
//      (fragment order), stores K scales * sm_scale * log2(e) as fp32, and
//      dequantises V exactly into an fp16 hi + lo pair (V = dV * code has at
//      most 18 significant bits; hi holds the rounded top 11, the fma residual
//      the rest), transposed into the MFMA fragment order of V^T;
//   2. per wave (16 query vectors): S^T = K Q^T on v_mfma_f32_16x16x32_f16, one
//      32-dim block per MFMA (q is split hi + lo when given in fp32, after a
//      per-vector power-of-two scaling that keeps both parts normal), each
//      block's dot scaled by its K scale in fp32 in fixed block order;
//   3. causal / range mask, online softmax in base 2 with a lazily moved
//      reference point, p split into fp16 hi + lo;
//   4. O^T += V^T P^T on the same MFMA as (Vhi,Phi) + (Vlo,Phi) + (Vhi,Plo).
//
// The page's accuracy contract ("hip: gfx12 (RDNA4) WMMA kernel for the
// int8-KV QSA prompt attention", How: fp16 hi+lo of q and p, fixed summation
// order, online softmax, V scale folded into p) is kept in spirit: here the V
// scale is folded into an exact hi+lo V tile instead of into p, which keeps the
// fold exact for any scale magnitude.
//
// The workgroup writes either split partials (m, l, o) or, when it covers every
// key its rows see, the normalised output.
#pragma once

#include "device_utils.h"

namespace attnq8 {

struct AttendArgs {
  const void* q;            // [n_rows][Hq][HD], fp32 or fp16
  const int8_t* kc;         // [Hkv][kv_stride][HD]
  const uint16_t* ks;       // [Hkv][kv_stride][HD/32]
  const int8_t* vc;
  const uint16_t* vs;
  float* part_o;            // [n_splits][n_rows][Hq][HD]   (partials mode)
  float2* part_ml;          // [n_splits][n_rows][Hq]
  float* out;               // [n_rows][Hq][HD]              (final mode)
  int Hq;
  int G;                    // Hq / Hkv
  int kv_stride;
  int pos0;                 // position of row 0
  int n_rows;
  int rows_per_wg;
  int n_splits;
  float kmul;               // sm_scale * log2(e)
};

// Reference-point policy of the online softmax (base-2 units): a new reference
// is taken only when a tile's maximum exceeds the current one by more than
// kRescaleSlack, and it is placed kRefBias below that maximum.  Probabilities
// then stay within [0, 2^15], inside fp16 range, and the largest ones sit well
// above fp16's subnormal range so that their hi + lo split keeps 22 bits.
constexpr float kRescaleSlack = 15.0f;
constexpr float kRefBias = 8.0f;

// One 32-key tile of K/V codes and scales, loaded with all of a thread's
// loads in flight at once and then converted into the LDS operand layouts:
//   Kf: K codes as fp16, A-operand fragments of S^T = K Q^T
//       [block b][subtile u][lane][8]: key 16u + lane%16, dims 32b + 8(lane/16) + e
//   Ks: K scale * sm_scale * log2(e), fp32 [block][key]
//   Vf: V = dV * code as an exact fp16 hi/lo pair, A-operand fragments of
//       O^T += V^T P^T: [dim tile d][hi|lo][lane][8]: dim 16d + lane%16, keys
//       4(lane/16) + e for e < 4 and 16 + 4(lane/16) + e - 4 for e >= 4
template <int HD, int NT>
struct RawTile {
  static constexpr int NB = HD / 32;
  static constexpr int KCH = 2 * HD;             // 16-byte K code chunks per tile
  static constexpr int CK = (KCH + NT - 1) / NT;
  static constexpr int VT = 2 * HD;              // V tasks: 4 keys x 4 dims
  static constexpr int CV = (VT + NT - 1) / NT;
  static constexpr int KS = 32 * NB;             // K scales per tile
  static constexpr int CS = (KS + NT - 1) / NT;

  uint4 k[CK];
  uint32_t v[CV][4];
  uint16_t vs[CV][4];
  uint16_t ks[CS];

  __device__ __forceinline__ void load(const int8_t* kc, const uint16_t* ksc, const int8_t* vc,
                                       const uint16_t* vsc, int key0, int k_end, int tid) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int f = tid + i * NT;
      const int kk = f / (HD / 16);
      const int c = f - kk * (HD / 16);
      const int key = key0 + kk;
      k[i] = make_uint4(0u, 0u, 0u, 0u);
      if (f < KCH && key < k_end) k[i] = *(const uint4*)(kc + (size_t)key * HD + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int f = tid + i * NT;
      const int c = f % (HD / 4);
      const int q4 = f / (HD / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key0 + 4 * q4 + j;
        v[i][j] = 0u;
        vs[i][j] = 0;
        if (f < VT && key < k_end) {
          v[i][j] = *(const uint32_t*)(vc + (size_t)key * HD + 4 * c);
          vs[i][j] = vsc[(size_t)key * NB + (c >> 3)];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CS; ++i) {
      const int f = tid + i * NT;
      const int kk = f / NB;
      const int b = f - kk * NB;
      const int key = key0 + kk;
      ks[i] = 0;
      if (f < KS && key < k_end) ks[i] = ksc[(size_t)key * NB + b];
    }
  }

  __device__ __forceinline__ void stage(half_t* Kf, float* Ksm, half_t* Vf, float kmul,
                                        int tid) const {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int f = tid + i * NT;
      if (f < KCH) {
        const int kk = f / (HD / 16);
        const int c = f - kk * (HD / 16);  // dims 16c .. 16c+15
        const int b = c >> 1, hh = 2 * (c & 1), u = kk >> 4;
        const half4_t x0 = dword_codes_to_f16(k[i].x);
        const half4_t x1 = dword_codes_to_f16(k[i].y);
        const half4_t x2 = dword_codes_to_f16(k[i].z);
        const half4_t x3 = dword_codes_to_f16(k[i].w);
        half_t* dst = &Kf[((b * 2 + u) * 64 + hh * 16 + (kk & 15)) * 8];
        *(half8_t*)dst = (half8_t){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        *(half8_t*)(dst + 16 * 8) = (half8_t){x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
      }
    }
#pragma unroll
    for (int i = 0; i < CS; ++i) {
      const int f = tid + i * NT;
      if (f < KS) {
        const int kk = f / NB;
        const int b = f - kk * NB;
        Ksm[b * 32 + kk] = (float)f16_from_bits(ks[i]) * kmul;
      }
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int f = tid + i * NT;
      if (f < VT) {
        const int c = f % (HD / 4);   // dims 4c .. 4c+3
        const int q4 = f / (HD / 4);  // keys 4 q4 .. 4 q4 + 3
        const half2_t dv01 = {f16_from_bits(vs[i][0]), f16_from_bits(vs[i][1])};
        const half2_t dv23 = {f16_from_bits(vs[i][2]), f16_from_bits(vs[i][3])};
        const int u = q4 >> 2, hh = q4 & 3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + j) << 16) | (uint32_t)j;
          const half2_t c01 = codes_to_f16(v[i][1], v[i][0], sel);
          const half2_t c23 = codes_to_f16(v[i][3], v[i][2], sel);
          const half2_t hi01 = c01 * dv01;
          const half2_t hi23 = c23 * dv23;
          const half2_t lo01 = __builtin_elementwise_fma(c01, dv01, -hi01);
          const half2_t lo23 = __builtin_elementwise_fma(c23, dv23, -hi23);
          const int D = 4 * c + j;
          const int d = D >> 4;
          const int ln = hh * 16 + (D & 15);
          *(half4_t*)&Vf[((d * 2 + 0) * 64 + ln) * 8 + 4 * u] =
              (half4_t){hi01[0], hi01[1], hi23[0], hi23[1]};
          *(half4_t*)&Vf[((d * 2 + 1) * 64 + ln) * 8 + 4 * u] =
              (half4_t){lo01[0], lo01[1], lo23[0], lo23[1]};
        }
      }
    }
  }
};

template <int HD, int NW, bool QF32, bool FINAL>
__global__ __launch_bounds__(64 * NW) void attend_q8_kernel(const AttendArgs a) {
  constexpr int NB = HD / 32;   // 32-dim blocks (one scale each)
  constexpr int ND = HD / 16;   // 16-dim output tiles
  constexpr int NT = 64 * NW;   // threads

  __shared__ __attribute__((aligned(16))) half_t Kf[NB * 2 * 64 * 8];
  __shared__ __attribute__((aligned(16))) float Ks[NB * 32];
  __shared__ __attribute__((aligned(16))) half_t Vf[ND * 2 * 64 * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h4 = lane >> 4;
  const int n16 = lane & 15;

  const int split = blockIdx.x;
  const int rg = blockIdx.y;
  const int g = blockIdx.z;
  const int r0 = rg * a.rows_per_wg;
  const int nr = min(a.rows_per_wg, a.n_rows - r0);
  const int M = nr * a.G;
  const int n_keys = a.pos0 + r0 + nr;  // keys 0 .. n_keys-1 are seen by some row
  const int n_tiles = (n_keys + 31) >> 5;
  const int t_begin = (int)(((long long)split * n_tiles) / a.n_splits);
  const int t_end = (int)(((long long)(split + 1) * n_tiles) / a.n_splits);
  const int k_end = min(n_keys, t_end * 32);

  // this lane's query vector (column of the S^T tile)
  const int v = wave * 16 + n16;
  const bool v_ok = v < M;
  const int vr = v_ok ? v / a.G : 0;
  const int vh = v_ok ? g * a.G + (v - vr * a.G) : 0;
  const int lim = v_ok ? a.pos0 + r0 + vr : -1;  // last key this vector sees

  // ---- q fragments: B operand of S^T = K Q^T (lane: vector n16, dims 32b + 8*h4 + e)
  half8_t qhi[NB];
  half8_t qlo[NB];
  float inv_qmul;
  {
    float qv[NB][8];
    float amax = 0.0f;
    const size_t qoff = ((size_t)(r0 + vr) * a.Hq + vh) * HD + 8 * h4;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (QF32) {
        float4_t x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
        if (v_ok) {
          const float4_t* p = (const float4_t*)((const float*)a.q + qoff + 32 * b);
          x0 = p[0];
          x1 = p[1];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[b][e] = x0[e];
          qv[b][4 + e] = x1[e];
        }
      } else {
        half8_t x = {0, 0, 0, 0, 0, 0, 0, 0};
        if (v_ok) x = *(const half8_t*)((const half_t*)a.q + qoff + 32 * b);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[b][e] = (float)x[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(qv[b][e]));
    }
    amax = wave_max_groups(amax);
    // power-of-two scaling so that max|q * 2^k| lies in [2^14, 2^15)
    int k = 0;
    if (amax > 0.0f) {
      int ex;
      (void)frexpf(amax, &ex);
      k = min(100, max(-100, 15 - ex));
    }
    const float qmul = ldexpf(1.0f, k);
    inv_qmul = ldexpf(1.0f, -k);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qv[b][e] * qmul;
        const half_t hi = (half_t)x;
        qhi[b][e] = hi;
        qlo[b][e] = QF32 ? (half_t)(x - (float)hi) : (half_t)0.0f;
      }
    }
  }

  float4_t O[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) O[d] = (float4_t){0, 0, 0, 0};
  float m_ref = -INFINITY;
  float l_part = 0.0f;

  const size_t head_rows = (size_t)g * a.kv_stride;
  const int8_t* kc_head = a.kc + head_rows * HD;
  const int8_t* vc_head = a.vc + head_rows * HD;
  const uint16_t* ks_head = a.ks + head_rows * NB;
  const uint16_t* vs_head = a.vs + head_rows * NB;

  // Raw bytes of one 32-key tile held in registers: the next tile's loads are
  // issued before the current tile is computed, so their latency overlaps it.
  RawTile<HD, NT> raw;
  if (t_begin < t_end) raw.load(kc_head, ks_head, vc_head, vs_head, t_begin * 32, k_end, tid);

  for (int t = t_begin; t < t_end; ++t) {
    const int key0 = t * 32;
    __syncthreads();  // every wave is done reading the previous tile
    raw.stage(Kf, Ks, Vf, a.kmul, tid);
    if (t + 1 < t_end) raw.load(kc_head, ks_head, vc_head, vs_head, key0 + 32, k_end, tid);
    __syncthreads();

    // ---- S^T = K Q^T for two 16-key subtiles
    float4_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = (float4_t){0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const half8_t ka = *(const half8_t*)&Kf[((b * 2 + u) * 64 + lane) * 8];
        float4_t acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qhi[b], acc, 0, 0, 0);
        if (QF32) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qlo[b], acc, 0, 0, 0);
        const float4_t ksc = *(const float4_t*)&Ks[b * 32 + 16 * u + 4 * h4];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[u][e] = fmaf(ksc[e], acc[e], s[u][e]);
      }
    }

    // ---- mask and online softmax (base 2)
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + 16 * u + 4 * h4 + e;
        const bool vis = (key < k_end) && (key <= lim);
        x[u][e] = vis ? s[u][e] * inv_qmul : -INFINITY;
        tmax = fmaxf(tmax, x[u][e]);
      }
    }
    tmax = wave_max_groups(tmax);
    const bool need = tmax > m_ref + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? tmax - kRefBias : m_ref;
      const float alpha = need ? exp2f(m_ref - m_new) : 1.0f;
#pragma unroll
      for (int d = 0; d < ND; ++d) O[d] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
    }
    const float mu = (m_ref == -INFINITY) ? 0.0f : m_ref;
    half8_t phi, plo;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = exp2f(x[u][e] - mu);
        l_part += p;
        const half_t ph = (half_t)p;
        phi[4 * u + e] = ph;
        plo[4 * u + e] = (half_t)(p - (float)ph);
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const half8_t vh = *(const half8_t*)&Vf[((d * 2 + 0) * 64 + lane) * 8];
      const half8_t vl = *(const half8_t*)&Vf[((d * 2 + 1) * 64 + lane) * 8];
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, phi, O[d], 0, 0, 0);
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, phi, O[d], 0, 0, 0);
      O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, plo, O[d], 0, 0, 0);
    }
  }

  // ---- epilogue
  const float l_tot = wave_sum_groups(l_part);
  if (!v_ok) return;
  const int row = r0 + vr;
  if (FINAL) {
    const float inv_l = 1.0f / l_tot;
    float* dst = a.out + ((size_t)row * a.Hq + vh) * HD + 4 * h4;
#pragma unroll
    for (int d = 0; d < ND; ++d) *(float4_t*)(dst + 16 * d) = O[d] * inv_l;
  } else {
    const size_t idx = ((size_t)split * a.n_rows + row) * a.Hq + vh;
    float* dst = a.part_o + idx * HD + 4 * h4;
#pragma unroll
    for (int d = 0; d < ND; ++d) *(float4_t*)(dst + 16 * d) = O[d];
    if (h4 == 0) a.part_ml[idx] = make_float2(m_ref, l_tot);
  }
}

// Merge split partials: one wave per (row, Q head), splits in fixed order.
template <int HD>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part_o,
                                                              const float2* __restrict__ part_ml,
                                                              int n_splits, int n_pairs,
                                                              float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= n_pairs) return;
  float M = -INFINITY;
  for (int s = lane; s < n_splits; s += 64) {
    const float2 ml = part_ml[(size_t)s * n_pairs + pair];
    if (ml.y > 0.0f) M = fmaxf(M, ml.x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  constexpr int NC = HD / 4;
  float4_t acc = {0, 0, 0, 0};
  float den = 0.0f;
  const bool active = lane < NC;
#pragma unroll 4
  for (int s = 0; s < n_splits; ++s) {
    const size_t idx = (size_t)s * n_pairs + pair;
    const float2 ml = part_ml[idx];
    const float w = (ml.y > 0.0f) ? exp2f(ml.x - M) : 0.0f;
    den = fmaf(w, ml.y, den);
    if (active) {
      const float4_t o = *(const float4_t*)(part_o + idx * HD + 4 * lane);
      acc += w * o;
    }
  }
  if (active) *(float4_t*)(out + (size_t)pair * HD + 4 * lane) = acc / den;
}

// All 65,536 byte pairs through the code conversion used by the kernels.
__global__ __launch_bounds__(256) void selftest_i8_to_f16_kernel(uint16_t* out) {
  const int p = blockIdx.x * 256 + threadIdx.x;  // 0 .. 65535
  uint32_t w = (uint32_t)p;                       // bytes: p & 255, p >> 8
  // Make the word opaque to the optimiser, as a word loaded from memory is in
  // the attention kernels; otherwise known-bits folding of the index rewrites
  // the conversion and the test would not exercise the kernels' instructions.
  asm volatile("" : "+v"(w));
  const half4_t h = dword_codes_to_f16(w);
  // store the pair as one word (bit-casting vector elements one at a time is
  // not reliable with this compiler)
  const half2_t pair = {h[0], h[1]};
  *(uint32_t*)(out + 2 * p) = __builtin_bit_cast(uint32_t, pair);
}

}  // namespace attnq8
