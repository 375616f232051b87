// The int8-KV attention kernel shared by the verify and prompt paths.
//
// One workgroup owns up to NW x 16 query vectors (row, Q head) of a group of
// consecutive rows that read one KV head -- the "one owner of several query
// rows shares every K/V scan" organisation of "perf(gfx1100): share Q8 KV scans
// across verifier rows" (Summary) -- and scans one range of that head's keys
// in 32-key tiles.  Each of its NW waves owns 16 of the vectors (waves past the
// last vector only help converting).
//
// Per tile:
//   1. copy: the tile's int8 codes and fp16 scales go from HBM straight into a
//      ring of DEPTH tiles in LDS (direct-to-LDS buffer loads; the copies of
//      the next DEPTH-1 tiles are in flight while one is used).  Buffer ranges
//      end at the split's last key, so the ragged last tile reads zeros.
//   2. convert, shared by all waves: K codes -> fp16 MFMA fragments (exact);
//      V codes, read transposed with the gfx950 ds_read_b64_tr_b8, times their
//      per-key scale -> an exact fp16 hi + lo pair of V^T fragments (dV * code
//      has at most 18 significant bits; hi is the rounded product, lo the fma
//      residual).  Each tile is converted once for all the workgroup's vectors.
//   3. compute, per wave: S^T = K Q^T on v_mfma_f32_16x16x32_f16, one 32-dim
//      block per MFMA (q in registers, split hi + lo when given in fp32 after
//      a per-vector power-of-two scaling that keeps both parts normal), each
//      block's dot scaled by its fp16 K scale in fp32 in fixed block order;
//      causal / range mask; online softmax in base 2 with a lazily moved
//      reference point; p split into fp16 hi + lo; O^T += V^T P^T as
//      (Vhi,Phi) + (Vlo,Phi) + (Vhi,Plo).
//
// The accuracy contract of "hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA
// prompt attention" (How: fp16 hi+lo of q and p, fixed summation order, online
// softmax, V scale folded into p) is kept in substance; the V scale is folded
// into an exact hi+lo V fragment instead of into p, which keeps the fold exact
// for any scale magnitude.
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
  int rows_per_wg;          // rows per workgroup
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
constexpr int kRingDepth = 3;

// LDS layout of one 32-key ring stage (bytes):
//   K codes  [32 keys][HD]  int8, 16-byte chunks of a row permuted by chunk_slot
//   V codes  [32 keys][HD]  int8, same permutation
//   K scales [32 keys][HD/32] fp16
//   V scales [32 keys][HD/32] fp16
template <int HD>
struct Stage {
  static constexpr int NB = HD / 32;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 32 * HD;
  static constexpr int KS_OFF = 64 * HD;
  static constexpr int VS_OFF = 66 * HD;
  static constexpr int BYTES = 68 * HD;
  static constexpr int CODE_OPS = HD / 32;                    // 1 KB copies per code tile
  static constexpr int SCALE_OPS = HD >= 128 ? HD / 128 : 1;  // 256 B copies per scale tile
  static constexpr int NOPS = 2 * CODE_OPS + 2 * SCALE_OPS;   // copies per tile
  static constexpr int C = HD / 16;                           // 16-byte chunks per key row
  static constexpr int R = 16 / C;                            // key rows per 256 bytes
};

// Converted fragments of one tile (bytes), one 1 KB fragment = 64 lanes x 16 B:
//   Kf [block b][subtile u]: K codes as fp16, A operand of S^T = K Q^T;
//      lane l: key 16u + l%16, dims 32b + 8(l/16) .. +7
//   Vf [dim tile d][hi|lo]: dV * code as fp16 hi/lo, A operand of O^T += V^T P^T;
//      lane l: dim 16d + l%16, keys pi(l/16, e), e = 0..7
//   with pi(h, e) = 4h + e for e < 4 and 16 + 4h + e - 4 for e >= 4.
template <int HD>
struct Frags {
  static constexpr int NB = HD / 32;
  static constexpr int ND = HD / 16;
  static constexpr int KF_OFF = 0;
  static constexpr int VF_OFF = NB * 2 * 1024;
  static constexpr int BYTES = VF_OFF + ND * 2 * 1024;
};

// Slot of 16-byte chunk `c` of tile row `key` (0..31) -- an involution in c.
// Chosen so that the rows read by one 16-lane group -- 16 consecutive keys for
// K fragments, keys {4h..4h+3, 16+4h..16+4h+3} for the transposing V reads --
// land in distinct 16-byte bank groups.
template <int HD>
__device__ __forceinline__ int chunk_slot(int key, int c) {
  constexpr int C = Stage<HD>::C, R = Stage<HD>::R;
  return c ^ (((key / R) ^ ((key >> 4) * (C / 2))) & (C - 1));
}

__device__ __forceinline__ int pi_key(int h, int e) { return (e < 4) ? 4 * h + e : 16 + 4 * h + (e - 4); }

// The workgroup's direct-to-LDS copies of one 32-key tile, split over its waves
// (wave w issues copies w, w + NW, ...).
template <int HD, int NW>
struct TileCopier {
  using L = Stage<HD>;
  static constexpr int MAXC = (L::NOPS + NW - 1) / NW;  // copies per wave (max)
  static constexpr int MINC = L::NOPS / NW;             // copies per wave (min)

  __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
  int wave, lane;

  __device__ __forceinline__ int count() const { return (L::NOPS - wave + NW - 1) / NW; }

  // Copy the tile starting at key0 into the stage at lds (zeros when !live).
  __device__ __forceinline__ void issue(uint32_t lds, int key0, bool live) const {
    constexpr int kOut = 0x7ffffff0;  // past every buffer range: stores zeros
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int o = wave + i * NW;
      if (o < L::NOPS) {
        if (o < 2 * L::CODE_OPS) {
          const bool is_v = o >= L::CODE_OPS;
          const int j = is_v ? o - L::CODE_OPS : o;
          const int pos = j * 1024 + 16 * lane;
          const int row = pos / HD;
          const int c = chunk_slot<HD>(row, (pos % HD) / 16);
          const int off = live ? (key0 + row) * HD + 16 * c : kOut;
          dma_b128(is_v ? vc : kc, lds + (is_v ? L::V_OFF : L::K_OFF) + j * 1024, off);
        } else {
          const int j = o - 2 * L::CODE_OPS;
          const bool is_v = j >= L::SCALE_OPS;
          const int jj = is_v ? j - L::SCALE_OPS : j;
          const int byte = jj * 256 + 4 * lane;
          const int off = (live && byte < 2 * HD) ? key0 * 2 * L::NB + byte : kOut;
          if (byte < 2 * HD)
            dma_b32(is_v ? vs : ks, lds + (is_v ? L::VS_OFF : L::KS_OFF) + jj * 256, off);
        }
      }
    }
  }

  // Wait until this wave's copies of all but the newest `newer` tiles landed.
  template <int newer>
  __device__ __forceinline__ void wait_all_but() const {
    if (count() == MAXC) wait_vmcnt<MAXC * newer>();
    else wait_vmcnt<MINC * newer>();
  }
};

// One key's NB fp16 block scales, read from LDS as a single vector.
template <int NB> struct ScaleRow;
template <> struct ScaleRow<8> {
  half8_t v;
  __device__ __forceinline__ void load(const half_t* p) { v = *(const half8_t*)p; }
  __device__ __forceinline__ half_t get(int b) const { return v[b]; }
};
template <> struct ScaleRow<4> {
  half4_t v;
  __device__ __forceinline__ void load(const half_t* p) { v = *(const half4_t*)p; }
  __device__ __forceinline__ half_t get(int b) const { return v[b]; }
};
template <> struct ScaleRow<2> {
  half2_t v;
  __device__ __forceinline__ void load(const half_t* p) { v = *(const half2_t*)p; }
  __device__ __forceinline__ half_t get(int b) const { return v[b]; }
};

// Convert unit j of a tile (j < NB: V dim tiles 2j, 2j+1; else K block j - NB)
// from the ring stage `st` into the fragment area `fr`.
template <int HD>
__device__ __forceinline__ void convert_unit(int j, const uint8_t* st, uint8_t* fr, int lane) {
  using L = Stage<HD>;
  using F = Frags<HD>;
  constexpr int NB = L::NB;
  const int h4 = lane >> 4;
  if (j < NB) {
    const int b = j;
    // per-key V scales of block b for keys pi(h4, e)
    const half_t* vsc = (const half_t*)(st + L::VS_OFF);
    half8_t sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = vsc[pi_key(h4, e) * NB + b];
    // transposing reads: lane 16h + 2k + s addresses key pi(h, k), dims 16d + 8s
    const int vkey = pi_key(h4, (lane & 15) >> 1);
    const uint8_t* vrow = st + L::V_OFF + vkey * HD + 8 * (lane & 1);
#pragma unroll
    for (int dd = 0; dd < 2; ++dd) {
      const int d = 2 * b + dd;
      const v2i32_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i32_t*)(vrow + 16 * chunk_slot<HD>(vkey, d)));
      const half8_t c = codes8_to_f16((uint32_t)w[0], (uint32_t)w[1]);
      const half8_t vh = c * sc;
      const half8_t vl = __builtin_elementwise_fma(c, sc, -vh);
      *(half8_t*)(fr + F::VF_OFF + ((d * 2 + 0) * 64 + lane) * 16) = vh;
      *(half8_t*)(fr + F::VF_OFF + ((d * 2 + 1) * 64 + lane) * 16) = vl;
    }
  } else {
    const int b = j - NB;
    const int c = 2 * b + (h4 >> 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = 16 * u + (lane & 15);
      const uint2 w = *(const uint2*)(st + L::K_OFF + kk * HD + 16 * chunk_slot<HD>(kk, c) + 8 * (h4 & 1));
      *(half8_t*)(fr + F::KF_OFF + ((b * 2 + u) * 64 + lane) * 16) = codes8_to_f16(w.x, w.y);
    }
  }
}

// Which wave converts unit j of a tile: waves that own no query vectors take
// four units for every one a computing wave takes, so that the conversion of
// the next tile finishes within the computing waves' time on this one.
__device__ __forceinline__ int convert_owner(int j, int n_compute, int nw) {
  const int n_idle = nw - n_compute;
  const int len = 4 * n_idle + n_compute;
  const int i = j % len;
  return (i < 4 * n_idle) ? n_compute + (i % n_idle) : i - 4 * n_idle;
}

template <int HD, int NW, bool QF32, bool FINAL>
__global__ __launch_bounds__(64 * NW) void attend_q8_kernel(const AttendArgs a) {
  using L = Stage<HD>;
  using F = Frags<HD>;
  constexpr int NB = L::NB;
  constexpr int ND = HD / 16;  // 16-dim output tiles
  constexpr int D = kRingDepth;
  constexpr int NU = 2 * NB;   // conversion units per tile

  __shared__ __attribute__((aligned(16))) uint8_t ring[D * L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t frag[2][F::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  const int n_compute = min(NW, (M + 15) >> 4);  // waves that own query vectors

  // ---- start the copies first so that their latency overlaps the q setup
  const size_t head_rows = (size_t)g * a.kv_stride;
  TileCopier<HD, NW> cp;
  cp.kc = make_rsrc(a.kc + head_rows * HD, k_end * HD);
  cp.vc = make_rsrc(a.vc + head_rows * HD, k_end * HD);
  cp.ks = make_rsrc(a.ks + head_rows * NB, k_end * NB * 2);
  cp.vs = make_rsrc(a.vs + head_rows * NB, k_end * NB * 2);
  cp.wave = wave;
  cp.lane = lane;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
#pragma unroll
  for (int s = 0; s < D - 1; ++s)
    cp.issue(ring0 + s * L::BYTES, (t_begin + s) * 32, t_begin + s < t_end);

  // ---- this wave's query vectors: column n16 of its S^T tile
  const int v = wave * 16 + n16;
  const bool v_ok = v < M;
  const bool computes = wave < n_compute;  // wave-uniform
  const int vr = v_ok ? v / a.G : 0;
  const int vh = v_ok ? g * a.G + (v - vr * a.G) : 0;
  const int lim = v_ok ? a.pos0 + r0 + vr : -1;  // last key this vector sees

  // q fragments: B operand of S^T = K Q^T (lane: vector n16, dims 32b + 8*h4 + e)
  half8_t qhi[NB];
  half8_t qlo[NB];
  float xmul;
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
    xmul = a.kmul * ldexpf(1.0f, -k);  // exact: a power-of-two factor
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

  // ---- prologue: convert the first tile
  if (t_begin < t_end) {
    cp.template wait_all_but<D - 2>();
    __syncthreads();
    for (int j = 0; j < NU; ++j)
      if (convert_owner(j, n_compute, NW) == wave) convert_unit<HD>(j, ring, frag[0], lane);
  }

  // Per tile t: one barrier, then copy tile t+D-1, convert tile t+1 and
  // compute tile t (the converted fragments are double-buffered).
  int slot = 0;
  int buf = 0;
  for (int t = t_begin; t < t_end; ++t) {
    const int key0 = t * 32;
    const bool has_next = t + 1 < t_end;
    if (has_next) cp.template wait_all_but<D - 3>();  // this wave's copies of tile t+1 landed
    __syncthreads();  // tile t converted; tile t-1 computed; copies of tile t+1 landed
    cp.issue(ring0 + ((slot + D - 1) % D) * L::BYTES, key0 + (D - 1) * 32, t + D - 1 < t_end);
    const uint8_t* st = ring + slot * L::BYTES;
    if (has_next) {
      const uint8_t* st_next = ring + ((slot + 1) % D) * L::BYTES;
      for (int j = 0; j < NU; ++j)
        if (convert_owner(j, n_compute, NW) == wave) convert_unit<HD>(j, st_next, frag[buf ^ 1], lane);
    }

    if (computes) {
      const uint8_t* fr = frag[buf];
      // ---- S^T = K Q^T, per 16-key subtile: the NB hi MFMAs, then the NB lo
      // MFMAs (independent ones in between), then the per-block K scales
      const half_t* Kst = (const half_t*)(st + L::KS_OFF);
      float4_t s[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float4_t acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const half8_t ka = *(const half8_t*)(fr + F::KF_OFF + ((b * 2 + u) * 64 + lane) * 16);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qhi[b], (float4_t){0, 0, 0, 0}, 0, 0, 0);
        }
        if (QF32) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const half8_t ka = *(const half8_t*)(fr + F::KF_OFF + ((b * 2 + u) * 64 + lane) * 16);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qlo[b], acc[b], 0, 0, 0);
          }
        }
        ScaleRow<NB> dk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dk[e].load(Kst + (16 * u + 4 * h4 + e) * NB);
        s[u] = (float4_t){0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[u][e] = fmaf((float)dk[e].get(b), acc[b][e], s[u][e]);
      }

      // ---- mask and online softmax (base 2), p -> fp16 hi + lo
      float x[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + 16 * u + 4 * h4 + e;
          const bool vis = (key < k_end) && (key <= lim);
          x[u][e] = vis ? s[u][e] * xmul : -INFINITY;
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

      // ---- O^T += V^T P^T: three passes over the dim tiles so that the
      // MFMAs on one accumulator are separated by independent ones
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const half8_t vh = *(const half8_t*)(fr + F::VF_OFF + ((d * 2 + 0) * 64 + lane) * 16);
        O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, phi, O[d], 0, 0, 0);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const half8_t vl = *(const half8_t*)(fr + F::VF_OFF + ((d * 2 + 1) * 64 + lane) * 16);
        O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, phi, O[d], 0, 0, 0);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const half8_t vh = *(const half8_t*)(fr + F::VF_OFF + ((d * 2 + 0) * 64 + lane) * 16);
        O[d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, plo, O[d], 0, 0, 0);
      }
    }
    slot = (slot + 1 == D) ? 0 : slot + 1;
    buf ^= 1;
  }
  // copies into the ring past the last tile may still be landing
  wait_vmcnt<0>();

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

// Merge split partials: one wave per (row, Q head); lane l owns dims 4l..4l+3.
// Splits are read 16 at a time with all loads in flight, and summed in fixed
// split order (run-to-run bitwise reproducible).
template <int HD>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part_o,
                                                              const float2* __restrict__ part_ml,
                                                              int n_splits, int n_pairs,
                                                              float* __restrict__ out) {
  constexpr int NC = HD / 4;  // lanes holding data
  constexpr int CH = 16;      // splits per batch
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
  const bool active = lane < NC;
  const int dl = active ? lane : 0;
  float4_t acc = {0, 0, 0, 0};
  float den = 0.0f;
  for (int s0 = 0; s0 < n_splits; s0 += CH) {
    float2 ml[CH];
    float4_t o[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int sp = min(s0 + i, n_splits - 1);
      const size_t idx = (size_t)sp * n_pairs + pair;
      ml[i] = part_ml[idx];
      o[i] = *(const float4_t*)(part_o + idx * HD + 4 * dl);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (s0 + i < n_splits) {
        const float w = (ml[i].y > 0.0f) ? exp2f(ml[i].x - M) : 0.0f;
        den = fmaf(w, ml[i].y, den);
        acc += w * o[i];
      }
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
