// Attention in a layout in which each compute wave owns 16 query vectors end
// to end.  The library launches it at head_dim 256 for row groups of six
// vector tiles (such as the prompt chunk's 8 queries x 12 heads) over an int8
// or fp16 cache, and over an fp16 cache also for three (the verify window's
// 8 rows x 6 heads); at head_dim 128 for row groups of five to eight vector
// tiles (such as the verify batch's 32 rows x 4 heads) over either cache.
//
// Waves 0..NQ-1 each own one vector tile: per 32-key tile they compute
// S^T = K Q^T, the mask and the online softmax, and then O^T += V^T P^T over all
// 16-dim tiles of the output with p straight from their own registers (no
// hand-off of p through LDS and no second barrier per tile).  The other waves
// feed them: they issue the direct-to-LDS copies of the int8 tiles and, one
// tile ahead, convert K to fp16 fragments and V to exact fp16 hi + lo
// fragments (dV * code, with the general body's power-of-two shift for a block
// holding a V scale above 512) in LDS, where every compute wave reads them.  The
// arithmetic of each output element is the same as in the general attention
// body (same q and p splits, same block order of the K scales, same three PV
// terms in the same order, same reference-point policy), so the two produce
// identical results.
//
// Head_dim 256 (eight waves): with six tiles, SIMDs 0 and 1 carry two compute
// waves each and SIMDs 2 and 3 one compute wave and one feeding wave; with
// three, SIMDs 0..2 carry one compute wave and one other wave each and SIMD 3
// two other waves (over an fp16 cache two of the five copy and three only keep
// the barriers).  Head_dim 128: eight compute waves (two per SIMD) and four
// feeders, one per SIMD (int8 cache: each a quarter of the copies and of the
// conversion), or two copying feeders (fp16 cache).
//
// LDS at head_dim 256: a ring of three int8 stages (a stage is free once its
// tile has been converted), double-buffered K fragments (16 KB), K scales
// (512 B) and V^T fragments (32 KB), and per tile a byte per block that carries
// the V fold's shift (0 unless the block holds a V scale above 512): 151,568 B
// in all (75,792 B at head_dim 128).  Over an fp16 cache nothing is converted:
// the compute waves read K and V^T fragments from a ring of four stages (32 KB
// each at head_dim 256, 16 KB at 128), and the feeders only copy.
//
// Per iteration t (one workgroup barrier each): the copying feeders have waited
// for their copies of tile t+1; after the barrier they copy tile t+3 into the
// stage of tile t and all feeders convert tile t+1, while the compute waves
// work on tile t.  The workgroup covers the key tiles [t_begin, t_end) of one
// split and writes split partials (m, l, o) or, with FINAL, the normalised
// output.
#pragma once

#include "attend_kernel.h"

namespace attnq8 {

// Feeder F of NF: its shares of the tile copies (the four shares of a
// four-wave TileCopier, share s going to feeder s % NF) and of the conversion
// (K units u = F, F + NF, ... of the 16 (block u >> 1, 16-key subtile u & 1);
// V blocks b = F, F + NF, ... of the 8).
template <int HD, int NF, int F>
struct OwnFeeder {
  using L = Stage<HD>;
  static constexpr int NB = L::NB;
  static_assert(HD == 128 || HD == 256, "head_dim 128 or 256");
  static_assert(NF == 2 || NF >= 4, "the four copy shares split evenly");
  static constexpr int NSHARE = NF >= 4 ? (F < 4 ? 1 : 0) : 4 / NF;  // copy shares
  static constexpr int NKU = (2 * NB - F + NF - 1) / NF;     // K units
  static constexpr int NVB = (NB - F + NF - 1) / NF;         // V blocks
  // copies per tile: share s of a four-wave TileCopier issues 2 CPW code
  // copies and, for s below its NS, one scale copy
  static constexpr int copies_per_tile() {
    using TC = TileCopier<L, 4>;
    int n = 0;
    for (int j = 0; j < NSHARE; ++j) n += 2 * TC::CPW + (F + NF * j < TC::NS ? 1 : 0);
    return n;
  }
  static constexpr int COPIES = copies_per_tile();
  // the K scale plane (64 NB bytes) goes in 256-byte parts to the first feeders
  static constexpr int NKSP = NB / 4;
  static constexpr int KSF = NF < NKSP ? NF : NKSP;
  static constexpr int NKS = F < KSF ? (NKSP - F + KSF - 1) / KSF : 0;  // this feeder's parts

  TileCopier<L, 4> cp[NSHARE > 0 ? NSHARE : 1];
  int k_rd[NKU > 0 ? NKU : 1];        // K unit j: the lane's 8 codes within a stage
  int v_rd[NVB > 0 ? NVB : 1][2];     // V block j, dim tile dd: the lane's transposing read
  int vs_rd;                          // V scale rows of the lane's keys pi(h4, e)
  // one key's NB V scales as NB / 2 dwords
  typedef uint32_t srow_t __attribute__((ext_vector_type(NB / 2)));

  __device__ __forceinline__ void init(const AttendArgs& a, size_t head_rows, int k_end, int lane) {
#pragma unroll
    for (int s = 0; s < NSHARE; ++s) {
      cp[s].kc = make_rsrc(a.kc + head_rows * HD, k_end * HD);
      cp[s].vc = make_rsrc(a.vc + head_rows * HD, k_end * HD);
      cp[s].ks = make_rsrc(a.ks + head_rows * NB, k_end * NB * 2);
      cp[s].vs = make_rsrc(a.vs + head_rows * NB, k_end * NB * 2);
      cp[s].init(F + NF * s, lane);
    }
    const int h4 = lane >> 4, n16 = lane & 15;
#pragma unroll
    for (int j = 0; j < NKU; ++j) {
      const int u = F + NF * j;
      const int key = 16 * (u & 1) + n16;
      k_rd[j] = L::K_OFF + key * HD + 16 * chunk_slot<HD>(key, 2 * (u >> 1) + (h4 >> 1)) + 8 * (h4 & 1);
    }
    const int vkey = pi_key(h4, n16 >> 1);
#pragma unroll
    for (int j = 0; j < NVB; ++j)
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
        v_rd[j][dd] = L::V_OFF + vkey * HD + 8 * (lane & 1) + 16 * chunk_slot<HD>(vkey, 2 * (F + NF * j) + dd);
    vs_rd = L::VS_OFF + 8 * NB * h4;  // key 4 h4 (a key row holds 2 NB bytes)
  }

  __device__ __forceinline__ void copy(uint32_t lds, int key0, bool live) const {
#pragma unroll
    for (int s = 0; s < NSHARE; ++s) cp[s].issue(lds, key0, live);
  }

  // this feeder's copies of all but the newest `newer` tiles landed
  template <int newer>
  __device__ __forceinline__ void wait() const {
    if constexpr (COPIES > 0) wait_vmcnt<COPIES * newer>();
  }

  // Tile in stage `st` -> K fragments `kf`, K scales `ksd`, V^T fragments `vf`
  // and the V fold shift of each of this feeder's blocks (one byte per block
  // in `vsd`; 0 unless the block holds a V scale above 512).  Every read of
  // the stage is issued before the first write, so the reads' latencies
  // overlap.
  __device__ __forceinline__ void convert(const uint8_t* st, uint8_t* kf, uint8_t* ksd, uint8_t* vf, uint8_t* vsd,
                                          int lane) const {
    uint2 kw[NKU > 0 ? NKU : 1];
#pragma unroll
    for (int j = 0; j < NKU; ++j) kw[j] = *(const uint2*)(st + k_rd[j]);
    v2i32_t vw[NVB > 0 ? NVB : 1][2];
#pragma unroll
    for (int j = 0; j < NVB; ++j)
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
        vw[j][dd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i32_t*)(st + v_rd[j][dd]));
    srow_t srow[8];
    if constexpr (NVB > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        srow[e] = *(const srow_t*)(st + vs_rd + 2 * NB * (e < 4 ? e : 16 + (e - 4)));
    }
    uint32_t ksw[NKS > 0 ? NKS : 1];
#pragma unroll
    for (int i = 0; i < NKS; ++i) ksw[i] = *(const uint32_t*)(st + L::KS_OFF + 256 * (F + KSF * i) + 4 * lane);

#pragma unroll
    for (int j = 0; j < NKU; ++j) {
      const int u = F + NF * j;
      *(half8_t*)(kf + (((u >> 1) * 2 + (u & 1)) * 64 + lane) * 16) = codes8_to_f16(kw[j].x, kw[j].y);
    }
#pragma unroll
    for (int i = 0; i < NKS; ++i) *(uint32_t*)(ksd + 256 * (F + KSF * i) + 4 * lane) = ksw[i];
#pragma unroll
    for (int j = 0; j < NVB; ++j) {
      const int b = F + NF * j;
      // scales of block b (half b & 1 of word b >> 1 of each row) for keys pi(h4, 0..7)
      constexpr uint32_t SEL0 = 0x05040100u, SEL1 = 0x07060302u;
      u32x4_t scw;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        scw[k] = __builtin_amdgcn_perm(srow[2 * k + 1][b >> 1], srow[2 * k][b >> 1], (b & 1) ? SEL1 : SEL0);
      half8_t sc = __builtin_bit_cast(half8_t, scw);
      const int sh = v_fold_prescale(sc);
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        const half8_t c = codes8_to_f16((uint32_t)vw[j][dd][0], (uint32_t)vw[j][dd][1]);
        const half8_t vh8 = c * sc;
        const half8_t vl8 = __builtin_elementwise_fma(c, sc, -vh8);
        const int d = 2 * b + dd;
        *(half8_t*)(vf + ((d * 2 + 0) * 64 + lane) * 16) = vh8;
        *(half8_t*)(vf + ((d * 2 + 1) * 64 + lane) * 16) = vl8;
      }
      if (lane == 0) vsd[b] = (uint8_t)sh;
    }
  }
};

// The feeders' loop: iteration t waits for this feeder's copies of tile t+1,
// passes the barrier, copies tile t+3 into the stage of tile t and converts
// tile t+1.  Iteration t_begin - 1 converts the first tile only.
template <int HD, int NF, int F, int D, class Ring>
__device__ __forceinline__ void own_feed(const AttendArgs& a, size_t head_rows, int k_end, int t_begin, int t_end,
                                         int lane, Ring& r) {
  using L = Stage<HD>;
  OwnFeeder<HD, NF, F> fd;
  fd.init(a, head_rows, k_end, lane);
  fd.copy(r.ring0 + 0 * L::BYTES, t_begin * 32, t_begin < t_end);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // q goes out with the first tile, the other tiles after
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 1; s < D; ++s) fd.copy(r.ring0 + s * L::BYTES, (t_begin + s) * 32, t_begin + s < t_end);
  int slot = 0;  // ring stage of tile t
  for (int t = t_begin - 1; t < t_end; ++t) {
    if (t < t_begin) fd.template wait<D - 1>();
    else fd.template wait<D - 2>();
    __syncthreads();  // tile t+1 landed; tile t converted; buffer (t+1) & 1 free
    if (t >= t_begin) {
      fd.copy(r.ring0 + slot * L::BYTES, (t + D) * 32, t + D < t_end);  // the stage of tile t is free
      slot = slot + 1 == D ? 0 : slot + 1;
    }
    if (t + 1 < t_end)
      fd.convert(r.ring + slot * L::BYTES, r.kfrag[(t + 1) & 1], r.kscale[(t + 1) & 1], r.vfrag[(t + 1) & 1],
                 r.vshift[(t + 1) & 1], lane);
  }
  wait_vmcnt<0>();  // copies past the last tile may still be landing
}

// The feeders' loop over an fp16 cache (no conversion: the compute waves read
// K and V^T fragments from the ring): iteration t waits for this feeder's
// copies of tile t, passes the barrier and copies tile t+D-1 into the stage of
// tile t-1.  Feeder F of NF takes code chunks F, F + NF, ... of each plane.
template <int HD, int NF, int F, int D>
__device__ __forceinline__ void own_feed16(const AttendArgs& a, size_t head_rows, int k_end, int t_begin, int t_end,
                                           int lane, uint32_t ring0) {
  using L = Stage16<HD>;
  TileCopier<L, NF> cp;
  cp.kc = make_rsrc((const uint8_t*)a.kc + head_rows * L::ROW, k_end * L::ROW);
  cp.vc = make_rsrc((const uint8_t*)a.vc + head_rows * L::ROW, k_end * L::ROW);
  cp.init(F, lane);
  cp.issue(ring0, t_begin * 32, t_begin < t_end);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // q goes out with the first tile, the other tiles after
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 1; s < D - 1; ++s) cp.issue(ring0 + s * L::BYTES, (t_begin + s) * 32, t_begin + s < t_end);
  int slot = D - 1;  // ring stage of tile t + D - 1
  for (int t = t_begin; t < t_end; ++t) {
    cp.template wait_all_but<D - 2>();
    __syncthreads();  // tile t landed; tile t-1 consumed
    cp.issue(ring0 + slot * L::BYTES, (t + D - 1) * 32, t + D - 1 < t_end);
    slot = slot + 1 == D ? 0 : slot + 1;
  }
  wait_vmcnt<0>();  // copies past the last tile may still be landing
}

// Feeding waves of an instance: at head_dim 256 the waves beyond the compute
// waves of eight; at 128 (eight compute waves) four over an int8 cache, one
// per copy share, and the two copying waves over an fp16 cache.
template <int HD, int NQ, bool KV16>
constexpr int own_feeders() { return HD == 256 ? kWaves - NQ : (KV16 ? 2 : 4); }
template <int HD, int NQ, bool KV16>
constexpr int own_waves() { return NQ + own_feeders<HD, NQ, KV16>(); }

template <int HD, bool QF32, bool FINAL, int NQ, bool KV16>
__device__ __forceinline__ void attend_own_body(const AttendArgs& a) {
  static_assert((HD == 256 && NQ <= 6) || (HD == 128 && NQ == 8), "instances");
  using L = std::conditional_t<KV16, Stage16<HD>, Stage<HD>>;
  constexpr int NB = L::NB;                    // 32-dim blocks
  constexpr int NDT = HD / 16;                 // 16-dim output tiles
  constexpr int NF = own_feeders<HD, NQ, KV16>();  // feeding waves
  // ring stages: an int8 stage is free once converted (tiles t+1 .. t+3 in it);
  // an fp16 stage is read in place (tiles t .. t+3)
  constexpr int D = KV16 ? 4 : 3;
  // converted K fragments [b][u][lane], V^T fragments [d][hi|lo][lane] and K
  // scales [key][b] (int8 only)
  constexpr int KF_BYTES = KV16 ? 16 : NB * 2 * 1024;
  constexpr int VF_BYTES = KV16 ? 16 : NDT * 2 * 1024;
  constexpr int KS_BYTES = KV16 ? 16 : 32 * NB * 2;
  static_assert(NQ >= 2 && NQ <= 8, "two to eight compute waves");
  static_assert(D * L::BYTES + 2 * (KF_BYTES + VF_BYTES + KS_BYTES) <= 160 * 1024, "LDS");

  struct Ring {
    uint8_t* ring;
    uint32_t ring0;
    uint8_t (*kfrag)[KF_BYTES];
    uint8_t (*vfrag)[VF_BYTES];
    uint8_t (*kscale)[KS_BYTES];
    uint8_t (*vshift)[8];
  };
  __shared__ __attribute__((aligned(16))) uint8_t ring[D * L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kfrag[2][KF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vfrag[2][VF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kscale[2][KS_BYTES];
  __shared__ __attribute__((aligned(8))) uint8_t vshift[2][8];  // V fold shift per block (int8 cache)
  Ring rg_{ring, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring, kfrag, vfrag, kscale,
           vshift};

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
  const int nq = (M + 15) >> 4;
  const int n_keys = a.pos0 + r0 + nr;  // keys 0 .. n_keys-1 are seen by some row
  const int n_tiles = (n_keys + 31) >> 5;
  int t_begin, t_end;
  if (n_tiles <= 32767 && a.n_splits <= 65535) {
    t_begin = (int)((uint32_t)(split * n_tiles) / (uint32_t)a.n_splits);
    t_end = (int)((uint32_t)((split + 1) * n_tiles) / (uint32_t)a.n_splits);
  } else {
    t_begin = (int)(((long long)split * n_tiles) / a.n_splits);
    t_end = (int)(((long long)(split + 1) * n_tiles) / a.n_splits);
  }
  const int k_end = min(n_keys, t_end * 32);
  const size_t head_rows = (size_t)g * a.kv_stride;

  if (wave >= NQ) {
    // ---- feeders (each specialised by its index, so that its shares are
    // compile-time)
    if constexpr (KV16) {
      // two waves copy; any others only keep the barriers
      if (wave == NQ) own_feed16<HD, 2, 0, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_.ring0);
      else if (wave == NQ + 1) own_feed16<HD, 2, 1, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_.ring0);
      else {
        __builtin_amdgcn_s_barrier();
        for (int t = t_begin; t < t_end; ++t) __syncthreads();
      }
    } else {
      switch (wave - NQ) {
        case 0: own_feed<HD, NF, 0, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_); break;
        case 1: if constexpr (NF > 1) own_feed<HD, NF, 1, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_); break;
        case 2: if constexpr (NF > 2) own_feed<HD, NF, 2, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_); break;
        case 3: if constexpr (NF > 3) own_feed<HD, NF, 3, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_); break;
        case 4: if constexpr (NF > 4) own_feed<HD, NF, 4, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_); break;
        default: if constexpr (NF > 5) own_feed<HD, NF, 5, D>(a, head_rows, k_end, t_begin, t_end, lane, rg_); break;
      }
    }
    return;
  }

  // ---- compute waves.  q of the wave's vector (lane: vector n16, dims
  // 32b + 8*h4 + e), split hi + lo when given in fp32
  const bool own = wave < nq;  // wave-uniform
  const int v = wave * 16 + n16;
  const bool v_ok = own && v < M;
  const int vr = v_ok ? v / a.G : 0;
  const int vh = v_ok ? g * a.G + (v - vr * a.G) : 0;
  constexpr int NREG = QF32 ? 2 * NB : NB;
  float4_t regs[NREG];
#define QR(k) (__builtin_bit_cast(half8_t, regs[(k)]))
#pragma unroll
  for (int k = 0; k < NREG; ++k) regs[k] = (float4_t){0, 0, 0, 0};
  float xmul = 0.0f;
  {
    float4_t qraw[NREG];
#pragma unroll
    for (int k = 0; k < NREG; ++k) qraw[k] = (float4_t){0, 0, 0, 0};
    const size_t qoff = ((size_t)(r0 + vr) * a.Hq + vh) * HD + 8 * h4;
    if (v_ok) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (QF32) {
          const float4_t* p = (const float4_t*)((const float*)a.q + qoff + 32 * b);
          qraw[2 * b] = p[0];
          qraw[2 * b + 1] = p[1];
        } else {
          qraw[b] = *(const float4_t*)((const half_t*)a.q + qoff + 32 * b);
        }
      }
    }
    // the feeders' first tile goes out with q, the other tiles after this barrier
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    float qv[NB][8];
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (QF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[b][e] = qraw[2 * b][e];
          qv[b][4 + e] = qraw[2 * b + 1][e];
        }
      } else {
        const half8_t x = __builtin_bit_cast(half8_t, qraw[b]);
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
      half8_t hi8, lo8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qv[b][e] * qmul;
        const half_t hi = (half_t)x;
        hi8[e] = hi;
        lo8[e] = (half_t)(x - (float)hi);
      }
      regs[b] = __builtin_bit_cast(float4_t, hi8);
      if (QF32) regs[NB + b] = __builtin_bit_cast(float4_t, lo8);
    }
  }

  // last key this vector sees within the split, and the smallest over the
  // wave's vectors (a vector's row grows with its index): tiles ending at or
  // before it need no mask
  const int lim = min(v_ok ? a.pos0 + r0 + vr : -1, k_end - 1);
  const int lim_min = min(a.pos0 + r0 + (wave * 16) / a.G, k_end - 1);

  float m_ref = -INFINITY;  // reference point of the lane's vector (base 2)
  float l_part = 0.0f;      // this lane's share of the vector's sum
  float4_t O[NDT];          // O^T tile d: lane holds dims 16d + 4*h4 .. +3 of vector n16
#pragma unroll
  for (int d = 0; d < NDT; ++d) O[d] = (float4_t){0, 0, 0, 0};

  // tile t from buffer t & 1 (an fp16 cache: from its ring stage `st`)
  auto own_tile = [&](int t, const uint8_t* st) {
    const int key0 = t * 32;
    const uint8_t* kf = kfrag[t & 1];
    const half_t* Kst = (const half_t*)kscale[t & 1];
    // S^T = K Q^T, two blocks at a time for both 16-key subtiles: the hi MFMAs,
    // the lo MFMAs, then the per-block K scales in fp32, in block order (an fp16
    // K has no scales: every block accumulates into S^T, in block order)
    constexpr int KG = 2;
    float4_t s[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    if constexpr (KV16) {
#pragma unroll
      for (int b0 = 0; b0 < NB; b0 += KG) {
        half8_t kv[2][KG];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < KG; ++j) {
            const int key = 16 * u + n16;
            kv[u][j] = *(const half8_t*)(st + L::K_OFF + key * L::ROW + 16 * L::slot(key, 4 * (b0 + j) + h4));
          }
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            s[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[u][j], QR(b0 + j), s[u], 0, 0, 0);
            if (QF32) s[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[u][j], QR(NB + b0 + j), s[u], 0, 0, 0);
          }
      }
    } else {
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += KG) {
      half8_t kv[2][KG];
      ScaleRow<KG> dk[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int j = 0; j < KG; ++j) kv[u][j] = *(const half8_t*)(kf + (((b0 + j) * 2 + u) * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) dk[u][e].load(Kst + (16 * u + 4 * h4 + e) * NB + b0);
      }
      float4_t acc[2][KG];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < KG; ++j)
          acc[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[u][j], QR(b0 + j), (float4_t){0, 0, 0, 0}, 0, 0, 0);
      if (QF32) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < KG; ++j)
            acc[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[u][j], QR(NB + b0 + j), acc[u][j], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[u][e] = fmaf((float)dk[u][e].get(j), acc[u][j][e], s[u][e]);
    }
    }
    // mask and online softmax (base 2) on the unscaled dots (xmul > 0)
    float x[2][4];
    float tmax = -INFINITY;
    if (key0 + 31 <= lim_min) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] = s[u][e];
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] = key0 + 16 * u + 4 * h4 + e <= lim ? s[u][e] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, x[u][e]);
    tmax = wave_max_groups(tmax) * xmul;
    const bool need = tmax > m_ref + kRescaleSlack;
    float alpha = 1.0f;
    if (__any(need)) {
      const float m_new = need ? tmax - kRefBias : m_ref;
      alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      l_part *= alpha;
      m_ref = m_new;
    }
    const float mu = (m_ref == -INFINITY) ? 0.0f : m_ref;
    // p as fp16 hi (truncated) + lo: the B operand of O^T += V^T P^T, keys
    // pi(h4, e) as held in the S^T accumulators
    float p[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[4 * u + e] = __builtin_amdgcn_exp2f(fmaf(x[u][e], xmul, -mu));
        l_part += p[4 * u + e];
      }
    half8_t phi, plo;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(p[i], p[i + 1]));
      const half2_t l = __builtin_bit_cast(
          half2_t, __builtin_amdgcn_cvt_pkrtz(fmaf(-(float)h[0], 1.0f, p[i]), fmaf(-(float)h[1], 1.0f, p[i + 1])));
      phi[i] = h[0];
      phi[i + 1] = h[1];
      plo[i] = l[0];
      plo[i + 1] = l[1];
    }
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int d = 0; d < NDT; ++d) O[d] *= alpha;
    }
    if constexpr (KV16) {
      // O^T += (V,Phi) + (V,Plo) (an fp16 V is exact), two blocks at a time
#pragma unroll
      for (int b0 = 0; b0 < NB; b0 += 2) {
        half8_t vh8[2][2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) read_v16<HD>(b0 + jb, st, lane, vh8[jb]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int dd = 0; dd < 2; ++dd)
            O[2 * (b0 + jb) + dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh8[jb][dd], phi, O[2 * (b0 + jb) + dd], 0, 0, 0);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int dd = 0; dd < 2; ++dd)
            O[2 * (b0 + jb) + dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh8[jb][dd], plo, O[2 * (b0 + jb) + dd], 0, 0, 0);
      }
    } else {
    // O^T += (Vhi,Phi) + (Vlo,Phi) + (Vhi,Plo), four output tiles at a time
    const uint8_t* vf = vfrag[t & 1];
    // a block with a shifted V fold (rare: a V scale above 512) takes this
    // tile's sum in units of 2^s: O *= 2^-s before its MFMAs, O *= 2^s after
    const uint2 shw = *(const uint2*)vshift[t & 1];
    const bool shifted = (shw.x | (NB > 4 ? shw.y : 0u)) != 0;  // bytes past NB are never written
    auto fold_scale = [&](int sign) {
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        const int b = d >> 1;
        const int sh = ((b < 4 ? shw.x : shw.y) >> (8 * (b & 3))) & 0xff;
        O[d] *= ldexpf(1.0f, sign * sh);
      }
    };
    if (__builtin_expect(shifted, 0)) fold_scale(-1);
#pragma unroll
    for (int d0 = 0; d0 < NDT; d0 += 4) {
      half8_t vh8[4], vl8[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vh8[i] = *(const half8_t*)(vf + (((d0 + i) * 2 + 0) * 64 + lane) * 16);
        vl8[i] = *(const half8_t*)(vf + (((d0 + i) * 2 + 1) * 64 + lane) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) O[d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh8[i], phi, O[d0 + i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl8[i], phi, O[d0 + i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[d0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh8[i], plo, O[d0 + i], 0, 0, 0);
    }
    if (__builtin_expect(shifted, 0)) fold_scale(1);
    }
  };

  // the same barriers as the feeders' loop: iteration t_begin - 1 converts the
  // first tile
  if constexpr (KV16) {
    int slot = 0;  // ring stage of tile t
    for (int t = t_begin; t < t_end; ++t) {
      __syncthreads();
      if (own) own_tile(t, ring + slot * L::BYTES);
      slot = slot + 1 == D ? 0 : slot + 1;
    }
  } else {
    for (int t = t_begin - 1; t < t_end; ++t) {
      __syncthreads();
      if (own && t >= t_begin) own_tile(t, nullptr);
    }
  }

  // ---- output of the wave's vectors
  if (own) {
    const float l_tot = wave_sum_groups(l_part);
    if (v_ok) {
      const int orow = r0 + vr;
      if (FINAL) {
        const float inv_l = 1.0f / l_tot;
        float* dst = a.out + ((size_t)orow * a.Hq + vh) * HD + 4 * h4;
#pragma unroll
        for (int d = 0; d < NDT; ++d) *(float4_t*)(dst + 16 * d) = O[d] * inv_l;
      } else {
        const size_t idx = ((size_t)split * a.n_rows + orow) * a.Hq + vh;
        float* dst = a.part_o + idx * HD + 4 * h4;
#pragma unroll
        for (int d = 0; d < NDT; ++d) *(float4_t*)(dst + 16 * d) = O[d];
        if (h4 == 0) a.part_ml[idx] = make_float2(m_ref, l_tot);
      }
    }
  }
#undef QR
}

template <int HD, bool QF32, bool FINAL, int NQ>
__global__ __launch_bounds__((64 * own_waves<HD, NQ, false>())) void attend_own_q8_kernel(const AttendArgs a) {
  attend_own_body<HD, QF32, FINAL, NQ, false>(a);
}

// The same layout over an fp16 K/V cache (no scales, no conversion).
template <int HD, bool QF32, bool FINAL, int NQ>
__global__ __launch_bounds__((64 * own_waves<HD, NQ, true>())) void attend_own_f16kv_kernel(const AttendArgs a) {
  attend_own_body<HD, QF32, FINAL, NQ, true>(a);
}

}  // namespace attnq8
