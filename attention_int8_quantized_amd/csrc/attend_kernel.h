// The int8-KV attention kernel shared by the verify and prompt paths.
//
// One workgroup of eight waves (twelve for two or three vector tiles at head_dim
// 256: body_waves) owns up to NQ x 16 query vectors (row, Q head)
// of a group of consecutive rows that read one KV head -- the "one owner of
// several query rows shares every K/V scan" organisation of "perf(gfx1100):
// share Q8 KV scans across verifier rows" (Summary) -- and scans one range of
// that head's keys in 32-key tiles.
//
// Per tile t (one workgroup barrier per tile):
//   copy     the tile's int8 codes and fp16 scales go from HBM straight into a
//            ring of tiles in LDS (direct-to-LDS buffer loads, kCopyLead tiles
//            in flight); buffer ranges end at the split's last key,
//            so the ragged last tile reads zeros.
//   convert  (tile t+1) K codes -> fp16 MFMA fragments in LDS, exact; each
//            PV wave reads its 32-dim blocks of V transposed with the gfx950
//            ds_read_b64_tr_b8 and keeps dV * code in registers as an exact
//            fp16 hi + lo pair (dV * code has at most 18 significant bits; hi
//            is the rounded product, lo the fma residual; a block with a V
//            scale above 512 takes a power-of-two shift, undone in fp32).
//   QK       (tile t, one wave per 16 vectors) S^T = K Q^T on
//            v_mfma_f32_16x16x32_f16, one 32-dim block per MFMA (q in registers,
//            split hi + lo when given in fp32 after a per-vector power-of-two
//            scaling that keeps both parts normal), each block's dot scaled by
//            its fp16 K scale in fp32 in fixed block order; causal / range
//            mask; online softmax in base 2 with a lazily moved reference point;
//            p split into fp16 hi + lo and handed to every wave through LDS
//            with the tile's rescale factor.
//   PV       (tile t-1) each PV wave owns 32-dim blocks of the output for
//            its share of the vectors: O^T *= alpha, then
//            O^T += V^T P^T as (Vhi,Phi) + (Vlo,Phi) + (Vhi,Plo).
// PV trails QK by one tile.  Which waves do QK, PV, the K conversion and the
// copies depends on the number of vector tiles (Roles below); each role runs
// its own loop with the same barriers, and the roles are spread so that every
// SIMD of the compute unit carries both MFMA and VALU work.
//
// The accuracy contract of "hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA
// prompt attention" (How: fp16 hi+lo of q and p, fixed summation order, online
// softmax, V scale folded into p) is kept in substance; the V scale is folded
// into an exact hi+lo V fragment instead of into p (converted once per tile
// for all of the workgroup's vectors).  The fold is exact for V scales up to
// 512; a block of a tile with a larger scale is folded with a power-of-two
// shift that the PV step undoes in fp32 (see kVScaleFoldMax).
//
// The workgroup writes either split partials (m, l, o) or, when it covers every
// key its rows see, the normalised output.
#pragma once

#include <type_traits>

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
constexpr int kCopyLead = 3;  // tiles in flight ahead of the one being converted

// LDS layout of one 32-key ring stage (bytes):
//   K codes  [32 keys][HD]  int8, 16-byte chunks of a row permuted by chunk_slot
//   V codes  [32 keys][HD]  int8, same permutation
//   K scales [32 keys][HD/32] fp16
//   V scales [32 keys][HD/32] fp16
template <int HD>
struct Stage {
  static constexpr int NB = HD / 32;
  static constexpr int ROW = HD;                              // bytes per key row of a plane
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
  __device__ static int slot(int key, int c);
};

// MFMA fragments, 64 lanes x 16 B = 1 KB each:
//   K fragment [block b][subtile u]: K codes as fp16, A operand of S^T = K Q^T;
//      lane l: key 16u + l%16, dims 32b + 8(l/16) .. +7
//   V^T fragment [dim tile d]: dV * code as fp16 (hi or lo), A operand of
//      O^T += V^T P^T; lane l: dim 16d + l%16, keys pi(l/16, e), e = 0..7
//   P^T fragment [vector tile n]: p as fp16 (hi or lo), B operand of the same;
//      lane l: vector 16n + l%16, keys pi(l/16, e), which are the keys that
//      the lane holds in the S^T accumulators of its two 16-key subtiles
//   with pi(h, e) = 4h + e for e < 4 and 16 + 4h + e - 4 for e >= 4.
// Slot of 16-byte chunk `c` of tile row `key` (0..31) -- an involution in c.
// Chosen so that the rows read by one 16-lane group -- 16 consecutive keys for
// K fragments, keys {4h..4h+3, 16+4h..16+4h+3} for the transposing V reads --
// land in distinct 16-byte bank groups.
template <int HD>
__device__ __forceinline__ int chunk_slot(int key, int c) {
  constexpr int C = Stage<HD>::C, R = Stage<HD>::R;
  return c ^ (((key / R) ^ ((key >> 4) * (C / 2))) & (C - 1));
}

template <int HD>
__device__ __forceinline__ int Stage<HD>::slot(int key, int c) { return chunk_slot<HD>(key, c); }

__device__ __forceinline__ int pi_key(int h, int e) { return (e < 4) ? 4 * h + e : 16 + 4 * h + (e - 4); }

// LDS layout of one 32-key ring stage of an fp16 cache (bytes):
//   K  [32 keys][HD] fp16, 16-byte chunks of a row permuted by slot()
//   V  [32 keys][HD] fp16, same permutation
// slot(key, c) = c ^ f(key) is an involution in c.  With 512- or 256-byte rows
// (head_dim 256, 128) a row starts on the same bank group, and f takes 16
// distinct values over any 16 consecutive keys (the K fragment reads) and 8
// distinct slots over the 4 keys x 2 chunks of a transposing V read; with
// 128-byte rows (head_dim 64) f spreads 16 consecutive keys over both halves of
// the 256-byte bank cycle.
template <int HD>
struct Stage16 {
  static constexpr int NB = HD / 32;
  static constexpr int ROW = 2 * HD;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 64 * HD;
  static constexpr int KS_OFF = 0;  // no scale planes
  static constexpr int VS_OFF = 0;
  static constexpr int BYTES = 128 * HD;
  static constexpr int CODE_OPS = HD / 16;  // 1 KB copies per plane
  static constexpr int SCALE_OPS = 0;
  static constexpr int C = HD / 8;          // 16-byte chunks per key row
  __device__ static int slot(int key, int c) {
    if constexpr (C >= 16) return c ^ (2 * (key & 7) + ((key >> 3) & 1));
    else return c ^ ((key >> 1) & (C - 1));
  }
};

// The workgroup's direct-to-LDS copies of one 32-key tile, split over NW of its
// waves.  A tile is CODE_OPS 1 KB copies of K codes, the same of V codes (the
// same rows and chunk permutation, so a K copy and a V copy share their lane
// offsets) and SCALE_OPS copies of each scale plane.  With CODE_OPS >= NW the
// wave with index w copies code chunks w, w + NW, ... of both planes; with
// fewer chunks than waves the first CODE_OPS waves copy one chunk of each.  The
// scale copies go one per wave to the waves after those (or from wave 0 when
// every wave copies codes).  Offsets are computed once; per tile only the key
// offset is added.
template <class L, int NW>
struct TileCopier {
  static constexpr int HD = L::NB * 32;
  static constexpr bool WIDE = L::CODE_OPS >= NW;
  static constexpr int CPW = WIDE ? L::CODE_OPS / NW : 1;  // code chunks per copying wave
  static constexpr int NS = 2 * L::SCALE_OPS;              // scale copies per tile
  static_assert(!WIDE || L::CODE_OPS % NW == 0, "code chunks must split evenly");
  static_assert((WIDE ? 0 : L::CODE_OPS) + NS <= NW, "one scale copy per wave at most");

  __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
  int lane;
  bool codes;        // this wave copies code chunks (wave-uniform)
  int s_op;          // scale copy of this wave (< 0: none; < SCALE_OPS: K, else V)
  int code_off[CPW]; // per lane: byte offset of the chunk within the tile's rows
  uint32_t code_lds[CPW];
  int s_off;         // per lane: byte offset within the tile's scale plane (< 0: lane idle)
  uint32_t s_lds;

  __device__ __forceinline__ void init(int w, int lane_) {
    lane = lane_;
    codes = WIDE || w < L::CODE_OPS;
#pragma unroll
    for (int r = 0; r < CPW; ++r) {
      const int j = WIDE ? w + NW * r : w;  // chunk index within a plane
      const int pos = j * 1024 + 16 * lane;
      const int row = pos / L::ROW;
      code_off[r] = row * L::ROW + 16 * L::slot(row, (pos % L::ROW) / 16);
      code_lds[r] = j * 1024;
    }
    s_op = w - (WIDE ? 0 : L::CODE_OPS);
    if (s_op >= NS) s_op = -1;
    if constexpr (L::SCALE_OPS > 0) {
      const int jj = s_op % L::SCALE_OPS;
      const int byte = jj * 256 + 4 * lane;
      s_off = byte < 2 * HD ? byte : -1;
      s_lds = (s_op >= L::SCALE_OPS ? L::VS_OFF : L::KS_OFF) + jj * 256;
    } else {
      s_off = -1;
      s_lds = 0;
    }
  }

  // copies per tile issued by this wave
  __device__ __forceinline__ int count() const { return (codes ? 2 * CPW : 0) + (s_op >= 0 ? 1 : 0); }

  // Copy the tile starting at key0 into the stage at lds (zeros when !live:
  // the key offset then lies past every buffer range).
  __device__ __forceinline__ void issue(uint32_t lds, int key0, bool live) const { issue_part(lds, key0, live, 0, 1); }

  // Part `part` of `nparts` of those copies (code chunks split evenly, the
  // scale copy with the last part), so that a wave can spread its copies
  // between other work instead of queueing them back to back.
  __device__ __forceinline__ void issue_part(uint32_t lds, int key0, bool live, int part, int nparts) const {
    const int k0 = live ? key0 : (1 << 22);  // wave-uniform
    if (codes) {
#pragma unroll
      for (int r = 0; r < CPW; ++r) {
        if (r * nparts < part * CPW || r * nparts >= (part + 1) * CPW) continue;
        const int off = k0 * L::ROW + code_off[r];
        dma_b128(kc, lds + L::K_OFF + code_lds[r], off);
        dma_b128(vc, lds + L::V_OFF + code_lds[r], off);
      }
    }
    if constexpr (L::SCALE_OPS > 0) {
      if (part == nparts - 1 && s_op >= 0 && s_off >= 0) {
        const int off = k0 * 2 * L::NB + s_off;
        if (s_op < L::SCALE_OPS) dma_b32(ks, lds + s_lds, off);
        else dma_b32(vs, lds + s_lds, off);
      }
    }
  }

  // Wait until this wave's copies of all but the newest `newer` tiles landed.
  template <int newer>
  __device__ __forceinline__ void wait_all_but() const {
    if (count() == 2 * CPW + 1) wait_vmcnt<(2 * CPW + 1) * newer>();
    else if (count() == 2 * CPW) wait_vmcnt<2 * CPW * newer>();
    else if (count() == 1) wait_vmcnt<newer>();
    else wait_vmcnt<0>();
  }
};

// SH consecutive shares (of NW) of a tile's copies, issued by one wave.
template <class L, int NW, int SH>
struct Copiers {
  TileCopier<L, NW> c[SH];

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t kc, __amdgpu_buffer_rsrc_t vc,
                                       __amdgpu_buffer_rsrc_t ks, __amdgpu_buffer_rsrc_t vs, int first,
                                       int lane) {
#pragma unroll
    for (int s = 0; s < SH; ++s) {
      c[s].kc = kc;
      c[s].vc = vc;
      c[s].ks = ks;
      c[s].vs = vs;
      c[s].init(first + s, lane);
    }
  }
  __device__ __forceinline__ int count() const {
    int n = 0;
#pragma unroll
    for (int s = 0; s < SH; ++s) n += c[s].count();
    return n;
  }
  __device__ __forceinline__ void issue(uint32_t lds, int key0, bool live) const {
#pragma unroll
    for (int s = 0; s < SH; ++s) c[s].issue(lds, key0, live);
  }
  __device__ __forceinline__ void issue_part(uint32_t lds, int key0, bool live, int part, int nparts) const {
#pragma unroll
    for (int s = 0; s < SH; ++s) c[s].issue_part(lds, key0, live, part, nparts);
  }
  // this wave's copies of all but the newest `newer` tiles landed
  template <int newer>
  __device__ __forceinline__ void wait_all_but() const {
    if constexpr (SH == 1) {
      c[0].template wait_all_but<newer>();
    } else {
      switch (count()) {  // wave-uniform
#define ATTNQ8_WAIT_CASE(k) \
  case k: wait_vmcnt<(k) * newer>(); break;
        ATTNQ8_WAIT_CASE(1) ATTNQ8_WAIT_CASE(2) ATTNQ8_WAIT_CASE(3) ATTNQ8_WAIT_CASE(4)
        ATTNQ8_WAIT_CASE(5) ATTNQ8_WAIT_CASE(6) ATTNQ8_WAIT_CASE(7) ATTNQ8_WAIT_CASE(8)
        ATTNQ8_WAIT_CASE(9) ATTNQ8_WAIT_CASE(10) ATTNQ8_WAIT_CASE(11) ATTNQ8_WAIT_CASE(12)
#undef ATTNQ8_WAIT_CASE
        default: wait_vmcnt<0>(); break;
      }
    }
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

// K codes of block b, subtile u of the ring stage `st` -> the K fragment in `kf`.
template <int HD>
__device__ __forceinline__ void convert_k(int b, int u, const uint8_t* st, uint8_t* kf, int lane) {
  using L = Stage<HD>;
  const int h4 = lane >> 4;
  const int c = 2 * b + (h4 >> 1);
  const int key = 16 * u + (lane & 15);
  const uint2 w = *(const uint2*)(st + L::K_OFF + key * HD + 16 * chunk_slot<HD>(key, c) + 8 * (h4 & 1));
  *(half8_t*)(kf + ((b * 2 + u) * 64 + lane) * 16) = codes8_to_f16(w.x, w.y);
}

// The V-scale fold.  The V^T fragments hold dV * code as an exact fp16 hi + lo
// pair: with |code| <= 127 the product has at most 18 significant bits, and
// while |dV| <= 512 its magnitude stays at most 65,024, inside fp16's range;
// every bit of it lies at or above dV's last bit, so the pair is exact down to
// fp16's subnormal scales.  A block of a tile that holds a larger scale (the
// Q8 format allows any fp16 scale: blocks whose largest element exceeds about
// 65,024 in magnitude) takes a shift s, the smallest with
// max |dV| * 2^-s <= 512: its scales are multiplied by 2^-s in fp16 (exact
// for every scale of at least 2^(s-14); a smaller one in such a block is
// rounded to fp16's subnormal step), the fragments hold
// (dV * 2^-s) * code, and the PV step brackets that tile's MFMAs for the block
// with O *= 2^-s and O *= 2^s (fold_scale; exact in fp32: the sum is taken in
// units of 2^s, with the same roundings relative to its magnitude).
constexpr uint16_t kVScaleFoldMax = 0x6000;  // 512.0 in fp16

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// Whether this lane's eight V scales include one above 512 in magnitude (or a
// negative, infinite or NaN one: every sign-bit pattern compares above).
__device__ __forceinline__ bool v_scales_large(half8_t sc) {
  const u16x8_t b = __builtin_bit_cast(u16x8_t, sc);
  const u16x4_t m4 = __builtin_elementwise_max(b.lo, b.hi);
  const u16x2_t m2 = __builtin_elementwise_max(m4.lo, m4.hi);
  return (m2.x > kVScaleFoldMax) | (m2.y > kVScaleFoldMax);
}

// The fold shift of a block (wave-uniform) from the scales of the tile's 32
// keys (each 16-lane group holds those of eight keys pi(h4, e)); when it is
// not 0 the scales are multiplied by 2^-s in place.
__device__ __forceinline__ int v_fold_prescale(half8_t& sc) {
  if (__builtin_expect(!__any(v_scales_large(sc)), 1)) return 0;
  float mx = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf((float)sc[e]));
  mx = wave_max_groups(mx);
  int ex = 0;
  (void)frexpf(mx, &ex);  // mx < 2^ex
  const int s = min(15, max(0, ex - 9));
  sc = sc * (half_t)ldexpf(1.0f, -s);  // 2^-s, s <= 15, is an fp16 value
  return s;
}

// O *= 2^(sign * s) for the accumulators O[jb][..][..] of each block jb with a
// shifted V fold: before a tile's PV MFMAs (sign -1) the block's sum is taken
// in units of 2^s, after them (sign +1) it returns to the plain units.
// Scaling by a power of two is exact in fp32 and commutes with the rescale by
// alpha, so the order of the two does not change a bit.
template <class Acc, int NBL>
__device__ __forceinline__ void fold_scale(Acc& O, const int (&sh)[NBL], int sign) {
#pragma unroll
  for (int jb = 0; jb < NBL; ++jb) {
    const float f = ldexpf(1.0f, sign * sh[jb]);
    constexpr int NI = std::extent<std::remove_reference_t<decltype(O[0])>>::value;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      O[jb][i][0] *= f;
      O[jb][i][1] *= f;
    }
  }
}

// K units k0, k0 + step, ... (unit k: block k >> 1, 16-key subtile k & 1) of the
// ring stage `st` -> K fragments in `kf`: every read is issued before the
// first conversion, so their latencies overlap.
template <int HD, int STEP>
__device__ __forceinline__ void convert_k_share(int k0, const uint8_t* st, uint8_t* kf, int lane) {
  using L = Stage<HD>;
  constexpr int NU = 2 * L::NB;
  static_assert(NU % STEP == 0, "units split evenly");
  constexpr int N = NU / STEP;
  const int h4 = lane >> 4;
  uint2 w[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int k = k0 + STEP * j;
    const int c = 2 * (k >> 1) + (h4 >> 1);
    const int key = 16 * (k & 1) + (lane & 15);
    w[j] = *(const uint2*)(st + L::K_OFF + key * HD + 16 * chunk_slot<HD>(key, c) + 8 * (h4 & 1));
  }
#pragma unroll
  for (int j = 0; j < N; ++j)
    *(half8_t*)(kf + ((k0 + STEP * j) * 64 + lane) * 16) = codes8_to_f16(w[j].x, w[j].y);
}

// What convert_v reads of block b (dim tiles 2b, 2b+1) from the ring stage
// `st`: the lane's eight per-key V scales (keys pi(h4, e)) and its two
// transposing reads of the codes (lane 16h + 2k + s addresses key pi(h, k),
// dims 16d + 8s).
struct VLoad {
  half8_t sc;
  v2i32_t w[2];
};
template <int HD>
__device__ __forceinline__ VLoad load_v(int b, const uint8_t* st, int lane) {
  using L = Stage<HD>;
  constexpr int NB = L::NB;
  const int h4 = lane >> 4;
  VLoad r;
  const half_t* vsc = (const half_t*)(st + L::VS_OFF);
#pragma unroll
  for (int e = 0; e < 8; ++e) r.sc[e] = vsc[pi_key(h4, e) * NB + b];
  const int vkey = pi_key(h4, (lane & 15) >> 1);
  const uint8_t* vrow = st + L::V_OFF + vkey * HD + 8 * (lane & 1);
#pragma unroll
  for (int dd = 0; dd < 2; ++dd)
    r.w[dd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i32_t*)(vrow + 16 * chunk_slot<HD>(vkey, 2 * b + dd)));
  return r;
}

// codes -> exact fp16, times the (possibly shifted) scales -> V^T fragments as
// exact fp16 hi + lo pairs.
__device__ __forceinline__ void fold_v(const v2i32_t (&w)[2], half8_t sc, half8_t (&vh)[2], half8_t (&vl)[2]) {
#pragma unroll
  for (int dd = 0; dd < 2; ++dd) {
    const half8_t c = codes8_to_f16((uint32_t)w[dd][0], (uint32_t)w[dd][1]);
    vh[dd] = c * sc;
    vl[dd] = __builtin_elementwise_fma(c, sc, -vh[dd]);
  }
}

// V codes of block b (dim tiles 2b, 2b+1) of the ring stage `st`, times their
// per-key scales -> V^T fragments as exact fp16 hi + lo pairs in registers.
// Returns the block's fold shift (wave-uniform; 0 unless a scale exceeds 512).
template <int HD>
__device__ __forceinline__ int convert_v(int b, const uint8_t* st, int lane, half8_t (&vh)[2], half8_t (&vl)[2]) {
  VLoad r = load_v<HD>(b, st, lane);
  const int s = v_fold_prescale(r.sc);
  fold_v(r.w, r.sc, vh, vl);
  return s;
}

// V of block b (dim tiles 2b, 2b+1) of an fp16 ring stage -> V^T fragments
// (exact: no lo part).  ds_read_b64_tr_b16: within a 16-lane group, lane j
// receives element j % 4 of the 8-byte segments addressed by lanes j / 4 + 4i,
// i = 0..3 (checked on the GPU with an in-bounds probe).  Lane q + 4i of group h
// addresses key pi(h, i) (then pi(h, 4 + i)) at dims 16d + 4q, so that lane j
// receives dim 16d + j of keys pi(h, 0..7): the same fragment as convert_v.
template <int HD>
__device__ __forceinline__ void read_v16(int b, const uint8_t* st, int lane, half8_t (&vh)[2]) {
  using L = Stage16<HD>;
  const int h4 = lane >> 4;
  const int q = lane & 3;
  const int i = (lane & 15) >> 2;
#pragma unroll
  for (int dd = 0; dd < 2; ++dd) {
    const int c = 4 * b + 2 * dd + (q >> 1);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int key = pi_key(h4, 4 * half + i);
      const uint8_t* p = st + L::V_OFF + key * L::ROW + 16 * L::slot(key, c) + 8 * (q & 1);
      const half4_t v = __builtin_bit_cast(
          half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)p));
#pragma unroll
      for (int e = 0; e < 4; ++e) vh[dd][4 * half + e] = v[e];
    }
  }
}

// Work split of a workgroup over its waves (eight, or twelve: body_waves).
// With at most four vector tiles (NQ <= 4: verify row groups) the roles are
// disjoint: waves 0..NQ-1 own one vector tile each for QK and do nothing
// else; waves 4.. own the 32-dim blocks for PV (one each with twelve waves;
// two each at head_dim 256 with eight; at 64 a block for half the vector
// tiles).  In an instance for two or three vector tiles K is converted by
// the waves NQ..3, which own no vector tile, in one for four by the PV waves.
// The tile copies are issued by the K-converting waves in the instance for
// two vector tiles over an int8 cache, else by the PV waves, so that the QK
// waves' loads of q never queue behind them.  With eight vector tiles
// (NQ == 8: prompt blocks) every wave owns a block (or a block for a share of
// the vector tiles) for PV, converts K and issues copies, and the first nq
// waves also own a vector tile for QK.
constexpr int kWaves = 8;

// Waves per workgroup of an attention-body instance: twelve (three per SIMD,
// one 32-dim block per PV wave) for row groups of two or three vector tiles at
// head_dim 256 over an int8 cache, else eight.
template <int HD, int NQ, bool KV16>
constexpr int body_waves() { return (!KV16 && HD == 256 && (NQ == 2 || NQ == 3)) ? 12 : kWaves; }

template <int HD, int NQ, bool KV16 = false>
struct Roles {
  static constexpr bool SPLIT = NQ <= 4;
  static constexpr int NW = body_waves<HD, NQ, KV16>();
  static constexpr int PV0 = SPLIT ? 4 : 0;  // first PV wave
  static constexpr int NPV = NW - PV0;       // PV waves
  static constexpr int NB = Stage<HD>::NB;
  static_assert(NQ == 2 || NQ == 3 || NQ == 4 || NQ == 8, "vector tiles per workgroup");
  static constexpr int BPW = NB > NPV ? NB / NPV : 1;  // PV blocks per wave
  static constexpr int GW = NPV > NB ? NPV / NB : 1;   // PV waves sharing one block
  static constexpr int NQW = NQ / GW;                  // vector tiles per PV wave
  static_assert(NQ % GW == 0, "vector tiles must split evenly over the waves");
  // PV block j of wave `wave` (NB: none)
  __device__ static int block(int wave, int j) { return wave >= PV0 ? (wave - PV0) % NB + NPV * j : NB; }
  // first vector tile of the wave's PV share (then every GW-th)
  __device__ static int qtile0(int wave) { return (wave - PV0) / NB; }
  // waves that convert K, and this wave's index among them (< 0: none)
  // (an instance for fewer than four vector tiles: waves NQ..3, which own none;
  // else the PV waves)
  static constexpr bool K_ON_QK_SIDE = SPLIT && NQ < 4;
  static constexpr int KW = K_ON_QK_SIDE ? 4 - NQ : NPV;
  __device__ static int k_workers(int) { return KW; }
  __device__ static int k_index(int wave, int) {
    return K_ON_QK_SIDE ? (wave >= NQ && wave < 4 ? wave - NQ : -1) : wave - PV0;
  }
  // waves that issue the tile copies: in the instance for two vector tiles
  // over an int8 cache the K-converting waves 2 and 3, two of four copy shares
  // each (the PV waves then only convert V and multiply); else the PV waves,
  // one share each.  copy_index: the wave's first share (< 0: none).
  static constexpr bool COPY_ON_K = !KV16 && K_ON_QK_SIDE && NQ == 2;
  static constexpr int NWI = COPY_ON_K ? 4 : NPV;
  static constexpr int SHARES = COPY_ON_K ? 4 / KW : 1;
  __device__ static int copy_index(int wave) {
    return COPY_ON_K ? (wave >= NQ && wave < 4 ? (wave - NQ) * SHARES : -1) : wave - PV0;
  }
};

// HD: head dim; QF32: q given in fp32 (else fp16); FINAL: write the normalised
// output (else split partials); NQ: most 16-vector tiles per workgroup; KV16:
// the cache holds fp16 K and V (no scales) instead of int8 blocks.
template <int HD, bool QF32, bool FINAL, int NQ, bool KV16>
__device__ __forceinline__ void attend_body(const AttendArgs& a) {
  using L = std::conditional_t<KV16, Stage16<HD>, Stage<HD>>;
  using R = Roles<HD, NQ, KV16>;
  constexpr int NW = R::NW;
  constexpr int NB = L::NB;
  // ring stages: tiles t (QK, V), t+1 (K conversion) and the copies in
  // flight, plus t-1 where PV converts V^T of its tile when it multiplies it.
  // An fp16 stage is twice as large, so the prompt layout keeps one copy
  // fewer in flight; with no K conversion a tile is needed only at its own
  // iteration, so one more copy stays in flight at the barrier.
  constexpr int LEAD = (KV16 && !R::SPLIT) ? kCopyLead - 1 : kCopyLead;
  constexpr int D = R::SPLIT ? LEAD + 1 : LEAD + 2;
  constexpr int WAIT_NEWER = KV16 ? LEAD - 1 : LEAD - 2;
  constexpr int BPW = R::BPW;
  constexpr int GW = R::GW;
  constexpr int NQW = R::NQW;
  constexpr int KF_BYTES = KV16 ? 16 : NB * 2 * 1024;
  constexpr int PB_BYTES = NQ * 2 * 1024;
  static_assert(NQ <= NW, "one QK wave per vector tile");
  static_assert(D * L::BYTES + 2 * KF_BYTES + 2 * PB_BYTES + 3 * NQ * 16 * 8 <= 160 * 1024,
                "LDS per workgroup");

  __shared__ __attribute__((aligned(16))) uint8_t ring[D * L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t kfrag[2][KF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t pfrag[2][PB_BYTES];  // [n][hi|lo][lane]
  __shared__ float alpha_s[2][NQ][16];
  __shared__ float2 ml_s[NQ][16];

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
  const int nq = (M + 15) >> 4;         // vector tiles (<= NQ, checked on the host)
  const int n_keys = a.pos0 + r0 + nr;  // keys 0 .. n_keys-1 are seen by some row
  const int n_tiles = (n_keys + 31) >> 5;
  // this split's tiles [t_begin, t_end): 32-bit arithmetic while the products
  // fit (the usual case), 64-bit otherwise
  int t_begin, t_end;
  if (n_tiles <= 32767 && a.n_splits <= 65535) {
    t_begin = (int)((uint32_t)(split * n_tiles) / (uint32_t)a.n_splits);
    t_end = (int)((uint32_t)((split + 1) * n_tiles) / (uint32_t)a.n_splits);
  } else {
    t_begin = (int)(((long long)split * n_tiles) / a.n_splits);
    t_end = (int)(((long long)(split + 1) * n_tiles) / a.n_splits);
  }
  const int k_end = min(n_keys, t_end * 32);

  // ---- QK role: vector tile `wave` (column n16 of its S^T tile)
  const int v = wave * 16 + n16;
  const bool v_ok = wave < nq && v < M;
  const int vr = v_ok ? v / a.G : 0;
  const int vh = v_ok ? g * a.G + (v - vr * a.G) : 0;

  // ---- the tile copier: tile t is copied D-2 iterations ahead into ring
  // stage t % D
  const size_t head_rows = (size_t)g * a.kv_stride;
  constexpr int NWI = R::NWI;
  const bool copies = R::copy_index(wave) >= 0;  // wave-uniform
  Copiers<L, NWI, R::SHARES> cp;
  {
    const auto kc = make_rsrc((const int8_t*)a.kc + head_rows * L::ROW, k_end * L::ROW);
    const auto vc = make_rsrc((const int8_t*)a.vc + head_rows * L::ROW, k_end * L::ROW);
    auto ks = kc, vs = vc;  // (unused over an fp16 cache)
    if constexpr (!KV16) {
      ks = make_rsrc(a.ks + head_rows * NB, k_end * NB * 2);
      vs = make_rsrc(a.vs + head_rows * NB, k_end * NB * 2);
    }
    cp.init(kc, vc, ks, vs, copies ? R::copy_index(wave) : NWI, lane);
  }
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  auto issue_first = [&](int n0, int n1) {
    if (copies) {
#pragma unroll
      for (int s = n0; s < n1; ++s)
        cp.issue(ring0 + s * L::BYTES, (t_begin + s) * 32, t_begin + s < t_end);
    }
  };

  // ---- the q loads and tile 0 go out first, the other tiles in flight only
  // after a barrier: at the start every CU requests its tiles at once, and q
  // (an L2 hit for all but the first workgroup of a head) and each CU's first
  // tile would otherwise return behind the others' later tiles.  Loads and their use stay in one block, so the
  // compiler's wait counting carries no q load into the other waves' loops
  // (a wait placed there for a q register would also wait for every copy).
  const bool qk = wave < nq;  // wave-uniform
  constexpr int NREG = QF32 ? 2 * NB : NB;
  float4_t regs[NREG];
#define QR(k) (__builtin_bit_cast(half8_t, regs[(k)]))
#pragma unroll
  for (int k = 0; k < NREG; ++k) regs[k] = (float4_t){0, 0, 0, 0};
  float xmul = 0.0f;
  if (qk) {
    constexpr int QRAW = QF32 ? 2 * NB : NB;
    float4_t qraw[QRAW];
    const size_t qoff = ((size_t)(r0 + vr) * a.Hq + vh) * HD + 8 * h4;
#pragma unroll
    for (int k = 0; k < QRAW; ++k) qraw[k] = (float4_t){0, 0, 0, 0};
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
    issue_first(0, 1);
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
  } else {
    issue_first(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  issue_first(1, LEAD);

  const int lim = v_ok ? a.pos0 + r0 + vr : -1;  // last key this vector sees
  const int lim_eff = min(lim, k_end - 1);        // ... within this split
  // the smallest of those over the wave's vectors (wave-uniform): tiles that end
  // at or before it need no mask.  A vector's row grows with its index, so it
  // is the wave's first vector's (valid for every QK wave).
  const int lim_min = min(a.pos0 + r0 + (wave * 16) / a.G, k_end - 1);

  // The q fragments of the QK role (set up above) are held across tiles as
  // the B operand of S^T = K Q^T (lane: vector n16, dims 32b + 8*h4 + e; hi
  // in QR(b), lo in QR(NB + b)).  Each role loop below keeps its own
  // accumulators.
  float m_ref = -INFINITY;  // QK role: reference point of the vector (base 2)
  float l_part = 0.0f;      // QK role: this lane's share of the vector's sum

  // ---- PV role: blocks R::block(wave, j), vector tiles q0, q0 + GW, ...
  const int q0 = R::qtile0(wave);
  int nblk = 0;  // PV blocks of this wave (wave-uniform)
#pragma unroll
  for (int jb = 0; jb < BPW; ++jb) nblk += R::block(wave, jb) < NB;
  const int kw = R::k_workers(nq);
  const int ki = R::k_index(wave, nq);

  // ---- prologue: K fragments of the first tile (an fp16 cache is read in place)
  if constexpr (!KV16) {
    if (t_begin < t_end) {
      if (copies) cp.template wait_all_but<LEAD - 1>();
      __syncthreads();
      for (int k = wave; k < 2 * NB; k += NW) convert_k<HD>(k >> 1, k & 1, ring, kfrag[t_begin & 1], lane);
    }
  }

  // QK of tile t: S^T, mask, online softmax, P^T fragments and rescale factor
  // into LDS buffer t & 1.
  auto qk_tile = [&](int t, const uint8_t* st, auto&& after_mfma) {
    const int key0 = t * 32;
    const uint8_t* kf = kfrag[t & 1];
    // S^T = K Q^T, KG blocks at a time for both 16-key subtiles: K fragments
    // and key scales first, then the hi MFMAs and the lo MFMAs (each block has
    // its own accumulator), then the per-block K scales in fp32, in block order
    constexpr int KG = NB < 4 ? NB : (R::SPLIT ? 2 : 4);  // blocks per group (registers)
    const half_t* Kst = (const half_t*)(st + L::KS_OFF);
    float4_t s[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    if constexpr (KV16) {
      // fp16 K fragments straight from the ring; no scales, so every block
      // accumulates into the same S^T tile (in block order)
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
    // (split instances: the fragments and scales of group b0 + KG are
    // requested before the products of group b0, so that their latency hides
    // behind those; the others have no registers to spare for that)
    constexpr bool AHEAD = R::SPLIT;
    half8_t kvn[2][KG];
    ScaleRow<KG> dkn[2][4];
    auto load_group = [&](int b0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int j = 0; j < KG; ++j) kvn[u][j] = *(const half8_t*)(kf + (((b0 + j) * 2 + u) * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) dkn[u][e].load(Kst + (16 * u + 4 * h4 + e) * NB + b0);
      }
    };
    if (AHEAD) load_group(0);
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += KG) {
      half8_t kv[2][KG];
      ScaleRow<KG> dk[2][4];
      if (!AHEAD) load_group(b0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int j = 0; j < KG; ++j) kv[u][j] = kvn[u][j];
#pragma unroll
        for (int e = 0; e < 4; ++e) dk[u][e] = dkn[u][e];
      }
      if (AHEAD && b0 + KG < NB) {
        load_group(b0 + KG);
        asm volatile("" ::: "memory");  // (those loads stay ahead of these products)
      }
      float4_t acc[2][KG];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < KG; ++j)
          acc[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[u][j], QR(b0 + j), (float4_t){0, 0, 0, 0}, 0, 0, 0);
      if (QF32) {
        half8_t ql[KG];
#pragma unroll
        for (int j = 0; j < KG; ++j)
          ql[j] = QR(NB + b0 + j);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < KG; ++j)
            acc[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv[u][j], ql[j], acc[u][j], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[u][e] = fmaf((float)dk[u][e].get(j), acc[u][j][e], s[u][e]);
    }
    }
    after_mfma();
    // mask and online softmax (base 2), p -> fp16 hi + lo
    // (lanes past the last vector of the wave hold q = 0, hence finite values
    // that only reach their own, never written, outputs)
    // (the maximum is taken on the unscaled dots: xmul > 0)
    float x[2][4];
    float tmax = -INFINITY;
    if (key0 + 31 <= lim_min) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] = s[u][e];
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + 16 * u + 4 * h4 + e;
          x[u][e] = key <= lim_eff ? s[u][e] : -INFINITY;
        }
      }
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
    // p split into fp16 hi + lo, two at a time: hi truncated (any hi works:
    // p - hi is exact in fp32 and its fp16 rounding keeps 22 bits of p)
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
    uint8_t* pf = pfrag[t & 1];
    *(half8_t*)(pf + ((wave * 2 + 0) * 64 + lane) * 16) = phi;
    *(half8_t*)(pf + ((wave * 2 + 1) * 64 + lane) * 16) = plo;
    if (h4 == 0) alpha_s[t & 1][wave][n16] = alpha;
  };

  // PV of tile t (ring stage st): V^T hi/lo of every owned block from the
  // ring, then for PG vector tiles at a time O^T *= alpha and
  // O^T += (Vhi,Phi) + (Vlo,Phi) + (Vhi,Plo).
  // (Oa: float4_t[NBL][NQW][2], the accumulators of the NBL blocks this wave owns)
  auto pv_tile = [&](int t, const uint8_t* st, auto& Oa) {
    constexpr int NBL = std::extent<std::remove_reference_t<decltype(Oa)>>::value;
    constexpr int PG = NBL > 1 ? 2 : (NQW < 4 ? NQW : 4);  // vector tiles per group (registers)
    half8_t vh[NBL][2], vl[NBL][2];
    int vsh[NBL];  // fold shifts of the blocks (wave-uniform)
    int any_sh = 0;
#pragma unroll
    for (int jb = 0; jb < NBL; ++jb) {
      vsh[jb] = 0;
      if constexpr (KV16) read_v16<HD>(R::block(wave, jb), st, lane, vh[jb]);
      else vsh[jb] = convert_v<HD>(R::block(wave, jb), st, lane, vh[jb], vl[jb]);
      any_sh |= vsh[jb];
    }
    if (any_sh) fold_scale(Oa, vsh, -1);
    const uint8_t* pf = pfrag[t & 1];
#pragma unroll
    for (int i0 = 0; i0 < NQW; i0 += PG) {
      half8_t ph[PG], pl[PG];
      float al[PG];
      bool rescale = false;
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        const int n = min(q0 + GW * (i0 + j), NQ - 1);
        ph[j] = *(const half8_t*)(pf + ((n * 2 + 0) * 64 + lane) * 16);
        pl[j] = *(const half8_t*)(pf + ((n * 2 + 1) * 64 + lane) * 16);
        al[j] = alpha_s[t & 1][n][n16];
        rescale |= al[j] != 1.0f;
      }
      if (__any(rescale)) {
#pragma unroll
        for (int jb = 0; jb < NBL; ++jb)
#pragma unroll
          for (int j = 0; j < PG; ++j) {
            Oa[jb][i0 + j][0] *= al[j];
            Oa[jb][i0 + j][1] *= al[j];
          }
      }
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        if (q0 + GW * (i0 + j) < nq) {
#pragma unroll
          for (int jb = 0; jb < NBL; ++jb)
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
              Oa[jb][i0 + j][dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[jb][dd], ph[j], Oa[jb][i0 + j][dd], 0, 0, 0);
          if constexpr (!KV16) {
#pragma unroll
            for (int jb = 0; jb < NBL; ++jb)
#pragma unroll
              for (int dd = 0; dd < 2; ++dd)
                Oa[jb][i0 + j][dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl[jb][dd], ph[j], Oa[jb][i0 + j][dd], 0, 0, 0);
          }
#pragma unroll
          for (int jb = 0; jb < NBL; ++jb)
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
              Oa[jb][i0 + j][dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[jb][dd], pl[j], Oa[jb][i0 + j][dd], 0, 0, 0);
        }
      }
    }
    if (any_sh) fold_scale(Oa, vsh, 1);
  };

  // Iteration t: barrier; copy tile t+D-2; QK of tile t; PV of tile t-1;
  // K fragments of tile t+1.  One extra iteration drains the last PV.  Every
  // wave passes the same barriers: one per iteration and one before the
  // output.
  if constexpr (R::SPLIT) {
    if (wave < R::PV0) {
      // ---- QK waves (and the waves among 0..3 without a vector tile,
      // converting K), in loops of their own: neither carries the other's
      // bookkeeping
      if (qk) {
        int slot = 0;  // ring stage of tile t
        for (int t = t_begin; t <= t_end; ++t) {
          __syncthreads();  // K(t) converted; P(t-2) consumed; tile t+1 landed
          if (t < t_end) qk_tile(t, ring + slot * L::BYTES, [] {});
          slot = (slot + 1 == D) ? 0 : slot + 1;
        }
      } else {
        int slot = 0;  // ring stage of tile t
        for (int t = t_begin; t <= t_end; ++t) {
          // (copying waves: their copies of tile t+1 landed)
          if (R::COPY_ON_K && copies && t + 1 < t_end) cp.template wait_all_but<WAIT_NEWER>();
          __syncthreads();  // K(t) converted; P(t-2) consumed; tile t+1 landed
          const uint8_t* stn = ring + ((slot + 1) % D) * L::BYTES;
          if (R::COPY_ON_K && copies && t < t_end)
            cp.issue(ring0 + ((slot + LEAD) % D) * L::BYTES, (t + LEAD) * 32, t + LEAD < t_end);
          if constexpr (!KV16 && R::K_ON_QK_SIDE) {
            if (ki >= 0 && t + 1 < t_end) convert_k_share<HD, R::KW>(ki, stn, kfrag[(t + 1) & 1], lane);
          }
          slot = (slot + 1 == D) ? 0 : slot + 1;
        }
        // copies into the ring past the last tile may still be landing
        if (R::COPY_ON_K && copies) wait_vmcnt<0>();
      }
      if (qk) {
        const float l_tot = wave_sum_groups(l_part);
        if (h4 == 0) ml_s[wave][n16] = make_float2(m_ref, l_tot);
      }
      __syncthreads();
    } else {
      // ---- PV waves: copies, K units of tile t+1 (unconditionally: past the
      // last tile the result is never read; only when wave 3 does not convert
      // K), V^T of tile t into registers for the next iteration, PV of tile t-1
      // (no copies here when the K-converting waves issue them: known at
      // compile time, so the loop carries none of their bookkeeping)
      const bool pv_copies = !R::COPY_ON_K && copies;
      float4_t O[BPW][NQW][2];
#pragma unroll
      for (int jb = 0; jb < BPW; ++jb)
#pragma unroll
        for (int i = 0; i < NQW; ++i) O[jb][i][0] = O[jb][i][1] = (float4_t){0, 0, 0, 0};
      half8_t vch[BPW][2], vcl[BPW][2];
      int vcs[BPW];   // fold shifts of those blocks (wave-uniform)
      int vc_any = 0;
#pragma unroll
      for (int jb = 0; jb < BPW; ++jb) vcs[jb] = 0;
      int slot = 0;  // ring stage of tile t
      for (int t = t_begin; t <= t_end; ++t) {
        const bool has_qk = t < t_end;
        // this wave's copies of tile t+1 (int8: K converted now) or t landed
        if (pv_copies && (KV16 ? has_qk : t + 1 < t_end)) cp.template wait_all_but<WAIT_NEWER>();
        __syncthreads();  // K(t) converted; P(t-1) written; tile t+1 landed
        const uint32_t cdst = ring0 + ((slot + LEAD) % D) * L::BYTES;
        const uint8_t* st = ring + slot * L::BYTES;
        const uint8_t* stn = ring + ((slot + 1) % D) * L::BYTES;
        uint8_t* kfn = kfrag[(t + 1) & 1];
        auto kconv = [&]() {
          if constexpr (!KV16 && !R::K_ON_QK_SIDE) convert_k_share<HD, R::NPV>(ki, stn, kfn, lane);
        };
        // the copies of tile t+LEAD go out one share before each block's V
        half8_t vnh[BPW][2], vnl[BPW][2];
        int vns[BPW];
        int vn_any = 0;
#pragma unroll
        for (int jb = 0; jb < BPW; ++jb) {
          if (pv_copies && has_qk) cp.issue_part(cdst, (t + LEAD) * 32, t + LEAD < t_end, jb, BPW);
          vns[jb] = 0;
          if constexpr (KV16) read_v16<HD>(R::block(wave, jb), st, lane, vnh[jb]);
          else vns[jb] = convert_v<HD>(R::block(wave, jb), st, lane, vnh[jb], vnl[jb]);
          vn_any |= vns[jb];
        }
        kconv();
        if (t > t_begin) {
          if (vc_any) fold_scale(O, vcs, -1);
          const uint8_t* pf = pfrag[(t - 1) & 1];
          // vector tiles in groups of PG (registers)
          constexpr int PG = NQW * BPW > 6 ? 2 : NQW;
#pragma unroll
          for (int i0 = 0; i0 < NQW; i0 += PG) {
            half8_t ph[PG], pl[PG];
            float al[PG];
            bool rescale = false;
#pragma unroll
            for (int j = 0; j < PG; ++j) {
              const int n = min(q0 + GW * (i0 + j), NQ - 1);
              ph[j] = *(const half8_t*)(pf + ((n * 2 + 0) * 64 + lane) * 16);
              pl[j] = *(const half8_t*)(pf + ((n * 2 + 1) * 64 + lane) * 16);
              al[j] = alpha_s[(t - 1) & 1][n][n16];
              rescale |= al[j] != 1.0f;
            }
            if (__any(rescale)) {
#pragma unroll
              for (int jb = 0; jb < BPW; ++jb)
#pragma unroll
                for (int j = 0; j < PG; ++j) {
                  O[jb][i0 + j][0] *= al[j];
                  O[jb][i0 + j][1] *= al[j];
                }
            }
#pragma unroll
            for (int hl = 0; hl < 3; ++hl) {
              if (KV16 && hl == 1) continue;  // an fp16 V has no lo part
#pragma unroll
              for (int j = 0; j < PG; ++j)
#pragma unroll
                for (int jb = 0; jb < BPW; ++jb)
#pragma unroll
                  for (int dd = 0; dd < 2; ++dd)
                    O[jb][i0 + j][dd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        hl == 1 ? vcl[jb][dd] : vch[jb][dd], hl == 2 ? pl[j] : ph[j], O[jb][i0 + j][dd], 0, 0, 0);
            }
          }
          if (vc_any) fold_scale(O, vcs, 1);
        }
#pragma unroll
        for (int jb = 0; jb < BPW; ++jb) {
#pragma unroll
          for (int dd = 0; dd < 2; ++dd) {
            vch[jb][dd] = vnh[jb][dd];
            if constexpr (!KV16) vcl[jb][dd] = vnl[jb][dd];
          }
          vcs[jb] = vns[jb];
        }
        vc_any = vn_any;
        slot = (slot + 1 == D) ? 0 : slot + 1;
      }
      // copies into the ring past the last tile may still be landing
      wait_vmcnt<0>();
      __syncthreads();  // (m, l) of every vector written by its QK wave
#pragma unroll
      for (int jb = 0; jb < BPW; ++jb) {
        const int b = R::block(wave, jb);
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
          const int n = q0 + GW * i;
          const int vv = n * 16 + n16;
          if (n >= nq || vv >= M) continue;
          const int orow = r0 + vv / a.G;
          const int ohead = g * a.G + vv % a.G;
          const float2 ml = ml_s[n][n16];
          const int dim0 = 32 * b + 4 * h4;
          if (FINAL) {
            const float inv_l = 1.0f / ml.y;
            float* dst = a.out + ((size_t)orow * a.Hq + ohead) * HD + dim0;
            *(float4_t*)dst = O[jb][i][0] * inv_l;
            *(float4_t*)(dst + 16) = O[jb][i][1] * inv_l;
          } else {
            const size_t idx = ((size_t)split * a.n_rows + orow) * a.Hq + ohead;
            float* dst = a.part_o + idx * HD + dim0;
            *(float4_t*)dst = O[jb][i][0];
            *(float4_t*)(dst + 16) = O[jb][i][1];
            if (b == 0 && h4 == 0) a.part_ml[idx] = ml;
          }
        }
      }
    }
  } else {
    // Each role runs its own loop (same barriers: one per iteration, one before
    // the output), so that its registers never meet another role's.
    auto role_loop = [&](auto do_qk, auto do_k, auto& Oa) {
      constexpr int NBL = std::extent<std::remove_reference_t<decltype(Oa)>>::value;
#pragma unroll
      for (int jb = 0; jb < NBL; ++jb)
#pragma unroll
        for (int i = 0; i < NQW; ++i) Oa[jb][i][0] = Oa[jb][i][1] = (float4_t){0, 0, 0, 0};
      int slot = 0;  // ring stage of tile t
      for (int t = t_begin; t <= t_end; ++t) {
        const bool has_qk = t < t_end;
        const bool has_next = t + 1 < t_end;
        // this wave's copies of tile t+1 (int8: K converted now) or t landed
        if (KV16 ? has_qk : has_next) cp.template wait_all_but<WAIT_NEWER>();
        __syncthreads();  // K(t) converted; P(t-1) written; tile t+1 landed; PV(t-2) done
        if (has_qk) cp.issue(ring0 + ((slot + LEAD) % D) * L::BYTES, (t + LEAD) * 32, t + LEAD < t_end);
        const uint8_t* st = ring + slot * L::BYTES;
        const uint8_t* st_prev = ring + ((slot + D - 1) % D) * L::BYTES;
        const uint8_t* stn = ring + ((slot + 1) % D) * L::BYTES;
        if (decltype(do_qk)::value && qk && has_qk) qk_tile(t, st, [] {});
        if (nblk > 0 && t > t_begin) pv_tile(t - 1, st_prev, Oa);
        if constexpr (!KV16 && decltype(do_k)::value)
          if (has_next)
            for (int k = ki; k < 2 * NB; k += kw) convert_k<HD>(k >> 1, k & 1, stn, kfrag[(t + 1) & 1], lane);
        slot = (slot + 1 == D) ? 0 : slot + 1;
      }
      // copies into the ring past the last tile may still be landing
      wait_vmcnt<0>();

      // ---- epilogue: (m, l) of every vector from its QK wave to the PV waves
      if (decltype(do_qk)::value && qk) {
        const float l_tot = wave_sum_groups(l_part);
        if (h4 == 0) ml_s[wave][n16] = make_float2(m_ref, l_tot);
      }
      __syncthreads();
#pragma unroll
      for (int jb = 0; jb < NBL; ++jb) {
        const int b = R::block(wave, jb);
        if (b >= NB) continue;
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
          const int n = q0 + GW * i;
          const int vv = n * 16 + n16;
          if (n >= nq || vv >= M) continue;
          const int orow = r0 + vv / a.G;
          const int ohead = g * a.G + vv % a.G;
          const float2 ml = ml_s[n][n16];
          const int dim0 = 32 * b + 4 * h4;
          if (FINAL) {
            const float inv_l = 1.0f / ml.y;
            float* dst = a.out + ((size_t)orow * a.Hq + ohead) * HD + dim0;
            *(float4_t*)dst = Oa[jb][i][0] * inv_l;
            *(float4_t*)(dst + 16) = Oa[jb][i][1] * inv_l;
          } else {
            const size_t idx = ((size_t)split * a.n_rows + orow) * a.Hq + ohead;
            float* dst = a.part_o + idx * HD + dim0;
            *(float4_t*)dst = Oa[jb][i][0];
            *(float4_t*)(dst + 16) = Oa[jb][i][1];
            if (b == 0 && h4 == 0) a.part_ml[idx] = ml;
          }
        }
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    float4_t Oa[BPW][NQW][2];
    role_loop(T_(), T_(), Oa);
  }
#undef QR
}

template <int HD, bool QF32, bool FINAL, int NQ>
__global__ __launch_bounds__((64 * body_waves<HD, NQ, false>())) void attend_q8_kernel(const AttendArgs a) {
  attend_body<HD, QF32, FINAL, NQ, false>(a);
}

// The same attention over an fp16 K/V cache (no scales).
template <int HD, bool QF32, bool FINAL, int NQ>
__global__ __launch_bounds__((64 * body_waves<HD, NQ, true>())) void attend_f16kv_kernel(const AttendArgs a) {
  attend_body<HD, QF32, FINAL, NQ, true>(a);
}

// Merge split partials: one 256-thread workgroup per (row, Q head, 64-dim
// chunk).  The largest reference point over the non-empty splits is found
// first; then the workgroup's 16 split slots (16 lanes each, 4 dims per lane)
// accumulate their splits (slot, slot + 16, ...) with up to B loads per lane in
// flight, and slot 0 adds the slot sums in slot order.  Every order is fixed,
// so results are run-to-run bitwise reproducible.
constexpr int kReduceThreads = 256;
constexpr int kReduceDims = 64;  // dims per workgroup
template <int HD>
__global__ __launch_bounds__(kReduceThreads) void reduce_partials_kernel(const float* __restrict__ part_o,
                                                                          const float2* __restrict__ part_ml,
                                                                          int n_splits, int n_pairs,
                                                                          float* __restrict__ out) {
  constexpr int LPS = kReduceDims / 4;          // lanes per split slot
  constexpr int NSLOT = kReduceThreads / LPS;   // split slots
  constexpr int NWAVE = kReduceThreads / 64;
  constexpr int B = 4;                          // splits in flight per lane
  __shared__ float wmax[NWAVE];
  __shared__ float4_t slot_acc[NSLOT][LPS];
  __shared__ float slot_den[NSLOT];
  const int pair = blockIdx.x;
  const int dim0 = blockIdx.y * kReduceDims;
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // the first batch of partials is requested before the maximum is known (the
  // loads do not depend on it), so the kernel makes one trip to memory, not two
  const int slot = tid / LPS;
  const int dl = tid % LPS;
  float2 ml[B];
  float4_t o[B];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int sp = min(s0 + i * NSLOT, n_splits - 1);
      const size_t idx = (size_t)sp * n_pairs + pair;
      ml[i] = part_ml[idx];
      o[i] = *(const float4_t*)(part_o + idx * HD + dim0 + 4 * dl);
    }
  };
  load_batch(slot);

  float M = -INFINITY;
  for (int s = tid; s < n_splits; s += kReduceThreads) {
    const float2 m = part_ml[(size_t)s * n_pairs + pair];
    if (m.y > 0.0f) M = fmaxf(M, m.x);
  }
  M = wave_max_all(M);
  if (lane == 0) wmax[tid >> 6] = M;
  __syncthreads();
  M = wmax[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) M = fmaxf(M, wmax[w]);

  float4_t acc = {0, 0, 0, 0};
  float den = 0.0f;
  for (int s0 = slot;;) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (s0 + i * NSLOT < n_splits) {
        // the hardware exponential: a weight below fp32's normal range reads
        // as 0 beside the split at M, whose weight is 1
        const float w = (ml[i].y > 0.0f) ? __builtin_amdgcn_exp2f(ml[i].x - M) : 0.0f;
        den = fmaf(w, ml[i].y, den);
        acc += w * o[i];
      }
    }
    s0 += NSLOT * B;
    if (s0 >= n_splits) break;
    load_batch(s0);
  }
  slot_acc[slot][dl] = acc;
  if (dl == 0) slot_den[slot] = den;
  __syncthreads();
  if (slot == 0) {
    float4_t a = slot_acc[0][dl];
    float d = slot_den[0];
#pragma unroll
    for (int k = 1; k < NSLOT; ++k) {
      a += slot_acc[k][dl];
      d += slot_den[k];
    }
    *(float4_t*)(out + (size_t)pair * HD + dim0 + 4 * dl) = a / d;
  }
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
