// Host side of the attnq8 C ABI: argument validation, launch planning and
// kernel launches on the caller's stream.  See include/attnq8.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <limits.h>
#include <math.h>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include "../../include/attnq8.h"
#include "append_kernel.h"
#include "attend_kernel.h"
#include "head_kernel.h"
#include "own_kernel.h"
#include "stream_kernel.h"

namespace {

using namespace attnq8;

constexpr int kMaxVectorsPerGroup = 128;  // query vectors of one row group
constexpr int kTargetCUs = 256;           // MI355X compute units
constexpr double kLog2e = 1.4426950408889634;
constexpr int kMaxAppendHeadDim = 4096;   // KV append: any multiple of 32 up to this
constexpr long long kAppendMaxBlocks = 8192;  // 32 workgroups per CU, then grid-stride
constexpr int kMaxGridYZ = 65535;         // largest second and third grid dimension

thread_local char g_last_path[192] = "none";

// The split partials of attn_verify_q8_static: one copy of this array on every
// GPU the library runs on, held until the process ends.  In host code its
// name stands for a host-side symbol, not a device address: kernels receive
// the address scratch_address() obtained with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[ATTNQ8_STATIC_SCRATCH_BYTES];

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept; nullptr with *status set when
// the runtime cannot provide it.
void* scratch_address(int* status) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *status = ATTNQ8_EHIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = ATTNQ8_EUNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = ATTNQ8_EHIP;
      return nullptr;
    }
    addr[dev] = p;
  }
  *status = ATTNQ8_OK;
  return addr[dev];
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool head_dim_ok(int hd) { return hd == 64 || hd == 128 || hd == 256; }

// Per-device architecture check, cached (0 = unknown, 1 = gfx950, 2 = other;
// atomic: threads that race on a device's first call store the same value).
int device_status() {
  static std::atomic<signed char> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTNQ8_EHIP;
  if (dev < 0 || dev >= 64) return ATTNQ8_EUNSUPPORTED;
  signed char c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTNQ8_EHIP;
    c = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1 ? ATTNQ8_OK : ATTNQ8_EUNSUPPORTED;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? ATTNQ8_OK : ATTNQ8_EHIP;
}

// Vector-tile capacity of the kernel instance for a row group of `vectors`
// query vectors (16 per tile): the smallest instance that holds them (at
// head_dim 256: 2, 3, 4, 6 or 8 tiles; at 128: 2, 4 or 8; at 64: 4 or 8).
int nq_for(int vectors, int hd) {
  const int n = (vectors + 15) / 16;
  if (n > 4) return (n <= 6 && hd == 256) ? 6 : 8;
  if (hd == 256) return n <= 2 ? 2 : n;
  if (hd == 128) return n <= 2 ? 2 : 4;
  return 4;
}

// Workgroups resident per CU: one at head_dim 128 and 256 (registers, LDS),
// two at head_dim 64.
int wgs_per_cu(int hd) { return hd == 64 ? 2 : 1; }  // register- and LDS-bound

int splits_for(int n_keys, int units, int hd) {
  const int tiles = (n_keys + 31) / 32;
  const int target = kTargetCUs * wgs_per_cu(hd);
  int s = (target + units - 1) / units;
  const int cap = tiles / 2;  // at least two 32-key tiles per split
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return s;
}

// Default row group: as many rows of a KV head as fit 64 query vectors (four
// vector tiles: the split-role instances).  Groups of up to 128 read the
// context half as often but write twice the split partials: at 32 rows of
// 32 / 8 heads and 8,192 keys, head_dim 128, one group of 128 vectors (the own
// layout) takes 25.0 against 25.6 us for the attention kernel and 31.9 against
// 30.5 us for the call with the reducer; at head_dim 64 the general
// eight-tile instance measured 30.1 against 24.5 us per call (fp16 cache: 29.2
// against 25.1 us).
int auto_rows_per_group(int G, int n_rows, int hd) {
  (void)hd;
  int rg = 64 / G;
  if (rg > n_rows) rg = n_rows;
  if (rg < 1) rg = 1;
  return rg;
}

using KernelFn = void (*)(AttendArgs);

template <int HD, bool QF32, bool FINAL, int NQ, bool KV16>
constexpr KernelFn kernel_of() {
  if constexpr (KV16) return attend_f16kv_kernel<HD, QF32, FINAL, NQ>;
  else return attend_q8_kernel<HD, QF32, FINAL, NQ>;
}

template <int HD, bool QF32, bool FINAL, bool KV16>
KernelFn pick_nq(int nq) {
  switch (nq) {
    case 2: if constexpr (HD >= 128) return kernel_of<HD, QF32, FINAL, 2, KV16>(); else return nullptr;
    case 3: if constexpr (HD == 256) return kernel_of<HD, QF32, FINAL, 3, KV16>(); else return nullptr;
    case 4: return kernel_of<HD, QF32, FINAL, 4, KV16>();
    case 6: return nullptr;  // (head_dim 256 with six tiles: the own layout)
    // an fp16 ring at head_dim 256 leaves no LDS for eight vector tiles
    case 8: if constexpr (!(KV16 && HD == 256)) return kernel_of<HD, QF32, FINAL, 8, KV16>(); else return nullptr;
    default: return nullptr;
  }
}

// Row groups of six vector tiles at head_dim 256 take the layout in which each
// compute wave owns its vectors end to end.  (With two or three tiles over an
// int8 cache that layout leaves the SIMDs' MFMA pipes to one wave each and
// gains nothing over the split roles; those row groups keep the general body.)
// At head_dim 128 the eight-tile row groups take it too (eight compute waves
// and their feeders).
bool own_layout(bool kv16, int hd, int nq) {
  return (hd == 256 && (nq == 6 || (kv16 && nq == 3))) || (hd == 128 && nq == 8);
}

template <bool FINAL, bool QF32, bool KV16>
KernelFn pick_own(int hd, int nq) {
  if (hd == 128) {
    if constexpr (KV16) return attend_own_f16kv_kernel<128, QF32, FINAL, 8>;
    else return attend_own_q8_kernel<128, QF32, FINAL, 8>;
  }
  if constexpr (KV16) return nq == 6 ? attend_own_f16kv_kernel<256, QF32, FINAL, 6> : attend_own_f16kv_kernel<256, QF32, FINAL, 3>;
  else return nq == 6 ? attend_own_q8_kernel<256, QF32, FINAL, 6> : nullptr;
}

// Threads per workgroup of the kernel pick_kernel returns.
template <bool KV16>
int threads_for(int hd, int nq) {
  if (own_layout(KV16, hd, nq)) return 64 * (hd == 128 ? own_waves<128, 8, KV16>() : kWaves);
  switch (hd) {
    case 256:
      switch (nq) {
        case 2: return 64 * body_waves<256, 2, KV16>();
        case 3: return 64 * body_waves<256, 3, KV16>();
        default: return 64 * kWaves;
      }
    default: return 64 * kWaves;
  }
}

template <bool FINAL, bool KV16 = false>
KernelFn pick_kernel(int hd, bool qf32, int nq) {
  if (own_layout(KV16, hd, nq)) return qf32 ? pick_own<FINAL, true, KV16>(hd, nq) : pick_own<FINAL, false, KV16>(hd, nq);
  switch (hd) {
    case 64: return qf32 ? pick_nq<64, true, FINAL, KV16>(nq) : pick_nq<64, false, FINAL, KV16>(nq);
    case 128: return qf32 ? pick_nq<128, true, FINAL, KV16>(nq) : pick_nq<128, false, FINAL, KV16>(nq);
    case 256: return qf32 ? pick_nq<256, true, FINAL, KV16>(nq) : pick_nq<256, false, FINAL, KV16>(nq);
    default: return nullptr;
  }
}

// Largest row group (query vectors) per workgroup: 128, except for an fp16
// cache at head_dim 256 (its ring leaves LDS for six vector tiles).
template <bool KV16>
int max_vectors(int hd) { return KV16 && hd == 256 ? 96 : kMaxVectorsPerGroup; }

// Checks shared by the attention calls (KV16: fp16 K/V, the scale pointers are unused).
template <bool KV16>
int check_kv(const void* q, int q_dtype, const void* kc, const uint16_t* ks, const void* vc,
             const uint16_t* vs, int hq, int hkv, int hd, int kv_stride) {
  if (!q || !kc || !vc) return ATTNQ8_EINVAL;
  if (!KV16 && (!ks || !vs)) return ATTNQ8_EINVAL;
  if (q_dtype != ATTNQ8_F32 && q_dtype != ATTNQ8_F16) return ATTNQ8_EINVAL;
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return ATTNQ8_EINVAL;
  if (hkv > kMaxGridYZ) return ATTNQ8_EINVAL;  // the KV heads are the launch's third grid dimension
  if (!head_dim_ok(hd)) return ATTNQ8_EUNSUPPORTED;
  if (hq / hkv > kMaxVectorsPerGroup) return ATTNQ8_EUNSUPPORTED;
  if (kv_stride <= 0) return ATTNQ8_EINVAL;
  // per-head cache bytes are addressed with 32-bit buffer offsets
  if ((long long)kv_stride * hd * (KV16 ? 2 : 1) >= (1LL << 31) - 64) return ATTNQ8_EINVAL;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16)) return ATTNQ8_EALIGN;
  if (!KV16 && (!aligned(ks, 4) || !aligned(vs, 4))) return ATTNQ8_EALIGN;
  return ATTNQ8_OK;
}

// Verify launch for either cache format (KV16: fp16 K/V in k, v; no scales).
// With dry set, only the host checks run (no HIP call, nothing launched) and
// the workspace pointer is not examined.
template <bool KV16>
int verify_launch(const void* q, int q_dtype, const void* k, const uint16_t* k_scales, const void* v,
                  const uint16_t* v_scales, int n_q_heads, int n_kv_heads, int head_dim,
                  int kv_stride, int ctx_len, int n_rows, int rows_per_group, int n_splits,
                  void* workspace, size_t workspace_bytes, float sm_scale, void* stream,
                  bool dry = false) {
  int st = check_kv<KV16>(q, q_dtype, k, k_scales, v, v_scales, n_q_heads, n_kv_heads, head_dim,
                          kv_stride);
  if (st) return st;
  if (ctx_len < 0 || n_rows < 1 || n_rows > 32) return ATTNQ8_EINVAL;
  if ((long long)ctx_len + n_rows > kv_stride) return ATTNQ8_EINVAL;
  if (rows_per_group < 0 || n_splits < 0) return ATTNQ8_EINVAL;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return ATTNQ8_EINVAL;
  const int G = n_q_heads / n_kv_heads;
  // (the product in 64 bits: a huge rows_per_group must not wrap into range)
  if ((long long)rows_per_group * G > kMaxVectorsPerGroup) return ATTNQ8_EINVAL;
  const int rg = rows_per_group > 0 ? rows_per_group : auto_rows_per_group(G, n_rows, head_dim);
  if (rg * G > max_vectors<KV16>(head_dim)) return ATTNQ8_EUNSUPPORTED;
  const int groups = (n_rows + rg - 1) / rg;
  const int n_keys = ctx_len + n_rows;
  const int tiles = (n_keys + 31) / 32;
  const int S = n_splits > 0 ? n_splits : splits_for(n_keys, groups * n_kv_heads, head_dim);
  if (S > tiles || S > 65535) return ATTNQ8_EINVAL;
  if (!dry && !workspace) return ATTNQ8_EINVAL;
  if (!dry && !aligned(workspace, 16)) return ATTNQ8_EALIGN;
  const size_t need = attn_verify_q8_workspace_bytes(n_rows, n_q_heads, head_dim, S);
  if (workspace_bytes < need) return ATTNQ8_EWORKSPACE;
  if (dry) return ATTNQ8_OK;

  st = device_status();
  if (st) return st;

  const int nq = nq_for(rg * G, head_dim);
  KernelFn fn = pick_kernel<false, KV16>(head_dim, q_dtype == ATTNQ8_F32, nq);
  if (!fn) return ATTNQ8_EUNSUPPORTED;
  AttendArgs a;
  a.q = q;
  a.kc = (const int8_t*)k;
  a.ks = k_scales;
  a.vc = (const int8_t*)v;
  a.vs = v_scales;
  a.part_o = (float*)workspace;
  a.part_ml = (float2*)((char*)workspace + (size_t)S * n_rows * n_q_heads * head_dim * sizeof(float));
  a.out = nullptr;
  a.Hq = n_q_heads;
  a.G = G;
  a.kv_stride = kv_stride;
  a.pos0 = ctx_len;
  a.n_rows = n_rows;
  a.rows_per_wg = rg;
  a.n_splits = S;
  const float scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)head_dim));
  a.kmul = (float)((double)scale * kLog2e);
  hipLaunchKernelGGL(fn, dim3(S, groups, n_kv_heads), dim3(threads_for<KV16>(head_dim, nq)), 0,
                     (hipStream_t)stream, a);
  st = launch_status();
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path),
           "verify kv%s hd%d q%s tiles%d%s rows_per_group%d groups%d splits%d kv_heads%d",
           KV16 ? "f16" : "q8", head_dim, q_dtype == ATTNQ8_F32 ? "f32" : "f16", nq,
           own_layout(KV16, head_dim, nq) ? " own" : "", rg, groups, S, n_kv_heads);
  return ATTNQ8_OK;
}

// Prompt launch for either cache format.
template <bool KV16>
int prompt_launch(const void* q, int q_dtype, const void* k, const uint16_t* k_scales, const void* v,
                  const uint16_t* v_scales, int n_q_heads, int n_kv_heads, int head_dim,
                  int kv_stride, int kv_len, int q_pos0, int n_queries, float sm_scale, float* out,
                  void* stream) {
  int st = check_kv<KV16>(q, q_dtype, k, k_scales, v, v_scales, n_q_heads, n_kv_heads, head_dim,
                          kv_stride);
  if (st) return st;
  if (!out) return ATTNQ8_EINVAL;
  if (!aligned(out, 16)) return ATTNQ8_EALIGN;
  if (n_queries < 1 || q_pos0 < 0 || kv_len < 1) return ATTNQ8_EINVAL;
  if ((long long)q_pos0 + n_queries > kv_len || kv_len > kv_stride) return ATTNQ8_EINVAL;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return ATTNQ8_EINVAL;
  const int G = n_q_heads / n_kv_heads;
  if (G > max_vectors<KV16>(head_dim)) return ATTNQ8_EUNSUPPORTED;
  // rows per workgroup: queries whose G heads fill up to 8 waves of 16 vectors,
  // keeping about one workgroup per CU for the chunk
  int rq = max_vectors<KV16>(head_dim) / G;
  if (rq < 1) rq = 1;
  const int per_cu = (n_queries * n_kv_heads + kTargetCUs - 1) / kTargetCUs;
  if (rq > per_cu) rq = per_cu;
  if (rq < 1) rq = 1;
  const int groups = (n_queries + rq - 1) / rq;
  if (groups > 65535) return ATTNQ8_EINVAL;
  st = device_status();
  if (st) return st;
  const int nq = nq_for(rq * G, head_dim);
  KernelFn fn = pick_kernel<true, KV16>(head_dim, q_dtype == ATTNQ8_F32, nq);
  const bool own = own_layout(KV16, head_dim, nq);
  if (!fn) return ATTNQ8_EUNSUPPORTED;
  AttendArgs a;
  a.q = q;
  a.kc = (const int8_t*)k;
  a.ks = k_scales;
  a.vc = (const int8_t*)v;
  a.vs = v_scales;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.out = out;
  a.Hq = n_q_heads;
  a.G = G;
  a.kv_stride = kv_stride;
  a.pos0 = q_pos0;
  a.n_rows = n_queries;
  a.rows_per_wg = rq;
  a.n_splits = 1;
  const float scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / sqrt((double)head_dim));
  a.kmul = (float)((double)scale * kLog2e);
  hipLaunchKernelGGL(fn, dim3(1, groups, n_kv_heads), dim3(threads_for<KV16>(head_dim, nq)), 0,
                     (hipStream_t)stream, a);
  st = launch_status();
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path),
           "prompt kv%s hd%d q%s tiles%d%s rows_per_group%d groups%d kv_heads%d", KV16 ? "f16" : "q8",
           head_dim, q_dtype == ATTNQ8_F32 ? "f32" : "f16", nq, own ? " own" : "", rq, groups, n_kv_heads);
  return ATTNQ8_OK;
}
}  // namespace

extern "C" {

const char* attnq8_status_string(int status) {
  switch (status) {
    case ATTNQ8_OK: return "ok";
    case ATTNQ8_EINVAL: return "invalid argument";
    case ATTNQ8_EUNSUPPORTED: return "unsupported device or shape";
    case ATTNQ8_EALIGN: return "misaligned pointer";
    case ATTNQ8_EWORKSPACE: return "workspace too small";
    case ATTNQ8_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attnq8_last_path(void) { return g_last_path; }

int attn_verify_q8_splits(int n_q_heads, int n_kv_heads, int head_dim, int ctx_len, int n_rows,
                          int rows_per_group) {
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads) return ATTNQ8_EINVAL;
  if (!head_dim_ok(head_dim)) return ATTNQ8_EUNSUPPORTED;
  if (ctx_len < 0 || n_rows < 1 || n_rows > 32) return ATTNQ8_EINVAL;
  const int G = n_q_heads / n_kv_heads;
  if (G > kMaxVectorsPerGroup) return ATTNQ8_EUNSUPPORTED;
  if (rows_per_group < 0 || (long long)rows_per_group * G > kMaxVectorsPerGroup) return ATTNQ8_EINVAL;
  const int rg = rows_per_group > 0 ? rows_per_group : auto_rows_per_group(G, n_rows, head_dim);
  const int groups = (n_rows + rg - 1) / rg;
  return splits_for(ctx_len + n_rows, groups * n_kv_heads, head_dim);
}

size_t attn_verify_q8_workspace_bytes(int n_rows, int n_q_heads, int head_dim, int n_splits) {
  if (n_rows <= 0 || n_q_heads <= 0 || head_dim <= 0 || n_splits <= 0) return 0;
  return (size_t)n_splits * n_rows * n_q_heads * (size_t)(head_dim + 2) * sizeof(float);
}

int attn_verify_q8(const void* q, int q_dtype, const int8_t* k_codes, const uint16_t* k_scales,
                   const int8_t* v_codes, const uint16_t* v_scales, int n_q_heads, int n_kv_heads,
                   int head_dim, int kv_stride, int ctx_len, int n_rows, int rows_per_group,
                   int n_splits, void* workspace, size_t workspace_bytes, float sm_scale,
                   void* stream) {
  return verify_launch<false>(q, q_dtype, k_codes, k_scales, v_codes, v_scales, n_q_heads,
                              n_kv_heads, head_dim, kv_stride, ctx_len, n_rows, rows_per_group,
                              n_splits, workspace, workspace_bytes, sm_scale, stream);
}

int attn_verify_f16kv(const void* q, int q_dtype, const uint16_t* k, const uint16_t* v,
                      int n_q_heads, int n_kv_heads, int head_dim, int kv_stride, int ctx_len,
                      int n_rows, int rows_per_group, int n_splits, void* workspace,
                      size_t workspace_bytes, float sm_scale, void* stream) {
  return verify_launch<true>(q, q_dtype, k, nullptr, v, nullptr, n_q_heads, n_kv_heads, head_dim,
                             kv_stride, ctx_len, n_rows, rows_per_group, n_splits, workspace,
                             workspace_bytes, sm_scale, stream);
}

int attn_reduce_partials(const void* workspace, size_t workspace_bytes, int n_rows, int n_q_heads,
                         int head_dim, int n_splits, float* out, void* stream) {
  if (!workspace || !out) return ATTNQ8_EINVAL;
  if (n_rows < 1 || n_q_heads < 1 || n_splits < 1 || n_splits > 65535) return ATTNQ8_EINVAL;
  if ((long long)n_rows * n_q_heads > INT_MAX) return ATTNQ8_EINVAL;  // (row, head) pairs: the grid's x
  if (!head_dim_ok(head_dim)) return ATTNQ8_EUNSUPPORTED;
  if (!aligned(workspace, 16) || !aligned(out, 16)) return ATTNQ8_EALIGN;
  if (workspace_bytes < attn_verify_q8_workspace_bytes(n_rows, n_q_heads, head_dim, n_splits))
    return ATTNQ8_EWORKSPACE;
  int st = device_status();
  if (st) return st;
  const int pairs = n_rows * n_q_heads;
  const float* po = (const float*)workspace;
  const float2* pml =
      (const float2*)((const char*)workspace + (size_t)n_splits * pairs * head_dim * sizeof(float));
  dim3 grid(pairs, head_dim / kReduceDims), block(kReduceThreads);
  hipStream_t s = (hipStream_t)stream;
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(reduce_partials_kernel<64>, grid, block, 0, s, po, pml, n_splits, pairs, out); break;
    case 128: hipLaunchKernelGGL(reduce_partials_kernel<128>, grid, block, 0, s, po, pml, n_splits, pairs, out); break;
    default: hipLaunchKernelGGL(reduce_partials_kernel<256>, grid, block, 0, s, po, pml, n_splits, pairs, out); break;
  }
  st = launch_status();
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path), "reduce hd%d pairs%d splits%d", head_dim, pairs, n_splits);
  return ATTNQ8_OK;
}

int attn_verify_q8_static(const void* q, int q_dtype, const int8_t* k_codes, const uint16_t* k_scales,
                          const int8_t* v_codes, const uint16_t* v_scales, int n_q_heads, int n_kv_heads,
                          int head_dim, int kv_stride, int ctx_len, int n_rows, int rows_per_group,
                          int n_splits, float sm_scale, float* out, void* stream) {
  // every check of both launches first, on the host
  if (!out) return ATTNQ8_EINVAL;
  if (!aligned(out, 16)) return ATTNQ8_EALIGN;
  if (n_splits < 0) return ATTNQ8_EINVAL;
  const int auto_splits =
      attn_verify_q8_splits(n_q_heads, n_kv_heads, head_dim, ctx_len, n_rows, rows_per_group);
  if (auto_splits < 0) return auto_splits;
  const size_t per_split = attn_verify_q8_workspace_bytes(n_rows, n_q_heads, head_dim, 1);
  const size_t fit = per_split ? (size_t)ATTNQ8_STATIC_SCRATCH_BYTES / per_split : 0;
  if (fit < 1) return ATTNQ8_EWORKSPACE;
  int S = n_splits;
  if (S == 0) S = (size_t)auto_splits <= fit ? auto_splits : (int)fit;
  else if ((size_t)S > fit) return ATTNQ8_EWORKSPACE;
  int st = verify_launch<false>(q, q_dtype, k_codes, k_scales, v_codes, v_scales, n_q_heads, n_kv_heads,
                                head_dim, kv_stride, ctx_len, n_rows, rows_per_group, S, nullptr,
                                ATTNQ8_STATIC_SCRATCH_BYTES, sm_scale, stream, /*dry=*/true);
  if (st) return st;
  st = device_status();
  if (st) return st;
  void* ws = scratch_address(&st);
  if (!ws) return st;
  st = verify_launch<false>(q, q_dtype, k_codes, k_scales, v_codes, v_scales, n_q_heads, n_kv_heads,
                            head_dim, kv_stride, ctx_len, n_rows, rows_per_group, S, ws,
                            ATTNQ8_STATIC_SCRATCH_BYTES, sm_scale, stream);
  if (st) return st;
  char verify_path[sizeof(g_last_path)];
  memcpy(verify_path, g_last_path, sizeof(verify_path));
  st = attn_reduce_partials(ws, ATTNQ8_STATIC_SCRATCH_BYTES, n_rows, n_q_heads, head_dim, S, out, stream);
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path), "static %.150s + reduce", verify_path);
  return ATTNQ8_OK;
}

int attn_prompt_q8(const void* q, int q_dtype, const int8_t* k_codes, const uint16_t* k_scales,
                   const int8_t* v_codes, const uint16_t* v_scales, int n_q_heads, int n_kv_heads,
                   int head_dim, int kv_stride, int kv_len, int q_pos0, int n_queries,
                   float sm_scale, float* out, void* stream) {
  return prompt_launch<false>(q, q_dtype, k_codes, k_scales, v_codes, v_scales, n_q_heads,
                              n_kv_heads, head_dim, kv_stride, kv_len, q_pos0, n_queries, sm_scale,
                              out, stream);
}

int attn_prompt_f16kv(const void* q, int q_dtype, const uint16_t* k, const uint16_t* v,
                      int n_q_heads, int n_kv_heads, int head_dim, int kv_stride, int kv_len,
                      int q_pos0, int n_queries, float sm_scale, float* out, void* stream) {
  return prompt_launch<true>(q, q_dtype, k, nullptr, v, nullptr, n_q_heads, n_kv_heads, head_dim,
                             kv_stride, kv_len, q_pos0, n_queries, sm_scale, out, stream);
}

int attn_kv_append_q8(const void* k, const void* v, int x_dtype, int n_tokens, int n_kv_heads,
                      int head_dim, int8_t* k_codes, uint16_t* k_scales, int8_t* v_codes,
                      uint16_t* v_scales, int kv_stride, int pos0, void* stream) {
  // the row pointers may be NULL only when there are no rows
  const bool has_v = v || v_codes || v_scales;
  if (!k_codes || !k_scales) return ATTNQ8_EINVAL;
  if (has_v && (!v_codes || !v_scales)) return ATTNQ8_EINVAL;
  if (n_tokens > 0 && (!k || (has_v && !v))) return ATTNQ8_EINVAL;
  if (x_dtype != ATTNQ8_F32 && x_dtype != ATTNQ8_F16) return ATTNQ8_EINVAL;
  if (n_tokens < 0 || n_kv_heads < 1 || kv_stride < 1 || pos0 < 0) return ATTNQ8_EINVAL;
  if (head_dim < 32 || head_dim > kMaxAppendHeadDim || head_dim % 32) return ATTNQ8_EUNSUPPORTED;
  if ((long long)pos0 + n_tokens > kv_stride) return ATTNQ8_EINVAL;
  if (!aligned(k, 16) || !aligned(k_codes, 16) || !aligned(k_scales, 4)) return ATTNQ8_EALIGN;
  if (has_v && (!aligned(v, 16) || !aligned(v_codes, 16) || !aligned(v_scales, 4)))
    return ATTNQ8_EALIGN;
  const long long row_units = (long long)n_kv_heads * head_dim / 8;
  if (row_units > (1LL << 30)) return ATTNQ8_EINVAL;
  const long long units = row_units * n_tokens;
  if (units == 0) {
    snprintf(g_last_path, sizeof(g_last_path), "kv_append empty");
    return ATTNQ8_OK;
  }
  int st = device_status();
  if (st) return st;
  AppendArgs a;
  a.x[0] = k;
  a.x[1] = v;
  a.codes[0] = k_codes;
  a.codes[1] = v_codes;
  a.scales[0] = k_scales;
  a.scales[1] = v_scales;
  a.units = units;
  a.row_units = (int)row_units;
  a.head_units = head_dim / 8;
  a.head_dim = head_dim;
  a.kv_stride = kv_stride;
  a.pos0 = pos0;
  long long blocks = (units + kAppendThreads - 1) / kAppendThreads;
  if (blocks > kAppendMaxBlocks) blocks = kAppendMaxBlocks;
  const long long step = blocks * kAppendThreads;
  a.step_tokens = (int)(step / row_units);
  a.step_in_row = (int)(step % row_units);
  const dim3 grid((unsigned)blocks, has_v ? 2 : 1);
  if (x_dtype == ATTNQ8_F32)
    hipLaunchKernelGGL(kv_append_q8_kernel<true>, grid, dim3(kAppendThreads), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(kv_append_q8_kernel<false>, grid, dim3(kAppendThreads), 0,
                       (hipStream_t)stream, a);
  st = launch_status();
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path), "kv_append hd%d x%s tensors%d blocks%lld units%lld",
           head_dim, x_dtype == ATTNQ8_F32 ? "f32" : "f16", has_v ? 2 : 1, blocks, units);
  return ATTNQ8_OK;
}

// Blocks per row of the greedy head: about one block per compute unit over
// all rows (at most kHeadMaxBlocks per row), each covering at least one quad of
// four logits per thread.
constexpr int kHeadBlocks = kTargetCUs;  // about one block per compute unit
static int head_blocks_per_row(int n_rows, int vocab) {
  const long long quads = vocab / 4;
  long long b = (kHeadBlocks + n_rows - 1) / n_rows;
  const long long by_size = (quads + kHeadThreads - 1) / kHeadThreads;
  if (b > by_size) b = by_size;
  if (b > kHeadMaxBlocks) b = kHeadMaxBlocks;
  if (b < 1) b = 1;
  return (int)b;
}

size_t attn_verify_head_workspace_bytes(int n_rows, int vocab) {
  if (n_rows < 1 || n_rows > kHeadMaxRows || vocab < 1) return 0;
  // the tickets first, at fixed offsets for every shape, then the block
  // states: n_rows * head_blocks_per_row() <= kHeadBlocks + n_rows - 1 for
  // every vocab, so the size grows with n_rows and a scratch sized for n rows
  // serves any call with fewer
  return kHeadTicketBytes + (size_t)(kHeadBlocks + n_rows) * sizeof(HeadSlot);
}

int attn_verify_head_greedy(const float* logits, int n_rows, int vocab, long long row_stride,
                            int* token, float* top_prob, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!logits || !token || !workspace) return ATTNQ8_EINVAL;
  if (n_rows < 1 || n_rows > kHeadMaxRows || vocab < 1 || row_stride < vocab) return ATTNQ8_EINVAL;
  if (!aligned(logits, 4) || !aligned(token, 4) || !aligned(workspace, 16)) return ATTNQ8_EALIGN;
  if (top_prob && !aligned(top_prob, 4)) return ATTNQ8_EALIGN;
  if (workspace_bytes < attn_verify_head_workspace_bytes(n_rows, vocab)) return ATTNQ8_EWORKSPACE;
  int st = device_status();
  if (st) return st;
  HeadArgs a;
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = vocab;
  a.blocks_per_row = head_blocks_per_row(n_rows, vocab);
  a.block_quads = (int)(((long long)(vocab / 4) + a.blocks_per_row - 1) / a.blocks_per_row);
  a.ticket = (unsigned*)workspace;
  a.slot = (HeadSlot*)((char*)workspace + kHeadTicketBytes);
  a.token = token;
  a.top_prob = top_prob;
  hipLaunchKernelGGL(head_greedy_kernel, dim3(a.blocks_per_row, n_rows), dim3(kHeadThreads), 0,
                     (hipStream_t)stream, a);
  st = launch_status();
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path), "verify_head rows%d vocab%d blocks_per_row%d", n_rows,
           vocab, a.blocks_per_row);
  return ATTNQ8_OK;
}

int attnq8_selftest_i8_to_f16(uint16_t* out, void* stream) {
  if (!out) return ATTNQ8_EINVAL;
  if (!aligned(out, 4)) return ATTNQ8_EALIGN;
  int st = device_status();
  if (st) return st;
  hipLaunchKernelGGL(selftest_i8_to_f16_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, out);
  return launch_status();
}

int attnq8_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  static_assert(ATTNQ8_STREAM_SINK_WORDS == kStreamBlocks, "one sink word per workgroup");
  if (!sink || (!buf && bytes > 0)) return ATTNQ8_EINVAL;
  if (!aligned(buf, 16) || bytes % 16 != 0 || !aligned(sink, 4)) return ATTNQ8_EALIGN;
  int st = device_status();
  if (st) return st;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamBlocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     (const uint4*)buf, bytes / 16, sink);
  st = launch_status();
  if (st) return st;
  snprintf(g_last_path, sizeof(g_last_path), "stream_read bytes%zu", bytes);
  return ATTNQ8_OK;
}

}  // extern "C"
