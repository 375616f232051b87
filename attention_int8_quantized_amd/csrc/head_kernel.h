// The verify head's greedy token and its probability, per row of logits.
//
// "[Engine] perf(hip): optimize MTP draft, shared expert, and verify/sampler
// head kernels on RDNA4" (Problem and result item 1, Summary item 1): the
// verifier's T rows of 248,320 fp32 logits are scanned by many blocks per row
// for the greedy token (argmax) and the row's top probability, with one scratch
// for 1..8 rows.  Per row x[0 .. V-1]:
//   token    = smallest i with x[i] = max of the non-NaN entries (-1: none)
//   top_prob = 1 / sum_i exp(x[i] - x[token]) over the non-NaN entries
//              (-inf entries add 0; NaN when no entry is finite)
//
// One pass over the logits: every lane keeps an online state (max, index of
// its first occurrence, sum of exp(x - max) rescaled when the max moves),
// lanes and waves merge in a fixed pattern, each block writes its state to the
// scratch and takes a ticket; the block that draws the row's last ticket merges
// the row's block states in block order, writes the result and puts the ticket
// back to zero.  The merge order never depends on arrival order, so results are
// run-to-run bitwise identical.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_utils.h"

namespace attnq8 {

constexpr int kHeadThreads = 256;
constexpr int kHeadPerLane = 16;                               // logits per lane per pass
constexpr int kHeadChunk = kHeadThreads * kHeadPerLane;        // 4,096 logits
constexpr int kHeadMaxBlocks = 256;                            // blocks per row
constexpr int kHeadNone = 0x7FFFFFFF;                          // no index yet
constexpr int kHeadMaxRows = 1024;
constexpr int kHeadTicketBytes = kHeadMaxRows * 4;             // at the scratch's start
constexpr float kHeadLog2e = 1.44269504088896341f;

struct HeadState {
  float m;  // largest non-NaN value so far (-inf: none or only -inf)
  float s;  // sum of exp(x - m) over the finite values so far
  int idx;  // first index holding m (kHeadNone: no non-NaN value yet)
  int pad;
};

struct HeadArgs {
  const float* logits;  // row r starts at logits + r * row_stride
  long long row_stride;
  int vocab;
  int blocks_per_row;
  HeadState* part;      // [n_rows][blocks_per_row]
  unsigned* ticket;     // [n_rows], zero between calls
  int* token;           // [n_rows]
  float* top_prob;      // [n_rows] (may be null)
};

__device__ __forceinline__ float head_exp(float d) { return exp2f(d * kHeadLog2e); }

// add logit x at index i (indices arrive in increasing order per lane)
__device__ __forceinline__ void head_push(HeadState& st, float x, int i) {
  if (x > st.m) {
    st.s = st.s * head_exp(st.m - x) + 1.0f;  // m = -inf: s is 0 and stays 0
    st.m = x;
    st.idx = i;
  } else if (x == st.m) {
    if (st.idx == kHeadNone) st.idx = i;
    if (x != -INFINITY) st.s += 1.0f;
  } else if (x == x && x != -INFINITY) {
    st.s += head_exp(x - st.m);
  }
}

// symmetric in its arguments (so every lane of a butterfly gets the same bits)
__device__ __forceinline__ HeadState head_merge(const HeadState& a, const HeadState& b) {
  HeadState r;
  r.m = fmaxf(a.m, b.m);
  r.s = r.m == -INFINITY ? 0.0f : a.s * head_exp(a.m - r.m) + b.s * head_exp(b.m - r.m);
  r.idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : min(a.idx, b.idx));
  r.pad = 0;
  return r;
}

__device__ __forceinline__ HeadState head_wave_merge(HeadState st) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    HeadState p;
    p.m = __shfl_xor(st.m, o, 64);
    p.s = __shfl_xor(st.s, o, 64);
    p.idx = __shfl_xor(st.idx, o, 64);
    st = head_merge(st, p);
  }
  return st;
}

// merge one state per thread of the block; every thread returns the block's state
__device__ __forceinline__ HeadState head_block_merge(HeadState st, HeadState* lds) {
  constexpr int NWAVE = kHeadThreads / 64;
  st = head_wave_merge(st);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = st;
  __syncthreads();
  HeadState r = lds[0];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) r = head_merge(r, lds[w]);
  return r;
}

__global__ __launch_bounds__(kHeadThreads) void head_greedy_kernel(HeadArgs a) {
  __shared__ HeadState lds[kHeadThreads / 64];
  __shared__ int last;
  const int row = blockIdx.y;
  const int blk = blockIdx.x;
  const float* x = a.logits + (long long)row * a.row_stride;

  HeadState st = {-INFINITY, 0.0f, kHeadNone, 0};
  const long long step = (long long)a.blocks_per_row * kHeadChunk;
  for (long long base = (long long)blk * kHeadChunk; base < a.vocab; base += step) {
    float v[kHeadPerLane];
#pragma unroll
    for (int j = 0; j < kHeadPerLane; ++j) {
      const long long i = base + j * kHeadThreads + threadIdx.x;
      v[j] = i < a.vocab ? x[i] : NAN;  // past the row: skipped like a NaN
    }
#pragma unroll
    for (int j = 0; j < kHeadPerLane; ++j)
      head_push(st, v[j], (int)(base + j * kHeadThreads + threadIdx.x));
  }
  st = head_block_merge(st, lds);

  // The block states go out as device-scope atomic stores (written through
  // to the device's coherence point) and are read back as device-scope atomic
  // loads, and the state's stores have completed (vmcnt 0) before the ticket
  // is taken; no full-cache fence is needed.
  HeadState* part = a.part + (long long)row * a.blocks_per_row;
  if (threadIdx.x == 0) {
    HeadState* p = part + blk;
    __hip_atomic_store(&p->m, st.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->s, st.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->idx, st.idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    const unsigned t =
        __hip_atomic_fetch_add(&a.ticket[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = t == (unsigned)a.blocks_per_row - 1;
  }
  __syncthreads();
  if (!last) return;

  // the last block of the row: merge the row's block states in block order
  HeadState r = {-INFINITY, 0.0f, kHeadNone, 0};
  if ((int)threadIdx.x < a.blocks_per_row) {
    HeadState* p = part + threadIdx.x;
    r.m = __hip_atomic_load(&p->m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.s = __hip_atomic_load(&p->s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.idx = __hip_atomic_load(&p->idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // lds is reused
  r = head_block_merge(r, lds);
  if (threadIdx.x == 0) {
    a.token[row] = r.idx == kHeadNone ? -1 : r.idx;
    if (a.top_prob) a.top_prob[row] = r.m == -INFINITY ? NAN : 1.0f / r.s;
    a.ticket[row] = 0u;  // ready for the next call
  }
}

}  // namespace attnq8
