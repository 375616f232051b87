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
// One pass over the logits, about one block per compute unit: a block covers
// a contiguous range of its row in quads of four logits (16-byte loads when
// the row starts 16-byte aligned); each lane takes the maximum of its values
// and the index of its first occurrence, then the sum of exp(x - max) as
// independent terms; lanes and waves merge in a fixed pattern, each block
// publishes its state in the scratch as self-validating atomic words and takes
// a ticket; the block that draws the row's last ticket merges the row's block
// states in block order, writes the result and clears the slots and the
// ticket.  The merge order never depends
// on arrival order, so results are run-to-run bitwise identical.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "device_utils.h"

namespace attnq8 {

constexpr int kHeadThreads = 256;
constexpr int kHeadQuads = 8;                                  // quads (4 logits) per lane per pass
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

// A block's state as published to the last block: three 64-bit words, each
// the 32-bit value (m, s, idx) with a valid flag in its high half, written and
// read as single atomic objects, so that a reader that sees the flag also sees
// that word's value; the reader clears the words after use.
struct HeadSlot {
  unsigned long long w[3];
};
constexpr unsigned long long kHeadValid = 1ull << 32;
constexpr int kHeadSpinLimit = 1 << 16;  // bounded wait for a published word

struct HeadArgs {
  const float* logits;  // row r starts at logits + r * row_stride
  long long row_stride;
  int vocab;
  int blocks_per_row;
  int block_quads;      // quads of four logits per block (the last block: the rest)
  HeadSlot* slot;       // [n_rows][blocks_per_row], all words zero between calls
  unsigned* ticket;     // [n_rows], zero between calls
  int* token;           // [n_rows]
  float* top_prob;      // [n_rows] (may be null)
};

// exp(d) for d <= 0 on the hardware exponential (v_exp_f32, about 1 ulp); a
// result below fp32's normal range reads as 0, which changes no sum here: every
// sum holds a term exp(0) = 1.
__device__ __forceinline__ float head_exp(float d) { return __builtin_amdgcn_exp2f(d * kHeadLog2e); }

// symmetric in its arguments (so every lane of a butterfly gets the same bits)
__device__ __forceinline__ HeadState head_merge(const HeadState& a, const HeadState& b) {
  HeadState r;
  r.m = fmaxf(a.m, b.m);
  r.s = r.m == -INFINITY ? 0.0f : a.s * head_exp(a.m - r.m) + b.s * head_exp(b.m - r.m);
  r.idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : min(a.idx, b.idx));
  r.pad = 0;
  return r;
}

// The partner's state under a lane involution: DPP within rows of 16 lanes
// (quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors), then
// the gfx950 row swaps (lanes l ^ 16, l ^ 32), which hand each lane its own
// value and its partner's in some order -- the merge is symmetric, so the order
// does not matter.  After each step a lane and its partner hold the same bits,
// so after the six steps every lane holds the wave's state.
template <int CTRL>
__device__ __forceinline__ HeadState head_dpp_merge(const HeadState& st) {
  HeadState p;
  p.m = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(st.m), CTRL, 0xF, 0xF, false));
  p.s = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(st.s), CTRL, 0xF, 0xF, false));
  p.idx = __builtin_amdgcn_update_dpp(0, st.idx, CTRL, 0xF, 0xF, false);
  return head_merge(st, p);
}

template <bool ROW32>
__device__ __forceinline__ HeadState head_swap_merge(const HeadState& st) {
  const uint32_t m = __float_as_uint(st.m), s = __float_as_uint(st.s), i = (uint32_t)st.idx;
  auto sm = ROW32 ? __builtin_amdgcn_permlane32_swap(m, m, false, false) : __builtin_amdgcn_permlane16_swap(m, m, false, false);
  auto ss = ROW32 ? __builtin_amdgcn_permlane32_swap(s, s, false, false) : __builtin_amdgcn_permlane16_swap(s, s, false, false);
  auto si = ROW32 ? __builtin_amdgcn_permlane32_swap(i, i, false, false) : __builtin_amdgcn_permlane16_swap(i, i, false, false);
  const HeadState a = {__uint_as_float(sm[0]), __uint_as_float(ss[0]), (int)si[0], 0};
  const HeadState b = {__uint_as_float(sm[1]), __uint_as_float(ss[1]), (int)si[1], 0};
  return head_merge(a, b);
}

__device__ __forceinline__ HeadState head_wave_merge(HeadState st) {
  st = head_dpp_merge<0xB1>(st);   // quad_perm [1,0,3,2]: lane ^ 1
  st = head_dpp_merge<0x4E>(st);   // quad_perm [2,3,0,1]: lane ^ 2
  st = head_dpp_merge<0x141>(st);  // row_half_mirror: lane i <-> 7 - i of its 8
  st = head_dpp_merge<0x140>(st);  // row_mirror: lane i <-> 15 - i of its 16
  st = head_swap_merge<false>(st);
  st = head_swap_merge<true>(st);
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

// The state of the values x[0..N) at indices idx[0..N), in increasing index
// order: the maximum and its first index, then the sum of exp(x - max) over the
// finite values as independent terms.
template <int N>
__device__ __forceinline__ HeadState head_state_of(const float (&x)[N], const int (&idx)[N]) {
  HeadState st = {-INFINITY, 0.0f, kHeadNone, 0};
#pragma unroll
  for (int k = 0; k < N; ++k) {
    // a NaN never compares; -inf is an ordinary value (first one wins);
    // selects rather than branches
    const bool gt = x[k] > st.m;
    const bool first = (x[k] == st.m) & (st.idx == kHeadNone);
    st.idx = (gt | first) ? idx[k] : st.idx;
    st.m = gt ? x[k] : st.m;
  }
  if (st.m != -INFINITY) {
    float e[N];
    // exp(-inf - m) is 0; a NaN term is dropped
#pragma unroll
    for (int k = 0; k < N; ++k) e[k] = x[k] == x[k] ? head_exp(x[k] - st.m) : 0.0f;
    // pairwise, in a fixed order
#pragma unroll
    for (int w = 1; w < N; w *= 2)
#pragma unroll
      for (int k = 0; k + w < N; k += 2 * w) e[k] += e[k + w];
    st.s = e[0];
  }
  return st;
}

__global__ __launch_bounds__(kHeadThreads) void head_greedy_kernel(HeadArgs a) {
  __shared__ HeadState lds[kHeadThreads / 64];
  __shared__ int last;
  const int row = blockIdx.y;
  const int blk = blockIdx.x;
  const int lane = threadIdx.x;
  const float* x = a.logits + (long long)row * a.row_stride;

  // quads [q0, q1) of the row; the last block also takes the vocab % 4 tail
  const long long nq = a.vocab >> 2;
  const long long q0 = (long long)blk * a.block_quads;
  const long long q1 = blk == a.blocks_per_row - 1 ? nq : min(nq, q0 + a.block_quads);
  HeadState st = {-INFINITY, 0.0f, kHeadNone, 0};
  // 16-byte loads when the row starts 16-byte aligned (block-uniform)
  auto scan = [&](auto vec) {
    for (long long base = q0; base < q1; base += (long long)kHeadQuads * kHeadThreads) {
      float v[4 * kHeadQuads];
      int vi[4 * kHeadQuads];
#pragma unroll
      for (int j = 0; j < kHeadQuads; ++j) {
        const long long q = base + (long long)j * kHeadThreads + lane;
        float4_t f = {NAN, NAN, NAN, NAN};  // past the range: skipped like NaN
        if (q < q1) {
          if constexpr (decltype(vec)::value) f = __builtin_nontemporal_load((const float4_t*)(x + 4 * q));
          else f = (float4_t){x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[4 * j + c] = f[c];
          vi[4 * j + c] = (int)(4 * q + c);
        }
      }
      st = head_merge(st, head_state_of(v, vi));
    }
  };
  if ((((uintptr_t)x) & 15) == 0) scan(std::true_type());
  else scan(std::false_type());
  if (blk == a.blocks_per_row - 1 && lane < (a.vocab & 3)) {
    float t[1] = {x[4 * nq + lane]};
    int ti[1] = {(int)(4 * nq + lane)};
    st = head_merge(st, head_state_of(t, ti));
  }
  st = head_block_merge(st, lds);

  // Hand-off: the block publishes its state as three self-validating atomic
  // words, then takes a ticket; the block that draws the row's last ticket
  // reads every slot of the row, waiting (boundedly) for each word's flag --
  // the writer stored it before taking its ticket, so it arrives -- merges the
  // states in block order, clears the slots and the ticket for the next call.
  HeadSlot* slots = a.slot + (long long)row * a.blocks_per_row;
  if (threadIdx.x == 0) {
    HeadSlot* p = slots + blk;
    __hip_atomic_store(&p->w[0], kHeadValid | __float_as_uint(st.m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->w[1], kHeadValid | __float_as_uint(st.s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->w[2], kHeadValid | (uint32_t)st.idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned t = __hip_atomic_fetch_add(&a.ticket[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = t == (unsigned)a.blocks_per_row - 1;
  }
  __syncthreads();
  if (!last) return;

  // the last block of the row: merge the row's block states in block order
  // (a row of at most 64 blocks: wave 0 alone; merging with the empty state
  // of an absent block leaves every bit unchanged, so both forms agree)
  const bool one_wave = a.blocks_per_row <= 64;
  if (one_wave && threadIdx.x >= 64) return;
  HeadState r = {-INFINITY, 0.0f, kHeadNone, 0};
  if ((int)threadIdx.x < a.blocks_per_row) {
    HeadSlot* p = slots + threadIdx.x;
    unsigned long long w[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) w[k] = __hip_atomic_load(&p->w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int spin = 0; !(w[0] & w[1] & w[2] & kHeadValid) && spin < kHeadSpinLimit; ++spin) {
#pragma unroll
      for (int k = 0; k < 3; ++k)
        if (!(w[k] & kHeadValid)) w[k] = __hip_atomic_load(&p->w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) __hip_atomic_store(&p->w[k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.m = __uint_as_float((uint32_t)w[0]);
    r.s = __uint_as_float((uint32_t)w[1]);
    r.idx = (int)(uint32_t)w[2];
  }
  if (one_wave) {
    r = head_wave_merge(r);
  } else {
    __syncthreads();  // lds is reused
    r = head_block_merge(r, lds);
  }
  if (threadIdx.x == 0) {
    a.token[row] = r.idx == kHeadNone ? -1 : r.idx;
    if (a.top_prob) a.top_prob[row] = r.m == -INFINITY ? NAN : 1.0f / r.s;
    __hip_atomic_store(&a.ticket[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
  }
}

}  // namespace attnq8
