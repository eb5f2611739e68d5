// dsa_common.h -- device helpers shared by the libdsa kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DSA_LDS __attribute__((address_space(3)))

namespace dsa {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int kWave = 64;

// Wait until at most N vector-memory instructions of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One HBM -> LDS copy instruction (global_load_lds_dwordx4): lane l's 16 bytes
// at src land at dst + 16 l; dst is wave-uniform.  Written out rather than
// through the compiler builtin because the compiler, which cannot tell LDS
// reads without type-based alias information (the transposing reads among
// them) apart from the copies, would wait for every copy in flight before each
// such read and so undo the prefetch.  The copy's completion is the caller's
// to track, with counted vmcnt waits and a barrier before the data is read.
// M0 carries the LDS base (one wait state separates its write from the copy);
// the kernels that use this keep nothing else in M0, which the compiler
// reserves and warns about naming as clobbered.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* src, DSA_LDS void* dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(src)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup rendezvous for the tile loop that does not drain vector memory:
// this wave's LDS operations complete (lgkmcnt 0), then every wave meets.
// The HBM -> LDS copies in flight are left alone; their completion is tracked
// by the counted vmcnt waits before this barrier.  (__syncthreads() carries a
// release fence, which would wait for every outstanding copy.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Where a query row sits in the ragged batch: position of the query, first
// key/latent row of its sequence.  Query row r of sequence b has position
// ctx_b - q_b + (r - cu_q[b]) and sees the candidates [0, pos].
struct RowInfo {
  int32_t pos;
  int32_t kbase;
};

__device__ inline RowInfo locate_row(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                                     int num_seqs, int32_t r) {
  int lo = 0, hi = num_seqs;  // invariant: cu_q[lo] <= r < cu_q[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= r) lo = mid; else hi = mid;
  }
  const int32_t q0 = cu_q[lo], q1 = cu_q[lo + 1];
  const int32_t k0 = cu_k[lo], k1 = cu_k[lo + 1];
  RowInfo ri;
  ri.pos = (k1 - k0) - (q1 - q0) + (r - q0);
  ri.kbase = k0;
  return ri;
}

// The same lookup for a row that is uniform over the wave, with every lane
// active.  For batches of at most 127 sequences the lanes hold the cu_q / cu_k
// entries, lane l entries l and 64 + l (load_seq_table, one load each, a
// second pair only for 64 sequences or more, for the whole kernel), and a row
// is located with one ballot per half; larger batches fall back to the
// binary search.
struct SeqTable {
  int32_t q, k;    // cu_q[lane], cu_k[lane] (lane <= num_seqs)
  int32_t q2, k2;  // cu_q[64 + lane], cu_k[64 + lane] (64 + lane <= num_seqs)
  int32_t n;       // num_seqs
};

__device__ inline SeqTable load_seq_table(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                                          int num_seqs) {
  const int lane = threadIdx.x & 63;
  SeqTable t;
  t.n = num_seqs;
  t.q = 0;
  t.k = 0;
  t.q2 = 0;
  t.k2 = 0;
  if (num_seqs < 128) {
    const int i = min(lane, num_seqs);
    t.q = cu_q[i];
    t.k = cu_k[i];
    if (num_seqs >= 64) {
      const int i2 = min(64 + lane, num_seqs);
      t.q2 = cu_q[i2];
      t.k2 = cu_k[i2];
    }
  }
  return t;
}

__device__ inline RowInfo locate_row_wave(const SeqTable& t, const int32_t* __restrict__ cu_q,
                                          const int32_t* __restrict__ cu_k, int32_t r) {
  if (t.n >= 128) return locate_row(cu_q, cu_k, t.n, r);
  const int lane = threadIdx.x & 63;
  // cu_q[0] = 0 <= r and cu_q is nondecreasing: entries 1 .. b are the ones <= r
  int b = __popcll(__ballot(lane >= 1 && lane <= t.n && t.q <= r));
  RowInfo ri;
  if (t.n < 64) {
    const int32_t q0 = __builtin_amdgcn_readlane(t.q, b), q1 = __builtin_amdgcn_readlane(t.q, b + 1);
    const int32_t k0 = __builtin_amdgcn_readlane(t.k, b), k1 = __builtin_amdgcn_readlane(t.k, b + 1);
    ri.pos = (k1 - k0) - (q1 - q0) + (r - q0);
    ri.kbase = k0;
    return ri;
  }
  b += __popcll(__ballot(64 + lane <= t.n && t.q2 <= r));
  // entry i: lane i of the first pair (i < 64) or lane i - 64 of the second
  auto q_at = [&](int i) { return i < 64 ? __builtin_amdgcn_readlane(t.q, i) : __builtin_amdgcn_readlane(t.q2, i - 64); };
  auto k_at = [&](int i) { return i < 64 ? __builtin_amdgcn_readlane(t.k, i) : __builtin_amdgcn_readlane(t.k2, i - 64); };
  const int32_t q0 = q_at(b), q1 = q_at(b + 1), k0 = k_at(b), k1 = k_at(b + 1);
  ri.pos = (k1 - k0) - (q1 - q0) + (r - q0);
  ri.kbase = k0;
  return ri;
}

__device__ inline float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over a wave (lane order).
__device__ inline int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ inline unsigned ballot_lo(bool p) { return (unsigned)__ballot(p); }

}  // namespace dsa
