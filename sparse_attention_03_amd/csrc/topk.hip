// topk.hip -- causal top-k selection on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), section
// "Step 2", and the gamebaike.com summary, 【细粒度Token选择机制】: each query
// keeps only the candidates whose index scores rank in the top k.  Order:
// score descending, ties to the lower position, -0 == +0, NaN lowest.
//
// One workgroup per score row, one pass over the row (few long rows -- decode
// batches -- split each row into segments first, see below).  Scores become
// order-preserving 32-bit keys.  The row is streamed in 2048-element chunks;
// candidates (key, position) that beat the running threshold are appended to
// an LDS buffer in position order (block-wide exclusive scan, so the buffer
// stays sorted by position).  When the buffer would overflow it is cut to
// exactly k entries by a histogram refinement over the buffer's own key
// range (LDS histograms, at most four passes) and a stable filter; the k-th key becomes the new threshold, and
// later elements (larger positions) must beat it strictly.  The final cut
// leaves the k winners already in ascending position order.  Integer work
// only: the selection is exact.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kPer = 8;
constexpr int kChunk = kTkThreads * kPer;  // 2048
constexpr int kMaxK = 2048;
constexpr int kCap = kMaxK + kChunk;       // 4096
constexpr int kSegMax = kCap / kTkThreads; // 16

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks below every number
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkShared {
  uint32_t key[kCap];
  int32_t pos[kCap];
  int hist[256];
  int wave_sum[2][kTkWaves];   // double-buffered: one barrier per scan
  uint32_t red[2][kTkWaves];
  int digit;
  int need;
  int parity;
};

// Exclusive prefix over the lanes of a small non-negative count (< 2^NBITS),
// from one ballot per bit: no cross-lane data movement.
template <int NBITS>
__device__ __forceinline__ int wave_excl_prefix_small(int v, int& wave_total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < NBITS; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    pre += below << b;
    tot += __popcll(m) << b;
  }
  wave_total = tot;
  return pre;
}

// Exclusive scan over the block (thread order) of a small count; every thread
// gets the total.  One barrier: the wave totals alternate between two slots.
template <int NBITS>
__device__ __forceinline__ int block_excl_scan(int v, TopkShared& sh, int& parity, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int wt;
  const int pre = wave_excl_prefix_small<NBITS>(v, wt);
  if (lane == 0) sh.wave_sum[parity][wave] = wt;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int t = sh.wave_sum[parity][w];
    off += (w < wave) ? t : 0;
    tot += t;
  }
  parity ^= 1;
  total = tot;
  return off + pre;
}

// Cut the first `cnt` (>= k) buffer entries to the k best, keeping position
// order; returns the k-th best key (the smallest kept key).  The k-th key T is
// located by histogram refinement over the buffer's own key range: each pass
// splits the current interval [lo, hi] (known to hold T) into at most 256
// equal power-of-two bins, so clustered scores still spread over the bins;
// at most four passes, none when every key is equal.
__device__ uint32_t cut_to_k(TopkShared& sh, int cnt, int k, int& parity) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int e = tid; e < cnt; e += kTkThreads) {
    const uint32_t key = sh.key[e];
    mn = min(mn, key);
    mx = max(mx, key);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  if (lane == 0) { sh.red[0][wave] = mn; sh.red[1][wave] = mx; }
  __syncthreads();
  uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < kTkWaves; ++w) { lo = min(lo, sh.red[0][w]); hi = max(hi, sh.red[1][w]); }
  int need = k;  // entries of [lo, hi] still to take, counted from the top
  while (hi > lo) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    const int nbins = (int)(span >> shift) + 1;  // <= 256
    sh.hist[tid] = 0;
    __syncthreads();
    for (int e = tid; e < cnt; e += kTkThreads) {
      const uint32_t key = sh.key[e];
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(key - lo) >> shift], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins nbins-1-4l .. nbins-4-4l (descending key order)
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = nbins - 1 - 4 * lane - j;
        c[j] = b >= 0 ? sh.hist[b] : 0;
        sum += c[j];
      }
      const int incl = wave_inclusive_scan(sum);
      const int excl = incl - sum;
      if (excl < need && need <= incl) {
        int run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < need && need <= run + c[j]) { sh.digit = nbins - 1 - 4 * lane - j; sh.need = need - run; }
          run += c[j];
        }
      }
    }
    __syncthreads();
    const uint32_t blo = lo + ((uint32_t)sh.digit << shift);
    const uint32_t bhi = blo + ((1u << shift) - 1u);
    lo = blo;
    hi = min(hi, bhi);
    need = sh.need;
  }
  const uint32_t T = lo;  // `need` entries equal to T are kept, the earliest ones
  // stable filter over contiguous per-thread segments
  const int per = (cnt + kTkThreads - 1) / kTkThreads;
  const int seg0 = min(tid * per, cnt), seg1 = min(seg0 + per, cnt);
  uint32_t kk[kSegMax];
  int32_t pp[kSegMax];
  int eq = 0;
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    const int e = seg0 + j;
    kk[j] = 0u;
    pp[j] = 0;
    if (e < seg1) { kk[j] = sh.key[e]; pp[j] = sh.pos[e]; eq += kk[j] == T; }
  }
  int tot;
  int rank = block_excl_scan<5>(eq, sh, parity, tot);
  int keep = 0;
  bool kf[kSegMax];
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    const bool in = seg0 + j < seg1;
    bool kp = in && kk[j] > T;
    if (in && kk[j] == T) { kp = rank < need; ++rank; }
    kf[j] = kp;
    keep += kp;
  }
  int off = block_excl_scan<5>(keep, sh, parity, tot);
  __syncthreads();  // every read of the buffer above precedes the writes below
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    if (kf[j]) { sh.key[off] = kk[j]; sh.pos[off] = pp[j]; ++off; }
  }
  __syncthreads();
  return T;
}

// ---------------------------------------------------------------------------
// Streaming selection over a sequence of `count` elements given in ascending
// position order.  Leaves the k best (or all, if fewer are valid) in
// sh.key/sh.pos[0 .. returned count), in ascending position order.  Src
// provides Fetch (the raw loads of one thread's kPer elements), fetch() and
// decode(); three chunks of loads are kept in flight ahead of the one being
// filtered, so the row streams at memory speed instead of load latency.
// ---------------------------------------------------------------------------
template <class Src>
__device__ int stream_select(TopkShared& sh, const Src& src, int32_t count, int k) {
  const int tid = threadIdx.x;
  int cnt = 0;
  bool have_tau = false;
  uint32_t tau = 0;
  int parity = 0;
  typename Src::Fetch f0, f1, f2, f3;
  src.fetch(0, f0);
  src.fetch(kChunk, f1);
  src.fetch(2 * kChunk, f2);
  for (int32_t c0 = 0; c0 < count; c0 += kChunk) {
    src.fetch(c0 + 3 * kChunk, f3);
    uint32_t key[kPer];
    int32_t pos[kPer];
    bool ok[kPer];
    src.decode(f0, c0 + tid * kPer, key, pos, ok);
    int c = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) c += ok[j] && (!have_tau || key[j] > tau);
    int total;
    int off = block_excl_scan<4>(c, sh, parity, total);
    if (cnt + total > kCap) {
      tau = cut_to_k(sh, cnt, k, parity);
      have_tau = true;
      cnt = k;
      c = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) c += ok[j] && key[j] > tau;
      off = block_excl_scan<4>(c, sh, parity, total);
    }
    off += cnt;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (ok[j] && (!have_tau || key[j] > tau)) { sh.key[off] = key[j]; sh.pos[off] = pos[j]; ++off; }
    }
    cnt += total;
    f0 = f1;
    f1 = f2;
    f2 = f3;
  }
  __syncthreads();
  if (cnt > k) {
    cut_to_k(sh, cnt, k, parity);
    cnt = k;
  }
  return cnt;
}

// Elements are the scores of one row at positions [lo, hi).
struct ScoreSrc {
  struct Fetch { f32x4 a, b; };
  const float* row;
  int32_t lo, hi;
  __device__ void fetch(int32_t c0, Fetch& f) const {
    const int32_t p = lo + c0 + (int32_t)threadIdx.x * kPer;  // lo is a multiple of kPer
    f.a = f32x4{0.f, 0.f, 0.f, 0.f};
    f.b = f.a;
    if (p < hi) f.a = *(const f32x4*)(row + p);
    if (p + 4 < hi) f.b = *(const f32x4*)(row + p + 4);
  }
  __device__ void decode(const Fetch& f, int32_t i0, uint32_t (&key)[kPer], int32_t (&pos)[kPer],
                         bool (&ok)[kPer]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) { key[j] = order_key(f.a[j]); key[4 + j] = order_key(f.b[j]); }
#pragma unroll
    for (int j = 0; j < kPer; ++j) { pos[j] = lo + i0 + j; ok[j] = pos[j] < hi; }
  }
};

// Elements are (key, position) candidates; position -1 marks padding.
struct CandSrc {
  struct Fetch { i32x4 ka, kb, pa, pb; };
  const uint32_t* key;
  const int32_t* pos;
  int32_t count;
  __device__ void fetch(int32_t c0, Fetch& f) const {
    const int32_t i = c0 + (int32_t)threadIdx.x * kPer;
    f.ka = f.kb = i32x4{0, 0, 0, 0};
    f.pa = f.pb = i32x4{-1, -1, -1, -1};
    if (i < count) {  // count is a multiple of kPer
      f.ka = *(const i32x4*)(key + i);
      f.kb = *(const i32x4*)(key + i + 4);
      f.pa = *(const i32x4*)(pos + i);
      f.pb = *(const i32x4*)(pos + i + 4);
    }
  }
  __device__ void decode(const Fetch& f, int32_t, uint32_t (&k)[kPer], int32_t (&p)[kPer], bool (&ok)[kPer]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      k[j] = (uint32_t)f.ka[j]; k[4 + j] = (uint32_t)f.kb[j];
      p[j] = f.pa[j]; p[4 + j] = f.pb[j];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) ok[j] = p[j] >= 0;
  }
};

// One workgroup per row: the whole selection in one pass over the row.
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                          int32_t row_begin, const float* __restrict__ scores,
                                                          int64_t ld, int32_t k, int32_t* __restrict__ idx) {
  __shared__ TopkShared sh;
  const int32_t r = row_begin + blockIdx.x;
  const RowInfo ri = locate_row(cu_q, cu_k, num_seqs, r);
  const int32_t n = ri.pos + 1;
  int32_t* out = idx + (int64_t)blockIdx.x * k;
  const int tid = threadIdx.x;
  if (n <= k) {
    for (int e = tid; e < k; e += kTkThreads) out[e] = e < n ? e : -1;
    return;
  }
  const ScoreSrc src{scores + (int64_t)blockIdx.x * ld, 0, n};
  const int cnt = stream_select(sh, src, n, k);
  for (int e = tid; e < k; e += kTkThreads) out[e] = e < cnt ? sh.pos[e] : -1;
}

// Few long rows: phase 1 selects the top k (>= the row's k_row) of each of
// `nseg` segments of a row (the global winners are winners of their segment,
// so nothing is lost), keeping (key, position) in position order, padded with
// position -1.
__global__ __launch_bounds__(kTkThreads) void topk_segment_kernel(const int32_t* __restrict__ cu_q,
                                                                  const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                                  int32_t row_begin, const float* __restrict__ scores,
                                                                  int64_t ld, int32_t k_row, int32_t k,
                                                                  int32_t seg_len,
                                                                  uint32_t* __restrict__ ckey,
                                                                  int32_t* __restrict__ cpos) {
  __shared__ TopkShared sh;
  const int32_t rl = blockIdx.x, seg = blockIdx.y, nseg = gridDim.y;
  const RowInfo ri = locate_row(cu_q, cu_k, num_seqs, row_begin + rl);
  const int32_t n = ri.pos + 1;
  if (n <= k_row) return;  // the merge writes every candidate directly
  const int32_t lo = seg * seg_len, hi = min(n, lo + seg_len);
  uint32_t* okey = ckey + ((int64_t)rl * nseg + seg) * k;
  int32_t* opos = cpos + ((int64_t)rl * nseg + seg) * k;
  int cnt = 0;
  if (lo < hi) {
    const ScoreSrc src{scores + (int64_t)rl * ld, lo, hi};
    cnt = stream_select(sh, src, hi - lo, k);
  }
  for (int e = threadIdx.x; e < k; e += kTkThreads) {
    okey[e] = e < cnt ? sh.key[e] : 0u;
    opos[e] = e < cnt ? sh.pos[e] : -1;
  }
}

// Phase 2: the same selection over the row's nseg * kp candidates (kp = k
// rounded up to a multiple of 8, the padded length of each segment's list).
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(const int32_t* __restrict__ cu_q,
                                                                const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                                int32_t row_begin, int32_t nseg, int32_t k,
                                                                int32_t kp, const uint32_t* __restrict__ ckey,
                                                                const int32_t* __restrict__ cpos,
                                                                int32_t* __restrict__ idx) {
  __shared__ TopkShared sh;
  const int32_t rl = blockIdx.x;
  const RowInfo ri = locate_row(cu_q, cu_k, num_seqs, row_begin + rl);
  const int32_t n = ri.pos + 1;
  int32_t* out = idx + (int64_t)rl * k;
  if (n <= k) {
    for (int e = threadIdx.x; e < k; e += kTkThreads) out[e] = e < n ? e : -1;
    return;
  }
  const CandSrc src{ckey + (int64_t)rl * nseg * kp, cpos + (int64_t)rl * nseg * kp, nseg * kp};
  const int cnt = stream_select(sh, src, nseg * kp, k);
  for (int e = threadIdx.x; e < k; e += kTkThreads) out[e] = e < cnt ? sh.pos[e] : -1;
}

}  // namespace

bool topk_may_segment(int max_ctx, int k) { return max_ctx / (4 * k) > 1; }

int topk_segments(int rows, int max_ctx, int k, int num_cus) {
  if (rows <= 0 || rows >= num_cus || !topk_may_segment(max_ctx, k)) return 1;
  // enough workgroups for the machine, but segments of at least 4k entries so
  // that phase 1 actually discards most of each segment
  int nseg = (2 * num_cus + rows - 1) / rows;
  const int by_len = max_ctx / (4 * k);
  if (nseg > by_len) nseg = by_len;
  return nseg > 1 ? nseg : 1;
}

size_t topk_workspace_bytes(int rows, int max_ctx, int k, int num_cus) {
  const int nseg = topk_segments(rows, max_ctx, k, num_cus);
  if (nseg <= 1) return 0;
  const size_t n = (size_t)rows * nseg * (size_t)((k + kPer - 1) / kPer * kPer);
  return 2 * ((n * 4 + 255) / 256 * 256);
}

hipError_t launch_topk(const TopkLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  if (L.k > kMaxK || L.k < 1) return hipErrorInvalidValue;
  const int nseg = topk_segments(rows, L.b.max_ctx, L.k, L.num_cus);
  if (nseg <= 1) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, L.b.cu_q, L.b.cu_k, L.b.num_seqs,
                       L.b.row_begin, L.scores, L.ld, L.k, L.idx);
    return hipGetLastError();
  }
  // candidate lists are padded to a multiple of kPer so that loads stay aligned
  const int kp = (L.k + kPer - 1) / kPer * kPer;
  const size_t n = (size_t)rows * nseg * kp;
  uint32_t* ckey = (uint32_t*)L.ws;
  int32_t* cpos = (int32_t*)((char*)L.ws + (n * 4 + 255) / 256 * 256);
  int32_t seg_len = (L.b.max_ctx + nseg - 1) / nseg;
  seg_len = (seg_len + kChunk - 1) / kChunk * kChunk;
  hipLaunchKernelGGL(topk_segment_kernel, dim3((unsigned)rows, (unsigned)nseg), dim3(kTkThreads), 0, s, L.b.cu_q,
                     L.b.cu_k, L.b.num_seqs, L.b.row_begin, L.scores, L.ld, L.k, kp, seg_len, ckey, cpos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, L.b.cu_q, L.b.cu_k,
                     L.b.num_seqs, L.b.row_begin, nseg, L.k, kp, ckey, cpos, L.idx);
  return hipGetLastError();
}

}  // namespace dsa
