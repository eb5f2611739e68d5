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
  int fcnt[2][kTkWaves];       // per-wave counts of the cut's filter
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

// The k-th best key T of the first `cnt` (>= k) buffer entries, and in `need`
// how many of the entries equal to T rank among the k best.  T is located by
// histogram refinement over the buffer's own key range: each pass splits the
// current interval [lo, hi] (known to hold T) into at most 256 equal
// power-of-two bins, so clustered scores still spread over the bins; at most
// four passes, none when every key is equal.
__device__ uint32_t kth_key(TopkShared& sh, int cnt, int k, int& need) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the thread's keys (entries tid + 256 j) stay in registers for every pass
  uint32_t kr[kSegMax];
  bool kv[kSegMax];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    const int e = tid + kTkThreads * j;
    kv[j] = e < cnt;
    kr[j] = kv[j] ? sh.key[e] : 0u;
    if (kv[j]) {
      mn = min(mn, kr[j]);
      mx = max(mx, kr[j]);
    }
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
  need = k;  // entries of [lo, hi] still to take, counted from the top
  while (hi > lo) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    const int nbins = (int)(span >> shift) + 1;  // <= 256
    sh.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSegMax; ++j)
      if (kv[j] && kr[j] >= lo && kr[j] <= hi) atomicAdd(&sh.hist[(kr[j] - lo) >> shift], 1);
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
  return lo;
}

// Cut the first `cnt` (>= k) buffer entries to the k best, keeping position
// order; returns the k-th best key (the smallest kept key).  The filter: wave
// w takes a contiguous range of 64-entry blocks (lane l: entry l of each
// block, conflict-free LDS reads) into registers, ballots order the lanes and
// one exchange of per-wave counts orders the waves; every read precedes the
// barrier of that exchange, so the kept entries are written back in place.
__device__ uint32_t cut_to_k(TopkShared& sh, int cnt, int k, int& parity) {
  (void)parity;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int need;
  const uint32_t T = kth_key(sh, cnt, k, need);
  const int L = (cnt + 64 * kTkWaves - 1) / (64 * kTkWaves) * 64;  // <= 64 * kSegMax
  const int w0 = min(wave * L, cnt), w1 = min(w0 + L, cnt);
  uint32_t kk[kSegMax];
  int32_t pp[kSegMax];
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    const int e = w0 + 64 * j + lane;
    const bool in = 64 * j < L && e < w1;
    kk[j] = in ? sh.key[e] : 0u;
    pp[j] = in ? sh.pos[e] : -1;  // buffered positions are >= 0: -1 marks an empty slot
    gt += __popcll(__ballot(in && kk[j] > T));
    eq += __popcll(__ballot(in && kk[j] == T));
  }
  if (lane == 0) { sh.fcnt[0][wave] = eq; sh.fcnt[1][wave] = gt; }
  __syncthreads();
  int eqrun = 0, keeprun = 0;
  {
    int eq_pre = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const int e_w = sh.fcnt[0][w], g_w = sh.fcnt[1][w];
      const int keep_w = g_w + min(max(need - eq_pre, 0), e_w);
      if (w < wave) { eqrun += e_w; keeprun += keep_w; }
      eq_pre += e_w;
    }
  }
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    const bool in = pp[j] >= 0;
    const bool is_eq = in && kk[j] == T;
    const uint64_t meq = __ballot(is_eq);
    const int rank = eqrun + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(meq >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)meq, 0u));
    const bool kept = (in && kk[j] > T) || (is_eq && rank < need);
    const uint64_t mk = __ballot(kept);
    const int o = keeprun + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    if (kept) { sh.key[o] = kk[j]; sh.pos[o] = pp[j]; }
    eqrun += __popcll(meq);
    keeprun += __popcll(mk);
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
// tau0 (have_tau0): start with the threshold tau0 -- only keys above it are
// admitted; *admitted: how many entries were admitted in all.
template <class Src>
__device__ int stream_select(TopkShared& sh, const Src& src, int32_t count, int k, bool have_tau0 = false,
                             uint32_t tau0 = 0, int* admitted = nullptr) {
  const int tid = threadIdx.x;
  int cnt = 0, adm = 0;
  bool have_tau = have_tau0;
  uint32_t tau = tau0;
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
    adm += total;
    f0 = f1;
    f1 = f2;
    f2 = f3;
  }
  __syncthreads();
  if (admitted) *admitted = adm;
  if (cnt > k) {
    cut_to_k(sh, cnt, k, parity);
    cnt = k;
  }
  return cnt;
}

// Long rows start from a sampled threshold: the key of rank ~1.5 k n_s / n
// among n_s = 4096 entries (four contiguous blocks spread over the row), so
// that about 1.5 k entries of the row reach it and the stream rarely needs a
// cut.  The result stays exact: if at least k entries reach the threshold,
// the k-th best key of the row is at least the threshold and every winner is
// admitted; otherwise the row is selected again without it.
constexpr int kSampleBlocks = 4;
constexpr int kSampleBlock = 4 * kTkThreads;      // 1024 entries, one 16-byte load per thread
constexpr int kSampleMinRow = 16384;
static_assert(kSampleBlocks * kSampleBlock <= kCap, "the sample is staged in the candidate buffer");

__device__ uint32_t sampled_threshold(TopkShared& sh, const float* row, int32_t n, int k) {
  const int tid = threadIdx.x;
  f32x4 v[kSampleBlocks];
#pragma unroll
  for (int b = 0; b < kSampleBlocks; ++b) {
    const int32_t start = (int32_t)((int64_t)b * (n - kSampleBlock) / (kSampleBlocks - 1)) & ~3;
    v[b] = *(const f32x4*)(row + start + 4 * tid);  // start + kSampleBlock <= n; rows are 16-byte aligned
  }
#pragma unroll
  for (int b = 0; b < kSampleBlocks; ++b)
    *(i32x4*)&sh.key[b * kSampleBlock + 4 * tid] = i32x4{(int)order_key(v[b][0]), (int)order_key(v[b][1]),
                                                         (int)order_key(v[b][2]), (int)order_key(v[b][3])};
  __syncthreads();
  constexpr int m = kSampleBlocks * kSampleBlock;
  const int rank = (int)min((int64_t)m, 3LL * k * m / (2LL * n) + 8);
  int need;
  return kth_key(sh, m, rank, need);
}

// Elements are the scores of one row at positions [lo, hi).
struct ScoreSrc {
  struct Fetch { f32x4 a, b; };
  const float* row;
  int32_t lo, hi;
  __device__ void fetch(int32_t c0, Fetch& f) const {
    const int32_t p = lo + c0 + (int32_t)threadIdx.x * kPer;  // lo is a multiple of kPer
    // raw buffer loads over the row's first hi entries: entries past hi read
    // as zero (and are masked in decode), and no load is conditional
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, (uint32_t)hi * 4, 0x00020000);
    f.a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)p * 4, 0, 0));
    f.b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)p * 4 + 16, 0, 0));
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
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, r);
  const int32_t n = ri.pos + 1;
  int32_t* out = idx + (int64_t)blockIdx.x * k;
  const int tid = threadIdx.x;
  if (n <= k) {
    for (int e = tid; e < k; e += kTkThreads) out[e] = e < n ? e : -1;
    return;
  }
  const float* row = scores + (int64_t)blockIdx.x * ld;
  const ScoreSrc src{row, 0, n};
  int cnt = -1;
  if (n >= kSampleMinRow) {
    const uint32_t ts = sampled_threshold(sh, row, n, k);
    int admitted;
    const int c = stream_select(sh, src, n, k, ts > 0u, ts - 1u, &admitted);  // admits keys >= ts
    if (admitted >= k) cnt = c;
    __syncthreads();
  }
  if (cnt < 0) cnt = stream_select(sh, src, n, k);
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
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, row_begin + rl);
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
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, row_begin + rl);
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

// ---------------------------------------------------------------------------
// Few long rows (decode batches).  One 1024-thread workgroup per row, or per
// segment of a row longer than kRxCap.  Each wave loads a contiguous range of
// the row into registers (16-byte loads, lane l holding entries 4l .. 4l + 3
// of every 256-entry block), so the row is read once and never staged in LDS.
// The k-th key is found by histogram refinement (the range-adaptive 256-bin
// passes of cut_to_k, LDS atomics fed from registers), and the winners are
// written in ascending position order: ballots order the lanes of a wave, one
// exchange of per-wave counts orders the waves.  Rows longer than kRxCap are
// cut into segments whose winners, (key, position) padded with position -1,
// go to a workspace; a second launch of the same kernel selects among them.
// A winner of the row is a winner of its segment and the candidates keep
// their keys, so the result is identical.
// ---------------------------------------------------------------------------
constexpr int kRxThreads = 1024;
constexpr int kRxWaves = kRxThreads / 64;
constexpr int kRxRowVecs = 9;                               // 16-byte vectors of keys per lane
constexpr int kRxCandVecs = 5;                              // ... of (key, position) candidates
constexpr int kRxCap = kRxWaves * 256 * kRxRowVecs;         // 36864 row entries per workgroup
constexpr int kRxCapPairs = kRxWaves * 256 * kRxCandVecs;   // 20480 candidates per workgroup

struct RadixShared {
  int hist[256];
  int cnt[kRxWaves];
  int fcnt[2][kRxWaves];
  uint32_t red[2][kRxWaves];
  int digit;
  int need;
};

// IN_CAND: the entries are (key, position) candidates [rows, kp] from the
// segment pass (position -1 = padding; launched with one segment); else the
// scores of one row at positions [seg * seg_len, (seg + 1) * seg_len).
// OUT_CAND: write the winners as candidates (kp slots, padded), else their
// positions to idx (k slots, padded with -1).
// NV: 16-byte vectors per lane, enough for the launch's longest segment
// (m <= 4096 NV).
template <bool IN_CAND, bool OUT_CAND, int NV>
__global__ __launch_bounds__(kRxThreads) void topk_radix_kernel(const int32_t* __restrict__ cu_q,
                                                                const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                                int32_t row_begin, const float* __restrict__ scores,
                                                                int64_t ld, int32_t k, int32_t seg_len, int32_t kp,
                                                                uint32_t* __restrict__ ckey,
                                                                int32_t* __restrict__ cpos,
                                                                int32_t* __restrict__ idx) {
  static_assert(NV <= (IN_CAND ? kRxCandVecs : kRxRowVecs), "too many vectors per lane");
  __shared__ RadixShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t rl = blockIdx.x, seg = blockIdx.y, nseg = gridDim.y;
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, row_begin + rl);
  const int32_t n = ri.pos + 1;
  if (!IN_CAND && OUT_CAND && n <= k) return;  // the selection pass writes every position directly
  if (!OUT_CAND && n <= k) {
    int32_t* out = idx + (int64_t)rl * k;
    for (int e = tid; e < k; e += kRxThreads) out[e] = e < n ? e : -1;
    return;
  }
  // ---- load: wave w owns entries [w0, w1), L a multiple of 256
  int32_t m, lo_pos = 0;
  if constexpr (IN_CAND) {
    m = kp;
  } else {
    lo_pos = seg * seg_len;  // seg_len is a multiple of 4
    m = max(0, min(n, lo_pos + seg_len) - lo_pos);
  }
  const int L = (m + 256 * kRxWaves - 1) / (256 * kRxWaves) * 256;  // <= 256 * NV
  const int w0 = min(wave * L, m), w1 = min(w0 + L, m);
  uint32_t key[NV][4];
  int32_t pos[NV][4];
  {
    // raw buffer loads over whole 16-byte vectors (they stay in the row:
    // lo_pos and ld are multiples of 4, candidate lists multiples of 8);
    // loads past the range read zero, and all are issued before the first use
    const uint32_t bytes = (uint32_t)((m + 3) / 4 * 16);
    const void* kbase = IN_CAND ? (const void*)(ckey + (int64_t)rl * kp)
                                : (const void*)(scores + (int64_t)rl * ld + lo_pos);
    const auto ks = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, bytes, 0x00020000);
    i32x4 kv[NV], pv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = w0 + 256 * i + 4 * lane;
      const uint32_t off = 256 * i < L ? (uint32_t)e * 4u : 0xfffffff0u;  // outside the wave's range: no access
      kv[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ks, off, 0, 0));
      if constexpr (IN_CAND) {
        const auto ps = __builtin_amdgcn_make_buffer_rsrc((void*)(cpos + (int64_t)rl * kp), 0, bytes, 0x00020000);
        pv[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ps, off, 0, 0));
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = w0 + 256 * i + 4 * lane + j;
        const bool in = 256 * i < L && e < w1;
        if constexpr (IN_CAND) {
          pos[i][j] = in ? pv[i][j] : -1;
          key[i][j] = (uint32_t)kv[i][j];
        } else {
          pos[i][j] = in ? lo_pos + e : -1;
          const int bits = kv[i][j];  // copied out first: a bit_cast of the element expression read element 0
          key[i][j] = order_key(__int_as_float(bits));
        }
      }
  }
  // ---- valid entries: count, min and max key
  uint32_t mn = 0xffffffffu, mx = 0u;
  int nv = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (pos[i][j] >= 0) {
        mn = min(mn, key[i][j]);
        mx = max(mx, key[i][j]);
        ++nv;
      }
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    nv += __shfl_xor(nv, o);
  }
  if (lane == 0) { sh.red[0][wave] = mn; sh.red[1][wave] = mx; sh.cnt[wave] = nv; }
  __syncthreads();
  uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
  int nvalid = sh.cnt[0];
#pragma unroll
  for (int w = 1; w < kRxWaves; ++w) {
    lo = min(lo, sh.red[0][w]);
    hi = max(hi, sh.red[1][w]);
    nvalid += sh.cnt[w];
  }

  // ---- the k-th key T: entries above it are kept, and `need` of those equal to it (the earliest)
  const int take = min((int)k, nvalid);
  int need;
  if (nvalid > k) {
    need = k;
    while (hi > lo) {
      const uint32_t span = hi - lo;
      const int bits = 32 - __clz(span);
      const int shift = bits > 8 ? bits - 8 : 0;
      const int nbins = (int)(span >> shift) + 1;  // <= 256
      if (tid < 256) sh.hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t kk = key[i][j];
          if (pos[i][j] >= 0 && kk >= lo && kk <= hi) atomicAdd(&sh.hist[(kk - lo) >> shift], 1);
        }
      __syncthreads();
      if (wave == 0) {
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
      lo = blo;
      hi = min(hi, blo + ((1u << shift) - 1u));
      need = sh.need;
    }
  } else {
    lo = 0u;  // every valid entry is kept
    need = 0x7fffffff;
  }
  const uint32_t T = lo;

  // ---- stable filter in position order
  int gt_w = 0, eq_w = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool v = pos[i][j] >= 0;
      gt_w += v && key[i][j] > T;
      eq_w += v && key[i][j] == T;
    }
  for (int o = 32; o >= 1; o >>= 1) {
    gt_w += __shfl_xor(gt_w, o);
    eq_w += __shfl_xor(eq_w, o);
  }
  if (lane == 0) { sh.fcnt[0][wave] = eq_w; sh.fcnt[1][wave] = gt_w; }
  __syncthreads();
  int eqrun = 0, keeprun = 0;
  {
    int eq_pre = 0;
#pragma unroll
    for (int w = 0; w < kRxWaves; ++w) {
      const int e_w = sh.fcnt[0][w], g_w = sh.fcnt[1][w];
      const int keep_w = g_w + min(max(need - eq_pre, 0), e_w);
      if (w < wave) { eqrun += e_w; keeprun += keep_w; }
      eq_pre += e_w;
    }
  }
  uint32_t* okey = nullptr;
  int32_t* opos = nullptr;
  int32_t* out = nullptr;
  if constexpr (OUT_CAND) {
    okey = ckey + ((int64_t)rl * nseg + seg) * kp;
    opos = cpos + ((int64_t)rl * nseg + seg) * kp;
  } else {
    out = idx + (int64_t)rl * k;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int eq_l = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) eq_l += pos[i][j] >= 0 && key[i][j] == T;
    int eq_tot;
    int rank = eqrun + wave_excl_prefix_small<3>(eq_l, eq_tot);
    bool kept[4];
    int keep_l = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool v = pos[i][j] >= 0;
      const bool is_eq = v && key[i][j] == T;
      kept[j] = (v && key[i][j] > T) || (is_eq && rank < need);
      rank += is_eq;
      keep_l += kept[j];
    }
    int keep_tot;
    int o = keeprun + wave_excl_prefix_small<3>(keep_l, keep_tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kept[j]) {
        if constexpr (OUT_CAND) {
          okey[o] = key[i][j];
          opos[o] = pos[i][j];
        } else {
          out[o] = pos[i][j];
        }
        ++o;
      }
    }
    eqrun += eq_tot;
    keeprun += keep_tot;
  }
  if constexpr (OUT_CAND) {
    for (int e = take + tid; e < kp; e += kRxThreads) { okey[e] = 0u; opos[e] = -1; }
  } else {
    for (int e = take + tid; e < k; e += kRxThreads) out[e] = -1;
  }
}

}  // namespace

namespace {

// How a batch is selected:
//   kStream:     one 256-thread workgroup streams each row (many rows: the
//                rows fill the machine, and each is read from HBM once);
//   kRadix:      few rows of at most kRxCap entries: LDS radix select per row;
//   kRadixSeg:   few longer rows: radix select per segment, then over the
//                segments' winners;
//   kStreamSeg:  few rows too long for the radix merge: streaming selection
//                per segment, then over the segments' winners.
enum TopkKind { kStream, kRadix, kRadixSeg, kStreamSeg };
struct TopkPlan {
  TopkKind kind;
  int nseg;
  int32_t seg_len;
};

TopkPlan topk_plan(int rows, int max_ctx, int k, int num_cus) {
  TopkPlan p{kStream, 1, 0};
  if (rows <= 0 || rows >= num_cus) return p;
  // Radix select: enough (row, segment) workgroups to cover the machine, but
  // segments of at least 4k entries (so that the segment pass discards most of
  // them); a segment must fit the registers, and the winners of all segments
  // of a row must fit one more radix pass.
  const int kp = (k + kPer - 1) / kPer * kPer;
  const int lo = (max_ctx + kRxCap - 1) / kRxCap;
  const int hi = kRxCapPairs / kp;
  int nseg = min((num_cus + rows - 1) / rows, max_ctx / (4 * k));
  nseg = max(nseg, lo);
  if (nseg <= 1) {
    p.kind = kRadix;
    return p;
  }
  if (nseg <= hi) {
    p.kind = kRadixSeg;
    p.nseg = nseg;
    p.seg_len = ((max_ctx + nseg - 1) / nseg + 3) / 4 * 4;  // <= kRxCap
    return p;
  }
  // rows too long for the radix merge: streaming selection per segment
  int ns = (2 * num_cus + rows - 1) / rows;
  const int by_len = max_ctx / (4 * k);
  if (ns > by_len) ns = by_len;
  if (ns <= 1) return p;
  p.kind = kStreamSeg;
  p.nseg = ns;
  const int32_t len = (max_ctx + ns - 1) / ns;
  p.seg_len = (len + kChunk - 1) / kChunk * kChunk;
  return p;
}

template <bool IN_CAND, bool OUT_CAND, int NV>
hipError_t launch_radix_nv(const TopkLaunch& L, dim3 grid, int32_t seg_len, int32_t kp, uint32_t* ckey,
                           int32_t* cpos, hipStream_t s) {
  hipLaunchKernelGGL((topk_radix_kernel<IN_CAND, OUT_CAND, NV>), grid, dim3(kRxThreads), 0, s, L.b.cu_q, L.b.cu_k,
                     L.b.num_seqs, L.b.row_begin, L.scores, L.ld, L.k, seg_len, kp, ckey, cpos, L.idx);
  return hipGetLastError();
}

// m_max: the most entries one workgroup holds (a segment, or a row's candidates)
template <bool IN_CAND, bool OUT_CAND>
hipError_t launch_radix(const TopkLaunch& L, dim3 grid, int32_t seg_len, int32_t kp, int32_t m_max, uint32_t* ckey,
                        int32_t* cpos, hipStream_t s) {
  const int nv = (m_max + 256 * kRxWaves - 1) / (256 * kRxWaves);
  if (nv <= 1) return launch_radix_nv<IN_CAND, OUT_CAND, 1>(L, grid, seg_len, kp, ckey, cpos, s);
  if (nv <= 2) return launch_radix_nv<IN_CAND, OUT_CAND, 2>(L, grid, seg_len, kp, ckey, cpos, s);
  if (nv <= 3) return launch_radix_nv<IN_CAND, OUT_CAND, 3>(L, grid, seg_len, kp, ckey, cpos, s);
  if (nv <= 5) return launch_radix_nv<IN_CAND, OUT_CAND, 5>(L, grid, seg_len, kp, ckey, cpos, s);
  if constexpr (!IN_CAND) {
    if (nv <= 9) return launch_radix_nv<IN_CAND, OUT_CAND, 9>(L, grid, seg_len, kp, ckey, cpos, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool topk_may_segment(int max_ctx, int k) { return k > 0 && (max_ctx > kRxCap || max_ctx / (4 * k) > 1); }

size_t topk_workspace_bytes(int rows, int max_ctx, int k, int num_cus) {
  const TopkPlan p = topk_plan(rows, max_ctx, k, num_cus);
  if (p.kind != kRadixSeg && p.kind != kStreamSeg) return 0;
  const size_t n = (size_t)rows * p.nseg * (size_t)((k + kPer - 1) / kPer * kPer);
  return 2 * ((n * 4 + 255) / 256 * 256);
}

hipError_t launch_topk(const TopkLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  if (L.k > kMaxK || L.k < 1) return hipErrorInvalidValue;
  const TopkPlan p = topk_plan(rows, L.b.max_ctx, L.k, L.num_cus);
  if (p.kind == kStream) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, L.b.cu_q, L.b.cu_k, L.b.num_seqs,
                       L.b.row_begin, L.scores, L.ld, L.k, L.idx);
    return hipGetLastError();
  }
  if (p.kind == kRadix)
    return launch_radix<false, false>(L, dim3((unsigned)rows), kRxCap, 0, L.b.max_ctx, nullptr, nullptr, s);
  // candidate lists are padded to a multiple of kPer so that loads stay aligned
  const int kp = (L.k + kPer - 1) / kPer * kPer;
  const size_t n = (size_t)rows * p.nseg * kp;
  uint32_t* ckey = (uint32_t*)L.ws;
  int32_t* cpos = (int32_t*)((char*)L.ws + (n * 4 + 255) / 256 * 256);
  if (p.kind == kRadixSeg) {
    hipError_t e = launch_radix<false, true>(L, dim3((unsigned)rows, (unsigned)p.nseg), p.seg_len, kp,
                                             min(p.seg_len, L.b.max_ctx), ckey, cpos, s);
    if (e != hipSuccess) return e;
    return launch_radix<true, false>(L, dim3((unsigned)rows), 0, p.nseg * kp, p.nseg * kp, ckey, cpos, s);
  }
  hipLaunchKernelGGL(topk_segment_kernel, dim3((unsigned)rows, (unsigned)p.nseg), dim3(kTkThreads), 0, s, L.b.cu_q,
                     L.b.cu_k, L.b.num_seqs, L.b.row_begin, L.scores, L.ld, L.k, kp, p.seg_len, ckey, cpos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, L.b.cu_q, L.b.cu_k,
                     L.b.num_seqs, L.b.row_begin, p.nseg, L.k, kp, ckey, cpos, L.idx);
  return hipGetLastError();
}

}  // namespace dsa
