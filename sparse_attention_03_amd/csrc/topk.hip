// topk.hip -- causal top-k selection on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), section
// "Step 2", and the gamebaike.com summary, 【细粒度Token选择机制】: each query
// keeps only the candidates whose index scores rank in the top k.  Order:
// score descending, ties to the lower position, -0 == +0, NaN lowest.
//
// One workgroup per score row, one pass over the row.  Scores become
// order-preserving 32-bit keys.  The row is streamed in 2048-element chunks;
// candidates (key, position) that beat the running threshold are appended to
// an LDS buffer in position order (block-wide exclusive scan, so the buffer
// stays sorted by position).  When the buffer would overflow it is cut to
// exactly k entries by a radix select on the keys (four 8-bit digits, LDS
// histograms) and a stable filter; the k-th key becomes the new threshold, and
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
  int wave_sum[kTkWaves];
  int digit;
  int need;
};

// Exclusive scan of one int per thread in thread order; every thread gets the total.
__device__ __forceinline__ int block_excl_scan(int v, TopkShared& sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) sh.wave_sum[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int t = sh.wave_sum[w];
    off += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// Cut the first `cnt` buffer entries to the k best, keeping position order.
// Returns the k-th best key (the smallest kept key).
__device__ uint32_t cut_to_k(TopkShared& sh, int cnt, int k) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, mask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0;  // 256 threads, 256 bins
    __syncthreads();
    for (int e = tid; e < cnt; e += kTkThreads) {
      const uint32_t key = sh.key[e];
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255-4l .. 252-4l (descending key order across lanes)
      int c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = sh.hist[255 - 4 * lane - j]; s += c[j]; }
      const int incl = wave_inclusive_scan(s);
      const int excl = incl - s;
      if (excl < need && need <= incl) {
        int run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < need && need <= run + c[j]) { sh.digit = 255 - 4 * lane - j; sh.need = need - run; }
          run += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << shift;
    mask |= 255u << shift;
    need = sh.need;
    __syncthreads();
  }
  const uint32_t T = prefix;  // k-th best key; `need` entries equal to T are kept
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
  int rank = block_excl_scan(eq, sh, tot);
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
  int off = block_excl_scan(keep, sh, tot);  // its barriers also order the reads above before the writes below
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    if (kf[j]) { sh.key[off] = kk[j]; sh.pos[off] = pp[j]; ++off; }
  }
  __syncthreads();
  return T;
}

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
  const float* row = scores + (int64_t)blockIdx.x * ld;

  auto load_chunk = [&](int32_t c0, f32x4& a, f32x4& b) {
    const int32_t base = c0 + tid * kPer;
    a = f32x4{0.f, 0.f, 0.f, 0.f};
    b = a;
    if (base < n) a = *(const f32x4*)(row + base);
    if (base + 4 < n) b = *(const f32x4*)(row + base + 4);
  };

  int cnt = 0;
  bool have_tau = false;
  uint32_t tau = 0;
  f32x4 ca, cb, na, nb;
  load_chunk(0, ca, cb);
  for (int32_t c0 = 0; c0 < n; c0 += kChunk) {
    if (c0 + kChunk < n) load_chunk(c0 + kChunk, na, nb);
    const int32_t base = c0 + tid * kPer;
    uint32_t key[kPer];
#pragma unroll
    for (int j = 0; j < 4; ++j) { key[j] = order_key(ca[j]); key[4 + j] = order_key(cb[j]); }
    int c = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) c += (base + j < n) && (!have_tau || key[j] > tau);
    int total;
    int off = block_excl_scan(c, sh, total);
    if (cnt + total > kCap) {
      tau = cut_to_k(sh, cnt, k);
      have_tau = true;
      cnt = k;
      c = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) c += (base + j < n) && key[j] > tau;
      off = block_excl_scan(c, sh, total);
    }
    off += cnt;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if ((base + j < n) && (!have_tau || key[j] > tau)) { sh.key[off] = key[j]; sh.pos[off] = base + j; ++off; }
    }
    cnt += total;
    ca = na;
    cb = nb;
  }
  __syncthreads();
  if (cnt > k) cut_to_k(sh, cnt, k);
  for (int e = tid; e < k; e += kTkThreads) out[e] = sh.pos[e];
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  if (L.k > kMaxK || L.k < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, L.b.cu_q, L.b.cu_k, L.b.num_seqs,
                     L.b.row_begin, L.scores, L.ld, L.k, L.idx);
  return hipGetLastError();
}

}  // namespace dsa
