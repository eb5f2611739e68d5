// topk.hip -- causal top-k selection on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), section
// "Step 2", and the gamebaike.com summary, 【细粒度Token选择机制】: each query
// keeps only the candidates whose index scores rank in the top k.  Order:
// score descending, ties to the lower position, -0 == +0, NaN lowest.
//
// One workgroup per score row, one pass over the row (few long rows -- decode
// batches -- split each row into segments first, see below).  The order is
// that of order-preserving 32-bit keys.  The row is streamed in 2048-element
// chunks; elements that beat the running threshold (one float comparison
// against the smallest float above the threshold key) are appended to an LDS
// buffer in position order, so the buffer stays sorted by position.  When the
// buffer would overflow it is cut to exactly k entries by a histogram
// refinement over the buffer's own key range (LDS histograms, at most four
// passes) and a stable filter; the k-th key becomes the new threshold, and
// later elements (larger positions) must beat it strictly.  The final cut
// leaves the k winners already in ascending position order.  Every decision
// is exact: key comparisons, or float comparisons equivalent to them.
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
constexpr int kHistBits = 8;               // bins per histogram pass: 256
constexpr int kHistBins = 1 << kHistBits;
constexpr int kBinsPerLane = kHistBins / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN ranks below every number
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The inverse of order_key on the keys it produces (NaN's key 0 gives a NaN,
// -0's key gives +0: equal under every comparison made here).
__device__ __forceinline__ uint32_t key_bits(uint32_t key) {
  return (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
}

// The smallest float f with order_key(x) > tau  <=>  x >= f for every x
// (NaN when no float qualifies).  The keys just above tau that no float takes
// (1 .. 0x007ffffe below -inf's key, 0x7fffffff which -0 gives up to +0) are
// skipped.  A float comparison is exact for the filter: NaN fails it, -0 and
// +0 compare equal, denormals compare by value.
__device__ __forceinline__ float admit_floor(uint32_t tau) {
  if (tau >= 0xff800000u) return __uint_as_float(0x7fc00000u);  // nothing ranks above +inf
  uint32_t k = tau + 1u;
  if (k < 0x007fffffu) k = 0x007fffffu;
  if (k == 0x7fffffffu) k = 0x80000000u;
  return __uint_as_float(key_bits(k));
}

// The candidate buffer holds order keys, or (RAW) the scores' float bits,
// which are turned into keys only when the buffer is cut.
template <bool RAW>
__device__ __forceinline__ uint32_t buf_key(uint32_t v) {
  return RAW ? order_key(__uint_as_float(v)) : v;
}

struct TopkShared {
  alignas(16) uint32_t key[kCap];
  alignas(16) int32_t pos[kCap];
  int hist[3][kHistBins];      // one per histogram pass, in rotation
  int wave_sum[2][kTkWaves];   // double-buffered: one barrier per scan
  int fcnt[2][kTkWaves];       // wave totals of the cut's two scans
  uint32_t red[2][kTkWaves];
  int list_total;              // the merge: entries in the row's lists
  int list_valid;              // the merge: the row's threshold was valid
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

// Wave-wide inclusive scan with op over lanes 0 .. 63 (every lane active):
// shifts within each 16-lane row, then the row totals carried across rows by
// broadcasts of lanes 15 and 31.  DPP moves, no LDS round trips.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x, uint32_t ident, Op op) {
  const int id = (int)ident;
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(x, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); }), 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(x, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }), 63);
}

// Entries in registers for a cut: thread t holds entries kSegMax t ..
// kSegMax t + kSegMax - 1 of the buffer, so that the thread order is the
// position order; valid are the first nv = cnt - kSegMax t of them.
__device__ __forceinline__ int thread_valid(int cnt) {
  return min(max(cnt - kSegMax * (int)threadIdx.x, 0), kSegMax);
}

template <bool RAW>
__device__ __forceinline__ void load_keys(const TopkShared& sh, uint32_t (&kr)[kSegMax]) {
  const int e0 = kSegMax * threadIdx.x;
#pragma unroll
  for (int i = 0; i < kSegMax / 4; ++i) {
    const i32x4 kv = *(const i32x4*)&sh.key[e0 + 4 * i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int kb = kv[c];
      kr[4 * i + c] = buf_key<RAW>((uint32_t)kb);
    }
  }
}

// Exclusive prefix of v over the workgroup's threads, and in `total` its sum;
// slot: kTkWaves ints of LDS (one barrier).
__device__ __forceinline__ int block_excl_scan(int v, int* slot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = (int)wave_scan_dpp((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 63) slot[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int t = slot[w];
    pre += w < wave ? t : 0;
    tot += t;
  }
  total = tot;
  return pre + incl - v;
}

// The k-th best key T among the keys kr[0 .. nv) of every thread (at least k
// in all), and in `need` how many of the entries equal to T rank among the k
// best.  T is located by histogram refinement over the keys' own range: each
// pass splits the current interval [lo, hi] (known to hold T) into at most
// kHistBins equal power-of-two bins, so clustered scores still spread over the
// bins; at most four passes, none when every key is equal.  After max_passes
// passes the lower end of the interval is returned instead: a key at most T,
// with `need` then meaningless.  When every entry of the bin holding the
// rank is kept, the bin's lower end is returned as T (a key at most the k-th
// best; every entry at or above it is among the k best, `need` = the bin's
// count) without refining further.  One barrier per pass: the histograms rotate
// over three buffers (a pass clears the next one, last read two passes
// before), and every wave scans the histogram itself.
__device__ uint32_t kth_key(TopkShared& sh, const uint32_t (&kr)[kSegMax], int nv, int k, int& need,
                            int max_passes = 4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(kHistBins == kTkThreads, "one histogram bin cleared per thread");
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int j = 0; j < kSegMax; ++j)
    if (j < nv) {
      mn = min(mn, kr[j]);
      mx = max(mx, kr[j]);
    }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) { sh.red[0][wave] = mn; sh.red[1][wave] = mx; }
  sh.hist[0][tid] = 0;
  __syncthreads();
  uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < kTkWaves; ++w) { lo = min(lo, sh.red[0][w]); hi = max(hi, sh.red[1][w]); }
  need = k;  // entries of [lo, hi] still to take, counted from the top
  int hb = 0;
  for (int pass = 0; hi > lo && pass < max_passes; ++pass) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > kHistBits ? bits - kHistBits : 0;
    const int nbins = (int)(span >> shift) + 1;  // <= kHistBins
    int* hist = sh.hist[hb];
#pragma unroll
    for (int j = 0; j < kSegMax; ++j)
      if (j < nv && kr[j] >= lo && kr[j] <= hi) atomicAdd(&hist[(kr[j] - lo) >> shift], 1);
    hb = hb == 2 ? 0 : hb + 1;
    sh.hist[hb][tid] = 0;
    __syncthreads();
    // lane l owns bins nbins-1-B l .. nbins-B-B l (descending key order, B = kBinsPerLane)
    int c[kBinsPerLane], sum = 0;
#pragma unroll
    for (int j = 0; j < kBinsPerLane; ++j) {
      const int b = nbins - 1 - kBinsPerLane * lane - j;
      c[j] = b >= 0 ? hist[b] : 0;
      sum += c[j];
    }
    const int incl = (int)wave_scan_dpp((uint32_t)sum, 0u, [](uint32_t a, uint32_t b) { return a + b; });
    const int excl = incl - sum;
    const bool mine = excl < need && need <= incl;  // exactly one lane: T lies in [lo, hi]
    int digit = 0, rest = 0, in_bin = 0;
    if (mine) {
      int run = excl;
#pragma unroll
      for (int j = 0; j < kBinsPerLane; ++j) {
        if (run < need && need <= run + c[j]) {
          digit = nbins - 1 - kBinsPerLane * lane - j;
          rest = need - run;
          in_bin = c[j];
        }
        run += c[j];
      }
    }
    const int owner = (int)__builtin_ctzll(__ballot(mine));
    digit = __builtin_amdgcn_readlane(digit, owner);
    rest = __builtin_amdgcn_readlane(rest, owner);
    in_bin = __builtin_amdgcn_readlane(in_bin, owner);
    const uint32_t blo = lo + ((uint32_t)digit << shift);
    const uint32_t bhi = blo + ((1u << shift) - 1u);
    lo = blo;
    hi = min(hi, bhi);
    need = rest;
    // every entry of the bin ranks among the k best: the bin's lower end
    // serves as T (the entries above it and all those equal to it are the
    // ones kept), with no further pass
    if (rest == in_bin) break;
  }
  return lo;
}

// Cut `cnt` (> k) entries held as above (keys kr; their positions are
// fetched by pos_of(pr) only once ranked, which keeps them out of the
// registers the histogram passes hold) to the k best and write them to the
// buffer's first k slots in position order (keys as RAW says); returns the
// k-th best key.  The stable filter: one scan of the per-thread counts of
// keys equal to T ranks the ties in position order (the earliest `need` are
// kept), a second scan of the kept counts gives each thread its output
// offset.  The buffer may be the entries' own source: every read of it
// (pos_of's included) precedes the second scan's barrier, every write follows.
template <bool RAW, class PosOf>
__device__ uint32_t cut_entries(TopkShared& sh, const uint32_t (&kr)[kSegMax], int cnt, int k, PosOf pos_of) {
  const int nv = thread_valid(cnt);
  int need;
  const uint32_t T = kth_key(sh, kr, nv, k, need);
  int eq = 0;
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) eq += j < nv && kr[j] == T;
  int eq_tot;
  int rank = block_excl_scan(eq, sh.fcnt[0], eq_tot);
  uint32_t kept = 0;
  int keep = 0;
#pragma unroll
  for (int j = 0; j < kSegMax; ++j) {
    const bool is_eq = j < nv && kr[j] == T;
    const bool kp = (j < nv && kr[j] > T) || (is_eq && rank < need);
    rank += is_eq;
    kept |= (uint32_t)kp << j;
    keep += kp;
  }
  int32_t pr[kSegMax];
  pos_of(pr);
  int keep_tot;
  int o = block_excl_scan(keep, sh.fcnt[1], keep_tot);
#pragma unroll
  for (int j = 0; j < kSegMax; ++j)
    if ((kept >> j) & 1u) {
      sh.key[o] = RAW ? key_bits(kr[j]) : kr[j];
      sh.pos[o] = pr[j];
      ++o;
    }
  __syncthreads();
  return T;
}

// Cut the first `cnt` (> k) buffer entries to the k best, keeping position
// order; returns the k-th best key (the smallest kept key).
template <bool RAW>
__device__ uint32_t cut_to_k(TopkShared& sh, int cnt, int k) {
  uint32_t kr[kSegMax];
  load_keys<RAW>(sh, kr);
  return cut_entries<RAW>(sh, kr, cnt, k, [&](int32_t (&pr)[kSegMax]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSegMax / 4; ++i) {
      const i32x4 pv = *(const i32x4*)&sh.pos[kSegMax * threadIdx.x + 4 * i];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int pb = pv[c];
        pr[4 * i + c] = pb;
      }
    }
  });
}

// ---------------------------------------------------------------------------
// Offset of this wave's admitted elements in the block's (wave order), from
// the admission masks of the wave's elements; every thread gets the block's
// total.  One barrier: the wave totals alternate between two slots.
__device__ __forceinline__ int block_base(const uint64_t (&m)[kPer], TopkShared& sh, int& parity, int& total) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int wt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) wt += __popcll(m[j]);
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
  return off;
}

// ---------------------------------------------------------------------------
// Streaming selection over a sequence of `count` elements given in ascending
// position order.  Leaves the k best (or all, if fewer are valid) in
// sh.key/sh.pos[0 .. returned count), in ascending position order (sh.key as
// Src::kRaw says).  A chunk of 2048 elements gives wave w elements
// 512 w .. 512 w + 511, lane l element 64 j + l of them for j < kPer, so the
// admission test of element j is one compare whose lane mask is also the
// lanes' order: element (j, l) lands at the wave's base plus the admitted
// elements of j' < j plus those of lanes below l (mbcnt).  Src provides Fetch
// (the raw loads of one thread's kPer elements), fetch(), admit() (the lane
// masks of the elements that beat the threshold: every valid one before there
// is one), value() and position(); three chunks of loads are kept in flight
// ahead of the one being filtered, so the row streams at memory speed instead
// of load latency.
// ---------------------------------------------------------------------------
// f: the ring, its first three chunks already fetched (prime_ring), so that a
// caller can overlap their latency with other work.  tau0 (have_tau0): start
// with the threshold tau0 -- only keys above it are admitted; *admitted: how
// many entries were admitted in all.  Without final_cut the buffer is left
// with up to kCap entries that hold the k best, cut only to make room.
template <class Src>
__device__ __forceinline__ void prime_ring(const Src& src, typename Src::Fetch (&f)[4]) {
  src.fetch(0, f[0]);
  src.fetch(kChunk, f[1]);
  src.fetch(2 * kChunk, f[2]);
}

template <class Src>
__device__ __forceinline__ int stream_select(TopkShared& sh, const Src& src, typename Src::Fetch (&f)[4], int32_t count, int k,
                             bool have_tau0 = false, uint32_t tau0 = 0, int* admitted = nullptr,
                             bool final_cut = true) {
  constexpr bool RAW = Src::kRaw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int cnt = 0, adm = 0;
  bool have_tau = have_tau0;
  uint32_t tau = tau0;
  float tfloor = admit_floor(tau0);
  int parity = 0;
  // a ring of four chunks' loads, unrolled so that every slot is a fixed set
  // of registers (a rotation by register copies would make each chunk wait
  // for the newest loads).  Whole groups of four chunks run without any exit
  // between them, so the compiler's wait before a chunk's keys covers that
  // chunk's loads only; the last partial group runs after them.
  // full: every element of the chunk lies before `count`
  auto step = [&](int32_t c0, int u, bool full) __attribute__((always_inline)) {
    src.fetch(c0 + 3 * kChunk, f[(u + 3) & 3]);
    const int32_t w0 = c0 + wave * (64 * kPer);  // the wave's first element
    uint64_t m[kPer];
    src.admit(f[u], w0, full, have_tau, tau, tfloor, m);
    int total;
    int base = block_base(m, sh, parity, total);
    if (cnt + total > kCap) {
      tau = cut_to_k<RAW>(sh, cnt, k);
      tfloor = admit_floor(tau);
      have_tau = true;
      cnt = k;
      src.admit(f[u], w0, full, true, tau, tfloor, m);
      base = block_base(m, sh, parity, total);
    }
    int o = cnt + base;  // uniform over the wave
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (__builtin_amdgcn_inverse_ballot_w64(m[j])) {
        const int e = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[j] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m[j], (uint32_t)o));
        sh.key[e] = src.value(f[u], j);
        sh.pos[e] = src.position(f[u], w0, j);
      }
      o += __popcll(m[j]);
    }
    cnt += total;
    adm += total;
  };
  int32_t c00 = 0;
  for (; c00 + 4 * kChunk <= count; c00 += 4 * kChunk) {
#pragma unroll
    for (int u = 0; u < 4; ++u) step(c00 + u * kChunk, u, true);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // count - c00 < 4 chunks: at most four, the last one partial
    if (c00 + u * kChunk >= count) break;
    step(c00 + u * kChunk, u, c00 + (u + 1) * kChunk <= count);
  }
  __syncthreads();
  if (admitted) *admitted = adm;
  if (final_cut && cnt > k) {
    cut_to_k<RAW>(sh, cnt, k);
    cnt = k;
  }
  return cnt;
}

// Long rows start from a sampled threshold: the key of rank 1.3 k n_s / n + 8
// among n_s = 4096 entries (four contiguous blocks spread over the row), so
// that about 1.3 k to 1.4 k entries of the row reach it and the stream rarely
// needs a cut.  The result stays exact: if at least k entries reach the threshold,
// the k-th best key of the row is at least the threshold and every winner is
// admitted; otherwise the row is selected again without it.
constexpr int kSampleBlocks = 4;
constexpr int kSampleBlock = 4 * kTkThreads;      // 1024 entries, one 16-byte load per thread
constexpr int kSampleMinRow = 16384;

__device__ __forceinline__ void load_sample(const float* row, int32_t n, f32x4 (&v)[kSampleBlocks]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int b = 0; b < kSampleBlocks; ++b) {
    const int32_t start = (int32_t)((int64_t)b * (n - kSampleBlock) / (kSampleBlocks - 1)) & ~3;
    v[b] = *(const f32x4*)(row + start + 4 * tid);  // start + kSampleBlock <= n; rows are 16-byte aligned
  }
}

// passes: histogram passes of the ranking; after one, the lower end of the
// bin holding that rank, which admits a few more entries.
__device__ __forceinline__ uint32_t sampled_threshold(TopkShared& sh, const f32x4 (&v)[kSampleBlocks], int32_t n, int k,
                                      int passes) {
  static_assert(4 * kSampleBlocks == kSegMax, "the sample's keys fill one thread's registers");
  uint32_t kr[kSegMax];
#pragma unroll
  for (int b = 0; b < kSampleBlocks; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c) kr[4 * b + c] = order_key(v[b][c]);
  constexpr int m = kSampleBlocks * kSampleBlock;
  const int rank = (int)min((int64_t)m, 13LL * k * m / (10LL * n) + 8);
  int need;
  return kth_key(sh, kr, kSegMax, rank, need, passes);
}

// Elements are the scores of one row at positions [lo, hi).  The filter
// compares floats against admit_floor(tau), which admits exactly the keys
// above tau, so no key is formed for the elements it rejects; the buffer keeps
// the admitted scores' bits.
struct ScoreSrc {
  static constexpr bool kRaw = true;
  struct Fetch { float v[kPer]; };
  const float* row;
  int32_t lo, hi;
  __device__ __forceinline__ void fetch(int32_t c0, Fetch& f) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int32_t p = lo + c0 + wave * (64 * kPer) + lane;
    // raw buffer loads over the row's first hi entries: entries past hi read
    // as zero (and are masked in admit), and no load is conditional
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, (uint32_t)hi * 4, 0x00020000);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      f.v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(p + 64 * j) * 4, 0, 0));
  }
  __device__ __forceinline__ void admit(const Fetch& f, int32_t w0, bool full, bool have_tau, uint32_t,
                                        float tfloor, uint64_t (&m)[kPer]) const {
    const int lane = threadIdx.x & 63;
    // the masks stay scalar: one compare per element, the rest is mask logic
    // (without a threshold every lane's element is admitted, NaN included)
    const uint64_t thr = have_tau ? ~0ull : 0ull, all = __ballot(true);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      uint64_t mj = (__ballot(f.v[j] >= tfloor) & thr) | (all & ~thr);
      if (!full) mj &= __ballot(lo + w0 + 64 * j + lane < hi);
      m[j] = mj;
    }
  }
  __device__ __forceinline__ uint32_t value(const Fetch& f, int j) const { return __float_as_uint(f.v[j]); }
  __device__ __forceinline__ int32_t position(const Fetch&, int32_t w0, int j) const {
    return lo + w0 + 64 * j + (int)(threadIdx.x & 63);
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
  ScoreSrc::Fetch f[4];
  if (n >= kSampleMinRow) {
    // the sample's loads, then the stream's first chunks (in flight while the
    // sample is ranked: waiting for the sample leaves them outstanding)
    f32x4 v[kSampleBlocks];
    load_sample(row, n, v);
    __builtin_amdgcn_sched_barrier(0);  // keep the sample's loads older than the stream's
    prime_ring(src, f);
    const uint32_t ts = sampled_threshold(sh, v, n, k, 1);
    int admitted;
    const int c = stream_select(sh, src, f, n, k, ts > 0u, ts - 1u, &admitted);  // admits keys >= ts
    if (admitted >= k) cnt = c;
    __syncthreads();
  }
  if (cnt < 0) {
    prime_ring(src, f);
    cnt = stream_select(sh, src, f, n, k);
  }
  for (int e = tid; e < k; e += kTkThreads) out[e] = e < cnt ? sh.pos[e] : -1;
}

// Few long rows, phase 1: each row is cut into `nseg` segments of seg_len
// entries, one workgroup each.  Every workgroup of a row derives the same
// threshold from the row's sample (rows of kSegSampleMinRow entries or more;
// shorter rows take none) and keeps the entries of its segment that reach it;
// should they overflow the buffer, it is cut to the segment's k best, which
// keeps every row winner of the segment.  Written per (row, segment), in a
// slot of `cap` (= min(kCap, seg_len)) entries: the kept entries' keys and
// positions in position order, and (count, admitted).
constexpr int kSegSampleMinRow = kSampleBlocks * kSampleBlock;  // the sample's blocks tile such a row
constexpr int kMaxSegs = 64;                                     // segments per row (one lane each in the merge)

__global__ __launch_bounds__(kTkThreads) void topk_segment_kernel(const int32_t* __restrict__ cu_q,
                                                                  const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                                  int32_t row_begin, const float* __restrict__ scores,
                                                                  int64_t ld, int32_t k, int32_t seg_len,
                                                                  int32_t cap, uint32_t* __restrict__ ckey,
                                                                  int32_t* __restrict__ cpos,
                                                                  int32_t* __restrict__ cstat) {
  __shared__ TopkShared sh;
  const int32_t rl = blockIdx.x, seg = blockIdx.y, nseg = gridDim.y;
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, row_begin + rl);
  const int32_t n = ri.pos + 1;
  if (n <= k) return;  // the merge writes every position directly
  const int32_t lo = seg * seg_len, hi = min(n, lo + seg_len);
  const int64_t slot = (int64_t)rl * nseg + seg;
  int cnt = 0, adm = 0;
  if (lo < hi) {
    const float* row = scores + (int64_t)rl * ld;
    const ScoreSrc src{row, lo, hi};
    ScoreSrc::Fetch f[4];
    if (n >= kSegSampleMinRow) {
      f32x4 v[kSampleBlocks];
      load_sample(row, n, v);
      __builtin_amdgcn_sched_barrier(0);  // keep the sample's loads older than the stream's
      prime_ring(src, f);
      // two passes: a tighter threshold keeps the row's lists within one buffer
      const uint32_t ts = sampled_threshold(sh, v, n, k, 2);
      cnt = stream_select(sh, src, f, hi - lo, k, ts > 0u, ts - 1u, &adm, false);  // admits keys >= ts
    } else {
      prime_ring(src, f);
      cnt = stream_select(sh, src, f, hi - lo, k, false, 0u, &adm, false);
    }
  }
  uint32_t* okey = ckey + slot * cap;
  int32_t* opos = cpos + slot * cap;
  for (int e = threadIdx.x; e < cnt; e += kTkThreads) {
    okey[e] = buf_key<ScoreSrc::kRaw>(sh.key[e]);
    opos[e] = sh.pos[e];
  }
  if (threadIdx.x == 0) {
    cstat[2 * slot] = cnt;
    cstat[2 * slot + 1] = adm;
  }
}

// Phase 2, one workgroup per row.  The threshold was valid when at least k
// entries of the row reached it: when no segment cut its list, the admitted
// counts add up to exactly that number, and a segment that did cut alone held
// more than k.  Then the row's k-th key is at least the threshold, every
// winner is in its segment's list, and the lists, concatenated in segment
// order (so in position order), are cut to the k best.  Otherwise, or when
// the lists exceed one buffer, the row is streamed again without a threshold.
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(const int32_t* __restrict__ cu_q,
                                                                const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                                int32_t row_begin, const float* __restrict__ scores,
                                                                int64_t ld, int32_t nseg, int32_t k, int32_t cap,
                                                                const uint32_t* __restrict__ ckey,
                                                                const int32_t* __restrict__ cpos,
                                                                const int32_t* __restrict__ cstat,
                                                                int32_t* __restrict__ idx) {
  __shared__ TopkShared sh;
  const int32_t rl = blockIdx.x;
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, row_begin + rl);
  const int32_t n = ri.pos + 1;
  const int tid = threadIdx.x;
  int32_t* out = idx + (int64_t)rl * k;
  if (n <= k) {
    for (int e = tid; e < k; e += kTkThreads) out[e] = e < n ? e : -1;
    return;
  }
  const int64_t s0 = (int64_t)rl * nseg;
  // list offsets: exclusive prefix of the counts over the segments (lane s of
  // wave 0), kept in sh.hist[0 .. nseg]
  if (tid < 64) {
    const int c = tid < nseg ? cstat[2 * (s0 + tid)] : 0;
    const int a = tid < nseg ? cstat[2 * (s0 + tid) + 1] : 0;
    const int incl = wave_inclusive_scan(c);
    int adm = a;
    for (int o = 32; o >= 1; o >>= 1) adm += __shfl_xor(adm, o);
    if (tid < nseg) sh.hist[0][tid] = incl - c;
    if (tid == 63) {
      sh.hist[0][nseg] = incl;
      sh.list_total = incl;
      sh.list_valid = adm >= k ? 1 : 0;
    }
  }
  __syncthreads();
  const int total = sh.list_total;
  int cnt;
  if (sh.list_valid && total <= kCap) {
    // where each buffer entry comes from (offset in the row's lists), written
    // segment by segment into sh.pos; each thread then reads the sources of
    // its own entries (kSegMax t .. kSegMax t + kSegMax - 1) and loads them
    const int wave = tid >> 6, lane = tid & 63;
    for (int sgi = wave; sgi < nseg; sgi += kTkWaves) {
      const int b = sh.hist[0][sgi], c = sh.hist[0][sgi + 1] - b;
      for (int o = lane; o < c; o += 64) sh.pos[b + o] = sgi * cap + o;
    }
    __syncthreads();
    const int nv = thread_valid(total);
    const uint32_t* lkey = ckey + s0 * cap;
    const int32_t* lpos = cpos + s0 * cap;
    uint32_t kr[kSegMax];
    int32_t pr[kSegMax];
#pragma unroll
    for (int i = 0; i < kSegMax / 4; ++i) {
      const i32x4 sv = *(const i32x4*)&sh.pos[kSegMax * tid + 4 * i];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int sb = sv[c];
        const int src = 4 * i + c < nv ? sb : 0;  // slots past the lists: any valid address
        kr[4 * i + c] = lkey[src];
        pr[4 * i + c] = lpos[src];
      }
    }
    if (total > k) {
      cut_entries<false>(sh, kr, total, k, [&](int32_t (&p)[kSegMax]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kSegMax; ++j) p[j] = pr[j];
      });
      cnt = k;
    } else {
#pragma unroll
      for (int j = 0; j < kSegMax; ++j)
        if (j < nv) sh.pos[kSegMax * tid + j] = pr[j];  // the thread's own slots
      __syncthreads();
      cnt = total;
    }
  } else {
    const ScoreSrc src{scores + (int64_t)rl * ld, 0, n};
    ScoreSrc::Fetch f[4];
    prime_ring(src, f);
    cnt = stream_select(sh, src, f, n, k);
  }
  for (int e = tid; e < k; e += kTkThreads) out[e] = e < cnt ? sh.pos[e] : -1;
}

// ---------------------------------------------------------------------------
// Few rows of at most kRxCap entries, too short to split: one 1024-thread
// workgroup per row.  Each wave loads a contiguous range of the row into
// registers (16-byte loads, lane l holding entries 4l .. 4l + 3 of every
// 256-entry block), so the row is read once and never staged in LDS.  The
// k-th key is found by histogram refinement (the range-adaptive 256-bin passes
// of kth_key, LDS atomics fed from registers, one barrier per pass), and the
// winners are written in ascending position order: ballots order the lanes of
// a wave, one exchange of per-wave counts orders the waves.
// ---------------------------------------------------------------------------
constexpr int kRxThreads = 1024;
constexpr int kRxWaves = kRxThreads / 64;
constexpr int kRxRowVecs = 4;                               // 16-byte vectors of keys per lane
constexpr int kRxCap = kRxWaves * 256 * kRxRowVecs;         // 16384 row entries per workgroup

struct RadixShared {
  int hist[3][256];  // one per pass, in rotation (as in kth_key)
  int cnt[kRxWaves];
  int fcnt[2][kRxWaves];
  uint32_t red[2][kRxWaves];
};

// NV: 16-byte vectors per lane, enough for the launch's longest row
// (n <= 4096 NV).
template <int NV>
__global__ __launch_bounds__(kRxThreads) void topk_radix_kernel(const int32_t* __restrict__ cu_q,
                                                                const int32_t* __restrict__ cu_k, int32_t num_seqs,
                                                                int32_t row_begin, const float* __restrict__ scores,
                                                                int64_t ld, int32_t k, int32_t* __restrict__ idx) {
  static_assert(NV <= kRxRowVecs, "too many vectors per lane");
  __shared__ RadixShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t rl = blockIdx.x;
  const RowInfo ri = locate_row_wave(load_seq_table(cu_q, cu_k, num_seqs), cu_q, cu_k, row_begin + rl);
  const int32_t n = ri.pos + 1;
  int32_t* out = idx + (int64_t)rl * k;
  if (n <= k) {
    for (int e = tid; e < k; e += kRxThreads) out[e] = e < n ? e : -1;
    return;
  }
  // ---- load: wave w owns entries [w0, w1), L a multiple of 256
  const int L = (n + 256 * kRxWaves - 1) / (256 * kRxWaves) * 256;  // <= 256 * NV
  const int w0 = min(wave * L, n), w1 = min(w0 + L, n);
  uint32_t key[NV][4];
  int32_t pos[NV][4];
  {
    // raw buffer loads over whole 16-byte vectors (they stay in the row: ld
    // is a multiple of 4); loads past the range read zero, and all are issued
    // before the first use
    const uint32_t bytes = (uint32_t)((n + 3) / 4 * 16);
    const auto ks = __builtin_amdgcn_make_buffer_rsrc((void*)(scores + (int64_t)rl * ld), 0, bytes, 0x00020000);
    i32x4 kv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = w0 + 256 * i + 4 * lane;
      const uint32_t off = 256 * i < L ? (uint32_t)e * 4u : 0xfffffff0u;  // outside the wave's range: no access
      kv[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ks, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = w0 + 256 * i + 4 * lane + j;
        pos[i][j] = 256 * i < L && e < w1 ? e : -1;
        const int bits = kv[i][j];  // copied out first: a bit_cast of the element expression read element 0
        key[i][j] = order_key(__int_as_float(bits));
      }
  }
  // ---- min and max key (n > k >= 1 entries are valid)
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (pos[i][j] >= 0) {
        mn = min(mn, key[i][j]);
        mx = max(mx, key[i][j]);
      }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) { sh.red[0][wave] = mn; sh.red[1][wave] = mx; }
  if (tid < 256) sh.hist[0][tid] = 0;
  __syncthreads();
  uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < kRxWaves; ++w) {
    lo = min(lo, sh.red[0][w]);
    hi = max(hi, sh.red[1][w]);
  }

  // ---- the k-th key T: entries above it are kept, and `need` of those equal to it (the earliest)
  int need = k;
  int hb = 0;
  while (hi > lo) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    const int nbins = (int)(span >> shift) + 1;  // <= 256
    int* hist = sh.hist[hb];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kk = key[i][j];
        if (pos[i][j] >= 0 && kk >= lo && kk <= hi) atomicAdd(&hist[(kk - lo) >> shift], 1);
      }
    hb = hb == 2 ? 0 : hb + 1;
    if (tid < 256) sh.hist[hb][tid] = 0;  // the next pass's histogram, last read two passes ago
    __syncthreads();
    int c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = nbins - 1 - 4 * lane - j;
      c[j] = b >= 0 ? hist[b] : 0;
      sum += c[j];
    }
    const int incl = (int)wave_scan_dpp((uint32_t)sum, 0u, [](uint32_t a, uint32_t b) { return a + b; });
    const int excl = incl - sum;
    const bool mine = excl < need && need <= incl;
    int digit = 0, rest = 0, in_bin = 0;
    if (mine) {
      int run = excl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run < need && need <= run + c[j]) { digit = nbins - 1 - 4 * lane - j; rest = need - run; in_bin = c[j]; }
        run += c[j];
      }
    }
    const int owner = (int)__builtin_ctzll(__ballot(mine));
    digit = __builtin_amdgcn_readlane(digit, owner);
    rest = __builtin_amdgcn_readlane(rest, owner);
    in_bin = __builtin_amdgcn_readlane(in_bin, owner);
    const uint32_t blo = lo + ((uint32_t)digit << shift);
    lo = blo;
    hi = min(hi, blo + ((1u << shift) - 1u));
    need = rest;
    if (rest == in_bin) break;  // the whole bin is kept: its lower end serves as T (as in kth_key)
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
      if (kept[j]) out[o++] = pos[i][j];
    }
    eqrun += eq_tot;
    keeprun += keep_tot;
  }
}

}  // namespace

namespace {

// How a batch is selected:
//   kStream:   one 256-thread workgroup streams each row (many rows: the rows
//              fill the machine, and each is read from HBM once);
//   kRadix:    few rows of at most kRxCap entries, too short to split: LDS
//              radix select per row;
//   kSegment:  few longer rows: sampled segments, then the merge of their
//              lists (topk_segment_kernel, topk_merge_kernel).
enum TopkKind { kStream, kRadix, kSegment };
struct TopkPlan {
  TopkKind kind;
  int nseg;
  int32_t seg_len;
};

constexpr int kSegWgsPerCu = 2;  // segment workgroups per CU the split aims for

TopkPlan topk_plan(int rows, int max_ctx, int k, int num_cus) {
  TopkPlan p{kStream, 1, 0};
  if (rows <= 0 || rows >= num_cus) return p;
  // one radix workgroup per row when the rows fit one and splitting would
  // not add workgroups: the machine is covered or segments would be shorter
  // than 4k entries
  const int by_cus = (num_cus + rows - 1) / rows, by_len = max_ctx / (4 * k);
  if (max_ctx <= kRxCap && min(by_cus, by_len) <= 1) {
    p.kind = kRadix;
    return p;
  }
  // segments of whole chunks, about kSegWgsPerCu workgroups per CU
  int ns = (kSegWgsPerCu * num_cus + rows - 1) / rows;
  ns = min(min(ns, kMaxSegs), max(1, max_ctx / kChunk));
  if (ns <= 1 && max_ctx <= kRxCap) {
    p.kind = kRadix;
    return p;
  }
  const int32_t len = (max_ctx + ns - 1) / ns;
  p.seg_len = (len + kChunk - 1) / kChunk * kChunk;
  p.nseg = (max_ctx + p.seg_len - 1) / p.seg_len;  // no trailing empty segment
  p.kind = kSegment;
  return p;
}

template <int NV>
hipError_t launch_radix_nv(const TopkLaunch& L, int rows, hipStream_t s) {
  hipLaunchKernelGGL((topk_radix_kernel<NV>), dim3((unsigned)rows), dim3(kRxThreads), 0, s, L.b.cu_q, L.b.cu_k,
                     L.b.num_seqs, L.b.row_begin, L.scores, L.ld, L.k, L.idx);
  return hipGetLastError();
}

hipError_t launch_radix(const TopkLaunch& L, int rows, hipStream_t s) {
  const int nv = (L.b.max_ctx + 256 * kRxWaves - 1) / (256 * kRxWaves);
  if (nv <= 1) return launch_radix_nv<1>(L, rows, s);
  if (nv <= 2) return launch_radix_nv<2>(L, rows, s);
  if (nv <= 4) return launch_radix_nv<4>(L, rows, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool topk_may_segment(int max_ctx, int k) { return k > 0 && (max_ctx > kRxCap || max_ctx / (4 * k) > 1); }

namespace {
// workspace of the segment plan: keys, positions, (count, admitted) per
// (row, segment)
struct SegWorkspace {
  size_t off_pos, off_stat, bytes;
};
int seg_cap(const TopkPlan& p) { return min(kCap, (int)p.seg_len); }
SegWorkspace seg_workspace(int rows, const TopkPlan& p) {
  const size_t n = (size_t)rows * p.nseg * (size_t)seg_cap(p);
  SegWorkspace w;
  w.off_pos = (n * 4 + 255) / 256 * 256;
  w.off_stat = 2 * w.off_pos;
  w.bytes = w.off_stat + ((size_t)rows * p.nseg * 8 + 255) / 256 * 256;
  return w;
}
}  // namespace

size_t topk_workspace_bytes(int rows, int max_ctx, int k, int num_cus) {
  const TopkPlan p = topk_plan(rows, max_ctx, k, num_cus);
  return p.kind == kSegment ? seg_workspace(rows, p).bytes : 0;
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
    return launch_radix(L, rows, s);
  const SegWorkspace w = seg_workspace(rows, p);
  const int cap = seg_cap(p);
  uint32_t* ckey = (uint32_t*)L.ws;
  int32_t* cpos = (int32_t*)((char*)L.ws + w.off_pos);
  int32_t* cstat = (int32_t*)((char*)L.ws + w.off_stat);
  hipLaunchKernelGGL(topk_segment_kernel, dim3((unsigned)rows, (unsigned)p.nseg), dim3(kTkThreads), 0, s, L.b.cu_q,
                     L.b.cu_k, L.b.num_seqs, L.b.row_begin, L.scores, L.ld, L.k, p.seg_len, cap, ckey, cpos, cstat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, L.b.cu_q, L.b.cu_k,
                     L.b.num_seqs, L.b.row_begin, L.scores, L.ld, p.nseg, L.k, cap, ckey, cpos, cstat, L.idx);
  return hipGetLastError();
}

}  // namespace dsa
