// align.hip -- the indexer's alignment loss on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), training
// "Step 1" (dense warm-up) and "Step 2" (sparse training); gamebaike.com
// summary 【密集预热阶段】 / 【稀疏训练阶段】: the indexer is trained to follow
// the main attention.  The target p_t (the heads' attention probabilities
// summed and L1-normalised, mla_target_kernel) is compared with the indexer's
// distribution softmax(I_t) over the same candidates through the KL
// divergence; in the sparse stage the candidates are the selected set S_t.
//
// indexer_kl_kernel: one workgroup per query row, two passes over the row's
// candidates (HBM-bound):
//   1. online max / sum of exp(I) and the sum of p (per thread, then merged);
//   2. dI_e = (sum p) softmax(I)_e - p_e, and the loss terms
//      p_e (log p_e - (I_e - lse)) for p_e > 0 (0 log 0 = 0).
// The per-entry form of the loss keeps its terms small; the row sums are fp32
// trees.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kKlThreads = 256;

struct KlArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t num_seqs, row_begin, row_end;
  const float* scores;   // [rows, ld_s]
  int64_t ld_s;
  const int32_t* idx;    // [rows, k] or null (dense: entry e = position e)
  int32_t k;
  const float* p;        // [rows, ld_p]
  int64_t ld_p;
  float* loss;           // [rows] or null
  float* dI;             // [rows, ld_p] or null
};

struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MaxSum{m, 0.0f};
  return MaxSum{m, a.s * expf(a.m - m) + b.s * expf(b.m - m)};
}

__global__ __launch_bounds__(kKlThreads) void indexer_kl_kernel(KlArgs a) {
  __shared__ float red_m[kKlThreads / 64], red_s[kKlThreads / 64], red_p[kKlThreads / 64];
  const int32_t rl = blockIdx.x, r = a.row_begin + rl;
  const RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, r);
  const bool dense = a.idx == nullptr;
  const int32_t m = dense ? ri.pos + 1 : a.k;  // entries of the row
  const float* srow = a.scores + (int64_t)rl * a.ld_s;
  const float* prow = a.p + (int64_t)rl * a.ld_p;
  const int32_t* irow = dense ? nullptr : a.idx + (int64_t)rl * a.k;
  auto pos_of = [&](int32_t e) -> int32_t {
    if (dense) return e;
    const int32_t s = irow[e];
    return s >= 0 && s <= ri.pos ? s : -1;
  };
  // pass 1
  MaxSum ms{-INFINITY, 0.0f};
  float psum = 0.0f;
  for (int32_t e = threadIdx.x; e < m; e += kKlThreads) {
    const int32_t s = pos_of(e);
    if (s < 0) continue;
    const float x = srow[s];
    ms = merge(ms, MaxSum{x, 1.0f});
    psum += prow[e];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ms = merge(ms, MaxSum{__shfl_xor(ms.m, o), __shfl_xor(ms.s, o)});
    psum += __shfl_xor(psum, o);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red_m[wave] = ms.m;
    red_s[wave] = ms.s;
    red_p[wave] = psum;
  }
  __syncthreads();
  ms = MaxSum{red_m[0], red_s[0]};
  psum = red_p[0];
#pragma unroll
  for (int w = 1; w < kKlThreads / 64; ++w) {
    ms = merge(ms, MaxSum{red_m[w], red_s[w]});
    psum += red_p[w];
  }
  const float lse = ms.m == -INFINITY ? 0.0f : ms.m + logf(ms.s);
  __syncthreads();  // red_* reused below
  // pass 2
  float kl = 0.0f;
  float* grow = a.dI ? a.dI + (int64_t)rl * a.ld_p : nullptr;
  for (int32_t e = threadIdx.x; e < m; e += kKlThreads) {
    const int32_t s = pos_of(e);
    float g = 0.0f;
    if (s >= 0) {
      const float x = srow[s] - lse;
      const float pe = prow[e];
      g = psum * expf(x) - pe;
      if (pe > 0.0f) kl += pe * (logf(pe) - x);
    }
    if (grow) grow[e] = g;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kl += __shfl_xor(kl, o);
  if (lane == 0) red_p[wave] = kl;
  __syncthreads();
  if (threadIdx.x == 0 && a.loss) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kKlThreads / 64; ++w) t += red_p[w];
    a.loss[rl] = t;
  }
}

}  // namespace

hipError_t launch_indexer_kl(const KlLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  KlArgs a;
  a.cu_q = L.b.cu_q;
  a.cu_k = L.b.cu_k;
  a.num_seqs = L.b.num_seqs;
  a.row_begin = L.b.row_begin;
  a.row_end = L.b.row_end;
  a.scores = L.scores;
  a.ld_s = L.ld_s;
  a.idx = L.idx;
  a.k = L.k;
  a.p = L.p;
  a.ld_p = L.ld_p;
  a.loss = L.loss;
  a.dI = L.dI;
  hipLaunchKernelGGL(indexer_kl_kernel, dim3((unsigned)rows), dim3(kKlThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
