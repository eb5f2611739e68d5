// indexer.hip -- lightning-indexer scores on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), section
// "Lightning indexer / Step 1": the index score of query row t against a
// preceding token s is sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]) over the few
// indexer heads j; the indexer is cheap because it has few heads and runs in
// FP8.  GELU (named instead of ReLU on the gamebaike.com summary,
// 【闪电索引器】) is a template switch.
//
// FP8 path: one v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit scales)
// computes a whole d_I = 128 dot product for 16 heads x 16 keys.  A wave holds
// the query fragments of two query rows (all heads) in VGPRs and streams key
// fragments straight from global memory (a 16-key fragment is 2 KB
// contiguous); the four waves of a workgroup sweep the same keys so the L1
// serves three of the four reads.  Epilogue per MFMA output element: max and
// fma with the head weight (fp32), accumulated in a fixed head order; the
// cross-lane head sum uses a transpose-reduce so that each lane group ends up
// owning one 16-key sub-tile and a 64-key slab is stored as one contiguous
// 256-byte row segment.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kIdxThreads = 256;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerBlock = 4 * kRowsPerWave;

// ReLU on the bit pattern: a float is >= +0 exactly when its int32 image is
// >= 0, so max(bits, 0) is max(x, 0) with -0 -> +0, in one integer op and
// without the NaN canonicalisation a float max would add.
__device__ __forceinline__ float relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

template <int ACT>
__device__ __forceinline__ float activation(float x) {
  if constexpr (ACT == 0) {
    return relu(x);
  } else {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  }
}

struct IdxArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t num_seqs, row_begin, row_end, skip_n;
  const uint8_t* q_idx;
  const uint8_t* k_idx;
  const float* w;
  float* scores;
  int64_t ld;
  int32_t key_chunk;
  int32_t H_I;
};

// NR query rows of one sequence against keys [kstart, kend).
template <int NR, int NHT, int ACT>
__device__ __forceinline__ void fp8_rows(const IdxArgs& a, const int32_t (&rows)[NR], const int32_t (&pos)[NR],
                                         int32_t kbase, int32_t kstart, int32_t kend) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  i32x8 qf[NR][NHT];
  float wv[NR][NHT][4];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const uint8_t* qrow = a.q_idx + (int64_t)rows[i] * a.H_I * 128;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const i32x4* p = (const i32x4*)(qrow + (16 * ht + li) * 128 + 32 * g);
      i32x4 lo = p[0], hi = p[1];
      qf[i][ht] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const f32x4 wq = *(const f32x4*)(a.w + (int64_t)rows[i] * a.H_I + 16 * ht + 4 * g);
      wv[i][ht][0] = wq[0]; wv[i][ht][1] = wq[1]; wv[i][ht][2] = wq[2]; wv[i][ht][3] = wq[3];
    }
  }
  const uint8_t* kb = a.k_idx + (int64_t)kbase * 128 + 32 * g;

  auto load_keys = [&](int32_t s0, i32x8 (&kf)[4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      int32_t s = min(s0 + 16 * st + li, kend - 1);
      const i32x4* p = (const i32x4*)(kb + (int64_t)s * 128);
      i32x4 lo = p[0], hi = p[1];
      kf[st] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  i32x8 kf[4], kn[4];
  load_keys(kstart, kf);
  for (int32_t s0 = kstart; s0 < kend; s0 += 64) {
    if (s0 + 64 < kend) load_keys(s0 + 64, kn);
    float part[NR][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        // NHT independent MFMAs, then one accumulator chain per head tile
        f32x4 x[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          x[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[i][ht], kf[st], f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                   0, 0, 127, 0, 127);
        float acc[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          acc[ht] = wv[i][ht][0] * activation<ACT>(x[ht][0]);
#pragma unroll
          for (int rr = 1; rr < 4; ++rr) acc[ht] = fmaf(wv[i][ht][rr], activation<ACT>(x[ht][rr]), acc[ht]);
        }
        float sum = acc[0];
#pragma unroll
        for (int ht = 1; ht < NHT; ++ht) sum += acc[ht];
        part[i][st] = sum;
      }
    }
    // transpose-reduce over the four lane groups: group g ends with sub-tile g
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bool hi2 = g >= 2;
      float keep0 = hi2 ? part[i][2] : part[i][0];
      float keep1 = hi2 ? part[i][3] : part[i][1];
      float send0 = hi2 ? part[i][0] : part[i][2];
      float send1 = hi2 ? part[i][1] : part[i][3];
      keep0 += __shfl_xor(send0, 32);
      keep1 += __shfl_xor(send1, 32);
      const bool odd = g & 1;
      float keep = odd ? keep1 : keep0;
      float send = odd ? keep0 : keep1;
      keep += __shfl_xor(send, 16);
      const int32_t s = s0 + 16 * g + li;
      if (s < kend && s <= pos[i]) a.scores[(int64_t)(rows[i] - a.row_begin) * a.ld + s] = keep;
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) kf[st] = kn[st];
  }
}

template <int NHT, int ACT>
__global__ __launch_bounds__(kIdxThreads) void indexer_fp8_kernel(IdxArgs a) {
  const int wave = threadIdx.x >> 6;
  const int32_t r0 = a.row_begin + blockIdx.x * kRowsPerBlock + wave * kRowsPerWave;
  const int32_t kstart = blockIdx.y * a.key_chunk;
  int32_t rows[2] = {r0, r0 + 1};
  int32_t pos[2];
  int32_t kbase[2];
  bool valid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    valid[i] = rows[i] < a.row_end;
    pos[i] = -1;
    kbase[i] = 0;
    if (valid[i]) {
      RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, rows[i]);
      pos[i] = ri.pos;
      kbase[i] = ri.kbase;
      valid[i] = ri.pos + 1 > a.skip_n && ri.pos >= kstart;
    }
  }
  const int32_t kchunk_end = kstart + a.key_chunk;
  if (valid[0] && valid[1] && kbase[0] == kbase[1]) {
    const int32_t kend = min(kchunk_end, max(pos[0], pos[1]) + 1);
    fp8_rows<2, NHT, ACT>(a, rows, pos, kbase[0], kstart, kend);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!valid[i]) continue;
      const int32_t r1[1] = {rows[i]};
      const int32_t p1[1] = {pos[i]};
      fp8_rows<1, NHT, ACT>(a, r1, p1, kbase[i], kstart, min(kchunk_end, pos[i] + 1));
    }
  }
}

// fp32 inputs: plain VALU dot products (used for small fp32 problems).
template <int ACT>
__global__ __launch_bounds__(256) void indexer_f32_kernel(IdxArgs a, int d_I) {
  extern __shared__ float qs[];  // [H_I * d_I] query row, then [H_I] weights
  const int32_t r = a.row_begin + blockIdx.x;
  if (r >= a.row_end) return;
  const RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, r);
  if (ri.pos + 1 <= a.skip_n) return;
  const int32_t kstart = blockIdx.y * a.key_chunk;
  const int32_t kend = min(kstart + a.key_chunk, ri.pos + 1);
  if (kstart >= kend) return;
  const float* q = (const float*)a.q_idx + (int64_t)r * a.H_I * d_I;
  float* ws = qs + a.H_I * d_I;
  for (int e = threadIdx.x; e < a.H_I * d_I; e += blockDim.x) qs[e] = q[e];
  for (int e = threadIdx.x; e < a.H_I; e += blockDim.x) ws[e] = a.w[(int64_t)r * a.H_I + e];
  __syncthreads();
  const float* kb = (const float*)a.k_idx + (int64_t)ri.kbase * d_I;
  for (int32_t s = kstart + threadIdx.x; s < kend; s += blockDim.x) {
    const float* kr = kb + (int64_t)s * d_I;
    float acc = 0.0f;
    for (int j = 0; j < a.H_I; ++j) {
      float dot = 0.0f;
      for (int d = 0; d < d_I; ++d) dot = fmaf(qs[j * d_I + d], kr[d], dot);
      acc = fmaf(ws[j], activation<ACT>(dot), acc);
    }
    a.scores[(int64_t)(r - a.row_begin) * a.ld + s] = acc;
  }
}

template <int NHT>
hipError_t launch_fp8(const IdxArgs& a, int act, dim3 grid, hipStream_t s) {
  if (act == 0) hipLaunchKernelGGL((indexer_fp8_kernel<NHT, 0>), grid, dim3(kIdxThreads), 0, s, a);
  else hipLaunchKernelGGL((indexer_fp8_kernel<NHT, 1>), grid, dim3(kIdxThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  IdxArgs a;
  a.cu_q = L.b.cu_q;
  a.cu_k = L.b.cu_k;
  a.num_seqs = L.b.num_seqs;
  a.row_begin = L.b.row_begin;
  a.row_end = L.b.row_end;
  a.skip_n = L.skip_n;
  a.q_idx = (const uint8_t*)L.q_idx;
  a.k_idx = (const uint8_t*)L.k_idx;
  a.w = L.w;
  a.scores = L.scores;
  a.ld = L.ld;
  a.H_I = L.H_I;
  if (L.fp8) {
    // key chunk: enough workgroups to cover every CU several times over
    const int64_t row_blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    int32_t chunk = 4096;
    while (chunk > 256 && row_blocks * ((L.b.max_ctx + chunk - 1) / chunk) < 4LL * L.num_cus) chunk >>= 1;
    a.key_chunk = chunk;
    dim3 grid((unsigned)row_blocks, (unsigned)((L.b.max_ctx + chunk - 1) / chunk));
    switch (L.H_I / 16) {
      case 1: return launch_fp8<1>(a, L.act, grid, s);
      case 2: return launch_fp8<2>(a, L.act, grid, s);
      case 3: return launch_fp8<3>(a, L.act, grid, s);
      case 4: return launch_fp8<4>(a, L.act, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  a.key_chunk = 4096;
  dim3 grid((unsigned)rows, (unsigned)((L.b.max_ctx + a.key_chunk - 1) / a.key_chunk));
  const size_t lds = (size_t)(L.H_I * L.d_I + L.H_I) * sizeof(float);
  if (L.act == 0) hipLaunchKernelGGL((indexer_f32_kernel<0>), grid, dim3(256), lds, s, a, L.d_I);
  else hipLaunchKernelGGL((indexer_f32_kernel<1>), grid, dim3(256), lds, s, a, L.d_I);
  return hipGetLastError();
}

}  // namespace dsa
