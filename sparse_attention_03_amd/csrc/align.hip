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

// ---------------------------------------------------------------------------
// Backward of the index score to the indexer's inputs (the indexer is what
// the alignment loss trains; its input is detached from the rest, training
// "Step 2").  For an upstream gradient g over a row's candidates, with
// x = q_I[t,j] . k[s] (k scaled per token if scales are given):
//   dw[t,j] += g act(x),  dq_I[t,j,:] += g w[t,j] act'(x) k[s,:],
//   dk_I[s,:] += g w[t,j] act'(x) q_I[t,j,:].
// One workgroup per (query row, key split), one wave per 16 indexer heads;
// the row's candidates go in chunks of 32 keys through a double-buffered LDS
// slab (key row kk: 16-byte chunk c at chunk c ^ ((kk >> 1) & 7)).  Per chunk
// and wave:
//   * x^T = K Q^T and x = Q K^T, two FP8 MFMAs each from the same fragments
//     (the per-token key scale in the MFMA's scale operand): lane (g, li)
//     holds keys 4g + r of head li, and heads 4g + r of key li;
//   * dq[head][dim] += G^T-as-A (head li, keys 4g..4g+3: exactly the x^T
//     lane layout) x K (keys 4g..4g+3 at dim li: four LDS bytes), bf16
//     16x16x16 MFMAs with fp32 accumulators kept for the whole row;
//   * dk[key][dim] = G-as-A (key li, heads 4g..4g+3: the x lane layout) x Q
//     (heads 4g..4g+3 at dim li, held in VGPRs); each wave stores its part
//     into its own LDS region (rows of 132 floats: the four lane groups land
//     on disjoint banks), and once per chunk the waves' parts are added in a
//     fixed order and scatter-added to dk in HBM (global float atomics).
//     (Adding the parts with LDS float atomics instead cost 5x the kernel.)
// G = g w act'(x) is rounded to bf16 for the two products (K and Q are E4M3
// values, exact in bf16).  dq, dw and dk are accumulated with float atomics:
// zero them first; the order of additions, and so the last bits, can vary.

constexpr int kBwChunk = 32;
constexpr int kBwStride = 132;  // floats per key row of a wave's dk part

struct IbArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t num_seqs, row_begin, row_end;
  const uint8_t* q_idx;
  const uint8_t* k_idx;
  const uint8_t* k_scale;
  const float* w;
  int32_t H_I;
  const int32_t* idx;
  int32_t k;
  const float* g;
  int64_t ld_g;
  float* dq;
  float* dw;
  float* dk;
  int32_t chunks_per_split;
};

typedef __attribute__((ext_vector_type(4))) short bf16x4_t;

__device__ __forceinline__ short bf16_bits(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(short, b);
}

template <int ACT>
__device__ __forceinline__ void act_and_slope(float x, float& a, float& da) {
  if constexpr (ACT == 0) {
    a = fmaxf(x, 0.0f);
    da = x > 0.0f ? 1.0f : 0.0f;
  } else {
    const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
    a = x * cdf;
    da = cdf + x * 0.39894228040143268f * expf(-0.5f * x * x);
  }
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// NR query rows per workgroup.  Over a selected set (NR = 1) every row has
// keys of its own.  In the dense warm-up (NR = 4, 2 with GELU) the rows of one sequence
// share their keys: one slab serves all of them and their dk contributions are
// summed in the MFMA accumulators before the scatter, so it issues a quarter of
// the atomics (which bound the kernel: about one fp32 atomic per L2 channel
// and clock).  Rows of different sequences are taken one at a time.
template <int ACT, int NR>
__global__ __launch_bounds__(256) void indexer_bwd_kernel(IbArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t slab[2][kBwChunk * 128];
  __shared__ float dk_part[4][kBwChunk * kBwStride];
  __shared__ int32_t kpos_s[2][kBwChunk];
  __shared__ float g_s[2][NR][kBwChunk];
  __shared__ int32_t ksc_s[2][kBwChunk];
  const int nthreads = blockDim.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const bool dense = a.idx == nullptr;
  const int h0 = 16 * wave;
  // the workgroup's rows (row i of the list is global row rb + i)
  const int32_t rb = a.row_begin + (int32_t)blockIdx.x * NR;
  int32_t pos[NR], kb[NR];
  bool live[NR];
  bool same = true;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    live[i] = rb + i < a.row_end;
    pos[i] = -1;
    kb[i] = 0;
    if (live[i]) {
      const RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, rb + i);
      pos[i] = ri.pos;
      kb[i] = ri.kbase;
      same = same && kb[i] == kb[0];
    }
  }
  // per-row fragments and weights (live rows; the others stay zero)
  i32x8 qf[NR];
  bf16x4_t qT[NR][8];
  float w_li[NR], w_g[NR][4];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    qf[i] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    w_li[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) w_g[i][j] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) qT[i][dt] = bf16x4_t{0, 0, 0, 0};
    if (!live[i]) continue;
    // heads past H_I (H_I a multiple of 4, not of 16) keep a zero query and
    // weight: they add nothing and store nothing
    const uint8_t* qrow = a.q_idx + (int64_t)(rb + i) * a.H_I * 128;
    const float* wrow = a.w + (int64_t)(rb + i) * a.H_I;
    if (h0 + li < a.H_I) {
      const i32x4* p = (const i32x4*)(qrow + (h0 + li) * 128 + 32 * g);
      const i32x4 lo = p[0], hi = p[1];
      qf[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      w_li[i] = wrow[h0 + li];
    }
    if (h0 + 4 * g < a.H_I) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        short v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = bf16_bits(e4m3_to_f32(qrow[(h0 + 4 * g + j) * 128 + 16 * dt + li]));
        qT[i][dt] = bf16x4_t{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) w_g[i][j] = wrow[h0 + 4 * g + j];
    }
  }
  f32x4 dq_acc[NR][8];
  float dw_acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    dw_acc[i] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dq_acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One pass over the chunks of the rows in `act` (a bit per row, all of one
  // sequence: base key row kbase), entries [0, mmax).
  auto run = [&](uint32_t act, int32_t kbase, int32_t mmax) {
    const int nchunks = (mmax + kBwChunk - 1) / kBwChunk;
    const int c0 = blockIdx.y * a.chunks_per_split;
    const int c1 = min(nchunks, c0 + a.chunks_per_split);
    if (c0 >= c1) return;  // uniform over the workgroup
    const uint8_t* kbytes = a.k_idx + (int64_t)kbase * 128;
    // position of entry e for row i (dense: e; selected: idx), -1 if no candidate
    auto entry_pos = [&](int i, int32_t e) -> int32_t {
      if (!((act >> i) & 1u)) return -1;
      if (dense) return e <= pos[i] ? e : -1;
      if (e >= a.k) return -1;
      const int32_t s = a.idx[(int64_t)(rb + i - a.row_begin) * a.k + e];
      return s >= 0 && s <= pos[i] ? s : -1;
    };
    // staging of one chunk: 256 pieces of 16 bytes (key kk = piece / 8, chunk
    // piece % 8), up to four per thread; positions, g of each row, scales
    i32x4 stage[4];
    int32_t st_pos = -1, st_sc = 127;
    float st_g[NR];
    auto fetch = [&](int c) {
      // the chunk's key rows: dense, one position list for all rows; selected,
      // the single row's
      const int irow = dense ? 0 : __builtin_ctz(act);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int piece = tid + u * nthreads;
        if (piece < kBwChunk * 8) {
          const int kk = piece >> 3, ch = piece & 7;
          const int32_t e = kBwChunk * c + kk;
          const int32_t s = dense ? (e < mmax ? e : -1) : entry_pos(irow, e);
          stage[u] = *(const i32x4*)(kbytes + (int64_t)(s < 0 ? 0 : s) * 128 + 16 * ch);
        }
      }
      if (tid < kBwChunk) {
        const int32_t e = kBwChunk * c + tid;
        st_pos = dense ? (e < mmax ? e : -1) : entry_pos(irow, e);
        st_sc = (st_pos >= 0 && a.k_scale) ? (int32_t)a.k_scale[kbase + st_pos] : 127;
#pragma unroll
        for (int i = 0; i < NR; ++i)
          st_g[i] = entry_pos(i, e) >= 0 ? a.g[(int64_t)(rb + i - a.row_begin) * a.ld_g + e] : 0.0f;
      }
    };
    auto store = [&](int buf) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int piece = tid + u * nthreads;
        if (piece < kBwChunk * 8) {
          const int kk = piece >> 3, ch = piece & 7;
          *(DSA_LDS i32x4*)((DSA_LDS uint8_t*)slab[buf] + kk * 128 + 16 * (ch ^ ((kk >> 1) & 7))) = stage[u];
        }
      }
      if (tid < kBwChunk) {
        kpos_s[buf][tid] = st_pos;
        ksc_s[buf][tid] = st_sc;
#pragma unroll
        for (int i = 0; i < NR; ++i) g_s[buf][i][tid] = st_g[i];
      }
    };
    __syncthreads();  // the buffers are free
    fetch(c0);
    store(0);
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
      const int buf = (c - c0) & 1;
      if (c + 1 < c1) fetch(c + 1);  // in flight during this chunk
      const DSA_LDS uint8_t* sb = (const DSA_LDS uint8_t*)slab[buf];
      // key fragments (key 16 kt + li, dims 32g .. 32g + 31) and their scales
      i32x8 kf[2];
      int ksc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int kk = 16 * kt + li;
        const int sw = (kk >> 1) & 7;
        const i32x4 lo = *(const DSA_LDS i32x4*)(sb + kk * 128 + 16 * ((2 * g) ^ sw));
        const i32x4 hi = *(const DSA_LDS i32x4*)(sb + kk * 128 + 16 * ((2 * g + 1) ^ sw));
        kf[kt] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        ksc[kt] = ksc_s[buf][kk];
      }
      // G of every row: x^T (keys 16 kt + 4g + rr of head h0 + li) gives G^T,
      // the A operand of dq; x (heads h0 + 4g + rr of key 16 kt + li) gives G,
      // the A operand of dk
      bf16x4_t gA[NR][2], gB[NR][2];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          gA[i][kt] = bf16x4_t{0, 0, 0, 0};
          gB[i][kt] = bf16x4_t{0, 0, 0, 0};
        }
        if (!((act >> i) & 1u)) continue;  // uniform
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x4 xt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt], qf[i], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                            0, 0, 0, ksc[kt], 0, 127);
          const f32x4 xx = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[i], kf[kt], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                            0, 0, 0, 127, 0, ksc[kt]);
          short va[4], vb[4];
          const float gl = g_s[buf][i][16 * kt + li];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float gk = g_s[buf][i][16 * kt + 4 * g + rr];
            float av, dv;
            act_and_slope<ACT>(xt[rr], av, dv);
            dw_acc[i] = fmaf(gk, av, dw_acc[i]);
            va[rr] = bf16_bits(gk * w_li[i] * dv);
            act_and_slope<ACT>(xx[rr], av, dv);
            vb[rr] = bf16_bits(gl * w_g[i][rr] * dv);
          }
          gA[i][kt] = bf16x4_t{va[0], va[1], va[2], va[3]};
          gB[i][kt] = bf16x4_t{vb[0], vb[1], vb[2], vb[3]};
        }
      }
      // per (key tile, column tile): K's column (keys 16 kt + 4g .. + 3 at dim
      // 16 dt + li) converted once, then every row's dq product and its dk
      // product, the latter summed over the rows:
      // dk[key 16 kt + 4g + rr][dim 16 dt + li] into this wave's LDS part
      float* part = dk_part[wave];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float kscale[4];
        int kk4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kk4[j] = 16 * kt + 4 * g + j;
          kscale[j] = __builtin_ldexpf(1.0f, ksc_s[buf][kk4[j]] - 127);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          short v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kk = kk4[j];
            const uint32_t byte = sb[kk * 128 + 16 * (dt ^ ((kk >> 1) & 7)) + li];
            v[j] = bf16_bits(e4m3_to_f32(byte) * kscale[j]);
          }
          const bf16x4_t kB = bf16x4_t{v[0], v[1], v[2], v[3]};
          f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            if (!((act >> i) & 1u)) continue;  // uniform
            dq_acc[i][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gA[i][kt], kB, dq_acc[i][dt], 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gB[i][kt], qT[i][dt], d, 0, 0, 0);
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) part[(16 * kt + 4 * g + rr) * kBwStride + 16 * dt + li] = d[rr];
        }
      }
      __syncthreads();  // every wave's dk part written, every wave done with slab[buf]
      if (c + 1 < c1) store(buf ^ 1);
      // the waves' parts added in order, scatter-added to the chunk's key rows
      const int nwaves = nthreads >> 6;
      for (int e = tid; e < kBwChunk * 128; e += nthreads) {
        const int kk = e >> 7;
        const int32_t s = kpos_s[buf][kk];
        float v = 0.0f;
        for (int w = 0; w < nwaves; ++w) v += dk_part[w][kk * kBwStride + (e & 127)];
        if (s >= 0 && v != 0.0f) atomicAdd(a.dk + (int64_t)(kbase + s) * 128 + (e & 127), v);
      }
      __syncthreads();
    }
  };

  if (dense && same) {
    uint32_t act = 0;
    int32_t pmax = -1;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (live[i]) {
        act |= 1u << i;
        pmax = max(pmax, pos[i]);
      }
    run(act, kb[0], pmax + 1);
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (live[i]) run(1u << i, kb[i], dense ? pos[i] + 1 : a.k);
  }
  // dw: sum over the lane groups; dq: this split's share
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (!live[i]) continue;
    const int32_t r = rb + i;
    float d = dw_acc[i];
    d += __shfl_xor(d, 16);
    d += __shfl_xor(d, 32);
    if (g == 0 && h0 + li < a.H_I) atomicAdd(a.dw + (int64_t)r * a.H_I + h0 + li, d);
    if (h0 + 4 * g < a.H_I) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          atomicAdd(a.dq + ((int64_t)r * a.H_I + h0 + 4 * g + rr) * 128 + 16 * dt + li, dq_acc[i][dt][rr]);
    }
  }
}

}  // namespace

hipError_t launch_indexer_bwd(const IndexerBwdLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  IbArgs a;
  a.cu_q = L.b.cu_q;
  a.cu_k = L.b.cu_k;
  a.num_seqs = L.b.num_seqs;
  a.row_begin = L.b.row_begin;
  a.row_end = L.b.row_end;
  a.q_idx = (const uint8_t*)L.q_idx;
  a.k_idx = (const uint8_t*)L.k_idx;
  a.k_scale = L.k_scale;
  a.w = L.w;
  a.H_I = L.H_I;
  a.idx = L.idx;
  a.k = L.k;
  a.g = L.g;
  a.ld_g = L.ld_g;
  a.dq = L.dq;
  a.dw = L.dw;
  a.dk = L.dk;
  const int m = L.idx ? L.k : L.b.max_ctx;
  // rows per workgroup: 4 in the dense warm-up (2 with GELU, whose epilogue
  // needs the registers), 1 over selected sets
  const int nr = L.idx ? 1 : (L.act == 0 ? 4 : 2);
  const int64_t blocks = (rows + nr - 1) / nr;
  const int nchunks = (m + kBwChunk - 1) / kBwChunk;
  int splits = 1;
  while (splits < nchunks && blocks * splits < 2LL * L.num_cus) splits <<= 1;
  if (splits > nchunks) splits = nchunks;
  a.chunks_per_split = (nchunks + splits - 1) / splits;
  const dim3 grid((unsigned)blocks, (unsigned)splits), block((unsigned)(64 * ((L.H_I + 15) / 16)));
  if (nr == 1) {
    if (L.act == 0) hipLaunchKernelGGL((indexer_bwd_kernel<0, 1>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((indexer_bwd_kernel<1, 1>), grid, block, 0, s, a);
  } else if (L.act == 0) {
    hipLaunchKernelGGL((indexer_bwd_kernel<0, 4>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((indexer_bwd_kernel<1, 2>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

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
