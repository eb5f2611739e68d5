// sparse_mla.hip -- sparse MLA attention in MQA mode on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com): section
// "Step 2" -- attention is computed between the query token and the selected
// entries only, and those entries are MLA's low-rank latent vectors; section
// "在MLA下實例化DSA" -- DSA runs on MLA's MQA mode, every latent is shared by
// all query heads of the token.  The key is the whole 576-wide latent row
// (512 latent + 64 rope columns) and the value is its first 512 columns.
//
// BF16 kernel, one workgroup per (query row, key split), NW waves each owning
// HPW query heads:
//   * gather: the 64 selected latent rows of a tile are copied HBM -> LDS with
//     global_load_lds_dwordx4 (16 B per lane, no register staging), double
//     buffered, each row stored as 72 16-byte chunks with an XOR swizzle of
//     the chunk index inside each group of 8 (bank spreading for both the
//     row-wise and the transposed reads);
//   * scores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 -- keys are the MFMA
//     rows (K fragments read from LDS with ds_read_b128), heads the columns (Q
//     fragments resident in VGPRs for the whole row), so each lane ends up
//     holding 16 keys of one head;
//   * softmax: fp32, base-2 exponent with the scale folded in, running max
//     updated only when a tile's max exceeds it by more than 8 (so the
//     accumulator rescale is rare), row sums kept per lane and reduced once;
//   * values: O^T = V^T P^T.  The lane's 8 probabilities of one head are
//     exactly the B fragment of the next MFMA (K index permuted consistently),
//     and the V^T A fragment comes from two ds_read_b64_tr_b16 transposed LDS
//     reads of the row-major tile.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;        // 1152
constexpr int kChunksPerRow = kRowBytes / 16;  // 72
constexpr int kTile = 64;                  // selected entries per tile
constexpr int kTileBytes = kTile * kRowBytes;  // 73728
constexpr int kQkSteps = kDqk / 32;        // 18
constexpr int kDvTiles = kDv / 16;         // 32
constexpr float kLazy = 8.0f;              // log2 headroom before a rescale

struct MlaArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t num_seqs, row_begin, row_end;
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* idx;
  int32_t k, H;
  float scale_log2;  // softmax scale * log2(e)
  uint16_t* out;
  float* lse;
  int32_t splits, tiles_per_split;
  float* ws_o;
  float* ws_lse;
};

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int chunk_at(int chunk, int row) { return (chunk & ~7) | ((chunk & 7) ^ swz(row)); }

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

template <int NW>
__device__ __forceinline__ void gather_tile(const MlaArgs& a, int32_t kbase, int32_t idx_lane, uint8_t* buf) {
  constexpr int RPW = kTile / NW;                      // rows gathered by one wave
  constexpr int NINS = RPW * kChunksPerRow / 64;       // wave instructions
  const int wave = threadIdx.x >> 6;
  int lane = threadIdx.x & 63;
  // keep the per-lane address arithmetic inside the tile loop (cheap integer
  // ops) instead of letting it be hoisted into registers for the whole kernel
  asm volatile("" : "+v"(lane));
  DSA_LDS uint8_t* lbase = (DSA_LDS uint8_t*)buf + (size_t)wave * RPW * kRowBytes;
#pragma unroll
  for (int q = 0; q < NINS; ++q) {
    const int slot = 64 * q + lane;
    const int riw = slot / kChunksPerRow;
    const int c_lds = slot - riw * kChunksPerRow;
    const int row = wave * RPW + riw;
    int32_t p = __shfl(idx_lane, row);
    p = p < 0 ? 0 : p;
    const int c_src = chunk_at(c_lds, row);
    const uint8_t* src = a.kv + ((int64_t)(kbase + p) * kChunksPerRow + c_src) * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (DSA_LDS void*)(lbase + 64 * q * 16), 16, 0, 0);
  }
}

template <int HPW, int NW>
__global__ __launch_bounds__(NW * 64, 1) void mla_bf16_kernel(MlaArgs a) {
  constexpr int NT = HPW / 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int32_t r = a.row_begin + blockIdx.x;
  const int32_t rl = blockIdx.x;
  const int sp = blockIdx.y;
  const RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, r);
  const int ntiles = (a.k + kTile - 1) / kTile;
  const int t0 = sp * a.tiles_per_split;
  const int t1 = min(ntiles, t0 + a.tiles_per_split);
  const int32_t* idx_row = a.idx + (int64_t)rl * a.k;
  auto load_idx = [&](int t) -> int32_t {
    const int e = t * kTile + lane;
    return (t < t1 && e < a.k) ? idx_row[e] : -1;
  };

  // query fragments: B operand of S^T = K Q^T (lane: head li of column tile nt, d = 32c + 8g .. +7)
  bf16x8 qf[NT][kQkSteps];
  const int head0 = wave * HPW;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint16_t* qrow = a.q + ((int64_t)r * a.H + head0 + 16 * nt + li) * kDqk + 8 * g;
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) qf[nt][c] = *(const bf16x8*)(qrow + 32 * c);
  }

  f32x4 oacc[kDvTiles][NT];
#pragma unroll
  for (int dt = 0; dt < kDvTiles; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.0f; }

  int32_t idx_cur = load_idx(t0);
  int32_t idx_nxt = load_idx(t0 + 1);
  if (t0 < t1) gather_tile<NW>(a, ri.kbase, idx_cur, smem);

  for (int t = t0; t < t1; ++t) {
    uint8_t* buf = smem + (size_t)((t - t0) & 1) * kTileBytes;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int32_t idx_nn = -1;
    if (t + 1 < t1) {
      gather_tile<NW>(a, ri.kbase, idx_nxt, smem + (size_t)((t + 1 - t0) & 1) * kTileBytes);
      idx_nn = load_idx(t + 2);
    }
    const uint64_t vmask = __ballot(idx_cur >= 0);
    if (vmask != 0) {
      const DSA_LDS uint8_t* lb = (const DSA_LDS uint8_t*)buf;
      // ---- scores: sacc[mt][nt] = S^T[keys 16mt.., heads 16nt..]
      f32x4 sacc[4][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K fragment of (key row 16mt + li, chunk 4c + g).  The swizzle of a row
      // with li = row mod 16 only depends on li, and chunk 4c + g = 8(c>>1) +
      // (4(c&1) | g), so the byte address is a per-lane base chosen by the
      // parity of c plus the compile-time offset 16*1152*mt + 128*(c>>1).
      const int sw = swz(li);
      const int vk0 = ((sw & 4)) + (g ^ (sw & 3));
      const int vk1 = ((sw & 4) ^ 4) + (g ^ (sw & 3));
      const DSA_LDS uint8_t* kbase0 = lb + li * kRowBytes + 16 * vk0;
      const DSA_LDS uint8_t* kbase1 = lb + li * kRowBytes + 16 * vk1;
      auto load_k = [&](int c, bf16x8 (&kf)[4]) {
        const DSA_LDS uint8_t* kb = (c & 1) ? kbase1 : kbase0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          kf[mt] = *(const DSA_LDS bf16x8*)(kb + (16 * kRowBytes * mt + 128 * (c >> 1)));
      };
      bf16x8 kcur[4], knxt[4];
      load_k(0, kcur);
#pragma unroll
      for (int c = 0; c < kQkSteps; ++c) {
        if (c + 1 < kQkSteps) load_k(c + 1, knxt);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kcur[mt], qf[nt][c], sacc[mt][nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) kcur[mt] = knxt[mt];
      }
      // ---- softmax (base 2), probabilities as the B fragments of the value product
      bf16x8 pf[2][NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float x[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int e = 16 * mt + 4 * g + rr;
            const bool v = (vmask >> e) & 1ull;
            x[mt][rr] = v ? sacc[mt][nt][rr] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, x[mt][rr]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = mx > m_run[nt] + kLazy;
        if (__ballot(need) != 0) {
          const float alpha = need ? exp2f(m_run[nt] - mx) : 1.0f;
          if (need) m_run[nt] = mx;
          l_run[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < kDvTiles; ++dt) oacc[dt][nt] *= alpha;
        }
        float ps = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            x[mt][rr] = exp2f(x[mt][rr] - m_run[nt]);
            ps += x[mt][rr];
          }
        l_run[nt] += ps;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pf[ks][nt] = bf16x8{(__bf16)x[2 * ks][0], (__bf16)x[2 * ks][1], (__bf16)x[2 * ks][2], (__bf16)x[2 * ks][3],
                              (__bf16)x[2 * ks + 1][0], (__bf16)x[2 * ks + 1][1], (__bf16)x[2 * ks + 1][2],
                              (__bf16)x[2 * ks + 1][3]};
      }
      // ---- values: O^T[d, h] += V^T[d, keys] P^T[keys, h], one step of V^T fragments ahead
      // V^T fragment rows 32ks + 4g + e4 (+16), columns 16dt + 4r4 .. +3.  With
      // row mod 8 = 4(g&1) + e4, the swizzled chunk of column chunk 2dt + (r4>>1)
      // is 8(dt>>2) + 2((dt&3) ^ e4) + ((r4>>1) ^ (g&1)): a per-lane base chosen
      // by dt&3 plus the compile-time offset 32*1152*ks + 128*(dt>>2).
      const int e4 = li >> 2, r4 = li & 3;
      const DSA_LDS uint8_t* vrow = lb + (4 * g + e4) * kRowBytes + 16 * ((r4 >> 1) ^ (g & 1)) + 8 * (r4 & 1);
      const DSA_LDS uint8_t* vb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vb[j] = vrow + 32 * (j ^ e4);
      auto load_v = [&](int step) -> bf16x8 {
        const int ks = step / kDvTiles, dt = step % kDvTiles;
        const DSA_LDS uint8_t* p = vb[dt & 3] + (32 * kRowBytes * ks + 128 * (dt >> 2));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS i16x4*)p);
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS i16x4*)(p + 16 * kRowBytes));
        return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
            v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]});
      };
      bf16x8 vcur = load_v(0), vnxt;
#pragma unroll
      for (int step = 0; step < 2 * kDvTiles; ++step) {
        const int ks = step / kDvTiles, dt = step % kDvTiles;
        if (step + 1 < 2 * kDvTiles) vnxt = load_v(step + 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          oacc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, pf[ks][nt], oacc[dt][nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        vcur = vnxt;
      }
    }
    idx_cur = idx_nxt;
    idx_nxt = idx_nn;
  }

  // ---- epilogue
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int h = head0 + 16 * nt + li;
    const bool empty = !(l > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / l;
    const float lse_v = empty ? -INFINITY : (m_run[nt] + log2f(l)) * 0.69314718055994531f;
    if (a.splits == 1) {
      uint16_t* orow = a.out + ((int64_t)r * a.H + h) * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) {
        const f32x4 o = oacc[dt][nt];
        const uint32_t lo = (uint32_t)to_bf16_bits(o[0] * inv) | ((uint32_t)to_bf16_bits(o[1] * inv) << 16);
        const uint32_t hi = (uint32_t)to_bf16_bits(o[2] * inv) | ((uint32_t)to_bf16_bits(o[3] * inv) << 16);
        *(uint2*)(orow + 16 * dt) = make_uint2(lo, hi);
      }
      if (a.lse && g == 0) a.lse[(int64_t)r * a.H + h] = lse_v;
    } else {
      const int64_t slot = ((int64_t)rl * a.splits + sp) * a.H + h;
      float* orow = a.ws_o + slot * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDvTiles; ++dt) *(f32x4*)(orow + 16 * dt) = oacc[dt][nt] * inv;
      if (g == 0) a.ws_lse[slot] = lse_v;
    }
  }
}

// Combine key-split partials: o = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
template <bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MlaArgs a, int d_v) {
  const int32_t rl = blockIdx.x;
  const int32_t r = a.row_begin + rl;
  const int S = a.splits;
  for (int e = threadIdx.x; e < a.H * d_v; e += blockDim.x) {
    const int h = e / d_v, d = e - h * d_v;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, a.ws_lse[((int64_t)rl * S + s) * a.H + h]);
    float num = 0.0f, den = 0.0f;
    if (M > -INFINITY) {
      for (int s = 0; s < S; ++s) {
        const int64_t slot = ((int64_t)rl * S + s) * a.H + h;
        const float ls = a.ws_lse[slot];
        if (ls == -INFINITY) continue;
        const float wgt = expf(ls - M);
        num = fmaf(wgt, a.ws_o[slot * d_v + d], num);
        den += wgt;
      }
    }
    const float o = den > 0.0f ? num / den : 0.0f;
    const int64_t oi = ((int64_t)r * a.H + h) * d_v + d;
    if constexpr (BF16) a.out[oi] = to_bf16_bits(o);
    else ((float*)a.out)[oi] = o;
    if (d == 0 && a.lse) a.lse[(int64_t)r * a.H + h] = den > 0.0f ? M + logf(den) : -INFINITY;
  }
}

// fp32 inputs: plain two-pass softmax per (row, head) on the VALU.
__global__ __launch_bounds__(256) void mla_f32_kernel(MlaArgs a, int d_qk, int d_v, float scale) {
  extern __shared__ float fs[];  // [d_qk] query, [k] logits, [8] reduction
  const int32_t rl = blockIdx.x, r = a.row_begin + rl;
  const int h = blockIdx.y;
  const RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, r);
  float* qs = fs;
  float* z = fs + d_qk;
  float* red = z + a.k;
  const float* q = (const float*)a.q + ((int64_t)r * a.H + h) * d_qk;
  const float* kv = (const float*)a.kv;
  const int32_t* sel = a.idx + (int64_t)rl * a.k;
  for (int d = threadIdx.x; d < d_qk; d += blockDim.x) qs[d] = q[d];
  __syncthreads();
  float mloc = -INFINITY;
  for (int e = threadIdx.x; e < a.k; e += blockDim.x) {
    const int32_t p = sel[e];
    float zz = -INFINITY;
    if (p >= 0) {
      const float* row = kv + (int64_t)(ri.kbase + p) * d_qk;
      float dot = 0.0f;
      for (int d = 0; d < d_qk; ++d) dot = fmaf(qs[d], row[d], dot);
      zz = dot * scale;
    }
    z[e] = zz;
    mloc = fmaxf(mloc, zz);
  }
  mloc = wave_max(mloc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mloc;
  __syncthreads();
  float m = -INFINITY;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  float lloc = 0.0f;
  for (int e = threadIdx.x; e < a.k; e += blockDim.x) {
    const float p = (m == -INFINITY) ? 0.0f : expf(z[e] - m);
    z[e] = p;
    lloc += p;
  }
  lloc = wave_sum(lloc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lloc;
  __syncthreads();
  float l = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) l += red[w];
  float* o = (float*)a.out + ((int64_t)r * a.H + h) * d_v;
  for (int d = threadIdx.x; d < d_v; d += blockDim.x) {
    float acc = 0.0f;
    for (int e = 0; e < a.k; ++e) {
      const int32_t p = sel[e];
      if (p < 0) continue;
      acc = fmaf(z[e], kv[(int64_t)(ri.kbase + p) * d_qk + d], acc);
    }
    o[d] = l > 0.0f ? acc / l : 0.0f;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)r * a.H + h] = l > 0.0f ? m + logf(l) : -INFINITY;
}

template <int HPW, int NW>
hipError_t launch_bf16(const MlaArgs& a, int rows, hipStream_t s) {
  const size_t lds = 2 * (size_t)kTileBytes;
  static bool attr_set = false;  // benign race: idempotent attribute call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_bf16_kernel<HPW, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((mla_bf16_kernel<HPW, NW>), dim3((unsigned)rows, (unsigned)a.splits), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int attention_splits(int rows, int k, bool bf16, int num_cus) {
  if (!bf16 || rows <= 0) return 1;
  const int ntiles = (k + kTile - 1) / kTile;
  int splits = 1;
  while (splits < ntiles && (int64_t)rows * splits < (int64_t)num_cus) splits <<= 1;
  if (splits > ntiles) splits = ntiles;
  return splits < 1 ? 1 : splits;
}

hipError_t launch_attention(const AttnLaunch& L, hipStream_t s) {
  const int32_t rows = L.b.row_end - L.b.row_begin;
  if (rows <= 0) return hipSuccess;
  MlaArgs a;
  a.cu_q = L.b.cu_q;
  a.cu_k = L.b.cu_k;
  a.num_seqs = L.b.num_seqs;
  a.row_begin = L.b.row_begin;
  a.row_end = L.b.row_end;
  a.q = (const uint16_t*)L.q;
  a.kv = (const uint8_t*)L.kv;
  a.idx = L.idx;
  a.k = L.k;
  a.H = L.H;
  a.scale_log2 = L.scale * 1.4426950408889634f;
  a.out = (uint16_t*)L.out;
  a.lse = L.lse;
  a.splits = L.bf16 ? L.splits : 1;
  const int ntiles = (L.k + kTile - 1) / kTile;
  a.tiles_per_split = (ntiles + a.splits - 1) / a.splits;
  a.ws_o = L.ws_o;
  a.ws_lse = L.ws_lse;
  if (!L.bf16) {
    const size_t lds = (size_t)(L.d_qk + L.k + 8) * sizeof(float);
    hipLaunchKernelGGL(mla_f32_kernel, dim3((unsigned)rows, (unsigned)L.H), dim3(256), lds, s, a, L.d_qk, L.d_v,
                       L.scale);
    return hipGetLastError();
  }
  hipError_t e;
  switch (L.H) {
    case 32: e = launch_bf16<16, 2>(a, rows, s); break;
    case 64: e = launch_bf16<16, 4>(a, rows, s); break;
    case 128: e = launch_bf16<16, 8>(a, rows, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((merge_kernel<true>), dim3((unsigned)rows), dim3(256), 0, s, a, kDv);
  return hipGetLastError();
}

}  // namespace dsa
