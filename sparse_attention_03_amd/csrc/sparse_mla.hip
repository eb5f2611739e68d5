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
// HPW = 32 query heads (one wave per SIMD; every K / V fragment read from LDS
// feeds two MFMAs, which halves LDS traffic against 16 heads per wave):
//   * gather: the 32 selected latent rows of a tile are copied HBM -> LDS with
//     global_load_lds_dwordx4 (16 B per lane, no register staging) into one of
//     four buffers, up to three tiles ahead; every 8 lanes of a copy read one
//     whole 128-byte line of a latent row, and the line-block layout keeps the
//     transposed V reads bank-conflict free;
//   * scores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 -- keys are the MFMA
//     rows (K fragments read from LDS with ds_read_b128), heads the columns (Q
//     fragments resident in VGPRs for the whole row), so each lane ends up
//     holding 16 keys of one head;
//   * softmax: fp32, base-2 exponent with the scale folded in, against a
//     per-head reference max fixed by the first tile (the accumulators are
//     only touched by MFMAs; a row whose sum leaves the safe range is
//     recomputed once with its true max), row sums kept per lane and reduced
//     once;
//   * values: O^T = V^T P^T.  The lane's 8 probabilities of one head are
//     exactly the B fragment of the next MFMA (K index permuted consistently),
//     and the V^T A fragment comes from two ds_read_b64_tr_b16 transposed LDS
//     reads of the row-major tile.
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "mla_tile.h"

namespace dsa {
namespace {

using namespace mla;

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
  int32_t dense;        // every candidate [0, pos] instead of idx (k = the longest row's candidate count)
  int32_t dense_short;  // rows with n <= k walk [0, pos] directly (their idx is 0 .. pos)
  uint16_t* ws_o;  // bf16 partial outputs, each split's own normalised average
  float* ws_lse;
  const float* lse_in;  // target: the main attention's lse per (row, head)
  float* p_out;         // target: [rows, ld_p]
  int64_t ld_p;
};

// DENSE: every candidate [0, pos] in position order (the masked mode of short
// prefill), tile t holding positions 32 t .. 32 t + 31, instead of the row's
// selected entries.  With a.dense_short, rows with n <= k (which select every
// candidate) take the same dense walk; their tiles and tile order equal those
// of the index walk over idx = 0 .. pos, so the result is the same.
// GHOST: H is not NW * 32; the heads past H compute on a copy of head H - 1
// and store nothing, and the recompute also triggers on a non-finite sum of
// the value accumulators.  (The H = 32, 64, 128 instances keep the plain code:
// at this register pressure the compiler's output changed with the shape of
// the code, and only the combinations in these two instances were validated.)
template <int HPW, int NW, bool DENSE, bool GHOST>
__global__ __launch_bounds__(NW * 64, 1) void mla_bf16_kernel(MlaArgs a) {
  constexpr int NT = HPW / 16;
  static_assert(4 % NW == 0, "a wave copies whole row groups");
  constexpr int RG = row_groups_per_wave<NW>();
  constexpr int NINS = kSegments * RG;  // copy instructions per tile per wave
  // tiles whose copies are issued ahead of the one being computed; the counted
  // wait below needs (AHEAD - 1) * NINS to fit the 6-bit vmcnt
  constexpr int AHEAD = 2 * NINS < 64 ? 3 : 1;
  static_assert(AHEAD + 1 <= kNumBuf, "not enough LDS buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  DSA_LDS int32_t* sel = (DSA_LDS int32_t*)((DSA_LDS uint8_t*)smem + kNumBuf * kTileBytes);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int32_t r = a.row_begin + blockIdx.x;
  const int32_t rl = blockIdx.x;
  const int sp = blockIdx.y;
  const RowInfo ri = locate_row_wave(load_seq_table(a.cu_q, a.cu_k, a.num_seqs), a.cu_q, a.cu_k, r);
  const int32_t n = ri.pos + 1;  // candidates of the row
  const bool dense = DENSE || (a.dense_short && n <= a.k);  // uniform over the workgroup
  const int ntiles = dense ? (n + kTile - 1) / kTile : (a.k + kTile - 1) / kTile;
  const int t0 = sp * a.tiles_per_split;
  const int t1 = min(ntiles, t0 + a.tiles_per_split);

  // the row's selected positions, -1 padded to whole tiles, and per tile the
  // mask of its valid entries (bit j: entry 32 t + j is >= 0)
  DSA_LDS uint32_t* tmask = (DSA_LDS uint32_t*)(sel + kMaxSel);
  const int32_t* idx_row = a.idx + (int64_t)rl * a.k;
  if (!dense) stage_selection<NW>(idx_row, a.k, ntiles, sel, tmask);

  // query fragments: B operand of S^T = K Q^T (lane: head li of column tile nt, d = 32c + 8g .. +7)
  bf16x8 qf[NT][kQkSteps];
  const int head0 = wave * HPW;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int hq = GHOST ? min(head0 + 16 * nt + li, a.H - 1) : head0 + 16 * nt + li;
    const uint16_t* qrow = a.q + ((int64_t)r * a.H + hq) * kDqk + 8 * g;
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) qf[nt][c] = *(const bf16x8*)(qrow + 32 * c);
  }
  // The query loads complete here: the tile copies are issued outside the
  // compiler's view, so a query load it still thought in flight would make it
  // wait on vmcnt inside the tile loop, and every such wait would also drain
  // the copies issued ahead.
  wait_vmcnt<0>();
  __syncthreads();  // sel[] and tmask[] visible
  const uint32_t tmask_lane = !dense && lane < kMaxSel / kTile ? tmask[lane] : 0u;  // tile t's mask: lane t
  // position copied by this lane for tile t, row group k (DENSE: invalid
  // entries copy position 0, always in bounds, and are masked)
  auto pos_at = [&](int t, int k) -> int32_t {
    const int e = t * kTile + gather_row(wave, NW, k, lane);
    return dense ? (e < n ? e : 0) : sel[e];
  };

  // Softmax reference point: the first tile's max of each head, fixed for the
  // whole row, so the accumulators are only ever touched by MFMAs and the
  // steady state needs no cross-lane reduction.  Later scores above it only
  // scale the probabilities up (exact in fp32 until they leave its range); if a
  // row sum reaches kSumLimit, a max-only pass rebuilds m_fix as the true max
  // and the row is recomputed against it (practically never taken).
  float m_fix[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) m_fix[nt] = -INFINITY;
  f32x4 oacc[kDvTiles][NT];

  // per-lane LDS byte offsets inside a tile (line blocks, see above):
  //   K fragment (row 16 mt + li, chunk 4c + g): koff[c & 1] + 4096 (c >> 1) + 2048 mt
  //   V^T rows 4g + e4 (+16), chunk 2dt + (r4 >> 1), half r4 & 1:
  //   voff[dt & 3] + 4096 (dt >> 2) (+2048)
  int koff[2], voff[4];
#pragma unroll
  for (int e = 0; e < 2; ++e) koff[e] = tile_off(li, 4 * e + g);
  const int e4 = li >> 2, r4 = li & 3;
#pragma unroll
  for (int m = 0; m < 4; ++m) voff[m] = tile_off(4 * g + e4, 2 * m + (r4 >> 1)) + 8 * (r4 & 1);

  for (int pass = 0; pass < 3; ++pass) {
    const bool max_only = pass == 1;
    if (max_only) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) m_fix[nt] = -INFINITY;  // rebuilt as the running max
    }
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_run[nt] = 0.0f;
    bool overflow = false;

    __syncthreads();  // the previous pass is done with every buffer
#pragma unroll
    for (int j = 0; j < AHEAD; ++j)
      if (t0 + j < t1) {
        int32_t pj[RG];
#pragma unroll
        for (int k = 0; k < RG; ++k) pj[k] = pos_at(t0 + j, k);
        gather_tile<NW>(a.kv, ri.kbase, pj, smem + (size_t)j * kTileBytes);
      }
    // positions for the next gather, read a tile ahead so their LDS latency hides
    int32_t p_next[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k)
      p_next[k] = t0 + AHEAD < t1 ? pos_at(t0 + AHEAD, k) : 0;

    for (int t = t0; t < t1; ++t) {
      // Tile t has landed once at most (copies issued after it) x NINS of this
      // wave's copy instructions are still in flight; the barrier then covers
      // the other waves' copies.
      const int issued_after = min(AHEAD - 1, t1 - 1 - t);
      if (issued_after >= 2) wait_vmcnt<(2 * NINS < 64 ? 2 * NINS : 0)>();
      else if (issued_after == 1) wait_vmcnt<(NINS < 64 ? NINS : 0)>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (t + AHEAD < t1) {
        gather_tile<NW>(a.kv, ri.kbase, p_next, smem + (size_t)((t + AHEAD - t0) % kNumBuf) * kTileBytes);
        if (t + AHEAD + 1 < t1) {
#pragma unroll
          for (int k = 0; k < RG; ++k) p_next[k] = pos_at(t + AHEAD + 1, k);
        }
      }
      const uint32_t vmask = dense ? (n - kTile * t >= kTile ? 0xffffffffu : (1u << (n - kTile * t)) - 1u)
                                   : (uint32_t)__builtin_amdgcn_readlane((int)tmask_lane, t);
      if (vmask != 0) {
        const DSA_LDS uint8_t* lb = (const DSA_LDS uint8_t*)smem + (size_t)((t - t0) % kNumBuf) * kTileBytes;
        // ---- scores: sacc[mt][nt] = S^T[keys 16mt.., heads 16nt..]
        f32x4 sacc[2][NT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const DSA_LDS uint8_t* kb[2] = {lb + koff[0], lb + koff[1]};
        auto load_k = [&](int c, bf16x8 (&kf)[2]) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) kf[mt] = *(const DSA_LDS bf16x8*)(kb[c & 1] + 4096 * (c >> 1) + 2048 * mt);
        };
        // K fragments kQkAhead steps ahead of the MFMAs (one wave per SIMD: the
        // wave itself must cover the LDS latency)
        bf16x8 kring[kQkAhead][2];
#pragma unroll
        for (int i = 0; i < kQkAhead; ++i) load_k(i, kring[i]);
#pragma unroll
        for (int c = 0; c < kQkSteps; ++c) {
          const bf16x8 kc0 = kring[c % kQkAhead][0], kc1 = kring[c % kQkAhead][1];
          if (c + kQkAhead < kQkSteps) load_k(c + kQkAhead, kring[c % kQkAhead]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            sacc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc0, qf[nt][c], sacc[0][nt], 0, 0, 0);
            sacc[1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc1, qf[nt][c], sacc[1][nt], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- softmax (base 2) against the fixed reference; the lane's 8
        //      probabilities of one head are the B fragment of the value product
        //      (MFMA K index 8g + e <-> key 4g + e for e < 4, 16 + 4g + e - 4 otherwise)
        const bool full = vmask == 0xffffffffu;
        if (max_only || m_fix[0] == -INFINITY) {
          // reference max of every head (first valid tile, or the max-only pass)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const bool v = (vmask >> (16 * mt + 4 * g + rr)) & 1u;
                mx = fmaxf(mx, v ? sacc[mt][nt][rr] * a.scale_log2 : -INFINITY);
              }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            m_fix[nt] = fmaxf(m_fix[nt], mx);
          }
          if (max_only) continue;
        }
        bf16x8 pf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(sacc[e >> 2][nt][e & 3], a.scale_log2, -m_fix[nt]);
          if (!full) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (!((vmask >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u)) x[e] = -INFINITY;
          }
          float ps = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = __builtin_amdgcn_exp2f(x[e]);  // v_exp_f32; exp2(-inf) = 0
            ps += x[e];
          }
          l_run[nt] += ps;
          pf[nt] = bf16x8{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                          (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
        }
        // ---- values: O^T[d, h] += V^T[d, keys] P^T[keys, h], one V^T fragment ahead.
        const DSA_LDS uint8_t* vb[4] = {lb + voff[0], lb + voff[1], lb + voff[2], lb + voff[3]};
        auto load_v = [&](int dt) -> bf16x8 {
          const DSA_LDS uint8_t* p = vb[dt & 3] + 4096 * (dt >> 2);
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS i16x4*)p);
          const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DSA_LDS i16x4*)(p + 2048));
          return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
              v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]});
        };
        bf16x8 vring[kPvAhead];
#pragma unroll
        for (int i = 0; i < kPvAhead; ++i) vring[i] = load_v(i);
#pragma unroll
        for (int dt = 0; dt < kDvTiles; ++dt) {
          const bf16x8 vc = vring[dt % kPvAhead];
          if (dt + kPvAhead < kDvTiles) vring[dt % kPvAhead] = load_v(dt + kPvAhead);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vc, pf[nt], oacc[dt][nt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (pass == 0) {
      // Against the first tile's max, a later score far above it scales its
      // probability up.  The row is recomputed against the true max when a
      // per-lane row sum reaches 2^60: below that the four lanes of a head keep
      // its row sum below 2^62, so every p is below 2^62 and every sum of p * v
      // stays finite in fp32 while the latent values are below 2^66 in
      // magnitude.  (Scores differ from the first tile's max by far less than
      // the 40 nats it takes to reach the limit.)  Every wave agrees on whether
      // the row is recomputed (the buffers are shared).
      if constexpr (GHOST) {
        // also on a non-finite accumulator: one running sum of the lane's
        // accumulators is non-finite when any of them is (x - x is NaN
        // exactly for inf and NaN; an overflow of the sum only costs a recompute)
        float sum = 0.0f;
#pragma unroll
        for (int dt = 0; dt < kDvTiles; ++dt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum += oacc[dt][nt][e];
        overflow = !(sum - sum == 0.0f);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) overflow |= !(l_run[nt] < kSumLimit);
      if (!__syncthreads_or(overflow)) break;
    }  // after the max-only pass m_fix holds the true max: every p <= 1, so the
       // recompute stays finite while 2048 max|v| does (|v| < 2^117)
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
    const float lse_v = empty ? -INFINITY : (m_fix[nt] + log2f(l)) * 0.69314718055994531f;
    if (GHOST && h >= a.H) continue;  // a head past H: nothing to store
    // one row of the output, or (key splits) this split's bf16 partial
    const bool direct = a.splits == 1;
    const int64_t slot = ((int64_t)rl * a.splits + sp) * a.H + h;
    uint16_t* orow = (direct ? a.out + ((int64_t)r * a.H + h) * kDv : a.ws_o + slot * kDv) + 4 * g;
#pragma unroll
    for (int dt = 0; dt < kDvTiles; ++dt) {
      const f32x4 o = oacc[dt][nt];
      const uint32_t lo = (uint32_t)to_bf16_bits(o[0] * inv) | ((uint32_t)to_bf16_bits(o[1] * inv) << 16);
      const uint32_t hi = (uint32_t)to_bf16_bits(o[2] * inv) | ((uint32_t)to_bf16_bits(o[3] * inv) << 16);
      *(uint2*)(orow + 16 * dt) = make_uint2(lo, hi);
    }
    if (g == 0) {
      if (!direct) a.ws_lse[slot] = lse_v;
      else if (a.lse) a.lse[(int64_t)r * a.H + h] = lse_v;
    }
  }
}

// Indexer-alignment target (blog "Deepseek v3.2 exp ..." training "Step 1"
// and "Step 2"): per query row and candidate entry e, the heads' attention
// probabilities exp(z_h,e - lse_h) summed over the heads and L1-normalised
// along the candidates.  With the main attention's lse given, each head's
// probabilities sum to 1, so the L1 norm of the head sum is H and the target
// is the head sum / H.  Same walk, gather and score MFMAs as mla_bf16_kernel,
// no value product.  Per tile, each wave reduces its heads within the lane
// groups and leaves a 32-entry partial in LDS; after the next barrier wave 0
// adds the waves' partials and stores the tile's 32 entries (0 for entries
// that are no candidate).
template <int HPW, int NW, bool DENSE>
__global__ __launch_bounds__(NW * 64, 1) void mla_target_kernel(MlaArgs a) {
  constexpr int NT = HPW / 16;
  static_assert(4 % NW == 0, "a wave copies whole row groups");
  constexpr int RG = row_groups_per_wave<NW>();
  constexpr int NINS = kSegments * RG;
  constexpr int AHEAD = 2 * NINS < 64 ? 3 : 1;
  static_assert(AHEAD + 1 <= kNumBuf, "not enough LDS buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  DSA_LDS int32_t* sel = (DSA_LDS int32_t*)((DSA_LDS uint8_t*)smem + kNumBuf * kTileBytes);
  DSA_LDS uint32_t* tmask = (DSA_LDS uint32_t*)(sel + kMaxSel);
  DSA_LDS float* psum = (DSA_LDS float*)(tmask + kMaxSel / kTile);  // [2][NW][kTile]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int32_t r = a.row_begin + blockIdx.x;
  const int32_t rl = blockIdx.x;
  const int sp = blockIdx.y;
  const RowInfo ri = locate_row_wave(load_seq_table(a.cu_q, a.cu_k, a.num_seqs), a.cu_q, a.cu_k, r);
  const int32_t n = ri.pos + 1;
  const bool dense = DENSE;
  const int ntiles = dense ? (n + kTile - 1) / kTile : (a.k + kTile - 1) / kTile;
  const int t0 = sp * a.tiles_per_split;
  const int t1 = min(ntiles, t0 + a.tiles_per_split);
  const int32_t* idx_row = a.idx + (int64_t)rl * a.k;
  if (!dense) stage_selection<NW>(idx_row, a.k, ntiles, sel, tmask);
  bf16x8 qf[NT][kQkSteps];
  float lse2[NT];
  const int head0 = wave * HPW;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int h = head0 + 16 * nt + li;
    const int hq = min(h, a.H - 1);  // heads past H copy head H - 1 and add nothing
    const uint16_t* qrow = a.q + ((int64_t)r * a.H + hq) * kDqk + 8 * g;
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) qf[nt][c] = *(const bf16x8*)(qrow + 32 * c);
    lse2[nt] = h < a.H ? a.lse_in[(int64_t)r * a.H + h] * 1.4426950408889634f : -INFINITY;  // -inf: adds nothing
  }
  wait_vmcnt<0>();  // the query loads complete before the tile loop (see mla_bf16_kernel)
  __syncthreads();
  const uint32_t tmask_lane = !dense && lane < kMaxSel / kTile ? tmask[lane] : 0u;
  auto pos_at = [&](int t, int k) -> int32_t {
    const int e = t * kTile + gather_row(wave, NW, k, lane);
    return dense ? (e < n ? e : 0) : sel[e];
  };
  auto tile_mask = [&](int t) -> uint32_t {
    return dense ? (n - kTile * t >= kTile ? 0xffffffffu : (1u << (n - kTile * t)) - 1u)
                 : (uint32_t)__builtin_amdgcn_readlane((int)tmask_lane, t);
  };
  const float inv_h = 1.0f / (float)a.H;
  float* prow = a.p_out + (int64_t)rl * a.ld_p;
  // wave 0 stores tile t from the waves' partials (every wave wrote its part
  // before the barrier that precedes this)
  auto finish = [&](int t) {
    if (wave == 0 && lane < kTile) {
      const uint32_t vm = tile_mask(t);
      float v = 0.0f;
      if ((vm >> lane) & 1u) {
#pragma unroll
        for (int w = 0; w < NW; ++w) v += psum[((t & 1) * NW + w) * kTile + lane];
        v *= inv_h;
      }
      prow[kTile * t + lane] = v;
    }
  };
  int koff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) koff[e] = tile_off(li, 4 * e + g);

#pragma unroll
  for (int j = 0; j < AHEAD; ++j)
    if (t0 + j < t1) {
      int32_t pj[RG];
#pragma unroll
      for (int k = 0; k < RG; ++k) pj[k] = pos_at(t0 + j, k);
      gather_tile<NW>(a.kv, ri.kbase, pj, smem + (size_t)j * kTileBytes);
    }
  int32_t p_next[RG];
#pragma unroll
  for (int k = 0; k < RG; ++k) p_next[k] = t0 + AHEAD < t1 ? pos_at(t0 + AHEAD, k) : 0;

  for (int t = t0; t < t1; ++t) {
    const int issued_after = min(AHEAD - 1, t1 - 1 - t);
    if (issued_after >= 2) wait_vmcnt<(2 * NINS < 64 ? 2 * NINS : 0)>();
    else if (issued_after == 1) wait_vmcnt<(NINS < 64 ? NINS : 0)>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (t + AHEAD < t1) {
      gather_tile<NW>(a.kv, ri.kbase, p_next, smem + (size_t)((t + AHEAD - t0) % kNumBuf) * kTileBytes);
      if (t + AHEAD + 1 < t1) {
#pragma unroll
        for (int k = 0; k < RG; ++k) p_next[k] = pos_at(t + AHEAD + 1, k);
      }
    }
    if (t > t0) finish(t - 1);
    const uint32_t vmask = tile_mask(t);
    if (vmask == 0) continue;
    const DSA_LDS uint8_t* lb = (const DSA_LDS uint8_t*)smem + (size_t)((t - t0) % kNumBuf) * kTileBytes;
    f32x4 sacc[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const DSA_LDS uint8_t* kb[2] = {lb + koff[0], lb + koff[1]};
    auto load_k = [&](int c, bf16x8 (&kf)[2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) kf[mt] = *(const DSA_LDS bf16x8*)(kb[c & 1] + 4096 * (c >> 1) + 2048 * mt);
    };
    bf16x8 kring[kQkAhead][2];
#pragma unroll
    for (int i = 0; i < kQkAhead; ++i) load_k(i, kring[i]);
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) {
      const bf16x8 kc0 = kring[c % kQkAhead][0], kc1 = kring[c % kQkAhead][1];
      if (c + kQkAhead < kQkSteps) load_k(c + kQkAhead, kring[c % kQkAhead]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sacc[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc0, qf[nt][c], sacc[0][nt], 0, 0, 0);
        sacc[1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc1, qf[nt][c], sacc[1][nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // probabilities of this lane's head(s), summed over the wave's heads:
    // lane (g, li) holds keys 16 mt + 4 g + rr of head 16 nt + li
    float ps[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float v = 0.0f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          v += lse2[nt] == -INFINITY ? 0.0f
                                     : __builtin_amdgcn_exp2f(fmaf(sacc[mt][nt][rr], a.scale_log2, -lse2[nt]));
        ps[mt][rr] = v;
      }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ps[mt][rr] += __shfl_xor(ps[mt][rr], m);
    if (li == 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) psum[((t & 1) * NW + wave) * kTile + 16 * mt + 4 * g + rr] = ps[mt][rr];
    }
  }
  __syncthreads();
  if (t1 > t0) finish(t1 - 1);
}

// Combine key-split partials: o = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// One wave per (row, head), lane l owning value columns 8 l .. 8 l + 7, so a
// split's partial is one 1-KB load of the wave and the reductions need no
// barrier.  Up to kMaxSplits splits: lane l holds the weights of splits
// l, l + 64, ...; the accumulation takes them by readlane.  The first four
// splits' partials are loaded before the weights are known, so their latency
// overlaps that of the lse loads.
template <bool BF16>
__global__ __launch_bounds__(64) void merge_kernel(MlaArgs a) {
  static_assert(kDv == 8 * 64, "one lane per eight value columns");
  constexpr int kW = kMaxSplits / 64;  // weights per lane
  const int32_t rl = blockIdx.x, r = a.row_begin + rl;
  const int h = blockIdx.y;
  const int S = a.splits;
  const int lane = threadIdx.x;
  const int d = 8 * lane;
  const int64_t slot0 = (int64_t)rl * S * a.H + h;  // split s: slot0 + s * H
  auto load_part = [&](int s) -> uint4 {
    return s < S ? *(const uint4*)(a.ws_o + (slot0 + (int64_t)s * a.H) * kDv + d) : make_uint4(0, 0, 0, 0);
  };
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = load_part(u);
  float wl[kW];
  float mloc = -INFINITY;
#pragma unroll
  for (int j = 0; j < kW; ++j) {
    const int s = 64 * j + lane;
    wl[j] = s < S ? a.ws_lse[slot0 + (int64_t)s * a.H] : -INFINITY;
    mloc = fmaxf(mloc, wl[j]);
  }
  const float M = wave_max(mloc);
  float dloc = 0.0f;
#pragma unroll
  for (int j = 0; j < kW; ++j) {
    wl[j] = (M == -INFINITY || wl[j] == -INFINITY) ? 0.0f : expf(wl[j] - M);
    dloc += wl[j];
  }
  const float den = wave_sum(dloc);
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
  auto lo16 = [](uint32_t x) { return __uint_as_float(x << 16); };
  auto hi16 = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };
  // four splits' bf16 partials in flight at a time; the weights of splits
  // 64 j .. 64 j + 63 sit in wl[j] of lanes 0 .. 63
#pragma unroll
  for (int j = 0; j < kW; ++j) {
    if (64 * j >= S) break;
    const int s_end = min(S, 64 * j + 64);
    for (int s0 = 64 * j; s0 < s_end; s0 += 4) {
      if (s0 > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = load_part(s0 + u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u;
        const float w = s < s_end ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl[j]), s - 64 * j)) : 0.0f;
        if (w != 0.0f) {
          acc0 += w * f32x4{lo16(v[u].x), hi16(v[u].x), lo16(v[u].y), hi16(v[u].y)};
          acc1 += w * f32x4{lo16(v[u].z), hi16(v[u].z), lo16(v[u].w), hi16(v[u].w)};
        }
      }
    }
  }
  acc0 *= inv;
  acc1 *= inv;
  const int64_t oi = ((int64_t)r * a.H + h) * kDv + d;
  if constexpr (BF16) {
    auto pack = [](float x, float y) { return (uint32_t)to_bf16_bits(x) | ((uint32_t)to_bf16_bits(y) << 16); };
    *(uint4*)(a.out + oi) = make_uint4(pack(acc0[0], acc0[1]), pack(acc0[2], acc0[3]), pack(acc1[0], acc1[1]),
                                       pack(acc1[2], acc1[3]));
  } else {
    *(f32x4*)((float*)a.out + oi) = acc0;
    *(f32x4*)((float*)a.out + oi + 4) = acc1;
  }
  if (lane == 0 && a.lse) a.lse[(int64_t)r * a.H + h] = den > 0.0f ? M + logf(den) : -INFINITY;
}

// fp32 inputs, alignment target: one workgroup per row, the heads in turn;
// each head's probabilities exp(z - lse_h) are added to the row's entries in
// LDS, which are stored / H at the end.
__global__ __launch_bounds__(256) void mla_target_f32_kernel(MlaArgs a, int d_qk, float scale, int m) {
  extern __shared__ float fs[];  // [d_qk] query of one head, [m] head sum
  const int32_t rl = blockIdx.x, r = a.row_begin + rl;
  const RowInfo ri = locate_row(a.cu_q, a.cu_k, a.num_seqs, r);
  float* qs = fs;
  float* acc = fs + d_qk;
  const float* kv = (const float*)a.kv;
  const int32_t* sel = a.dense ? nullptr : a.idx + (int64_t)rl * a.k;
  for (int e = threadIdx.x; e < m; e += blockDim.x) acc[e] = 0.0f;
  for (int h = 0; h < a.H; ++h) {
    __syncthreads();
    const float* q = (const float*)a.q + ((int64_t)r * a.H + h) * d_qk;
    for (int d = threadIdx.x; d < d_qk; d += blockDim.x) qs[d] = q[d];
    __syncthreads();
    const float lse = a.lse_in[(int64_t)r * a.H + h];
    if (lse == -INFINITY) continue;
    for (int e = threadIdx.x; e < m; e += blockDim.x) {
      const int32_t p = a.dense ? (e <= ri.pos ? e : -1) : (e < a.k ? sel[e] : -1);
      if (p < 0) continue;
      const float* row = kv + (int64_t)(ri.kbase + p) * d_qk;
      float dot = 0.0f;
      for (int d = 0; d < d_qk; ++d) dot = fmaf(qs[d], row[d], dot);
      acc[e] += expf(dot * scale - lse);
    }
  }
  const float inv_h = 1.0f / (float)a.H;
  for (int e = threadIdx.x; e < m; e += blockDim.x) a.p_out[(int64_t)rl * a.ld_p + e] = acc[e] * inv_h;
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
  const int32_t* sel = a.dense ? nullptr : a.idx + (int64_t)rl * a.k;
  for (int d = threadIdx.x; d < d_qk; d += blockDim.x) qs[d] = q[d];
  __syncthreads();
  float mloc = -INFINITY;
  for (int e = threadIdx.x; e < a.k; e += blockDim.x) {
    const int32_t p = a.dense ? (e <= ri.pos ? e : -1) : sel[e];
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
      const int32_t p = a.dense ? (e <= ri.pos ? e : -1) : sel[e];
      if (p < 0) continue;
      acc = fmaf(z[e], kv[(int64_t)(ri.kbase + p) * d_qk + d], acc);
    }
    o[d] = l > 0.0f ? acc / l : 0.0f;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)r * a.H + h] = l > 0.0f ? m + logf(l) : -INFINITY;
}

template <int HPW, int NW, bool DENSE>
hipError_t launch_target(const MlaArgs& a, int rows, hipStream_t s) {
  const size_t lds = (size_t)kNumBuf * kTileBytes + kMaxSel * sizeof(int32_t) + (kMaxSel / kTile) * sizeof(uint32_t) +
                     2 * NW * kTile * sizeof(float);
  static bool attr_set = false;  // benign race: idempotent attribute call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_target_kernel<HPW, NW, DENSE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((mla_target_kernel<HPW, NW, DENSE>), dim3((unsigned)rows, (unsigned)a.splits), dim3(NW * 64),
                     lds, s, a);
  return hipGetLastError();
}

template <int HPW, int NW, bool DENSE, bool GHOST>
hipError_t launch_bf16_g(const MlaArgs& a, int rows, hipStream_t s) {
  const size_t lds = (size_t)kNumBuf * kTileBytes + kMaxSel * sizeof(int32_t) + (kMaxSel / kTile) * sizeof(uint32_t);
  static bool attr_set = false;  // benign race: idempotent attribute call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_bf16_kernel<HPW, NW, DENSE, GHOST>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((mla_bf16_kernel<HPW, NW, DENSE, GHOST>), dim3((unsigned)rows, (unsigned)a.splits),
                     dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int HPW, int NW, bool DENSE>
hipError_t launch_bf16(const MlaArgs& a, int rows, hipStream_t s) {
  return a.H == NW * HPW ? launch_bf16_g<HPW, NW, DENSE, false>(a, rows, s)
                         : launch_bf16_g<HPW, NW, DENSE, true>(a, rows, s);
}

}  // namespace

// Waves of 32 heads per workgroup for H heads (heads past H are masked).
int attention_waves(int H) { return H <= 32 ? 1 : H <= 64 ? 2 : 4; }

// A workgroup fills a CU (its LDS and one wave per SIMD), so a launch of more
// workgroups than CUs runs in rounds: the splits are as many as fit beside
// each other, rows * splits <= num_cus, with the tiles dealt out evenly and no
// split left empty (40 rows of 64 tiles on 256 CUs: 6 splits of 11 tiles, one
// round, where 8 splits of 8 would take two).
int attention_splits(int rows, int k, bool bf16, int num_cus) {
  if (!bf16 || rows <= 0) return 1;
  const int ntiles = (k + kTile - 1) / kTile;
  int64_t target = (int64_t)num_cus / rows;
  if (target > ntiles) target = ntiles;
  if (target > kMaxSplits) target = kMaxSplits;
  if (target <= 1) return 1;
  const int tps = (int)((ntiles + target - 1) / target);  // tiles per split
  return (ntiles + tps - 1) / tps;
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
  a.dense = L.dense ? 1 : 0;
  a.dense_short = L.dense_short ? 1 : 0;
  a.lse_in = L.lse_in;
  a.p_out = L.p_out;
  a.ld_p = L.ld_p;
  if (L.target) {
    if (!L.bf16) {
      // entries written per row: the candidates' span, whole tiles of the walk
      const int m = L.dense ? L.b.max_ctx : L.k;
      const size_t lds = (size_t)(L.d_qk + m) * sizeof(float);
      hipLaunchKernelGGL(mla_target_f32_kernel, dim3((unsigned)rows), dim3(256), lds, s, a, L.d_qk, L.scale, m);
      return hipGetLastError();
    }
    switch (attention_waves(L.H) * 2 + (L.dense ? 1 : 0)) {
      case 2: return launch_target<32, 1, false>(a, rows, s);
      case 4: return launch_target<32, 2, false>(a, rows, s);
      case 8: return launch_target<32, 4, false>(a, rows, s);
      case 3: return launch_target<32, 1, true>(a, rows, s);
      case 5: return launch_target<32, 2, true>(a, rows, s);
      case 9: return launch_target<32, 4, true>(a, rows, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (!L.bf16) {
    const size_t lds = (size_t)(L.d_qk + L.k + 8) * sizeof(float);
    hipLaunchKernelGGL(mla_f32_kernel, dim3((unsigned)rows, (unsigned)L.H), dim3(256), lds, s, a, L.d_qk, L.d_v,
                       L.scale);
    return hipGetLastError();
  }
  hipError_t e;
  switch (attention_waves(L.H) * 2 + (L.dense ? 1 : 0)) {
    case 2: e = launch_bf16<32, 1, false>(a, rows, s); break;
    case 4: e = launch_bf16<32, 2, false>(a, rows, s); break;
    case 8: e = launch_bf16<32, 4, false>(a, rows, s); break;
    case 3: e = launch_bf16<32, 1, true>(a, rows, s); break;
    case 5: e = launch_bf16<32, 2, true>(a, rows, s); break;
    case 9: e = launch_bf16<32, 4, true>(a, rows, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((merge_kernel<true>), dim3((unsigned)rows, (unsigned)a.H), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
