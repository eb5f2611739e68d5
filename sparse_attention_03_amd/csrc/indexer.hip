// indexer.hip -- lightning-indexer scores on gfx950.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), section
// "Lightning indexer / Step 1": the index score of query row t against a
// preceding token s is sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]) over the few
// indexer heads j; the indexer is cheap because it has few heads and runs in
// FP8.  GELU (named instead of ReLU on the gamebaike.com summary,
// 【闪电索引器】) is a template switch.
//
// FP8 path: one v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3) computes a
// whole d_I = 128 dot product for 16 heads x 16 keys.  A wave holds the query
// fragments of two query rows (all heads) in VGPRs and streams key fragments
// straight from global memory (a 16-key fragment is 2 KB contiguous; the four
// waves of a workgroup sweep the same keys so the L1 serves most reads).
//
// ReLU epilogue.  With ReLU(x) = (x + |x|) / 2 the score splits into
//   I = 1/2 * qt . k  +  1/2 * sum_j w_j |x_j|,   qt = sum_j w_j q_I[j],
// a linear term and a term that costs one fma per head (|x| is a free source
// modifier), instead of a max and an fma.  The linear term runs on the MFMA
// too: a pre-pass writes qt per row as four E4M3 terms, each with E8M0 scales
// per 32-element K block of the MFMA (the residual after four terms is about
// 2^-16 of the block maximum; six would represent the fp32 qt exactly).  The terms of row i
// sit in MFMA rows {i, i+4, i+8, i+12}, so every lane group holds one term per
// key and the cross-lane head sum adds the terms up for free.  The GELU
// epilogue applies the activation per head.
//
// Cross-lane head sum: a transpose-reduce with the gfx950 permlane swaps, so
// that each lane group ends up owning one 16-key sub-tile and a 64-key slab is
// one contiguous 256-byte store per row.  Key loads and score stores are
// buffer instructions whose range check replaces per-lane clamps: keys past
// the chunk read as zero, scores past the causal bound are dropped.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kIdxThreads = 256;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerBlock = 4 * kRowsPerWave;
constexpr int kSlabBytes = 64 * 128;                         // 64 keys
constexpr int kRing = 3;                                      // LDS slabs: one read, two in flight
constexpr int kPrivSlots = 4;                                 // per-wave LDS ring of the streaming kernel
constexpr int kStreamRows = 4;                                // rows per workgroup of the streaming kernel
constexpr int kScaleArea = 256;                               // LDS bytes per slab's key scales (a dword per key)
constexpr int kLinTerms = 4;
constexpr int kLinScaleOff = kLinTerms * 128;                 // E8M0 scales [term][32-dim block]
constexpr int kLinRowBytes = kLinScaleOff + kLinTerms * 4;    // 528
constexpr uint32_t kBufFlags = 0x00020000;                    // raw buffer, dword data format

template <int ACT>
__device__ __forceinline__ float activation(float x) {
  if constexpr (ACT == 0) {
    return fmaxf(x, 0.0f);
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
  const uint8_t* lin;      // [row_end - row_begin, kLinRowBytes] linear-term fragments (ReLU)
  uint8_t* lin_out;
  const uint8_t* k_scale;  // [total_k] E8M0 per-key scales, or null
};

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Sum over the four lane groups of part[st], leaving sub-tile g's total in lane
// group g: a permlane32 swap pairs groups {0,2} and {1,3}, a permlane16 swap
// then pairs {0,1} and {2,3}.
__device__ __forceinline__ float transpose_reduce(float p0, float p1, float p2, float p3) {
  auto a = __builtin_amdgcn_permlane32_swap(f_bits(p0), f_bits(p2), false, false);
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(p1), f_bits(p3), false, false);
  const float ka = bits_f(a[0]) + bits_f(a[1]);  // groups 0,1: sub-tile 0; groups 2,3: sub-tile 2
  const float kb = bits_f(b[0]) + bits_f(b[1]);  // groups 0,1: sub-tile 1; groups 2,3: sub-tile 3
  auto c = __builtin_amdgcn_permlane16_swap(f_bits(ka), f_bits(kb), false, false);
  return bits_f(c[0]) + bits_f(c[1]);
}

// Linear-term pre-pass, one wave per query row: qt = sum_j w[j] q_I[j] in
// fp32, then four E4M3 terms with per-32-block power-of-two scales, each the
// rounding of what the previous ones left.
__global__ __launch_bounds__(256) void indexer_lin_kernel(IdxArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t r = a.row_begin + blockIdx.x * 4 + wave;
  if (r >= a.row_end) return;
  const uint8_t* qrow = a.q_idx + (int64_t)r * a.H_I * 128 + 2 * lane;
  const float* wr = a.w + (int64_t)r * a.H_I;
  float q0 = 0.0f, q1 = 0.0f;
  for (int h = 0; h < a.H_I; h += 4) {  // H_I is a multiple of 4
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t two = *(const uint16_t*)(qrow + (h + u) * 128);
      const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
      const float wh = wr[h + u];
      q0 = fmaf(wh, f[0], q0);
      q1 = fmaf(wh, f[1], q1);
    }
  }
  uint8_t* out = a.lin_out + (int64_t)(r - a.row_begin) * kLinRowBytes;
  // The MFMA reads a lane's 32 fragment bytes as K = 16 g + (0..15) and
  // 64 + 16 g + (0..15) (g = lane / 16), and lane group b's E8M0 scale covers
  // K = 32 b .. 32 b + 31.  In memory order (fragment bytes = dims 32 g ..
  // 32 g + 31) scale block b is therefore dims {0-15, 32-47} (b = 0),
  // {64-79, 96-111} (1), {16-31, 48-63} (2), {80-95, 112-127} (3): for this
  // lane's dims 2 lane, 2 lane + 1:
  const int blk = ((lane >> 5) & 1) + 2 * ((lane >> 3) & 1);
#pragma unroll
  for (int t = 0; t < kLinTerms; ++t) {
    float m = fmaxf(fabsf(q0), fabsf(q1));
    // max over the 16 lanes of this scale block (lane bits 0-2 and 4 vary)
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    m = fmaxf(m, __shfl_xor(m, 16));
    int e = 0;
    if (m > 0.0f) {
      int E;
      (void)frexpf(m, &E);
      e = E - 8;  // m * 2^-e in [128, 256): below the E4M3 maximum 448
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(q0, -e), ldexpf(q1, -e), 0, false);
    const auto back = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
    q0 -= ldexpf(back[0], e);
    q1 -= ldexpf(back[1], e);
    *(uint16_t*)(out + t * 128 + 2 * lane) = (uint16_t)pk;
    if ((lane & 0x17) == 0) out[kLinScaleOff + t * 4 + blk] = (uint8_t)(127 + e);
  }
}

// Where the keys come from.
enum KeySource {
  kKeysShared = 0,    // the four waves run the same key range and take the keys from an LDS ring
                      // that they fill together (one 8-KB slab per barrier)
  kKeysPlain = 2,     // each wave streams its keys, one slab at a time (fewest registers)
  kKeysPrivate = 3,   // each wave streams its keys through its own LDS ring (global_load_lds),
                      // kPrivSlots - 1 slabs in flight, no register staging and no barriers
};

// NR query rows of one sequence against keys [kstart, kend); lim[i]: row i's
// scores are stored for keys below lim[i] only.  LIN: ReLU through the
// linear-term MFMA and |x| (rows need the pre-pass fragments); otherwise the
// activation is applied per head.  SC: every key carries an E8M0 scale, which
// goes into the MFMA's B-operand scale (lane (g, li) of sub-tile st: key
// 16 st + li).  On the LDS paths a slab's scales travel with its keys: one
// byte copy per lane into the wave's kScaleArea bytes at `sarea` (key i of the
// slab in the low byte of dword i), counted by the same waits.
template <int NR, int NHT, int ACT, int KEYS, bool SC, bool LIN = ACT == 0>
__device__ __forceinline__ void fp8_rows(const IdxArgs& a, const int32_t (&rows)[NR], const int32_t (&lim)[NR],
                                         int32_t kbase, int32_t kstart, int32_t kend, DSA_LDS uint8_t* ring,
                                         DSA_LDS uint8_t* sarea) {
  static_assert(!LIN || ACT == 0, "the linear-term split is ReLU's");
  constexpr int NST = 4;                          // 16-key sub-tiles per 64-key slab
  constexpr int NPS = (LIN ? 1 : 0) + NR * NHT;   // MFMAs per sub-tile
  constexpr int NM = NST * NPS;                   // MFMAs per slab
  constexpr int LAG = 2;                          // epilogue of MFMA j follows MFMA j + LAG
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  i32x8 qf[NR][NHT];
  float wv[NR][NHT][4];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const uint8_t* qrow = a.q_idx + (int64_t)rows[i] * a.H_I * 128;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      // heads past H_I (H_I a multiple of 4, not of 16) have a zero query and
      // a zero weight: x = 0 and they add nothing
      qf[i][ht] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (16 * ht + li < a.H_I) {
        const i32x4* p = (const i32x4*)(qrow + (16 * ht + li) * 128 + 32 * g);
        i32x4 lo = p[0], hi = p[1];
        qf[i][ht] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      f32x4 wq = f32x4{0.f, 0.f, 0.f, 0.f};
      if (16 * ht + 4 * g < a.H_I) wq = *(const f32x4*)(a.w + (int64_t)rows[i] * a.H_I + 16 * ht + 4 * g);
      wv[i][ht][0] = wq[0]; wv[i][ht][1] = wq[1]; wv[i][ht][2] = wq[2]; wv[i][ht][3] = wq[3];
    }
  }
  // linear-term A fragment: MFMA row li holds term li / 4 of row li % 4
  i32x8 lf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  int lscale = 127;
  if constexpr (LIN) {
    const int i = li & 3, t = li >> 2;
    if (i < NR) {
      const int32_t row = i == 0 ? rows[0] : rows[NR - 1];
      const uint8_t* src = a.lin + (int64_t)(row - a.row_begin) * kLinRowBytes;
      const i32x4* p = (const i32x4*)(src + t * 128 + 32 * g);
      i32x4 lo = p[0], hi = p[1];
      lf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      lscale = src[kLinScaleOff + t * 4 + g];
    }
  }
  // keys: [kbase, kbase + kend) in range, everything past it reads as zero
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_idx + (int64_t)kbase * 128), 0, kend * 128, kBufFlags);
  const int kvo = li * 128 + 32 * g;
  __amdgpu_buffer_rsrc_t srs[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    srs[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.scores + (int64_t)(rows[i] - a.row_begin) * a.ld), 0,
                                               lim[i] * 4, kBufFlags);
  const int svo = (16 * g + li) * 4;
  // per-key scales (SC), straight from memory (plain path): [kbase, kbase + kend)
  // in range, past it reads 0 (those scores are dropped)
  auto load_scales = [&](int32_t s0, int (&ks)[NST]) {
    if constexpr (SC) {
      const __amdgpu_buffer_rsrc_t ksrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_scale + kbase), 0, kend, kBufFlags);
      const int so = __builtin_amdgcn_readfirstlane(s0);
#pragma unroll
      for (int st = 0; st < NST; ++st) ks[st] = __builtin_amdgcn_raw_buffer_load_b8(ksrs, li + 16 * st, so, 0);
    } else {
#pragma unroll
      for (int st = 0; st < NST; ++st) ks[st] = 127;
    }
  };
  // ... and through LDS (ring paths): the copy of slab s0's scales into one
  // scale area, and the read of this lane's four
  auto copy_scales = [&](int32_t s0, DSA_LDS uint8_t* dst) {
    if constexpr (SC)
      __builtin_amdgcn_global_load_lds((const void*)(a.k_scale + kbase + min(s0 + lane, kend - 1)),
                                       (DSA_LDS void*)dst, 1, 0, 0);
  };
  auto read_scales = [&](const DSA_LDS uint8_t* src, int (&ks)[NST]) {
#pragma unroll
    for (int st = 0; st < NST; ++st) ks[st] = SC ? (int)src[4 * (li + 16 * st)] : 127;
  };

  // LDS rings: a 64-key slab is eight 1-KB blocks of eight whole key rows.
  // Block b holds rows 8 b .. 8 b + 7; 16-byte chunk c of its row 8 b + q sits
  // in slot 8 q + (c ^ q ^ (b & 1)).  Copy instruction b of a slab fills block
  // b, every eight lanes one whole 128-byte key row (lane l: row 8 b + l / 8,
  // the chunk its slot l holds), so each instruction touches eight lines.  A
  // fragment read (lane group g: chunks 2 g, 2 g + 1 of rows 16 st + li) has
  // the 16 rows of a lane group on 16 different bank slots: within a block the
  // slots of one chunk are c ^ q, offset by 8 for odd q, and block 2 st + 1
  // flips the low bit, which moves each row to the other parity's free slots.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t* kglob = a.k_idx + (int64_t)kbase * 128;
  const int crow = lane >> 3;                       // copy lane: row within its block
  auto copy_src = [&](int32_t s0, int b) {
    const int c = (lane & 7) ^ crow ^ (b & 1);
    return kglob + (int64_t)min(s0 + 8 * b + crow, kend - 1) * 128 + 16 * c;  // rows past kend: a valid key
  };
  auto copy_slab = [&](int32_t s0, int slot) {
    copy_scales(s0, sarea + slot * 4 * kScaleArea);
    DSA_LDS uint8_t* dst = ring + slot * kSlabBytes;
    __builtin_amdgcn_global_load_lds((const void*)copy_src(s0, wave), (DSA_LDS void*)(dst + 1024 * wave), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)copy_src(s0, wave + 4), (DSA_LDS void*)(dst + 1024 * (wave + 4)),
                                     16, 0, 0);
  };
  // this lane's chunks 2 g (lo) and 2 g + 1 (hi) of row li of sub-tile 0:
  // block li / 8, row q = li % 8; the two slots differ in their low bit
  const int rq = li & 7, rb = li >> 3;
  const int lo_slot = 8 * rq + ((2 * g) ^ rq ^ rb);
  const int ro = rb * 1024 + 16 * lo_slot, rh = rb * 1024 + 16 * (lo_slot ^ 1);
  auto read_keys = [&](int slot, i32x8 (&kf)[NST]) {
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const DSA_LDS uint8_t* base = ring + slot * kSlabBytes + st * 2048;
      const i32x4 lo = *(const DSA_LDS i32x4*)(base + ro);
      const i32x4 hi = *(const DSA_LDS i32x4*)(base + rh);
      kf[st] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  auto load_keys = [&](int32_t s0, i32x8 (&kf)[NST]) {
    const int so = __builtin_amdgcn_readfirstlane(s0 * 128);  // keep the offset scalar
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, kvo + st * 2048, so, 0));
      const i32x4 hi = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, kvo + st * 2048 + 16, so, 0));
      kf[st] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  // One 64-key slab with the keys in kf and their scales in ks.
  auto slab = [&](int32_t s0, i32x8 (&kf)[NST], const int (&ks)[NST]) {
    float acc[NST][NR];
    f32x4 x[LAG + 1];
#pragma unroll
    for (int j = 0; j < NM + LAG; ++j) {
      if (j < NM) {
        const int st = j / NPS, u = j % NPS;
        if (LIN && u == 0) {
          x[j % (LAG + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lf, kf[st], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                              0, 0, 0, lscale, 0, SC ? ks[st] : 127);
        } else {
          const int v = u - (LIN ? 1 : 0), i = v / NHT, ht = v % NHT;
          x[j % (LAG + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[i][ht], kf[st],
                                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127,
                                                                              0, SC ? ks[st] : 127);
        }
      }
      // Order pins (empty volatile asm, kept in program order): MFMA j's result
      // and the one whose epilogue runs now (MFMA j - LAG) pass through the
      // first, the accumulators that epilogue wrote and the keys of MFMA j + 1
      // through the second.  So the epilogue of MFMA j - LAG runs after MFMA j
      // issues and before MFMA j + 1: left alone, the compiler runs each
      // epilogue straight after its own MFMA, and the wave waits out every one.
      if (j < NM) asm volatile("" : "+v"(x[j % (LAG + 1)]));
      if (j >= LAG) asm volatile("" : "+v"(x[(j - LAG) % (LAG + 1)]));
      if (j >= LAG) {
        const int e = j - LAG;
        const int st = e / NPS, u = e % NPS;
        const f32x4 xv = x[e % (LAG + 1)];
        if (LIN && u == 0) {
#pragma unroll
          for (int i = 0; i < NR; ++i) acc[st][i] = xv[i];  // this lane group's term of row i
        } else {
          const int v = u - (LIN ? 1 : 0), i = v / NHT, ht = v % NHT;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (LIN) {
              acc[st][i] = fmaf(wv[i][ht][r], fabsf(xv[r]), acc[st][i]);
            } else {
              const float av = activation<ACT>(xv[r]);
              acc[st][i] = (ht == 0 && r == 0) ? wv[i][ht][r] * av : fmaf(wv[i][ht][r], av, acc[st][i]);
            }
          }
        }
        if (LIN && u == 0) {
#pragma unroll
          for (int i = 0; i < NR; ++i) asm volatile("" : "+v"(acc[st][i]));
        } else {
          asm volatile("" : "+v"(acc[st][(u - (LIN ? 1 : 0)) / NHT]));
        }
      }
      if (j + 1 < NM) asm volatile("" : "+v"(kf[(j + 1) / NPS]));
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      float v = transpose_reduce(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      if constexpr (LIN) v *= 0.5f;
      __builtin_amdgcn_raw_buffer_store_b32(f_bits(v), srs[i], svo, __builtin_amdgcn_readfirstlane(s0 * 4), 0);
    }
  };

  if constexpr (KEYS == kKeysShared) {
    // per slab n: this wave's copies of slab n done (after them it issued the
    // stores of n-2, the copies of n+1 and the stores of n-1), barrier (every
    // wave's copies landed, every wave done reading slab n-1), copy slab n+2
    // into the slot slab n-1 used, read and compute slab n
    // (each wave also copies the slab's scales into its own scale area)
    constexpr int C = SC ? 3 : 2;  // copies per slab and wave
    copy_slab(kstart, 0);
    copy_slab(kstart + 64, 1);
    int slot = 0, n = 0;
    for (int32_t s0 = kstart; s0 < kend; s0 += 64, ++n) {
      if (n == 0) wait_vmcnt<C>();
      else if (n == 1) wait_vmcnt<C + NR>();
      else wait_vmcnt<C + 2 * NR>();
      lds_barrier();
      copy_slab(s0 + 128, slot == 0 ? 2 : slot - 1);
      i32x8 kf[NST];
      int ks[NST];
      read_keys(slot, kf);
      read_scales(sarea + slot * 4 * kScaleArea, ks);
      slab(s0, kf, ks);
      slot = slot == 2 ? 0 : slot + 1;
    }
  } else if constexpr (KEYS == kKeysPrivate) {
    // ring: this wave's kPrivSlots slabs.  Slab n sits in slot n % kPrivSlots;
    // its 8 copies (copy b: block b, eight whole key rows) are issued
    // kPrivSlots - 1 slabs ahead.  Ahead of slab n's wait, this wave issued the
    // copies of slabs n + 1 .. n + kPrivSlots - 2 and the score stores of the
    // (at most kPrivSlots - 1) slabs before n, all counted by vmcnt.
    constexpr int P = kPrivSlots;
    constexpr int C = SC ? 9 : 8;  // copies per slab
    auto copy_own = [&](int32_t s0, int slot) {
      copy_scales(s0, sarea + slot * kScaleArea);
      DSA_LDS uint8_t* dst = ring + slot * kSlabBytes;
#pragma unroll
      for (int b = 0; b < 8; ++b)
        __builtin_amdgcn_global_load_lds((const void*)copy_src(s0, b), (DSA_LDS void*)(dst + 1024 * b), 16, 0, 0);
    };
#pragma unroll
    for (int j = 0; j < P - 1; ++j) copy_own(kstart + 64 * j, j);
    int n = 0;
    for (int32_t s0 = kstart; s0 < kend; s0 += 64, ++n) {
      static_assert(P == 4, "the counted waits below assume four slots");
      if (n == 0) wait_vmcnt<C * (P - 2)>();
      else if (n == 1) wait_vmcnt<C * (P - 2) + NR>();
      else if (n == 2) wait_vmcnt<C * (P - 2) + 2 * NR>();
      else wait_vmcnt<C * (P - 2) + 3 * NR>();
      copy_own(s0 + 64 * (P - 1), (n + P - 1) % P);  // the slot slab n - 1 used, read before this point
      i32x8 kf[NST];
      int ks[NST];
      read_keys(n % P, kf);
      read_scales(sarea + (n % P) * kScaleArea, ks);
      slab(s0, kf, ks);
    }
    wait_vmcnt<0>();  // no copy into LDS outlives the wave
  } else {
    for (int32_t s0 = kstart; s0 < kend; s0 += 64) {
      i32x8 kf[NST];
      int ks[NST];
      load_keys(s0, kf);
      load_scales(s0, ks);
      slab(s0, kf, ks);
    }
  }
}

// Prefill-like batches: workgroups whose eight rows are one sequence's share
// the keys through an LDS ring; workgroups whose rows span two sequences fall
// back to the lean per-wave path.
template <int NHT, int ACT, bool SC>
__global__ __launch_bounds__(kIdxThreads) void indexer_fp8_kernel(IdxArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kSlabBytes + (SC ? kRing * 4 * kScaleArea : 0)];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t rb = a.row_begin + blockIdx.x * kRowsPerBlock;
  const int32_t kstart = blockIdx.y * a.key_chunk;
  const int32_t kchunk_end = kstart + a.key_chunk;
  // the workgroup's rows (wave-uniform values: readfirstlane lets the buffer
  // descriptors built from them live in scalar registers)
  int32_t pos[kRowsPerBlock], kb[kRowsPerBlock];
  bool live[kRowsPerBlock];
  bool same = true;
  int32_t kend_blk = kstart;
  const SeqTable seqs = load_seq_table(a.cu_q, a.cu_k, a.num_seqs);
#pragma unroll
  for (int j = 0; j < kRowsPerBlock; ++j) {
    const int32_t r = rb + j;
    pos[j] = -1;
    kb[j] = 0;
    if (r < a.row_end) {
      const RowInfo ri = locate_row_wave(seqs, a.cu_q, a.cu_k, r);
      pos[j] = __builtin_amdgcn_readfirstlane(ri.pos);
      kb[j] = __builtin_amdgcn_readfirstlane(ri.kbase);
      same = same && kb[j] == kb[0];
    }
    live[j] = pos[j] >= 0 && pos[j] + 1 > a.skip_n && pos[j] >= kstart;
    if (live[j]) kend_blk = max(kend_blk, min(kchunk_end, pos[j] + 1));
  }
  if (kend_blk <= kstart) return;  // nothing to score in this key chunk (uniform over the workgroup)
  if (same) {
    int32_t rows[2], lim[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = wave * kRowsPerWave + i;
      rows[i] = min(rb + j, a.row_end - 1);
      lim[i] = __builtin_amdgcn_readfirstlane(live[j] ? min(kchunk_end, pos[j] + 1) : 0);
    }
    fp8_rows<2, NHT, ACT, kKeysShared, SC>(a, rows, lim, kb[0], kstart, kend_blk, (DSA_LDS uint8_t*)ring,
                                           (DSA_LDS uint8_t*)ring + kRing * kSlabBytes + wave * kScaleArea);
    return;
  }
  // rows of several sequences: each wave on its own
  const int j0 = wave * kRowsPerWave;
  bool v[2];
  int32_t l[2], k[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v[i] = __builtin_amdgcn_readfirstlane((int)live[j0 + i]) != 0;
    l[i] = __builtin_amdgcn_readfirstlane(min(kchunk_end, pos[j0 + i] + 1));
    k[i] = __builtin_amdgcn_readfirstlane(kb[j0 + i]);
  }
  if (v[0] && v[1] && k[0] == k[1]) {
    const int32_t rows[2] = {rb + j0, rb + j0 + 1};
    const int32_t lim[2] = {l[0], l[1]};
    fp8_rows<2, NHT, ACT, kKeysPlain, SC>(a, rows, lim, k[0], kstart, max(l[0], l[1]), nullptr, nullptr);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!v[i]) continue;
      const int32_t r1[1] = {rb + j0 + i};
      const int32_t l1[1] = {l[i]};
      fp8_rows<1, NHT, ACT, kKeysPlain, SC>(a, r1, l1, k[i], kstart, l[i], nullptr, nullptr);
    }
  }
}

// Decode-like batches (fewer than 8 query rows per sequence): one row per
// wave, kStreamRows rows per workgroup.  Every wave streams its row's keys
// through its own LDS ring, so it needs no barrier and returns on its own.
// The path is bound by the key bytes, so the activation is applied per head
// (no linear-term pre-pass).
template <int NHT, int ACT, bool SC>
__global__ __launch_bounds__(kIdxThreads) void indexer_fp8_stream_kernel(IdxArgs a) {
  // kStreamRows x kPrivSlots slabs, then (SC) kStreamRows x kPrivSlots scale areas
  extern __shared__ __attribute__((aligned(16))) uint8_t pring[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const RowInfo ri = locate_row_wave(load_seq_table(a.cu_q, a.cu_k, a.num_seqs), a.cu_q, a.cu_k,
                                     min(a.row_begin + (int32_t)blockIdx.x * kStreamRows + wave, a.row_end - 1));
  const int32_t r = a.row_begin + blockIdx.x * kStreamRows + wave;
  const int32_t pos = __builtin_amdgcn_readfirstlane(ri.pos);
  const int32_t kstart = blockIdx.y * a.key_chunk;
  if (r >= a.row_end || pos < kstart || pos + 1 <= a.skip_n) return;
  const int32_t kend = min(kstart + a.key_chunk, pos + 1);
  const int32_t rows[1] = {r}, lim[1] = {kend};
  fp8_rows<1, NHT, ACT, kKeysPrivate, SC, false>(a, rows, lim, __builtin_amdgcn_readfirstlane(ri.kbase), kstart, kend,
                                             (DSA_LDS uint8_t*)pring + wave * kPrivSlots * kSlabBytes,
                                             (DSA_LDS uint8_t*)pring + kStreamRows * kPrivSlots * kSlabBytes +
                                                 wave * kPrivSlots * kScaleArea);
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
  const bool sc = a.k_scale != nullptr;
  if (act == 0) {
    if (sc) hipLaunchKernelGGL((indexer_fp8_kernel<NHT, 0, true>), grid, dim3(kIdxThreads), 0, s, a);
    else hipLaunchKernelGGL((indexer_fp8_kernel<NHT, 0, false>), grid, dim3(kIdxThreads), 0, s, a);
  } else {
    if (sc) hipLaunchKernelGGL((indexer_fp8_kernel<NHT, 1, true>), grid, dim3(kIdxThreads), 0, s, a);
    else hipLaunchKernelGGL((indexer_fp8_kernel<NHT, 1, false>), grid, dim3(kIdxThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int NHT, int ACT, bool SC>
hipError_t launch_stream_act(const IdxArgs& a, dim3 grid, hipStream_t s) {
  constexpr size_t lds = (size_t)kStreamRows * kPrivSlots * (kSlabBytes + (SC ? kScaleArea : 0));  // 128 (132) KB
  static bool attr_set = false;  // benign race: idempotent attribute call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)indexer_fp8_stream_kernel<NHT, ACT, SC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((indexer_fp8_stream_kernel<NHT, ACT, SC>), grid, dim3(kIdxThreads), lds, s, a);
  return hipGetLastError();
}

template <int NHT>
hipError_t launch_stream(const IdxArgs& a, int act, dim3 grid, hipStream_t s) {
  if (a.k_scale) return act == 0 ? launch_stream_act<NHT, 0, true>(a, grid, s) : launch_stream_act<NHT, 1, true>(a, grid, s);
  return act == 0 ? launch_stream_act<NHT, 0, false>(a, grid, s) : launch_stream_act<NHT, 1, false>(a, grid, s);
}

}  // namespace

size_t indexer_workspace_bytes(int rows, bool fp8, int act) {
  if (!fp8 || act != 0 || rows <= 0) return 0;
  return ((size_t)rows * kLinRowBytes + 255) / 256 * 256;
}

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
  a.lin = (const uint8_t*)L.ws;
  a.lin_out = (uint8_t*)L.ws;
  a.k_scale = L.fp8 ? L.k_scale : nullptr;
  if (L.fp8) {
    // prefill-like batches (sequences of many query rows): workgroups of eight
    // rows share their keys; otherwise every row streams its own
    const bool shared = indexer_prefill_like(L.batch_rows >= 0 ? L.batch_rows : rows, L.b.num_seqs);
    if (!shared) {
      // one workgroup per CU (128 KB of LDS): key chunks that cover the CUs once
      const int64_t row_blocks = (rows + kStreamRows - 1) / kStreamRows;
      int32_t chunk = 8192;
      while (chunk > 256 && row_blocks * ((L.b.max_ctx + chunk - 1) / chunk) < L.num_cus) chunk >>= 1;
      a.key_chunk = chunk;
      dim3 grid((unsigned)row_blocks, (unsigned)((L.b.max_ctx + chunk - 1) / chunk));
      switch ((L.H_I + 15) / 16) {
        case 1: return launch_stream<1>(a, L.act, grid, s);
        case 2: return launch_stream<2>(a, L.act, grid, s);
        case 3: return launch_stream<3>(a, L.act, grid, s);
        case 4: return launch_stream<4>(a, L.act, grid, s);
        default: return hipErrorInvalidValue;
      }
    }
    if (L.act == 0) {
      if (!L.ws) return hipErrorInvalidValue;
      hipLaunchKernelGGL(indexer_lin_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    // key chunk: enough workgroups to cover every CU several times over
    const int64_t row_blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    int32_t chunk = 4096;
    while (chunk > 256 && row_blocks * ((L.b.max_ctx + chunk - 1) / chunk) < 4LL * L.num_cus) chunk >>= 1;
    a.key_chunk = chunk;
    dim3 grid((unsigned)row_blocks, (unsigned)((L.b.max_ctx + chunk - 1) / chunk));
    switch ((L.H_I + 15) / 16) {
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
