// cache_append.hip -- writing new tokens into the key and latent caches.
//
// Blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), section
// "Lightning indexer": the indexer runs in FP8, so each token's indexer key
// k_I is kept as E4M3 codes; section "在MLA下實例化DSA": one latent row per
// token serves every query head.  This kernel takes the keys and latent rows
// of new tokens (a prefill, or one token per sequence in decode) and writes
// them at their rows of the caches:
//   * key part: k_I (fp32 or bf16) rounded to OCP E4M3FN, ties to even,
//     saturating at +-448, NaN -> 0x7F; optionally with a per-token power of
//     two 2^e (the smallest e with max|k_I| <= 448 * 2^e), stored as the E8M0
//     byte 127 + e, which the indexer's scaled MFMA applies for free;
//   * latent part: a plain row copy.
// Both parts stream HBM once (no LDS, one or two 16-byte loads per lane), so
// they share one launch: workgroups [0, key_blocks) quantise keys, the rest
// copy latent rows.
#include <algorithm>

#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte chunks per lane in the latent part

struct AppendArgs {
  const uint8_t* k_new;   // [n, d_I] fp32 or bf16
  uint8_t* k_cache;       // [cache_rows, d_I] E4M3 codes
  uint8_t* k_scale;       // [cache_rows] E8M0, or null
  const uint8_t* kv_new;  // [n, row_bytes]
  uint8_t* kv_cache;      // [cache_rows, row_bytes]
  const int32_t* dst;     // [n] destination rows, or null (row t -> t)
  int64_t n;
  int64_t cache_rows;
  int32_t d_I;
  int32_t row_chunks;     // latent row bytes / 16
  int32_t key_blocks;
};

__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// One E4M3FN code per input (in the byte of its position): the hardware
// conversion rounds to nearest even; saturation, NaN and the sign of results
// that round to zero are settled here so that they do not depend on the
// conversion's clamp and denormal modes.
__device__ __forceinline__ uint32_t e4m3_pack4(const float (&y)[4]) {
  float c[4];
  uint32_t nan = 0, sign = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool isn = y[i] != y[i];
    nan |= (isn ? 0xFFu : 0u) << (8 * i);
    sign |= ((f_bits(y[i]) >> 31) << 7) << (8 * i);
    c[i] = isn ? 0.0f : fminf(fmaxf(y[i], -448.0f), 448.0f);
  }
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], r, true);
  const uint32_t code = ((uint32_t)r & 0x7F7F7F7Fu) | sign;
  return (code & ~nan) | (0x7F7F7F7Fu & nan);
}

// LPR lanes per key row, 8 elements per lane.
template <int LPR, bool BF16, bool SCALED>
__device__ __forceinline__ void append_keys(const AppendArgs& a) {
  const int lane_in_row = threadIdx.x % LPR;
  const int64_t t = (int64_t)blockIdx.x * (kAppendThreads / LPR) + threadIdx.x / LPR;
  if (t >= a.n) return;  // whole row groups leave together
  float x[8];
  if constexpr (BF16) {
    const i32x4 v = *(const i32x4*)(a.k_new + (t * a.d_I + 8 * lane_in_row) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = (uint32_t)v[i];
      x[2 * i] = __builtin_bit_cast(float, u << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, u & 0xFFFF0000u);
    }
  } else {
    const f32x4* p = (const f32x4*)(a.k_new + (t * a.d_I + 8 * lane_in_row) * 4);
    const f32x4 lo = p[0], hi = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = lo[i];
      x[4 + i] = hi[i];
    }
  }
  int e = 0;
  if constexpr (SCALED) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));  // NaN is ignored by fmaxf
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    // amax = f 2^ex with f in [0.5, 1); 448 = 0.875 * 2^9
    if (__builtin_isinf(amax)) {
      e = 127;
    } else if (amax > 0.0f) {
      int ex;
      const float f = frexpf(amax, &ex);
      e = min(127, max(-127, ex - 9 + (f > 0.875f ? 1 : 0)));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ldexpf(x[i], -e);  // exact unless the result is far below E4M3's range
  }
  const float lo4[4] = {x[0], x[1], x[2], x[3]};
  const float hi4[4] = {x[4], x[5], x[6], x[7]};
  const uint32_t c0 = e4m3_pack4(lo4), c1 = e4m3_pack4(hi4);
  const int64_t d = a.dst ? (int64_t)a.dst[t] : t;
  if (d < 0 || d >= a.cache_rows) return;  // outside the cache: not written
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  *(u32x2*)(a.k_cache + d * a.d_I + 8 * lane_in_row) = u32x2{c0, c1};
  if constexpr (SCALED) {
    if (lane_in_row == 0) a.k_scale[d] = (uint8_t)(127 + e);
  }
}

__device__ __forceinline__ void append_latent(const AppendArgs& a, int64_t blk) {
  const int64_t total = a.n * a.row_chunks;
  i32x4 v[kCopyUnroll];
  int64_t dst_off[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t q = (blk * kCopyUnroll + u) * kAppendThreads + threadIdx.x;
    dst_off[u] = -1;
    if (q < total) {
      const int32_t t = (int32_t)(q / a.row_chunks);
      const int32_t c = (int32_t)(q - (int64_t)t * a.row_chunks);
      v[u] = *(const i32x4*)(a.kv_new + q * 16);
      const int64_t d = a.dst ? (int64_t)a.dst[t] : t;
      if (d >= 0 && d < a.cache_rows) dst_off[u] = (d * a.row_chunks + c) * 16;
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    if (dst_off[u] >= 0) *(i32x4*)(a.kv_cache + dst_off[u]) = v[u];
}

template <int LPR, bool BF16, bool SCALED>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(AppendArgs a) {
  if ((int32_t)blockIdx.x < a.key_blocks) append_keys<LPR, BF16, SCALED>(a);
  else append_latent(a, (int64_t)blockIdx.x - a.key_blocks);
}

template <int LPR>
hipError_t launch_lpr(const AppendArgs& a, bool bf16, bool scaled, unsigned grid, hipStream_t s) {
  if (bf16) {
    if (scaled) hipLaunchKernelGGL((cache_append_kernel<LPR, true, true>), dim3(grid), dim3(kAppendThreads), 0, s, a);
    else hipLaunchKernelGGL((cache_append_kernel<LPR, true, false>), dim3(grid), dim3(kAppendThreads), 0, s, a);
  } else {
    if (scaled) hipLaunchKernelGGL((cache_append_kernel<LPR, false, true>), dim3(grid), dim3(kAppendThreads), 0, s, a);
    else hipLaunchKernelGGL((cache_append_kernel<LPR, false, false>), dim3(grid), dim3(kAppendThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

namespace {
// dst row r (out_stride bytes) = the first copy_bytes of src row r (in_stride
// bytes), zero-filled up to out_stride; every size a multiple of 16.  One
// thread per 16-byte chunk of the output, grid-stride.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint8_t* __restrict__ src, int64_t in_stride,
                                                       uint8_t* __restrict__ dst, int64_t out_stride, int64_t rows,
                                                       int64_t copy_bytes) {
  const int64_t per_row = out_stride / 16, total = rows * per_row;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / per_row, c = e - r * per_row;
    i32x4 v = i32x4{0, 0, 0, 0};
    if (16 * c < copy_bytes) v = *(const i32x4*)(src + r * in_stride + 16 * c);
    *(i32x4*)(dst + r * out_stride + 16 * c) = v;
  }
}
}  // namespace

hipError_t launch_copy_rows(const void* src, int64_t in_stride, void* dst, int64_t out_stride, int64_t rows,
                            int64_t copy_bytes, int num_cus, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((in_stride | out_stride | copy_bytes) % 16 != 0 || copy_bytes > in_stride) return hipErrorInvalidValue;
  const int64_t total = rows * (out_stride / 16);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8LL * num_cus);
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)src, in_stride,
                     (uint8_t*)dst, out_stride, rows, copy_bytes);
  return hipGetLastError();
}

hipError_t launch_cache_append(const AppendLaunch& L, hipStream_t s) {
  if (L.n <= 0) return hipSuccess;
  AppendArgs a;
  a.k_new = (const uint8_t*)L.k_new;
  a.k_cache = L.k_cache;
  a.k_scale = L.k_scale;
  a.kv_new = (const uint8_t*)L.kv_new;
  a.kv_cache = (uint8_t*)L.kv_cache;
  a.dst = L.dst;
  a.n = L.n;
  a.cache_rows = L.cache_rows;
  a.d_I = L.d_I;
  a.row_chunks = L.kv_new ? (int32_t)(L.kv_row_bytes / 16) : 0;
  const int lpr = L.k_new ? L.d_I / 8 : 8;
  const int64_t key_blocks = L.k_new ? (L.n + kAppendThreads / lpr - 1) / (kAppendThreads / lpr) : 0;
  const int64_t copy_blocks =
      L.kv_new ? (L.n * a.row_chunks + kCopyUnroll * kAppendThreads - 1) / (kCopyUnroll * kAppendThreads) : 0;
  if (key_blocks + copy_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  a.key_blocks = (int32_t)key_blocks;
  const unsigned grid = (unsigned)(key_blocks + copy_blocks);
  switch (lpr) {
    case 8: return launch_lpr<8>(a, L.k_bf16, L.k_scale != nullptr, grid, s);
    case 16: return launch_lpr<16>(a, L.k_bf16, L.k_scale != nullptr, grid, s);
    case 32: return launch_lpr<32>(a, L.k_bf16, L.k_scale != nullptr, grid, s);
    case 64: return launch_lpr<64>(a, L.k_bf16, L.k_scale != nullptr, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsa
