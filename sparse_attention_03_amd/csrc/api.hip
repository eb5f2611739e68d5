// api.hip -- the libdsa C interface: host-side argument checks, workspace
// layout and kernel launches.  Every check runs before the first HIP call, so
// invalid calls never touch the device (and work without one).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/libdsa.h"
#include "dsa_kernels.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dsa_status hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];
std::once_flag g_once[kMaxDevices];

dsa_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev] = n;
  });
  *cus = g_cus[dev];
  return DSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

dsa_status check_batch(const dsa_batch* b) {
  if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is NULL");
  if (b->num_seqs < 1) return fail(DSA_ERR_INVALID_ARG, "num_seqs = %d, need >= 1", b->num_seqs);
  if (!b->cu_q || !b->cu_k) return fail(DSA_ERR_INVALID_ARG, "cu_q / cu_k is NULL");
  if (b->total_q < 0) return fail(DSA_ERR_INVALID_ARG, "total_q = %d < 0", b->total_q);
  if (b->total_k < 1) return fail(DSA_ERR_INVALID_ARG, "total_k = %d, need >= 1", b->total_k);
  if (b->max_ctx < 1 || b->max_ctx > b->total_k)
    return fail(DSA_ERR_INVALID_ARG, "max_ctx = %d outside [1, total_k = %d]", b->max_ctx, b->total_k);
  if (b->total_q > b->total_k) return fail(DSA_ERR_INVALID_ARG, "total_q %d > total_k %d", b->total_q, b->total_k);
  return DSA_OK;
}

dsa::BatchView view(const dsa_batch* b, int32_t r0, int32_t r1) {
  return dsa::BatchView{b->cu_q, b->cu_k, b->num_seqs, r0, r1, b->max_ctx};
}

dsa_status check_indexer(const dsa_batch* b, const void* q_idx, const void* k_idx, dsa_dtype dt, const float* w,
                         int32_t H_I, int32_t d_I, dsa_act act) {
  if (!q_idx || !k_idx || !w) return fail(DSA_ERR_INVALID_ARG, "indexer input pointer is NULL");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w))
    return fail(DSA_ERR_INVALID_ARG, "indexer inputs must be 16-byte aligned");
  if (act != DSA_ACT_RELU && act != DSA_ACT_GELU) return fail(DSA_ERR_INVALID_ARG, "unknown activation %d", (int)act);
  if (H_I < 1 || d_I < 1) return fail(DSA_ERR_INVALID_ARG, "H_I = %d, d_I = %d", H_I, d_I);
  if (dt == DSA_FP8_E4M3) {
    if (d_I % 16 != 0 || d_I > 128)
      return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer needs d_I a multiple of 16, <= 128 (got %d)", d_I);
    if (H_I % 4 != 0 || H_I > 64) return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer needs H_I a multiple of 4, <= 64 (got %d)", H_I);
    if (b->max_ctx > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer needs max_ctx <= 2^24 (got %d)", b->max_ctx);
  } else if (dt == DSA_F32) {
    if (d_I > 256 || H_I > 64 || H_I * d_I > 8192)
      return fail(DSA_ERR_UNSUPPORTED, "F32 indexer needs d_I <= 256, H_I <= 64, H_I * d_I <= 8192");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype must be FP8_E4M3 or F32");
  }
  return DSA_OK;
}

// FP8 indexer inputs with d_I < 128 are widened to 128-byte rows (zero-filled)
// in the workspace: q_I rows of `q_rows` query rows, then the k_I rows.
size_t fp8_pad_q_bytes(int64_t q_rows, int32_t H_I, int32_t d_I, bool fp8) {
  return fp8 && d_I < 128 ? round_up((size_t)q_rows * (size_t)H_I * 128, 256) : 0;
}
size_t fp8_pad_k_bytes(int64_t k_rows, int32_t d_I, bool fp8) {
  return fp8 && d_I < 128 ? round_up((size_t)k_rows * 128, 256) : 0;
}

dsa_status check_scores(const dsa_batch* b, const void* scores, int64_t ld) {
  if (!scores) return fail(DSA_ERR_INVALID_ARG, "scores is NULL");
  if (!aligned16(scores)) return fail(DSA_ERR_INVALID_ARG, "scores must be 16-byte aligned");
  if (ld < b->max_ctx || ld % 4 != 0)
    return fail(DSA_ERR_INVALID_ARG, "ld_scores = %lld must be >= max_ctx (%d) and a multiple of 4", (long long)ld,
                b->max_ctx);
  return DSA_OK;
}

dsa_status check_k(int32_t k) {
  if (k < 1 || k > 2048) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside [1, 2048]", k);
  return DSA_OK;
}

dsa_status check_attention(const void* q, const void* kv, dsa_dtype dt, const int32_t* idx, int32_t k, int32_t H,
                           int32_t d_qk, int32_t d_v, float scale, const void* out, const float* lse) {
  if (!q || !kv || !idx || !out) return fail(DSA_ERR_INVALID_ARG, "attention pointer is NULL");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || !aligned16(idx))
    return fail(DSA_ERR_INVALID_ARG, "attention buffers must be 16-byte aligned");
  (void)lse;
  if (dsa_status s = check_k(k)) return s;
  if (!(scale == scale)) return fail(DSA_ERR_INVALID_ARG, "softmax_scale is NaN");
  if (H < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk) return fail(DSA_ERR_INVALID_ARG, "bad H / d_qk / d_v");
  if (dt == DSA_BF16) {
    if (d_qk % 16 != 0 || d_qk > 576 || d_v % 16 != 0 || d_v > 512)
      return fail(DSA_ERR_UNSUPPORTED, "BF16 attention needs d_qk and d_v multiples of 16, d_qk <= 576, d_v <= 512");
    if (H % 8 != 0 || H > 128) return fail(DSA_ERR_UNSUPPORTED, "BF16 attention needs H a multiple of 8, <= 128");
  } else if (dt == DSA_F32) {
    if (d_qk > 1024 || H > 128) return fail(DSA_ERR_UNSUPPORTED, "F32 attention needs d_qk <= 1024, H <= 128");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "attention dtype must be BF16 or F32");
  }
  return DSA_OK;
}

// BF16 shapes other than d_qk = 576, d_v = 512 run the 576 / 512 kernels on
// widened copies in the workspace: q and kv rows widened to 576 columns with
// zeros (which add nothing to q . kv), and the output staged at 512 value
// columns, of which the first d_v are kept (the value is the first d_v columns
// of kv either way).
constexpr int64_t kQkW = 576, kVW = 512;  // the kernels' widths
struct AttnWiden {
  bool in;   // d_qk < 576: q and kv widened
  bool out;  // d_v < 512: output staged
  int32_t d_qk, d_v;  // the widths the kernels run
};
AttnWiden attn_widen(dsa_dtype dt, int32_t d_qk, int32_t d_v) {
  const bool in = dt == DSA_BF16 && d_qk != kQkW, out = dt == DSA_BF16 && d_v != kVW;
  return AttnWiden{in, out, in ? (int32_t)kQkW : d_qk, out ? (int32_t)kVW : d_v};
}
size_t widen_q_bytes(int64_t rows, int32_t H, const AttnWiden& w) {
  return w.in ? round_up((size_t)rows * H * kQkW * 2, 256) : 0;
}
size_t widen_kv_bytes(int64_t total_k, const AttnWiden& w) {
  return w.in ? round_up((size_t)total_k * kQkW * 2, 256) : 0;
}
size_t stage_out_bytes(int64_t rows, int32_t H, const AttnWiden& w) {
  return w.out ? round_up((size_t)rows * H * kVW * 2, 256) : 0;
}

// key-split partials: bf16 outputs [rows, splits, H, d_v], then fp32 lse
// [rows, splits, H]
size_t partial_o_bytes(int32_t rows, int splits, int32_t H, int32_t d_v) {
  return round_up((size_t)rows * splits * H * d_v * sizeof(uint16_t), 256);
}
size_t attention_ws_bytes(int32_t rows, int splits, int32_t H, int32_t d_v) {
  if (splits <= 1) return 0;
  return partial_o_bytes(rows, splits, H, d_v) + round_up((size_t)rows * splits * H * sizeof(float), 256);
}

}  // namespace

namespace dsa {
// The error reporting of the C interface for the library's other sources.
dsa_status report_error(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}
}  // namespace dsa

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_err; }

const char* dsa_version(void) { return "libdsa 0.1 gfx950"; }

dsa_status dsa_indexer_workspace_size(const dsa_batch* batch, dsa_dtype idx_dtype, int32_t H_I, int32_t d_I,
                                      dsa_act act, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (dsa_status s = check_batch(batch)) return s;
  static const uint8_t kDummy[16] __attribute__((aligned(16))) = {};
  if (dsa_status s = check_indexer(batch, kDummy, kDummy, idx_dtype, (const float*)kDummy, H_I, d_I, act)) return s;
  const bool fp8 = idx_dtype == DSA_FP8_E4M3;
  *bytes = round_up(dsa::indexer_workspace_bytes(batch->total_q, fp8, (int)act), 256) +
           fp8_pad_q_bytes(batch->total_q, H_I, d_I, fp8) + fp8_pad_k_bytes(batch->total_k, d_I, fp8);
  return DSA_OK;
}

dsa_status dsa_indexer_scores(const dsa_batch* batch, const void* q_idx, const void* k_idx, dsa_dtype idx_dtype,
                              const uint8_t* k_idx_scale, const float* w, int32_t H_I, int32_t d_I, dsa_act act,
                              float* scores, int64_t ld_scores, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_indexer(batch, q_idx, k_idx, idx_dtype, w, H_I, d_I, act)) return s;
  if (k_idx_scale && idx_dtype != DSA_FP8_E4M3) return fail(DSA_ERR_INVALID_ARG, "k_idx_scale needs FP8 keys");
  if (dsa_status s = check_scores(batch, scores, ld_scores)) return s;
  const bool fp8 = idx_dtype == DSA_FP8_E4M3;
  const size_t lin = dsa::indexer_workspace_bytes(batch->total_q, fp8, (int)act);
  const size_t pad_q = fp8_pad_q_bytes(batch->total_q, H_I, d_I, fp8);
  const size_t need = round_up(lin, 256) + pad_q + fp8_pad_k_bytes(batch->total_k, d_I, fp8);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(DSA_ERR_WORKSPACE, "indexer workspace: need %zu bytes (got %zu)", need, ws_bytes);
  if (batch->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  hipStream_t st = (hipStream_t)stream;
  if (pad_q) {  // FP8 with d_I < 128: the kernels read 128-byte rows, zero-filled past d_I
    char* pq = (char*)ws + round_up(lin, 256);
    char* pk = pq + pad_q;
    hipError_t e = dsa::launch_copy_rows(q_idx, d_I, pq, 128, (int64_t)batch->total_q * H_I, d_I, cus, st);
    if (e == hipSuccess) e = dsa::launch_copy_rows(k_idx, d_I, pk, 128, batch->total_k, d_I, cus, st);
    if (e != hipSuccess) return hip_fail(e, "indexer input widening");
    q_idx = pq;
    k_idx = pk;
    d_I = 128;
  }
  dsa::IndexerLaunch L{view(batch, 0, batch->total_q), 0, q_idx, k_idx, w, scores, ld_scores, H_I, d_I, (int32_t)act,
                       fp8, cus, lin > 0 ? ws : nullptr};
  L.k_scale = k_idx_scale;
  hipError_t e = dsa::launch_indexer(L, st);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer launch");
}

dsa_status dsa_topk_workspace_size(const dsa_batch* batch, int32_t k, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_k(k)) return s;
  if (!dsa::topk_may_segment(batch->max_ctx, k)) {
    *bytes = 0;
    return DSA_OK;
  }
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  *bytes = dsa::topk_workspace_bytes(batch->total_q, batch->max_ctx, k, cus);
  return DSA_OK;
}

dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores, int32_t k, int32_t* idx,
                    void* ws, size_t ws_bytes, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_scores(batch, scores, ld_scores)) return s;
  if (dsa_status s = check_k(k)) return s;
  if (!idx || !aligned16(idx)) return fail(DSA_ERR_INVALID_ARG, "idx is NULL or not 16-byte aligned");
  if (batch->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  const size_t need = dsa::topk_workspace_bytes(batch->total_q, batch->max_ctx, k, cus);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace: need %zu bytes (got %zu)", need, ws_bytes);
  dsa::TopkLaunch L{view(batch, 0, batch->total_q), scores, ld_scores, k, idx, ws, cus};
  hipError_t e = dsa::launch_topk(L, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "topk launch");
}

dsa_status dsa_sparse_mla_attn_workspace_size(const dsa_batch* batch, dsa_dtype dtype, int32_t H, int32_t k,
                                              int32_t d_qk, int32_t d_v, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_k(k)) return s;
  if (H < 1 || d_qk < 1 || d_v < 1) return fail(DSA_ERR_INVALID_ARG, "bad H / d_qk / d_v");
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  const AttnWiden w = attn_widen(dtype, d_qk, d_v);
  const int splits = dsa::attention_splits(batch->total_q, k, dtype == DSA_BF16, cus);
  *bytes = round_up(attention_ws_bytes(batch->total_q, splits, H, w.d_v), 256) +
           widen_q_bytes(batch->total_q, H, w) + widen_kv_bytes(batch->total_k, w) +
           stage_out_bytes(batch->total_q, H, w);
  return DSA_OK;
}

// One attention launch over the whole batch (sparse or dense), with the
// widening of other BF16 shapes around it.
dsa_status run_attention(const dsa_batch* batch, dsa::AttnLaunch L, int32_t d_qk, int32_t d_v, dsa_dtype dtype,
                         void* ws, size_t ws_bytes, int cus, hipStream_t st, const char* what) {
  const int32_t rows = batch->total_q, H = L.H;
  const AttnWiden w = attn_widen(dtype, d_qk, d_v);
  const size_t part = round_up(attention_ws_bytes(rows, L.splits, H, w.d_v), 256);
  const size_t wq = widen_q_bytes(rows, H, w), wkv = widen_kv_bytes(batch->total_k, w);
  const size_t need = part + wq + wkv + stage_out_bytes(rows, H, w);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(DSA_ERR_WORKSPACE, "%s workspace: need %zu bytes (got %zu)", what, need, ws_bytes);
  char* base = (char*)ws;
  if (L.splits > 1) {
    L.ws_o = (uint16_t*)base;
    L.ws_lse = (float*)(base + partial_o_bytes(rows, L.splits, H, w.d_v));
  }
  if (w.in) {
    hipError_t e = dsa::launch_copy_rows(L.q, 2 * d_qk, base + part, 2 * kQkW, (int64_t)rows * H, 2 * d_qk, cus, st);
    if (e == hipSuccess)
      e = dsa::launch_copy_rows(L.kv, 2 * d_qk, base + part + wq, 2 * kQkW, batch->total_k, 2 * d_qk, cus, st);
    if (e != hipSuccess) return hip_fail(e, "attention input widening");
    L.q = base + part;
    L.kv = base + part + wq;
  }
  void* out = L.out;
  if (w.out) L.out = base + part + wq + wkv;
  L.d_qk = w.d_qk;
  L.d_v = w.d_v;
  hipError_t e = dsa::launch_attention(L, st);
  if (e != hipSuccess) return hip_fail(e, what);
  if (w.out) {
    e = dsa::launch_copy_rows(L.out, 2 * kVW, out, 2 * d_v, (int64_t)rows * H, 2 * d_v, cus, st);
    if (e != hipSuccess) return hip_fail(e, "attention output narrowing");
  }
  return DSA_OK;
}

dsa_status dsa_sparse_mla_attn(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype,
                               const int32_t* idx, int32_t k, int32_t H, int32_t d_qk, int32_t d_v,
                               float softmax_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                               dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_attention(q, kv, dtype, idx, k, H, d_qk, d_v, softmax_scale, out, lse)) return s;
  if (batch->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  const int splits = dsa::attention_splits(batch->total_q, k, dtype == DSA_BF16, cus);
  dsa::AttnLaunch L{view(batch, 0, batch->total_q), q, kv, idx, k, H, d_qk, d_v, softmax_scale, out, lse,
                    dtype == DSA_BF16, splits, nullptr, nullptr};
  return run_attention(batch, L, d_qk, d_v, dtype, ws, ws_bytes, cus, (hipStream_t)stream, "attention");
}

dsa_status dsa_dense_mla_attn_workspace_size(const dsa_batch* batch, dsa_dtype dtype, int32_t H, int32_t d_qk,
                                             int32_t d_v, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (dsa_status s = check_batch(batch)) return s;
  if (H < 1 || d_qk < 1 || d_v < 1) return fail(DSA_ERR_INVALID_ARG, "bad H / d_qk / d_v");
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  const AttnWiden w = attn_widen(dtype, d_qk, d_v);
  const int splits = dsa::attention_splits(batch->total_q, batch->max_ctx, dtype == DSA_BF16, cus);
  *bytes = round_up(attention_ws_bytes(batch->total_q, splits, H, w.d_v), 256) +
           widen_q_bytes(batch->total_q, H, w) + widen_kv_bytes(batch->total_k, w) +
           stage_out_bytes(batch->total_q, H, w);
  return DSA_OK;
}

dsa_status dsa_dense_mla_attn(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype, int32_t H,
                              int32_t d_qk, int32_t d_v, float softmax_scale, void* out, float* lse, void* ws,
                              size_t ws_bytes, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  // the same checks as the sparse call, with a stand-in index pointer and k
  static const int32_t no_idx[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  if (dsa_status s = check_attention(q, kv, dtype, no_idx, 1, H, d_qk, d_v, softmax_scale, out, lse)) return s;
  if (dtype == DSA_F32 && (int64_t)batch->max_ctx + d_qk + 8 > 16384)
    return fail(DSA_ERR_UNSUPPORTED, "F32 dense attention needs max_ctx + d_qk <= 16376");
  if (batch->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  const int splits = dsa::attention_splits(batch->total_q, batch->max_ctx, dtype == DSA_BF16, cus);
  dsa::AttnLaunch L{view(batch, 0, batch->total_q), q, kv, nullptr, batch->max_ctx, H, d_qk, d_v, softmax_scale,
                    out, lse, dtype == DSA_BF16, splits, nullptr, nullptr};
  L.dense = true;
  return run_attention(batch, L, d_qk, d_v, dtype, ws, ws_bytes, cus, (hipStream_t)stream, "dense attention");
}

dsa_status dsa_sparse_mla_backward_workspace_size(const dsa_batch* batch, int32_t H, int32_t k, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_k(k)) return s;
  if (H != 32 && H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "backward needs H in {32, 64, 128}");
  *bytes = dsa::mla_backward_workspace_bytes(batch->total_q, H, k);
  return DSA_OK;
}

dsa_status dsa_sparse_mla_backward(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype,
                                   const int32_t* idx, int32_t k, int32_t H, int32_t d_qk, int32_t d_v,
                                   float softmax_scale, const float* lse, const void* dout, float* dq, float* dkv,
                                   void* ws, size_t ws_bytes, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_attention(q, kv, dtype, idx, k, H, d_qk, d_v, softmax_scale, dq, lse)) return s;
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "attention backward needs BF16");
  if (d_qk != 576 || d_v != 512) return fail(DSA_ERR_UNSUPPORTED, "attention backward needs d_qk = 576, d_v = 512");
  if (H != 32 && H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "attention backward needs H in {32, 64, 128}");
  if (!lse || !dout || !dq || !dkv) return fail(DSA_ERR_INVALID_ARG, "lse / dout / dq / dkv is NULL");
  if (!aligned16(dout) || !aligned16(dkv)) return fail(DSA_ERR_INVALID_ARG, "dout and dkv must be 16-byte aligned");
  if (batch->total_q == 0) return DSA_OK;
  const size_t need = dsa::mla_backward_workspace_bytes(batch->total_q, H, k);
  if (!ws || ws_bytes < need || !aligned16(ws))
    return fail(DSA_ERR_WORKSPACE, "attention backward workspace: need %zu bytes (got %zu)", need, ws_bytes);
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  dsa::MlaBwdLaunch L{view(batch, 0, batch->total_q), q, kv, idx, k, H, softmax_scale, lse, dout, dq, dkv, ws, cus};
  hipError_t e = dsa::launch_mla_backward(L, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "attention backward launch");
}

dsa_status dsa_attn_target(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype,
                           const int32_t* idx, int32_t k, int32_t H, int32_t d_qk, float softmax_scale,
                           const float* lse, float* p, int64_t ld_p, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  static const int32_t no_idx[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  const bool dense = idx == nullptr;
  // the attention's checks (d_v is the value width; the target has none: pass a valid one)
  const int32_t d_v = dtype == DSA_BF16 ? 512 : d_qk;
  if (dsa_status s = check_attention(q, kv, dtype, dense ? no_idx : idx, dense ? 1 : k, H, d_qk, d_v, softmax_scale,
                                     p, lse))
    return s;
  if (!lse || !p) return fail(DSA_ERR_INVALID_ARG, "lse / p is NULL");
  if (dtype == DSA_BF16 && d_qk != 576) return fail(DSA_ERR_UNSUPPORTED, "BF16 target needs d_qk = 576");
  const int64_t m = dense ? batch->max_ctx : k;
  if (ld_p < (m + 31) / 32 * 32 || ld_p % 4 != 0)
    return fail(DSA_ERR_INVALID_ARG, "ld_p = %lld must be >= %lld (whole 32-entry tiles) and a multiple of 4",
                (long long)ld_p, (long long)((m + 31) / 32 * 32));
  if (dtype == DSA_F32 && m + d_qk > 16384) return fail(DSA_ERR_UNSUPPORTED, "F32 target needs m + d_qk <= 16384");
  if (batch->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  dsa::AttnLaunch L{view(batch, 0, batch->total_q), q, kv, idx, dense ? batch->max_ctx : k, H, d_qk, d_v,
                    softmax_scale, nullptr, nullptr, dtype == DSA_BF16, 1, nullptr, nullptr};
  L.splits = dsa::attention_splits(batch->total_q, L.k, dtype == DSA_BF16, cus);
  L.dense = dense;
  L.target = true;
  L.lse_in = lse;
  L.p_out = p;
  L.ld_p = ld_p;
  hipError_t e = dsa::launch_attention(L, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "target launch");
}

dsa_status dsa_indexer_kl(const dsa_batch* batch, const float* scores, int64_t ld_scores, const int32_t* idx,
                          int32_t k, const float* p, int64_t ld_p, float* loss, float* dI, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_scores(batch, scores, ld_scores)) return s;
  if (!p || !aligned16(p) || (dI && !aligned16(dI))) return fail(DSA_ERR_INVALID_ARG, "p / dI NULL or misaligned");
  const int64_t m = idx ? k : batch->max_ctx;
  if (idx && (k < 1 || !aligned16(idx))) return fail(DSA_ERR_INVALID_ARG, "idx misaligned or k < 1");
  if (ld_p < m) return fail(DSA_ERR_INVALID_ARG, "ld_p = %lld < %lld", (long long)ld_p, (long long)m);
  if (batch->total_q == 0) return DSA_OK;
  dsa::KlLaunch L{view(batch, 0, batch->total_q), scores, ld_scores, idx, k, p, ld_p, loss, dI};
  hipError_t e = dsa::launch_indexer_kl(L, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer kl launch");
}

dsa_status dsa_indexer_backward(const dsa_batch* batch, const void* q_idx, const void* k_idx, dsa_dtype idx_dtype,
                                const uint8_t* k_idx_scale, const float* w, int32_t H_I, int32_t d_I, dsa_act act,
                                const int32_t* idx, int32_t k, const float* g, int64_t ld_g, float* dq_idx,
                                float* dw, float* dk_idx, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_batch(batch)) return s;
  if (dsa_status s = check_indexer(batch, q_idx, k_idx, idx_dtype, w, H_I, d_I, act)) return s;
  if (idx_dtype != DSA_FP8_E4M3) return fail(DSA_ERR_UNSUPPORTED, "indexer backward needs FP8 inputs");
  if (d_I != 128) return fail(DSA_ERR_UNSUPPORTED, "indexer backward needs d_I = 128 (got %d)", d_I);
  if (!g || !dq_idx || !dw || !dk_idx) return fail(DSA_ERR_INVALID_ARG, "g / dq_idx / dw / dk_idx is NULL");
  if (!aligned16(g) || !aligned16(dq_idx) || !aligned16(dw) || !aligned16(dk_idx))
    return fail(DSA_ERR_INVALID_ARG, "g and the gradients must be 16-byte aligned");
  if (idx && (k < 1 || !aligned16(idx))) return fail(DSA_ERR_INVALID_ARG, "idx misaligned or k < 1");
  const int64_t m = idx ? k : batch->max_ctx;
  if (ld_g < m) return fail(DSA_ERR_INVALID_ARG, "ld_g = %lld < %lld", (long long)ld_g, (long long)m);
  if (batch->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  dsa::IndexerBwdLaunch L{view(batch, 0, batch->total_q), q_idx, k_idx, k_idx_scale, w, H_I, (int32_t)act, idx, k,
                          g, ld_g, dq_idx, dw, dk_idx, cus};
  hipError_t e = dsa::launch_indexer_bwd(L, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "indexer backward launch");
}

dsa_status dsa_cache_append(int64_t n, const int32_t* dst_rows, int64_t cache_rows, const void* k_new,
                            dsa_dtype k_dtype, int32_t d_I, uint8_t* k_cache, uint8_t* k_scale, const void* kv_new,
                            dsa_dtype kv_dtype, int32_t d_qk, void* kv_cache, dsa_stream_t stream) {
  g_err[0] = 0;
  if (n < 0 || cache_rows < 0) return fail(DSA_ERR_INVALID_ARG, "n = %lld, cache_rows = %lld", (long long)n,
                                          (long long)cache_rows);
  dsa::AppendLaunch L{};
  L.n = n;
  L.dst = dst_rows;
  L.cache_rows = cache_rows;
  if (k_new) {
    if (k_dtype != DSA_F32 && k_dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "k_new must be F32 or BF16");
    if (d_I != 64 && d_I != 128 && d_I != 256 && d_I != 512)
      return fail(DSA_ERR_UNSUPPORTED, "d_I = %d not in {64, 128, 256, 512}", d_I);
    if (!k_cache) return fail(DSA_ERR_INVALID_ARG, "k_cache is NULL");
    if (!aligned16(k_new) || (reinterpret_cast<uintptr_t>(k_cache) & 7u))
      return fail(DSA_ERR_INVALID_ARG, "k_new must be 16-byte and k_cache 8-byte aligned");
    L.k_new = k_new;
    L.k_bf16 = k_dtype == DSA_BF16;
    L.d_I = d_I;
    L.k_cache = k_cache;
    L.k_scale = k_scale;
  } else if (k_scale) {
    return fail(DSA_ERR_INVALID_ARG, "k_scale without k_new");
  }
  if (kv_new) {
    if (kv_dtype != DSA_F32 && kv_dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "kv_new must be F32 or BF16");
    const int64_t row_bytes = (int64_t)d_qk * (kv_dtype == DSA_F32 ? 4 : 2);
    if (d_qk < 1 || row_bytes % 16) return fail(DSA_ERR_INVALID_ARG, "latent row of %lld bytes is not a multiple of 16",
                                                (long long)row_bytes);
    if (!kv_cache || !aligned16(kv_new) || !aligned16(kv_cache))
      return fail(DSA_ERR_INVALID_ARG, "kv_new / kv_cache NULL or not 16-byte aligned");
    if (n * (row_bytes / 16) >= (1LL << 31)) return fail(DSA_ERR_UNSUPPORTED, "latent part too large for one call");
    L.kv_new = kv_new;
    L.kv_cache = kv_cache;
    L.kv_row_bytes = row_bytes;
  }
  if (n == 0 || (!k_new && !kv_new)) return DSA_OK;
  hipError_t e = dsa::launch_cache_append(L, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "cache append launch");
}

}  // extern "C"

namespace {

struct ForwardPlan {
  int32_t qb;       // rows per chunk
  int64_t ld;       // score row stride
  size_t off_scores, off_idx, off_topk, off_attn, off_lin, off_pad_q, off_pad_k, off_wq, off_wkv, off_stage, total;
  bool pad;         // FP8 with d_I < 128: q_I (per chunk) and k_I widened to 128-byte rows
  AttnWiden w;      // BF16 attention shapes other than 576 / 512: q (per chunk), kv, output staging
  int max_splits;
};

dsa_status check_forward(const dsa_forward_params* p) {
  if (!p) return fail(DSA_ERR_INVALID_ARG, "params is NULL");
  if (dsa_status s = check_batch(p->batch)) return s;
  if (dsa_status s = check_indexer(p->batch, p->q_idx, p->k_idx, p->idx_dtype, p->w, p->H_I, p->d_I, p->act)) return s;
  if (p->k_idx_scale && p->idx_dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_INVALID_ARG, "k_idx_scale needs FP8 keys");
  if (p->q_block < 0) return fail(DSA_ERR_INVALID_ARG, "q_block = %d < 0", p->q_block);
  if (p->out_idx && !aligned16(p->out_idx)) return fail(DSA_ERR_INVALID_ARG, "out_idx must be 16-byte aligned");
  // idx pointer is internal (workspace or out_idx); check the rest with a placeholder
  static const int32_t kDummy[4] = {0, 0, 0, 0};
  return check_attention(p->q, p->kv, p->dtype, kDummy, p->k, p->H, p->d_qk, p->d_v, p->softmax_scale, p->out,
                         p->lse);
}

dsa_status plan_forward(const dsa_forward_params* p, int cus, ForwardPlan* f) {
  const dsa_batch* b = p->batch;
  f->qb = p->q_block > 0 ? p->q_block : 4096;
  if (f->qb > b->total_q) f->qb = b->total_q > 0 ? b->total_q : 1;
  f->ld = (int64_t)round_up((size_t)b->max_ctx, 64);
  size_t off = 0;
  f->off_scores = off;
  off += round_up((size_t)f->qb * (size_t)f->ld * sizeof(float), 256);
  f->off_idx = off;
  if (!p->out_idx) off += round_up((size_t)f->qb * p->k * sizeof(int32_t), 256);
  f->off_topk = off;
  {
    const int32_t last_rows = b->total_q % f->qb;
    const size_t t_full = dsa::topk_workspace_bytes(f->qb, b->max_ctx, p->k, cus);
    const size_t t_last = last_rows ? dsa::topk_workspace_bytes(last_rows, b->max_ctx, p->k, cus) : 0;
    off += round_up(t_full > t_last ? t_full : t_last, 256);
  }
  f->off_attn = off;
  const int32_t last = b->total_q % f->qb;
  const int s_full = dsa::attention_splits(f->qb, p->k, p->dtype == DSA_BF16, cus);
  const int s_last = last ? dsa::attention_splits(last, p->k, p->dtype == DSA_BF16, cus) : 1;
  f->w = attn_widen(p->dtype, p->d_qk, p->d_v);
  const size_t a_full = attention_ws_bytes(f->qb, s_full, p->H, f->w.d_v);
  const size_t a_last = last ? attention_ws_bytes(last, s_last, p->H, f->w.d_v) : 0;
  off += round_up(a_full > a_last ? a_full : a_last, 256);
  f->max_splits = s_full > s_last ? s_full : s_last;
  f->off_lin = off;
  const bool fp8 = p->idx_dtype == DSA_FP8_E4M3;
  off += round_up(dsa::indexer_workspace_bytes(f->qb, fp8, (int)p->act), 256);
  f->pad = fp8 && p->d_I < 128;
  f->off_pad_q = off;
  off += fp8_pad_q_bytes(f->qb, p->H_I, p->d_I, fp8);
  f->off_pad_k = off;
  off += fp8_pad_k_bytes(b->total_k, p->d_I, fp8);
  f->off_wq = off;
  off += widen_q_bytes(f->qb, p->H, f->w);
  f->off_wkv = off;
  off += widen_kv_bytes(b->total_k, f->w);
  f->off_stage = off;
  off += stage_out_bytes(f->qb, p->H, f->w);
  f->total = off;
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_forward_workspace_size(const dsa_forward_params* p, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (dsa_status s = check_forward(p)) return s;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  ForwardPlan f;
  if (dsa_status s = plan_forward(p, cus, &f)) return s;
  *bytes = f.total;
  return DSA_OK;
}

dsa_status dsa_forward(const dsa_forward_params* p, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  g_err[0] = 0;
  if (dsa_status s = check_forward(p)) return s;
  const dsa_batch* b = p->batch;
  if (b->total_q == 0) return DSA_OK;
  int cus = 0;
  if (dsa_status s = device_cus(&cus)) return s;
  ForwardPlan f;
  if (dsa_status s = plan_forward(p, cus, &f)) return s;
  if (!ws || ws_bytes < f.total || !aligned16(ws))
    return fail(DSA_ERR_WORKSPACE, "forward workspace: need %zu bytes (got %zu)", f.total, ws_bytes);
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  float* scores = (float*)(base + f.off_scores);
  const void* k_idx = p->k_idx;
  int32_t d_I = p->d_I;
  const void* kv = p->kv;
  if (f.w.in) {  // BF16 with d_qk < 576: latent rows widened to 576 columns, zero-filled
    hipError_t e = dsa::launch_copy_rows(p->kv, 2 * p->d_qk, base + f.off_wkv, 2 * kQkW, b->total_k, 2 * p->d_qk, cus, st);
    if (e != hipSuccess) return hip_fail(e, "forward latent widening");
    kv = base + f.off_wkv;
  }
  if (f.pad) {  // FP8 with d_I < 128: the kernels read 128-byte rows, zero-filled past d_I
    hipError_t e = dsa::launch_copy_rows(p->k_idx, p->d_I, base + f.off_pad_k, 128, b->total_k, p->d_I, cus, st);
    if (e != hipSuccess) return hip_fail(e, "forward key widening");
    k_idx = base + f.off_pad_k;
    d_I = 128;
  }
  for (int32_t r0 = 0; r0 < b->total_q; r0 += f.qb) {
    const int32_t r1 = r0 + f.qb < b->total_q ? r0 + f.qb : b->total_q;
    const dsa::BatchView v = view(b, r0, r1);
    int32_t* idx = p->out_idx ? p->out_idx + (int64_t)r0 * p->k : (int32_t*)(base + f.off_idx);
    const void* q_idx = p->q_idx;
    if (f.pad) {
      // the chunk's query rows widened; the indexer addresses q_I by global row,
      // so it gets the buffer's address less r0 rows
      const size_t row_bytes = (size_t)p->H_I * 128;
      hipError_t e = dsa::launch_copy_rows((const char*)p->q_idx + (size_t)r0 * p->H_I * p->d_I, p->d_I,
                                           base + f.off_pad_q, 128, (int64_t)(r1 - r0) * p->H_I, p->d_I, cus, st);
      if (e != hipSuccess) return hip_fail(e, "forward query widening");
      q_idx = (const void*)((uintptr_t)(base + f.off_pad_q) - (uintptr_t)r0 * row_bytes);
    }
    // rows with pos + 1 <= k select every candidate: their scores are never read
    dsa::IndexerLaunch IL{v, p->k, q_idx, k_idx, p->w, scores, f.ld, p->H_I, d_I, (int32_t)p->act,
                          p->idx_dtype == DSA_FP8_E4M3, cus, base + f.off_lin};
    IL.k_scale = p->k_idx_scale;
    IL.batch_rows = b->total_q;  // every chunk scores its rows as the whole batch does
    hipError_t e = dsa::launch_indexer(IL, st);
    if (e != hipSuccess) return hip_fail(e, "forward indexer launch");
    dsa::TopkLaunch TL{v, scores, f.ld, p->k, idx, base + f.off_topk, cus};
    e = dsa::launch_topk(TL, st);
    if (e != hipSuccess) return hip_fail(e, "forward topk launch");
    const int splits = dsa::attention_splits(r1 - r0, p->k, p->dtype == DSA_BF16, cus);
    // q and out are addressed by global row: widened / staged copies of this
    // chunk's rows are passed as their buffer's address less r0 rows
    const void* q = p->q;
    void* out = p->out;
    if (f.w.in) {
      const size_t row = (size_t)p->H * kQkW * 2;
      e = dsa::launch_copy_rows((const char*)p->q + (size_t)r0 * p->H * p->d_qk * 2, 2 * p->d_qk, base + f.off_wq,
                                2 * kQkW, (int64_t)(r1 - r0) * p->H, 2 * p->d_qk, cus, st);
      if (e != hipSuccess) return hip_fail(e, "forward query widening");
      q = (const void*)((uintptr_t)(base + f.off_wq) - (uintptr_t)r0 * row);
    }
    if (f.w.out) out = (void*)((uintptr_t)(base + f.off_stage) - (uintptr_t)r0 * ((size_t)p->H * kVW * 2));
    dsa::AttnLaunch AL{v, q, kv, idx, p->k, p->H, f.w.d_qk, f.w.d_v, p->softmax_scale, out, p->lse,
                       p->dtype == DSA_BF16, splits, nullptr, nullptr};
    AL.dense_short = true;  // rows with pos + 1 <= k: the masked mode, same result as their idx = 0 .. pos
    if (splits > 1) {
      AL.ws_o = (uint16_t*)(base + f.off_attn);
      AL.ws_lse = (float*)(base + f.off_attn + partial_o_bytes(r1 - r0, splits, p->H, f.w.d_v));
    }
    e = dsa::launch_attention(AL, st);
    if (e != hipSuccess) return hip_fail(e, "forward attention launch");
    if (f.w.out) {
      e = dsa::launch_copy_rows(base + f.off_stage, 2 * kVW, (char*)p->out + (size_t)r0 * p->H * p->d_v * 2,
                                2 * p->d_v, (int64_t)(r1 - r0) * p->H, 2 * p->d_v, cus, st);
      if (e != hipSuccess) return hip_fail(e, "forward output narrowing");
    }
  }
  return DSA_OK;
}

}  // extern "C"
