// dsa_kernels.h -- internal launch interface between the C ABI layer and the
// kernels.  Not installed; the public interface is include/libdsa.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Rows [row_begin, row_end) of the global query-row space are processed; row
// r's outputs go to row (r - row_begin) of the output arrays, except the
// query-side inputs, which are always indexed by the global row.
struct BatchView {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t num_seqs;
  int32_t row_begin;
  int32_t row_end;
  int32_t max_ctx;
};

struct IndexerLaunch {
  BatchView b;
  int32_t skip_n;          // rows with pos + 1 <= skip_n are not computed
  const void* q_idx;       // [total_q, H_I, d_I]
  const void* k_idx;       // [total_k, d_I]
  const float* w;          // [total_q, H_I]
  float* scores;           // [row_end - row_begin, ld]
  int64_t ld;
  int32_t H_I, d_I;
  int32_t act;             // 0 relu, 1 gelu
  bool fp8;
  int32_t num_cus;
  void* ws;                // indexer_workspace_bytes(rows, fp8, act) bytes, or null when that is 0
  const uint8_t* k_scale = nullptr;  // [total_k] E8M0 per-key scales (FP8), or null
  // FP8 kernel family: prefill-like batches (at least 8 query rows per
  // sequence) share key slabs between rows and, with ReLU, take the
  // linear-term form of the score; other batches stream keys per row.  The
  // two differ in the last bits of a score, so the choice is made from the
  // whole batch (its total rows), not from the rows of one launch: a chunk of
  // a batch scores its rows as the batch does.
  int32_t batch_rows = -1;  // total query rows of the batch; -1: this launch's rows
};
// True when a batch of `total_rows` query rows in `num_seqs` sequences takes
// the prefill-like (shared key slab) FP8 indexer.
inline bool indexer_prefill_like(int64_t total_rows, int num_seqs) { return total_rows >= 8LL * num_seqs; }

struct TopkLaunch {
  BatchView b;
  const float* scores;     // [row_end - row_begin, ld]
  int64_t ld;
  int32_t k;
  int32_t* idx;            // [row_end - row_begin, k]
  void* ws;                // topk_workspace_bytes(...) bytes, or null when that is 0
  int32_t num_cus;
};

struct AttnLaunch {
  BatchView b;
  const void* q;           // [total_q, H, d_qk]
  const void* kv;          // [total_k, d_qk]
  const int32_t* idx;      // [row_end - row_begin, k]
  int32_t k;
  int32_t H, d_qk, d_v;
  float scale;
  void* out;               // [total_q, H, d_v] (global rows)
  float* lse;              // [total_q, H] or null (global rows)
  bool bf16;
  int32_t splits;          // >1: partials in ws, then a merge
  uint16_t* ws_o;          // [rows, splits, H, d_v] bf16: each split's normalised output
  float* ws_lse;           // [rows, splits, H]
  bool dense = false;      // every candidate [0, pos] (idx unused; k = max_ctx)
  bool dense_short = false;  // rows with pos + 1 <= k walk [0, pos] without reading idx
  // alignment target instead of attention: p_out[row, e] = sum_h exp(z_h,e - lse_in[row, h]) / H
  bool target = false;
  const float* lse_in = nullptr;  // [total_q, H] (global rows)
  float* p_out = nullptr;         // [rows, ld_p]
  int64_t ld_p = 0;
};

// New tokens into the caches: indexer keys quantised to E4M3 (optionally with
// per-token E8M0 scales), latent rows copied.  Either part may be absent.
struct AppendLaunch {
  int64_t n;               // new tokens
  const int32_t* dst;      // [n] cache rows, or null (token t -> row t)
  int64_t cache_rows;      // rows outside [0, cache_rows) are not written
  const void* k_new;       // [n, d_I] fp32 or bf16, or null
  bool k_bf16;
  int32_t d_I;             // 64, 128, 256 or 512
  uint8_t* k_cache;        // [cache_rows, d_I]
  uint8_t* k_scale;        // [cache_rows] or null (unscaled)
  const void* kv_new;      // [n, kv_row_bytes], or null
  void* kv_cache;          // [cache_rows, kv_row_bytes]
  int64_t kv_row_bytes;    // multiple of 16
};

// KL(p || softmax(I)) per row over its candidates and dI (indexer alignment).
struct KlLaunch {
  BatchView b;
  const float* scores;     // [rows, ld_s] index scores by position
  int64_t ld_s;
  const int32_t* idx;      // [rows, k] selected positions, or null (dense: entry e = position e)
  int32_t k;
  const float* p;          // [rows, ld_p] target by entry
  int64_t ld_p;
  float* loss;             // [rows] or null
  float* dI;               // [rows, ld_p] by entry, or null
};

// Backward of the FP8 index score to q_I, w and k_I (accumulated with atomics).
struct IndexerBwdLaunch {
  BatchView b;
  const void* q_idx;       // [total_q, H_I, 128] e4m3
  const void* k_idx;       // [total_k, 128] e4m3
  const uint8_t* k_scale;  // [total_k] or null
  const float* w;          // [total_q, H_I]
  int32_t H_I;
  int32_t act;
  const int32_t* idx;      // [rows, k] or null (dense)
  int32_t k;
  const float* g;          // [rows, ld_g] by entry
  int64_t ld_g;
  float* dq;               // [total_q, H_I, 128]
  float* dw;               // [total_q, H_I]
  float* dk;               // [total_k, 128]
  int32_t num_cus;
};

// Backward of the bf16 sparse MQA attention (dq and dkv accumulated).
struct MlaBwdLaunch {
  BatchView b;
  const void* q;           // [total_q, H, 576] bf16
  const void* kv;          // [total_k, 576] bf16
  const int32_t* idx;      // [rows, k]
  int32_t k, H;
  float scale;
  const float* lse;        // [total_q, H]
  const void* dout;        // [total_q, H, 512] bf16
  float* dq;               // [total_q, H, 576]
  float* dkv;              // [total_k, 576]
  void* ws;                // mla_backward_workspace_bytes(rows, H, k)
  int32_t num_cus;
};
size_t mla_backward_workspace_bytes(int rows, int H, int k);
hipError_t launch_mla_backward(const MlaBwdLaunch& a, hipStream_t s);

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t s);
hipError_t launch_indexer_bwd(const IndexerBwdLaunch& a, hipStream_t s);
hipError_t launch_indexer_kl(const KlLaunch& a, hipStream_t s);
hipError_t launch_cache_append(const AppendLaunch& a, hipStream_t s);

// Workspace of the indexer for `rows` query rows (the FP8 ReLU path keeps the
// linear-term fragments of every row there).
size_t indexer_workspace_bytes(int rows, bool fp8, int act);
// Row reshaping (sizes in bytes, multiples of 16): dst row r of out_stride
// bytes gets the first copy_bytes (<= in_stride) of src row r, zero-filled up
// to out_stride.  Widens narrow FP8 indexer rows and attention rows, and keeps
// the first d_v columns of a staged attention output.
hipError_t launch_copy_rows(const void* src, int64_t in_stride, void* dst, int64_t out_stride, int64_t rows,
                            int64_t copy_bytes, int num_cus, hipStream_t s);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t s);
hipError_t launch_attention(const AttnLaunch& a, hipStream_t s);

// Workspace of the segmented top-k for `rows` rows (0: single pass per row).
size_t topk_workspace_bytes(int rows, int max_ctx, int k, int num_cus);
// False when no batch with this max_ctx and k is ever split into segments
// (then the workspace is 0 bytes on every device).
bool topk_may_segment(int max_ctx, int k);

// Number of key-splits the attention uses for `rows` query rows.
int attention_splits(int rows, int k, bool bf16, int num_cus);
// Waves (of 32 heads each) of the bf16 attention workgroup for H heads.
int attention_waves(int H);

}  // namespace dsa
