/*
 * libdsa.h -- C interface of the MI355X (gfx950) DeepSeek Sparse Attention
 * hot path: lightning-indexer scores, causal top-k selection, and sparse MLA
 * attention in MQA mode, plus the three fused into one call.
 *
 * Sources (web pages on DeepSeek-V3.2-Exp, cited by title and section):
 *   [P1] blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com), sections
 *        "Lightning indexer / Step 1", "Step 2", "在MLA下實例化DSA".
 *   [P2] "DeepSeek 发布新模型 V3.2-Exp：基于DSA稀疏注意力机制的长上下文优化"
 *        (gamebaike.com), items 【闪电索引器】, 【细粒度Token选择机制】,
 *        【MLA架构集成】, 【推理成本评估】.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated otherwise; tensors are
 *     row-major with the innermost dimension contiguous.
 *   - The caller owns every buffer, the workspace and the stream.  The library
 *     never allocates, frees or synchronises, and keeps no pointer after the
 *     call returns; buffers must stay alive until the stream work completes.
 *   - Calls are asynchronous: DSA_OK means "enqueued on `stream`".
 *   - All argument checks run on the host before anything is enqueued; on an
 *     error nothing is enqueued, outputs are untouched, and dsa_last_error()
 *     holds a description (thread-local).  A failed kernel launch returns
 *     DSA_ERR_HIP.  Device array CONTENTS (cu_q/cu_k consistent with the host
 *     totals, selected positions in [0, pos] or -1) are the caller's contract
 *     and are not checked.
 *   - The library is stateless apart from a per-device property cache and is
 *     safe to call from several threads.
 */
#ifndef LIBDSA_H
#define LIBDSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dsa_stream_t; /* a hipStream_t; NULL = default stream */

/* The enums are int-sized in C and C++ alike.  In C++ they have a fixed int
 * underlying type, so a value a C caller passes outside the listed ones is
 * still a value of the type, which the library then rejects. */
#ifdef __cplusplus
#define DSA_ENUM_BASE : int
#else
#define DSA_ENUM_BASE
#endif

typedef enum DSA_ENUM_BASE {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, inconsistent sizes */
  DSA_ERR_UNSUPPORTED = 2,  /* a valid shape / dtype the library does not implement */
  DSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the size query */
  DSA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} dsa_status;

typedef enum DSA_ENUM_BASE {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2          /* OCP E4M3FN: bias 7, max 448, no infinities */
} dsa_dtype;

typedef enum DSA_ENUM_BASE {
  DSA_ACT_RELU = 0,         /* [P1] "Lightning indexer / Step 1": ReLU, chosen for throughput */
  DSA_ACT_GELU = 1          /* [P2] 【闪电索引器】 names GELU: x * Phi(x), erf form */
} dsa_act;

/*
 * Ragged batch of B sequences (a HOST struct; the arrays it points to are on
 * the device).  Query row r of sequence b (cu_q[b] <= r < cu_q[b+1]) sits at
 * position pos = ctx_b - q_b + (r - cu_q[b]), where q_b = cu_q[b+1]-cu_q[b]
 * and ctx_b = cu_k[b+1]-cu_k[b] (the context includes the query rows).  Its
 * candidates are the positions s in [0, pos]: "a preceding token" of [P1]
 * "Lightning indexer / Step 1", read inclusively.  Key / latent row of
 * position s is cu_k[b] + s.  Prefill: q_b = ctx_b.  Decode: q_b = 1.
 */
typedef struct {
  int32_t num_seqs;         /* B >= 1 */
  const int32_t* cu_q;      /* device [B+1], cu_q[0] = 0, non-decreasing */
  const int32_t* cu_k;      /* device [B+1], cu_k[0] = 0, non-decreasing */
  int32_t total_q;          /* host copy of cu_q[B] (>= 0) */
  int32_t total_k;          /* host copy of cu_k[B] (>= 1) */
  int32_t max_ctx;          /* host: max over b of ctx_b (an upper bound is fine) */
} dsa_batch;

/* Human-readable name of a status code (static string). */
const char* dsa_status_string(dsa_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* dsa_last_error(void);

/* Library version string, e.g. "libdsa 0.1 gfx950". */
const char* dsa_version(void);

/*
 * Lightning-indexer scores.  [P1] "Lightning indexer / Step 1", [P2] 【闪电索引器】:
 *   I[r, s] = sum_{j < H_I} w[r, j] * act(q_idx[r, j, :] . k_idx[kbase + s, :])
 * for every query row r and every candidate s in [0, pos_r].
 *   q_idx   [total_q, H_I, d_I]   idx_dtype (FP8_E4M3 or F32), 16-B aligned
 *   k_idx   [total_k, d_I]        idx_dtype, 16-B aligned (one key per token,
 *                                 shared by all indexer heads)
 *   w       [total_q, H_I]        fp32, 16-B aligned
 *   scores  [total_q, ld_scores]  fp32 output, 16-B aligned; only s <= pos_r
 *                                 is written; ld_scores >= max_ctx, % 4 == 0
 * Arithmetic: FP8 x FP8 products are exact in fp32; dot products accumulate in
 * fp32 (MFMA); the weighted head sum is fp32 in a fixed order.  With ReLU,
 * FP8 inputs and at least 8 query rows per sequence (prefill-like batches) the
 * score is evaluated as 1/2 (qt . k + sum_j w[r,j] |q_idx[r,j,:] . k|) with
 * qt = sum_j w[r,j] q_idx[r,j,:] (the same function, since
 * ReLU(x) = (x + |x|) / 2); qt is carried as four E4M3 terms with power-of-two
 * scales per 32 elements, within about 2^-16 of each block's largest value.
 * Other batches (decode) apply the activation per head.  The two forms differ
 * in the last bits of a score.  The form is chosen from the whole batch
 * (batch->total_q >= 8 * num_seqs), and dsa_forward makes the same choice for
 * every chunk it scores, so a row gets the same score from dsa_forward as
 * from dsa_indexer_scores over the batch, whatever q_block is.
 * k_idx_scale [total_k] uint8 E8M0, or NULL: FP8 keys with a per-token
 *   power-of-two scale (as dsa_cache_append writes them); key s is then
 *   value(k_idx[s, :]) * 2^(k_idx_scale[s] - 127).  The MFMA applies the
 *   scale to each key's dot products, so the products stay exact.  FP8 only.
 * Workspace: dsa_indexer_workspace_size bytes (528 per query row for FP8 with
 * ReLU; for FP8 with d_I < 128 also 128 * H_I per query row and 128 per key
 * row, where q_idx and k_idx are widened to 128-byte rows with zero bytes,
 * which add nothing to the dot products; else 0), 16-B aligned; ws may be
 * NULL when that is 0; a smaller workspace gives DSA_ERR_WORKSPACE.  The size
 * needs no device.
 * Supported: FP8 with d_I a multiple of 16 up to 128 (one MFMA covers 128),
 * H_I a multiple of 4 up to 64 (heads are taken 16 at a time; past H_I the
 * query and weight are zero) and max_ctx <= 2^24;
 * F32 with d_I <= 256, H_I <= 64 and H_I * d_I <= 8192.
 */
dsa_status dsa_indexer_workspace_size(const dsa_batch* batch, dsa_dtype idx_dtype, int32_t H_I, int32_t d_I,
                                      dsa_act act, size_t* bytes /* host */);
dsa_status dsa_indexer_scores(const dsa_batch* batch,
                              const void* q_idx, const void* k_idx, dsa_dtype idx_dtype,
                              const uint8_t* k_idx_scale,
                              const float* w, int32_t H_I, int32_t d_I, dsa_act act,
                              float* scores, int64_t ld_scores,
                              void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * Causal top-k selection.  [P1] "Step 2", [P2] 【细粒度Token选择机制】: for each
 * query keep only the candidates whose index scores rank in the top k.
 * Order: score descending, ties to the lower position; -0 equals +0; NaN
 * ranks below every number.  With n = pos_r + 1 candidates:
 *   n <= k: idx[r] = 0, 1, ..., n-1 followed by -1 (every candidate);
 *   n >  k: the k best positions in ascending order.
 *   scores [total_q, ld_scores] fp32 (only s <= pos_r is read), 16-B aligned,
 *          ld_scores >= max_ctx, % 4 == 0
 *   idx    [total_q, k] int32 output, 16-B aligned
 * Integer / bit operations only: the result is exact.  Supported: 1 <= k <= 2048.
 * Workspace: dsa_topk_workspace_size bytes, 16-B aligned, for batches with
 * fewer rows than the device has compute units and max_ctx >= 8 k or
 * max_ctx > 16384: each row is then split into segments that keep their
 * entries reaching a threshold sampled from the row, and the segments' lists
 * are selected again (same result).  The size depends on the current device's
 * compute-unit count, so query it on the device the call will run on
 * (DSA_ERR_HIP if none is usable; batches with max_ctx < 8 k and
 * max_ctx <= 16384 need no device and get 0).  ws may be NULL when the size
 * is 0; a smaller workspace gives DSA_ERR_WORKSPACE.
 */
dsa_status dsa_topk_workspace_size(const dsa_batch* batch, int32_t k, size_t* bytes /* host */);
dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * Sparse MLA attention in MQA mode.  [P1] "Step 2" (attention between the
 * query and the selected latent entries only) and "在MLA下實例化DSA" / [P2]
 * 【MLA架构集成】 (one latent vector shared by all query heads).  For every
 * query row r and head h, over S_r = the entries of idx[r, :] that are >= 0:
 *   z_s = softmax_scale * q[r, h, :] . kv[kbase + s, :]        (all d_qk columns)
 *   out[r, h, :] = sum_s softmax(z)_s * kv[kbase + s, 0:d_v]    (value = first d_v)
 *   lse[r, h] = log sum_s exp(z_s)
 * An empty S_r gives out = 0 and lse = -inf.
 *   q    [total_q, H, d_qk]  dtype (BF16 or F32), 16-B aligned
 *   kv   [total_k, d_qk]     dtype, 16-B aligned
 *   idx  [total_q, k]        int32 positions within the sequence, or -1
 *   out  [total_q, H, d_v]   dtype output, 16-B aligned
 *   lse  [total_q, H]        fp32 output, or NULL
 * Arithmetic (BF16): bf16 MFMA with fp32 accumulation, fp32 softmax
 * statistics, probabilities rounded to bf16 for the value product, output
 * rounded to nearest even.  Range: the scores z must be finite in fp32 and
 * the value columns below 2^66 in magnitude; within that the output is
 * finite, also when a late entry's score dominates the first ones (a row
 * whose probabilities, taken against its first tile's maximum, grow past
 * 2^60 is recomputed against its true maximum).  Supported: BF16 with d_qk and d_v
 * multiples of 16, d_qk <= 576, d_v <= min(d_qk, 512) (the kernels are 576 /
 * 512 wide; other widths run on copies in the workspace: q and kv rows widened
 * with zeros, which add nothing to q . kv, and the output staged at 512
 * columns, of which the first d_v are kept), H a multiple of 8 up to 128 (the
 * kernel runs waves of 32 heads; heads past H in the last wave are computed on
 * a copy and not stored);
 * F32 with d_qk <= 1024, d_v <= d_qk, H <= 128;
 * 1 <= k <= 2048.  The workspace (possibly 0 bytes) holds split partials and
 * the widened copies.
 */
dsa_status dsa_sparse_mla_attn_workspace_size(const dsa_batch* batch, dsa_dtype dtype, int32_t H,
                                              int32_t k, int32_t d_qk, int32_t d_v, size_t* bytes /* host */);
dsa_status dsa_sparse_mla_attn(const dsa_batch* batch,
                               const void* q, const void* kv, dsa_dtype dtype,
                               const int32_t* idx, int32_t k,
                               int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                               void* out, float* lse,
                               void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * Dense causal MQA attention: the masked mode of short prefill.  [P2]
 * 【推理成本评估】 says short prefill runs DSA as a mask over dense attention;
 * [P1] "在MLA下實例化DSA" gives the MQA form.  For every query row r and head h
 * the candidate set is every position s in [0, pos_r] (no index tensor):
 *   z_s = softmax_scale * q[r, h, :] . kv[kbase + s, :]
 *   out[r, h, :] = sum_s softmax(z)_s * kv[kbase + s, 0:d_v],  lse[r, h] = log sum_s exp(z_s)
 * Shapes, layouts, arithmetic and support as dsa_sparse_mla_attn.  When
 * neither call splits rows over keys (batches with at least as many rows as
 * the device has compute units) the result is bit-identical to
 * dsa_sparse_mla_attn with idx[r] = 0, 1, ..., pos_r (-1 padded): the tiles
 * and their order are the same.  batch->max_ctx must be at least every
 * sequence's context length.
 * F32 additionally needs max_ctx + d_qk <= 16376.  Workspace:
 * dsa_dense_mla_attn_workspace_size bytes (split partials for batches with
 * fewer rows than compute units, and the widened copies of BF16 shapes other
 * than 576 / 512 as in dsa_sparse_mla_attn), 16-B aligned; ws may be NULL when
 * that is 0.
 */
dsa_status dsa_dense_mla_attn_workspace_size(const dsa_batch* batch, dsa_dtype dtype, int32_t H, int32_t d_qk,
                                             int32_t d_v,
                                             size_t* bytes /* host */);
dsa_status dsa_dense_mla_attn(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype,
                              int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                              void* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * Backward of the sparse MLA attention.  [P2] 【稀疏训练阶段】 / [P5]: the
 * sparse training stage optimises every parameter through the sparse
 * attention, so the gradient reaches the query and, by scatter-add, the
 * selected latent rows.  With z_s = softmax_scale q[r,h,:] . kv[s,:], P the
 * softmax over the entries of idx[r] >= 0, out = P V (V = first d_v columns)
 * and the upstream dout:
 *   dP_s = dout[r,h,:] . V_s,  D = dout[r,h,:] . out[r,h,:],
 *   dS_s = softmax_scale P_s (dP_s - D),
 *   dq[r,h,:]   += sum_s dS_s kv[kbase + s, :]
 *   dkv[kbase + s, :] += sum_h dS_s q[r,h,:]  (all d_qk columns)
 *                      + sum_h P_s dout[r,h,:] (first d_v columns)
 *   q, kv, idx, k, H, d_qk, d_v, softmax_scale as dsa_sparse_mla_attn (BF16 only,
 *        H in {32, 64, 128})
 *   lse  [total_q, H] fp32: the forward's log-sum-exp (P is recomputed against
 *        it; D = sum_s P_s dP_s is formed in fp32 over the row's entries)
 *   dout [total_q, H, d_v] bf16, 16-B aligned
 *   dq   [total_q, H, d_qk] fp32 and dkv [total_k, d_qk] fp32, 16-B aligned:
 *        ACCUMULATED (zero them first); dkv by float atomics, so the order of
 *        its additions (its last bits) may vary between runs
 * Arithmetic: bf16 MFMAs with fp32 accumulation; P and dS are kept in the
 * workspace as bf16, dS for dq as a hi + lo pair of bf16 (dq sums terms that
 * cancel).
 * Workspace: dsa_sparse_mla_backward_workspace_size bytes (4 x rows x H x k
 * rounded up to 32, bf16), 16-B aligned.
 */
dsa_status dsa_sparse_mla_backward_workspace_size(const dsa_batch* batch, int32_t H, int32_t k,
                                                  size_t* bytes /* host */);
dsa_status dsa_sparse_mla_backward(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype,
                                   const int32_t* idx, int32_t k, int32_t H, int32_t d_qk, int32_t d_v,
                                   float softmax_scale, const float* lse, const void* dout,
                                   float* dq, float* dkv, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * Indexer-alignment target.  [P1] training "Step 1" (dense warm-up) and
 * "Step 2" (sparse training), [P2] 【密集预热阶段】 / 【稀疏训练阶段】: for each
 * query row the main attention's probabilities of every head are summed over
 * the heads and L1-normalised along the candidates, giving the distribution
 * the indexer is trained to follow.  With lse the main attention's log-sum-exp
 * over the same candidates (as dsa_sparse_mla_attn / dsa_dense_mla_attn return
 * it) each head's probabilities sum to 1, so
 *   p[r, e] = (1/H) sum_h exp(softmax_scale * q[r, h, :] . kv[kbase + s_e, :] - lse[r, h])
 * (sum_e p[r, e] = 1 up to rounding).  Candidates: idx == NULL, every
 * position s_e = e <= pos_r (dense warm-up); else s_e = idx[r, e] for the
 * entries >= 0 (the selected set of the sparse stage).
 *   q, kv   as dsa_sparse_mla_attn (BF16: d_qk = 576, H a multiple of 8 up to 128;
 *           F32: d_qk <= 1024, H <= 128)
 *   idx     [total_q, k] int32 or NULL; k as dsa_sparse_mla_attn (ignored when NULL)
 *   lse     [total_q, H] fp32 (natural log); a head with lse = -inf adds nothing
 *   p       [total_q, ld_p] fp32 output, 16-B aligned.  Entries that are no
 *           candidate are written as 0, up to the walk's whole 32-entry tiles
 *           (dense: positions up to pos_r rounded up; selected: k rounded up),
 *           so ld_p >= 32 * ceil(m / 32) with m = max_ctx (dense) or k.
 * Arithmetic: bf16 MFMA scores, fp32 exponent and head sums.  F32 needs
 * m + d_qk <= 16384.  No workspace.
 */
dsa_status dsa_attn_target(const dsa_batch* batch, const void* q, const void* kv, dsa_dtype dtype,
                           const int32_t* idx, int32_t k, int32_t H, int32_t d_qk, float softmax_scale,
                           const float* lse, float* p, int64_t ld_p, dsa_stream_t stream);

/*
 * Indexer-alignment loss and its gradient.  [P1] training "Step 1": a KL
 * divergence between the target p and the indexer's output, read as
 * softmax(I) over the same candidates; "Step 2": over the selected set only.
 * For each query row r, with candidates s_e as in dsa_attn_target:
 *   loss[r] = sum_e p[r, e] (log p[r, e] - log softmax(I)_e)       (0 log 0 = 0)
 *   dI[r, e] = (sum_e' p[r, e']) softmax(I)_e - p[r, e]             (d loss[r] / d I[r, s_e])
 * where I_e = scores[r, s_e] (dense: s_e = e, so dI is by position; selected:
 * dI is by entry, aligned with idx; entries that are no candidate get 0).
 *   scores [total_q, ld_scores] fp32 (the indexer's output), 16-B aligned
 *   p      [total_q, ld_p] fp32; dI [total_q, ld_p] fp32 output or NULL;
 *   loss   [total_q] fp32 output or NULL
 * Arithmetic: fp32, row sums as trees.  No workspace.
 */
dsa_status dsa_indexer_kl(const dsa_batch* batch, const float* scores, int64_t ld_scores, const int32_t* idx,
                          int32_t k, const float* p, int64_t ld_p, float* loss, float* dI, dsa_stream_t stream);

/*
 * Backward of the index score to the indexer's inputs: what the alignment
 * loss trains.  [P1] training "Step 2": the indexer's input is detached from
 * the computational graph, so its gradient ends at q_I, w and k_I (the
 * projections that make them are outside this library).  For an upstream
 * gradient g over each row's candidates (as dsa_attn_target: dense, entry
 * e = position e; else entry e = position idx[r, e] when >= 0), with
 * x = q_idx[r, j, :] . k[s, :] and k the (scaled) key:
 *   dw[r, j]        += sum_e g[r, e] act(x)
 *   dq_idx[r, j, :] += sum_e g[r, e] w[r, j] act'(x) k[s_e, :]
 *   dk_idx[s, :]    += sum over rows and heads of g w act'(x) q_idx[r, j, :]
 * act' of ReLU is 1 for x > 0 and 0 otherwise (0 at x = 0); of GELU
 * Phi(x) + x phi(x).  dk is by key row of the batch (kbase + s); with scales it
 * is the gradient with respect to the scaled key.
 *   q_idx, k_idx, k_idx_scale, w, H_I, act as dsa_indexer_scores (FP8 only,
 *           d_I = 128 only)
 *   g       [total_q, ld_g] fp32, ld_g >= max_ctx (dense) or k
 *   dq_idx  [total_q, H_I, d_I] fp32, dw [total_q, H_I] fp32, dk_idx [total_k, d_I]
 *           fp32: ACCUMULATED with float atomics (zero them first; the order
 *           of the additions, and so the last bits, may vary between runs)
 * Arithmetic: x by FP8 MFMA (exact products, fp32 sums); g w act'(x) rounded
 * to bf16 for the two bf16 MFMA products (k and q_idx are exact in bf16); fp32
 * accumulation.  No workspace.
 */
dsa_status dsa_indexer_backward(const dsa_batch* batch, const void* q_idx, const void* k_idx, dsa_dtype idx_dtype,
                                const uint8_t* k_idx_scale, const float* w, int32_t H_I, int32_t d_I, dsa_act act,
                                const int32_t* idx, int32_t k, const float* g, int64_t ld_g,
                                float* dq_idx, float* dw, float* dk_idx, dsa_stream_t stream);

/*
 * New tokens into the caches.  [P1] "Lightning indexer": the indexer runs in
 * FP8, so the indexer key of every token is stored as E4M3 codes;
 * "在MLA下實例化DSA": one latent row per token serves all query heads.  For
 * each new token t < n, with d = dst_rows[t] (or t when dst_rows is NULL):
 *   k_cache[d, :]  = E4M3FN(k_new[t, :] / 2^e_t)   (when k_new != NULL)
 *   k_scale[d]     = 127 + e_t                      (when k_scale != NULL)
 *   kv_cache[d, :] = kv_new[t, :]                   (when kv_new != NULL)
 * E4M3FN(x): nearest value, ties to the even code, magnitudes above 448 give
 * +-448, NaN gives 0x7F, the sign of x is kept (results that round to zero
 * give +0 or -0).  e_t = 0 without k_scale; with it, e_t is the smallest
 * integer with max_j |k_new[t, j]| <= 448 * 2^e_t (NaN ignored), clamped to
 * [-127, 127], e_t = 0 for an all-zero row and 127 for a row holding an
 * infinity.  Scaling by 2^-e_t is exact except for values that round to zero
 * in E4M3 anyway.
 *   k_new     [n, d_I]           k_dtype F32 or BF16, 16-B aligned
 *   k_cache   [cache_rows, d_I]  uint8 E4M3FN codes, 8-B aligned
 *   k_scale   [cache_rows]       uint8 E8M0, or NULL (unscaled codes)
 *   kv_new    [n, d_qk]          kv_dtype (F32 or BF16), 16-B aligned; d_qk
 *                                 times the element size a multiple of 16
 *   kv_cache  [cache_rows, d_qk] kv_dtype, 16-B aligned
 *   dst_rows  [n] int32 device, or NULL.  Tokens whose row lies outside
 *             [0, cache_rows) are not written.  Two tokens with the same row
 *             race (either result may stay).
 * Supported: d_I in {64, 128, 256, 512}; n * d_qk * element size / 16 < 2^31.
 * No workspace; the result is exact (bit-for-bit definition above).
 */
dsa_status dsa_cache_append(int64_t n, const int32_t* dst_rows, int64_t cache_rows,
                            const void* k_new, dsa_dtype k_dtype, int32_t d_I,
                            uint8_t* k_cache, uint8_t* k_scale,
                            const void* kv_new, dsa_dtype kv_dtype, int32_t d_qk, void* kv_cache,
                            dsa_stream_t stream);

/*
 * The three steps fused in one call, on one stream, with no host
 * synchronisation.  Query rows are processed in chunks of q_block rows
 * (bounded score workspace).  Rows with pos + 1 <= k skip the indexer and the
 * selection: every candidate is selected, which is the masked dense-equivalent
 * mode [P2] 【推理成本评估】 describes for short prefill.  The indices equal
 * those of dsa_topk(dsa_indexer_scores(...)) bit for bit.
 */
typedef struct {
  const dsa_batch* batch;
  /* indexer */
  const void* q_idx; const void* k_idx; dsa_dtype idx_dtype;
  const uint8_t* k_idx_scale;  /* [total_k] E8M0 per-token key scales (FP8), or NULL */
  const float* w; int32_t H_I; int32_t d_I; dsa_act act;
  /* attention */
  const void* q; const void* kv; dsa_dtype dtype;
  int32_t H; int32_t d_qk; int32_t d_v; float softmax_scale;
  int32_t k;                /* tokens selected per query (2048 in the pages) */
  int32_t q_block;          /* query rows per chunk; 0 = library default (4096) */
  void* out; float* lse;    /* lse may be NULL */
  int32_t* out_idx;         /* [total_q, k] selected positions, or NULL */
} dsa_forward_params;

dsa_status dsa_forward_workspace_size(const dsa_forward_params* p, size_t* bytes /* host */);
dsa_status dsa_forward(const dsa_forward_params* p, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * workspace is the library's own static device array of 128 MiB (134217728
 * bytes), which each device the library runs on holds until the process
 * ends; the caller still passes every input and output.  The call allocates
 * nothing and enqueues exactly the kernels dsa_forward enqueues, so the
 * results are identical.  A batch whose dsa_forward_workspace_size exceeds
 * 128 MiB gives DSA_ERR_WORKSPACE with nothing enqueued (decode steps of tens
 * of sequences fit; long prefills need dsa_forward with their own workspace).
 * Nothing in the array needs to start at zero: a call writes every byte it
 * reads.  Every call on one device shares that device's array, so calls that
 * overlap on one device (other streams, other threads) race: serialise them.
 * The first call on a device takes the array's device address (HIP error:
 * DSA_ERR_HIP).
 */
dsa_status dsa_forward_noalloc(const dsa_forward_params* p, dsa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBDSA_H */
