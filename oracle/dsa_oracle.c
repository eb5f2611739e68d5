/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DeepSeek Sparse Attention (DSA)
 * hot path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
 * baseline leg of the benchmark call it; the library never does.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Everything is computed in double precision with the plain definitions:
 * no tiling, no online softmax, no radix select, no fused steps.  OpenMP
 * parallelises over independent query rows only.
 *
 * Sources (web pages on DeepSeek-V3.2-Exp; cited by title and section):
 *   [P1] blog "Deepseek v3.2 exp 加班快樂 ... 論文原文" (hdetylss.com):
 *        "Lightning indexer / Step 1" (index score), "Step 2" (top-k selection,
 *        attention over the selected entries), "在MLA下實例化DSA" (MQA mode,
 *        one latent shared by all heads).
 *   [P2] "DeepSeek 发布新模型 V3.2-Exp：基于DSA稀疏注意力机制的长上下文优化"
 *        (gamebaike.com): 【闪电索引器】, 【细粒度Token选择机制】, 【MLA架构集成】.
 *
 * Batch convention (shared with the library's C interface, restated here):
 *   row r of sequence b (cu_q[b] <= r < cu_q[b+1]) sits at position
 *   pos = ctx_b - q_b + (r - cu_q[b]) with q_b = cu_q[b+1]-cu_q[b] and
 *   ctx_b = cu_k[b+1]-cu_k[b]; its candidates are the positions s in [0, pos]
 *   ("a preceding token", read inclusively); the key / latent row of position s
 *   is cu_k[b] + s.
 *
 * Every function takes an explicit list of rows so that a caller can evaluate
 * a sample of a large problem; query-side inputs and all outputs are compact
 * arrays indexed by the position in that list.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8_E4M3 = 2 };
enum { OR_ACT_RELU = 0, OR_ACT_GELU = 1 };

/* ------------------------------------------------------------------ */
/* Exact decoding of the stored element formats.                       */
/* ------------------------------------------------------------------ */

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
double dsa_oracle_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load_elem(const void* base, int dtype, int64_t i, const double* e4m3_table) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[i];
    case OR_BF16: return bf16_value(((const uint16_t*)base)[i]);
    default: return e4m3_table[((const uint8_t*)base)[i]];
    }
}

/* Locate a row in the ragged batch: sequence index, position, first key row. */
static int locate_row(int nseq, const int32_t* cu_q, const int32_t* cu_k, int32_t r,
                      int64_t* pos, int64_t* kbase) {
    for (int b = 0; b < nseq; ++b) {
        if (r >= cu_q[b] && r < cu_q[b + 1]) {
            int64_t qb = cu_q[b + 1] - cu_q[b], ctx = cu_k[b + 1] - cu_k[b];
            *pos = ctx - qb + (r - cu_q[b]);
            *kbase = cu_k[b];
            return (*pos >= 0 && *pos < ctx) ? 0 : -1;
        }
    }
    return -1;
}

/* ------------------------------------------------------------------ */
/* Step 1: lightning-indexer scores.                                   */
/* [P1] "Lightning indexer / Step 1": the index score between query token t
 * and a preceding token s sums, over the few indexer heads j, a weight w[t,j]
 * derived from the query token times a ReLU of the dot product of the head's
 * indexer query q_I[t,j] with the preceding token's indexer key k_I[s]; ReLU
 * was chosen for throughput.  [P2] 【闪电索引器】 names GELU instead; it is kept
 * as a switch (exact erf form).  An FP8 key cache may carry a per-token
 * power-of-two scale (E8M0 byte, see the quantisation below); the key is
 * then value(code) * 2^(scale - 127).                                  */
/* ------------------------------------------------------------------ */
static double activation(double x, int act) {
    if (act == OR_ACT_GELU) return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    return x > 0.0 ? x : 0.0;
}

int dsa_oracle_indexer(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                       int nrows, const int32_t* rows,
                       const void* q_idx, const void* k_idx, int dtype, const uint8_t* k_scale,
                       const float* w, int H_I, int d_I, int act,
                       double* scores, int64_t ld) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < nrows; ++i) {
        int64_t pos, kbase;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0 || pos + 1 > ld) { bad |= 1; continue; }
        double* out = scores + (int64_t)i * ld;
        for (int64_t s = 0; s <= pos; ++s) {
            /* per-token key scale: the key is value(code) * 2^(scale - 127) */
            const double ks = k_scale ? ldexp(1.0, (int)k_scale[kbase + s] - 127) : 1.0;
            double score = 0.0;
            for (int j = 0; j < H_I; ++j) {
                double dot = 0.0;
                for (int d = 0; d < d_I; ++d) {
                    double q = load_elem(q_idx, dtype, ((int64_t)i * H_I + j) * d_I + d, table);
                    double k = load_elem(k_idx, dtype, (kbase + s) * d_I + d, table) * ks;
                    dot += q * k;
                }
                score += (double)w[(int64_t)i * H_I + j] * activation(dot, act);
            }
            out[s] = score;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Step 2: fine-grained token selection.                                */
/* [P1] "Step 2" / [P2] 【细粒度Token选择机制】: for each query keep only the
 * tokens whose index scores rank in the top k.  Ties go to the lower position;
 * -0 equals +0 (numeric comparison); NaN ranks below every number.  The
 * selected positions are returned in ascending order, padded with -1 when the
 * row has fewer than k candidates (then every candidate is selected).    */
/* ------------------------------------------------------------------ */
typedef struct { float score; int32_t pos; } cand_t;

static int better_first(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    int an = isnan(a->score), bn = isnan(b->score);
    if (!an && !bn) {
        if (a->score > b->score) return -1;
        if (a->score < b->score) return 1;
    } else if (an != bn) {
        return an ? 1 : -1;
    }
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos);
}

static int ascending_int(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

int dsa_oracle_topk(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                    int nrows, const int32_t* rows,
                    const float* scores, int64_t ld, int k, int32_t* idx) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < nrows; ++i) {
        int64_t pos, kbase;
        int32_t* out = idx + (int64_t)i * k;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0 || pos + 1 > ld) { bad |= 1; continue; }
        int64_t n = pos + 1;
        int64_t take = n < k ? n : k;
        if (n <= k) {
            for (int64_t s = 0; s < n; ++s) out[s] = (int32_t)s;
        } else {
            cand_t* c = (cand_t*)malloc((size_t)n * sizeof(cand_t));
            for (int64_t s = 0; s < n; ++s) { c[s].score = scores[(int64_t)i * ld + s]; c[s].pos = (int32_t)s; }
            qsort(c, (size_t)n, sizeof(cand_t), better_first);
            for (int64_t s = 0; s < take; ++s) out[s] = c[s].pos;
            free(c);
            qsort(out, (size_t)take, sizeof(int32_t), ascending_int);
        }
        for (int64_t s = take; s < k; ++s) out[s] = -1;
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Step 3: attention over the selected latent entries, MQA mode.        */
/* [P1] "Step 2": the attention output is computed between the query token
 * and the selected entries only; the entries are the MLA low-rank latent
 * vectors.  [P1] "在MLA下實例化DSA" / [P2] 【MLA架构集成】: DSA runs on MLA's
 * MQA mode, so one latent vector is shared by every query head.  The key is
 * the whole latent row (d_qk columns); the value is its first d_v columns.
 * Plain softmax: z_s = scale * q.c_s; o = sum_s softmax(z)_s * c_s[:d_v];
 * lse = log sum_s exp z_s.  An empty selection gives o = 0, lse = -inf;
 * repeated positions count as often as listed.                         */
/* ------------------------------------------------------------------ */
int dsa_oracle_sparse_mla(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                          int nrows, const int32_t* rows,
                          const void* q, const void* kv, int dtype,
                          const int32_t* idx, int k, int H, int d_qk, int d_v,
                          double scale, double* out, double* lse) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < nrows; ++i) {
        int64_t pos, kbase;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0) { bad |= 1; continue; }
        const int32_t* sel = idx + (int64_t)i * k;
        double* z = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
        for (int h = 0; h < H; ++h) {
            double* o = out + ((int64_t)i * H + h) * d_v;
            int nvalid = 0;
            double m = -INFINITY;
            for (int e = 0; e < k; ++e) {
                if (sel[e] < 0) continue;
                if (sel[e] > pos) bad |= 2;
                double dot = 0.0;
                for (int d = 0; d < d_qk; ++d)
                    dot += load_elem(q, dtype, ((int64_t)i * H + h) * d_qk + d, table) *
                           load_elem(kv, dtype, (kbase + sel[e]) * d_qk + d, table);
                z[e] = scale * dot;
                if (z[e] > m) m = z[e];
                ++nvalid;
            }
            for (int d = 0; d < d_v; ++d) o[d] = 0.0;
            if (nvalid == 0) {
                if (lse) lse[(int64_t)i * H + h] = -INFINITY;
                continue;
            }
            double l = 0.0;
            for (int e = 0; e < k; ++e) {
                if (sel[e] < 0) continue;
                double p = exp(z[e] - m);
                l += p;
                for (int d = 0; d < d_v; ++d)
                    o[d] += p * load_elem(kv, dtype, (kbase + sel[e]) * d_qk + d, table);
            }
            for (int d = 0; d < d_v; ++d) o[d] /= l;
            if (lse) lse[(int64_t)i * H + h] = m + log(l);
        }
        free(z);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Indexer-key quantisation to OCP E4M3FN.  [P1] "Lightning indexer": the
 * indexer runs in FP8, so its key cache holds FP8 codes.  Rounding is to the
 * nearest representable value, ties to the even code; magnitudes beyond the
 * largest finite value (448) saturate to it; NaN gives 0x7F; the sign is kept
 * (so values that round to zero give +0 or -0).
 * With per-token scaling each key row t gets the power of two 2^e_t with the
 * smallest e_t such that max_d |x[t,d]| <= 448 * 2^e_t (NaN ignored; e_t = 0
 * for an all-zero row; clamped to [-127, 127], so a row holding an infinity
 * gets 127); the codes encode x[t,d] / 2^e_t and
 * the scale is stored as an E8M0 byte 127 + e_t, so the key is
 * value(code) * 2^e_t. */
/* ------------------------------------------------------------------ */
static int e4m3_encode(double x) {
    if (x != x) return 0x7F;
    const int sign = (x < 0.0 || (x == 0.0 && signbit(x))) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    /* nearest of the 127 non-negative finite codes 0x00 .. 0x7E; codes are
     * monotone in value, ties go to the even code */
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(dsa_oracle_e4m3_value(c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    return sign | best;
}

int dsa_oracle_quantize_keys(const void* src, int dtype, int64_t n, int d, int scaled,
                             uint8_t* codes, uint8_t* scale_e8m0) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    if (dtype != OR_F32 && dtype != OR_BF16) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int e = 0;
        if (scaled) {
            double amax = 0.0;
            for (int j = 0; j < d; ++j) {
                const double v = fabs(load_elem(src, dtype, t * d + j, table));
                if (v > amax) amax = v;  /* NaN never compares greater */
            }
            if (isinf(amax)) {
                e = 127;
            } else if (amax > 0.0) {
                int ex;
                const double f = frexp(amax / 448.0, &ex);  /* amax / 448 = f 2^ex, f in [0.5, 1) */
                e = (f == 0.5) ? ex - 1 : ex;               /* ceil(log2(amax / 448)) */
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            scale_e8m0[t] = (uint8_t)(127 + e);
        }
        for (int j = 0; j < d; ++j)
            codes[t * d + j] = (uint8_t)e4m3_encode(ldexp(load_elem(src, dtype, t * d + j, table), -e));
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Indexer alignment, the training objective of the indexer.  [P1] training
 * "Step 1" (dense warm-up) and [P2] 【密集预热阶段】: for query token t the main
 * attention scores (the softmax probabilities of each head) are summed over
 * the heads and L1-normalised along the sequence, giving the target p_t; the
 * loss is the KL divergence from p_t to the indexer's distribution, read as
 * softmax(I_t) over the same candidates.  [P1] "Step 2" / [P2] 【稀疏训练阶段】:
 * in the sparse stage only the selected set S_t is considered, and the
 * indexer's input is detached, so this loss trains the indexer alone.
 *
 * Candidate lists: dense (idx == NULL) entry e of row i is position e, for
 * e <= pos; sparse: entry e is position idx[i, e] when that is >= 0.  Row i's
 * arrays have m entries; entries that are no candidate are 0 on output. */
/* ------------------------------------------------------------------ */
static int cand_pos(const int32_t* idx, int m, int i, int e, int64_t pos) {
    if (!idx) return e <= pos ? e : -1;
    const int32_t s = idx[(int64_t)i * m + e];
    return s >= 0 && s <= pos ? s : -1;
}

int dsa_oracle_attn_target(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                           int nrows, const int32_t* rows,
                           const void* q, const void* kv, int dtype,
                           const int32_t* idx, int m, int H, int d_qk, double scale, double* p) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < nrows; ++i) {
        int64_t pos, kbase;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0 || (!idx && pos + 1 > m)) { bad |= 1; continue; }
        double* pr = p + (int64_t)i * m;
        double* z = (double*)malloc((size_t)m * sizeof(double));
        for (int e = 0; e < m; ++e) pr[e] = 0.0;
        for (int h = 0; h < H; ++h) {
            /* this head's attention probabilities over the candidates */
            double mx = -INFINITY;
            for (int e = 0; e < m; ++e) {
                const int s = cand_pos(idx, m, i, e, pos);
                if (s < 0) continue;
                double dot = 0.0;
                for (int d = 0; d < d_qk; ++d)
                    dot += load_elem(q, dtype, ((int64_t)i * H + h) * d_qk + d, table) *
                           load_elem(kv, dtype, (kbase + s) * d_qk + d, table);
                z[e] = scale * dot;
                if (z[e] > mx) mx = z[e];
            }
            double l = 0.0;
            for (int e = 0; e < m; ++e)
                if (cand_pos(idx, m, i, e, pos) >= 0) l += exp(z[e] - mx);
            /* summed over the heads */
            for (int e = 0; e < m; ++e)
                if (cand_pos(idx, m, i, e, pos) >= 0) pr[e] += exp(z[e] - mx) / l;
        }
        /* L1-normalised along the sequence */
        double norm = 0.0;
        for (int e = 0; e < m; ++e) norm += fabs(pr[e]);
        if (norm > 0.0)
            for (int e = 0; e < m; ++e) pr[e] /= norm;
        free(z);
    }
    return bad ? -1 : 0;
}

/* KL(p || softmax(I)) per row over its first cnt[i] entries, and its gradient
 * with respect to I: d/dI_e = (sum_e' p_e') softmax(I)_e - p_e.  Terms with
 * p_e = 0 contribute 0 (0 log 0 = 0).  Entries past cnt[i] get dI = 0. */
int dsa_oracle_indexer_kl(int nrows, int m, const int32_t* cnt, const double* I, const double* p,
                          double* loss, double* dI) {
    int bad = 0;
    for (int i = 0; i < nrows; ++i) {
        const int n = cnt[i];
        if (n < 0 || n > m) { bad = 1; continue; }
        const double* Ir = I + (int64_t)i * m;
        const double* pr = p + (int64_t)i * m;
        double mx = -INFINITY, psum = 0.0;
        for (int e = 0; e < n; ++e) {
            if (Ir[e] > mx) mx = Ir[e];
            psum += pr[e];
        }
        double l = 0.0;
        for (int e = 0; e < n; ++e) l += exp(Ir[e] - mx);
        const double lse = mx + log(l);
        double kl = 0.0;
        for (int e = 0; e < n; ++e)
            if (pr[e] > 0.0) kl += pr[e] * (log(pr[e]) - (Ir[e] - lse));
        if (loss) loss[i] = n > 0 ? kl : 0.0;
        if (dI) {
            double* g = dI + (int64_t)i * m;
            for (int e = 0; e < m; ++e) g[e] = e < n ? psum * exp(Ir[e] - lse) - pr[e] : 0.0;
        }
    }
    return bad ? -1 : 0;
}

/* Backward of the index score (R1) for an upstream gradient g over each row's
 * candidates: with x = q_idx[i,j,:] . k[s,:] (k scaled per token if k_scale),
 *   dw[i,j]        += g_e act(x)
 *   dq_idx[i,j,:]  += g_e w[i,j] act'(x) k[s,:]
 *   dk_idx[s,:]    += g_e w[i,j] act'(x) q_idx[i,j,:]      (all rows, summed)
 * act' of ReLU is 1 for x > 0 and 0 otherwise; of GELU Phi(x) + x phi(x).
 * The outputs are accumulated: the caller zeroes them. */
int dsa_oracle_indexer_backward(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                                int nrows, const int32_t* rows,
                                const void* q_idx, const void* k_idx, int dtype, const uint8_t* k_scale,
                                const float* w, int H_I, int d_I, int act,
                                const int32_t* idx, int m, const double* g,
                                double* dq_idx, double* dw, double* dk_idx) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    for (int i = 0; i < nrows; ++i) {
        int64_t pos, kbase;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0 || (!idx && pos + 1 > m)) return -1;
        for (int e = 0; e < m; ++e) {
            const int s = cand_pos(idx, m, i, e, pos);
            const double ge = g[(int64_t)i * m + e];
            if (s < 0 || ge == 0.0) continue;
            const double ks = k_scale ? ldexp(1.0, (int)k_scale[kbase + s] - 127) : 1.0;
            for (int j = 0; j < H_I; ++j) {
                double x = 0.0;
                for (int d = 0; d < d_I; ++d)
                    x += load_elem(q_idx, dtype, ((int64_t)i * H_I + j) * d_I + d, table) *
                         load_elem(k_idx, dtype, (kbase + s) * d_I + d, table) * ks;
                const double wij = (double)w[(int64_t)i * H_I + j];
                double a, da;
                if (act == OR_ACT_GELU) {
                    const double cdf = 0.5 * (1.0 + erf(x / sqrt(2.0)));
                    a = x * cdf;
                    da = cdf + x * exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846);
                } else {
                    a = x > 0.0 ? x : 0.0;
                    da = x > 0.0 ? 1.0 : 0.0;
                }
                dw[(int64_t)i * H_I + j] += ge * a;
                const double c = ge * wij * da;
                if (c == 0.0) continue;
                for (int d = 0; d < d_I; ++d) {
                    dq_idx[((int64_t)i * H_I + j) * d_I + d] += c * load_elem(k_idx, dtype, (kbase + s) * d_I + d, table) * ks;
                    dk_idx[(kbase + s) * d_I + d] += c * load_elem(q_idx, dtype, ((int64_t)i * H_I + j) * d_I + d, table);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Backward of the sparse MQA attention.  [P2] 【稀疏训练阶段】 / [P5]: the
 * sparse training stage updates every parameter through the sparse attention,
 * so its gradient flows to the query and, by scatter-add, to the latent rows
 * that were selected.  For row i, head h, selected positions S (entries of
 * idx >= 0), z_s = scale q_h . kv_s, P = softmax(z), out_h = sum_s P_s v_s
 * (v_s = kv_s[0:d_v]) and the upstream gradient dout_h:
 *   dP_s = dout_h . v_s,  D_h = dout_h . out_h = sum_s P_s dP_s,
 *   dz_s = P_s (dP_s - D_h),
 *   dq_h   = scale sum_s dz_s kv_s
 *   dkv_s += scale dz_s q_h   (all d_qk columns)  +  P_s dout_h   (first d_v)
 * dkv is accumulated over rows and heads (the caller zeroes it). */
/* ------------------------------------------------------------------ */
int dsa_oracle_sparse_mla_backward(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                                   int nrows, const int32_t* rows,
                                   const void* q, const void* kv, int dtype,
                                   const int32_t* idx, int k, int H, int d_qk, int d_v, double scale,
                                   const double* dout, double* dq, double* dkv) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    double* z = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
    double* dp = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
    double* o = (double*)malloc((size_t)(d_v > 0 ? d_v : 1) * sizeof(double));
    int rc = 0;
    for (int i = 0; i < nrows && rc == 0; ++i) {
        int64_t pos, kbase;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0) { rc = -1; break; }
        const int32_t* sel = idx + (int64_t)i * k;
        for (int h = 0; h < H; ++h) {
            const int64_t qo = ((int64_t)i * H + h) * d_qk;
            double* dqh = dq + qo;
            for (int d = 0; d < d_qk; ++d) dqh[d] = 0.0;
            double m = -INFINITY;
            int nvalid = 0;
            for (int e = 0; e < k; ++e) {
                if (sel[e] < 0) continue;
                if (sel[e] > pos) { rc = -1; break; }
                double dot = 0.0;
                for (int d = 0; d < d_qk; ++d)
                    dot += load_elem(q, dtype, qo + d, table) * load_elem(kv, dtype, (kbase + sel[e]) * d_qk + d, table);
                z[e] = scale * dot;
                if (z[e] > m) m = z[e];
                ++nvalid;
            }
            if (rc != 0 || nvalid == 0) continue;
            double l = 0.0;
            for (int e = 0; e < k; ++e)
                if (sel[e] >= 0) l += exp(z[e] - m);
            /* probabilities, the output and dP */
            const double* dO = dout + ((int64_t)i * H + h) * d_v;
            for (int d = 0; d < d_v; ++d) o[d] = 0.0;
            for (int e = 0; e < k; ++e) {
                if (sel[e] < 0) continue;
                z[e] = exp(z[e] - m) / l;  /* now P */
                double acc = 0.0;
                for (int d = 0; d < d_v; ++d) {
                    const double v = load_elem(kv, dtype, (kbase + sel[e]) * d_qk + d, table);
                    o[d] += z[e] * v;
                    acc += dO[d] * v;
                }
                dp[e] = acc;
            }
            double D = 0.0;
            for (int d = 0; d < d_v; ++d) D += dO[d] * o[d];
            for (int e = 0; e < k; ++e) {
                if (sel[e] < 0) continue;
                const double dz = z[e] * (dp[e] - D);
                double* row = dkv + (kbase + sel[e]) * d_qk;
                for (int d = 0; d < d_qk; ++d) {
                    const double c = load_elem(kv, dtype, (kbase + sel[e]) * d_qk + d, table);
                    dqh[d] += scale * dz * c;
                    row[d] += scale * dz * load_elem(q, dtype, qo + d, table);
                }
                for (int d = 0; d < d_v; ++d) row[d] += z[e] * dO[d];
            }
        }
    }
    free(z);
    free(dp);
    free(o);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Dense causal MQA: attention of every query row over all its candidates
 * [0, pos], no selection.  [P2] 【推理成本评估】 describes this "masked mode"
 * for short prefill, where DSA is emulated by a mask over the dense
 * attention; [P1] "在MLA下實例化DSA" gives the MQA form (one latent per
 * position, key = all columns, value = the first d_v).  Same plain
 * definition as above with the candidate set S = [0, pos]. */
/* ------------------------------------------------------------------ */
int dsa_oracle_dense_mla(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                         int nrows, const int32_t* rows,
                         const void* q, const void* kv, int dtype,
                         int H, int d_qk, int d_v, double scale, double* out, double* lse) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = dsa_oracle_e4m3_value(c);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < nrows; ++i) {
        int64_t pos, kbase;
        if (locate_row(nseq, cu_q, cu_k, rows[i], &pos, &kbase) != 0) { bad |= 1; continue; }
        const int64_t n = pos + 1;
        double* z = (double*)malloc((size_t)n * sizeof(double));
        for (int h = 0; h < H; ++h) {
            double* o = out + ((int64_t)i * H + h) * d_v;
            double m = -INFINITY;
            for (int64_t s = 0; s < n; ++s) {
                double dot = 0.0;
                for (int d = 0; d < d_qk; ++d)
                    dot += load_elem(q, dtype, ((int64_t)i * H + h) * d_qk + d, table) *
                           load_elem(kv, dtype, (kbase + s) * d_qk + d, table);
                z[s] = scale * dot;
                if (z[s] > m) m = z[s];
            }
            double l = 0.0;
            for (int d = 0; d < d_v; ++d) o[d] = 0.0;
            for (int64_t s = 0; s < n; ++s) {
                double p = exp(z[s] - m);
                l += p;
                for (int d = 0; d < d_v; ++d) o[d] += p * load_elem(kv, dtype, (kbase + s) * d_qk + d, table);
            }
            for (int d = 0; d < d_v; ++d) o[d] /= l;
            if (lse) lse[(int64_t)i * H + h] = m + log(l);
        }
        free(z);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* The three steps in order for a list of rows.  The scores are rounded to
 * binary32 (round-to-nearest-even, the C cast) before selection, since the
 * score tensor the method ranks is fp32.  scores_out / idx_out may be NULL. */
/* ------------------------------------------------------------------ */
int dsa_oracle_forward(int nseq, const int32_t* cu_q, const int32_t* cu_k,
                       int nrows, const int32_t* rows,
                       const void* q_idx, const void* k_idx, int idx_dtype, const uint8_t* k_scale,
                       const float* w, int H_I, int d_I, int act,
                       const void* q, const void* kv, int dtype,
                       int H, int d_qk, int d_v, double scale, int k,
                       int64_t ld, double* out, double* lse,
                       float* scores_out, int32_t* idx_out) {
    double* sc = (double*)malloc((size_t)nrows * (size_t)ld * sizeof(double));
    float* sf = (float*)malloc((size_t)nrows * (size_t)ld * sizeof(float));
    int32_t* sel = (int32_t*)malloc((size_t)nrows * (size_t)(k > 0 ? k : 1) * sizeof(int32_t));
    int rc = -1;
    if (!sc || !sf || !sel) goto done;
    for (int64_t e = 0; e < (int64_t)nrows * ld; ++e) sc[e] = 0.0;
    if (dsa_oracle_indexer(nseq, cu_q, cu_k, nrows, rows, q_idx, k_idx, idx_dtype, k_scale, w, H_I, d_I, act, sc, ld)) goto done;
    for (int64_t e = 0; e < (int64_t)nrows * ld; ++e) sf[e] = (float)sc[e];
    if (dsa_oracle_topk(nseq, cu_q, cu_k, nrows, rows, sf, ld, k, sel)) goto done;
    if (dsa_oracle_sparse_mla(nseq, cu_q, cu_k, nrows, rows, q, kv, dtype, sel, k, H, d_qk, d_v, scale, out, lse)) goto done;
    if (scores_out) memcpy(scores_out, sf, (size_t)nrows * (size_t)ld * sizeof(float));
    if (idx_out) memcpy(idx_out, sel, (size_t)nrows * (size_t)k * sizeof(int32_t));
    rc = 0;
done:
    free(sc);
    free(sf);
    free(sel);
    return rc;
}
