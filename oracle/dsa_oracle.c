/*
 * CPU oracle for the DSA lightning-indexer -> top-k -> sparse MQA attention
 * path. TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
 * CPU-baseline leg may call it; the product path never does. It shares no
 * code, header or constant with the GPU library.
 *
 * Source of the method: the DeepSeek-V3.2 DSA page (kwkr.cn/news/60693).
 *   section 3.2  the lightning indexer: scores = relu(q k^T * dim^-0.5)
 *   section 3.3  each query keeps its top-k keys, then ordinary attention
 *                runs over those keys only
 *   section 4.1  FP8 index stage, comparison-based selection, BF16 attention
 *   section 4.2  all query heads share one K/V set (MQA)
 * Threshold-mode selection follows the sparse-attention explainer page
 * (yunthe.com/news/469461.html), section 2.2: keys whose similarity exceeds
 * a threshold are kept.
 * Readings where the page is silent (causal inclusion j <= pos, ties to the
 * lower key index, ascending output order with -1 padding, fp32 rounding of
 * the scale) are listed with the design notes of this repository.
 *
 * Everything is plain loops; floating point is accumulated in double. OpenMP
 * runs only across independent query rows, so results do not depend on the
 * thread count. Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC.
 * Parity status: every function here is pinned by tests (brute force, closed
 * forms, invariants, hand-worked example); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_FP8_E4M3FN = 0, ORACLE_BF16 = 1 };

/* OCP FP8 E4M3 ("fn": no infinities): 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN. */
static double dec_e4m3fn(uint8_t v) {
    int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
    double x;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) x = ldexp((double)m, -9);
    else x = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -x : x;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double dec_bf16(uint16_t v) {
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double dec_idx(const void* base, int dtype, size_t i) {
    if (dtype == ORACLE_FP8_E4M3FN) return dec_e4m3fn(((const uint8_t*)base)[i]);
    return dec_bf16(((const uint16_t*)base)[i]);
}

/* Encoding a float32 value as e4m3fn: the nearest representable value, ties
 * to the code with an even mantissa (its low bit 0), magnitudes beyond the
 * largest finite value 448 saturating to +-448, NaN to the NaN code; the sign
 * (also of a zero) is kept. The nearest code is found by bisection over the
 * non-negative finite codes 0x00..0x7e, whose values increase with the code. */
static uint8_t enc_e4m3fn_sat(float v) {
    if (v != v) return 0x7f;
    uint8_t s = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return s | 0x7e;
    int lo = 0, hi = 0x7e;               /* dec(lo) <= a < dec(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (dec_e4m3fn((uint8_t)mid) <= a) lo = mid;
        else hi = mid;
    }
    double dl = a - dec_e4m3fn((uint8_t)lo), dh = dec_e4m3fn((uint8_t)hi) - a;
    int c = dl < dh ? lo : dh < dl ? hi : ((lo & 1) ? hi : lo);
    return s | (uint8_t)c;
}

/* Encoding a float32 value as bfloat16: of the two bfloat16 values around it
 * (the upper half of its bits, and the next value away from zero) the nearer,
 * ties to the even one; NaN to the quiet NaN 0x7fc0. */
static uint16_t enc_bf16(float v) {
    if (v != v) return 0x7fc0;
    uint32_t u;
    memcpy(&u, &v, 4);
    uint16_t t = (uint16_t)(u >> 16);
    if ((u & 0xffffu) == 0) return t;
    double a = fabs((double)v);
    double dl = a - fabs(dec_bf16(t)), dh = fabs(dec_bf16((uint16_t)(t + 1))) - a;
    return dl < dh ? t : dh < dl ? (uint16_t)(t + 1) : ((t & 1) ? (uint16_t)(t + 1) : t);
}

/* The indexer's scale, dim^-0.5, evaluated in double as the page's Python
 * expression does and then rounded once to float32, the type the scores are
 * multiplied in. */
float oracle_index_scale(int d) { return (float)pow((double)d, -0.5); }

/* One indexer score (DSA page section 3.2): the dot product of the query and
 * key indexer vectors, rounded to float32, times the float32 scale, then ReLU.
 * A negative or zero product becomes +0.0. */
static float index_score(const void* q_idx, const void* k_idx, int dtype,
                         size_t qoff, size_t koff, int d, float scale) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c)
        acc += dec_idx(q_idx, dtype, qoff + c) * dec_idx(k_idx, dtype, koff + c);
    float x = (float)acc;
    float s = x * scale;
    return s > 0.0f ? s : 0.0f;
}

/* scores[b][r][j] for query rows i = q_begin + r of every sequence b, all keys
 * j < n_k. Query i sits at position q_pos0 + i and sees keys j <= pos; keys
 * past pos are not candidates and read -inf. Returns 0, or -1 on bad sizes. */
int oracle_index_scores(int B, int n_q, int n_k, int q_pos0, int d, int dtype,
                        const void* q_idx, const void* k_idx,
                        int q_begin, int q_end, float* scores) {
    if (B < 0 || n_q < 0 || n_k < 0 || d <= 0 || q_begin < 0 || q_end > n_q ||
        q_begin > q_end || (dtype != ORACLE_FP8_E4M3FN && dtype != ORACLE_BF16))
        return -1;
    const float scale = oracle_index_scale(d);
    const int rows = q_end - q_begin;
    const long total = (long)B * rows;
#pragma omp parallel for schedule(dynamic, 4)
    for (long t = 0; t < total; ++t) {
        int b = (int)(t / rows), r = (int)(t % rows), i = q_begin + r;
        long pos = (long)q_pos0 + i;
        float* out = scores + ((size_t)b * rows + r) * n_k;
        size_t qoff = ((size_t)b * n_q + i) * d;
        for (int j = 0; j < n_k; ++j) {
            if (j > pos) { out[j] = -INFINITY; continue; }
            out[j] = index_score(q_idx, k_idx, dtype, qoff,
                                 ((size_t)b * n_k + j) * d, d, scale);
        }
    }
    return 0;
}

typedef struct { float s; int32_t j; } cand_t;

/* Total order of the selection (DSA page section 3.3 keeps the k highest
 * scores; ties go to the lower key index): a precedes b iff a's score is
 * higher, or the scores are equal and a's index is lower. */
static int cmp_rank(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int cmp_int(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/* Top-k of one row: the first min(k, pos+1) candidates j <= pos under the
 * total order above, written in ascending j, the rest of the k slots -1. */
static void topk_row(const float* row, int n_k, long pos, int k, cand_t* buf,
                     int32_t* out) {
    int n = (int)(pos + 1 < n_k ? pos + 1 : n_k);
    for (int j = 0; j < n; ++j) { buf[j].s = row[j]; buf[j].j = j; }
    qsort(buf, (size_t)n, sizeof(cand_t), cmp_rank);
    int m = n < k ? n : k;
    for (int t = 0; t < m; ++t) out[t] = buf[t].j;
    qsort(out, (size_t)m, sizeof(int32_t), cmp_int);
    for (int t = m; t < k; ++t) out[t] = -1;
}

/* Threshold-mode selection of one row. The sparse-attention explainer page
 * (yunthe.com/news/469461.html, section 2.2) keeps, for each query, the keys
 * whose similarity exceeds a threshold; here the similarity is the indexer
 * score and the kept set is bounded by the k output slots: the candidates
 * j <= pos with score > tau, and when more than k of them pass, the first k
 * under the total order above. Written in ascending j, the rest -1. */
static void thresh_row(const float* row, int n_k, long pos, int k, float tau, cand_t* buf,
                       int32_t* out) {
    int n = (int)(pos + 1 < n_k ? pos + 1 : n_k);
    int c = 0;
    for (int j = 0; j < n; ++j)
        if (row[j] > tau) { buf[c].s = row[j]; buf[c].j = j; ++c; }
    qsort(buf, (size_t)c, sizeof(cand_t), cmp_rank);
    int m = c < k ? c : k;
    for (int t = 0; t < m; ++t) out[t] = buf[t].j;
    qsort(out, (size_t)m, sizeof(int32_t), cmp_int);
    for (int t = m; t < k; ++t) out[t] = -1;
}

/* idx[b][r][0..k) for score rows scores[b][r][0..n_k) whose query sits at
 * position pos_begin + r. Returns 0, -1 on bad sizes, -2 on no memory. */
int oracle_topk(int B, int rows, int n_k, int pos_begin, int k,
                const float* scores, int32_t* idx) {
    if (B < 0 || rows < 0 || n_k < 0 || k < 1 || pos_begin < 0) return -1;
    const long total = (long)B * rows;
    int fail = 0;
#pragma omp parallel
    {
        cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n_k > 0 ? n_k : 1));
        if (!buf) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long t = 0; t < total; ++t) {
            if (!buf) continue;
            int r = (int)(t % rows);
            topk_row(scores + (size_t)t * n_k, n_k, (long)pos_begin + r, k, buf,
                     idx + (size_t)t * k);
        }
        free(buf);
    }
    return fail ? -2 : 0;
}

/* The indexer projections (DSA page section 3.2: query_proj and key_proj are
 * bias-free linear maps from the model width to the indexer width; section
 * 4.1 runs the index stage in FP8): for each input row r,
 *   y[o] = sum_c X[r][c] * W[o][c]      (W in nn.Linear's [d_idx][d_model] layout)
 * accumulated in double, rounded to float32, then encoded as e4m3fn
 * (enc_e4m3fn_sat) or bfloat16 (enc_bf16) into out row out_rows[r] (row r
 * when out_rows is NULL) of out [n_out][d_idx]; other rows of out are left
 * as they are (a decode step appends its new key rows to the cache this way).
 * X [rows][d_model] and W are bfloat16 bit patterns. Returns 0, -1 on bad
 * sizes or a destination row outside [0, n_out). */
int oracle_index_project(int rows, int d_model, int d_idx, int out_dtype, const uint16_t* X,
                         const uint16_t* W, const int32_t* out_rows, int n_out, void* out) {
    if (rows < 0 || d_model < 1 || d_idx < 1 || n_out < 0 ||
        (out_dtype != ORACLE_FP8_E4M3FN && out_dtype != ORACLE_BF16))
        return -1;
    for (int r = 0; r < rows; ++r) {
        int dst = out_rows ? out_rows[r] : r;
        if (dst < 0 || dst >= n_out) return -1;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int r = 0; r < rows; ++r) {
        int dst = out_rows ? out_rows[r] : r;
        for (int o = 0; o < d_idx; ++o) {
            double acc = 0.0;
            for (int c = 0; c < d_model; ++c)
                acc += dec_bf16(X[(size_t)r * d_model + c]) * dec_bf16(W[(size_t)o * d_model + c]);
            float y = (float)acc;
            if (out_dtype == ORACLE_FP8_E4M3FN)
                ((uint8_t*)out)[(size_t)dst * d_idx + o] = enc_e4m3fn_sat(y);
            else
                ((uint16_t*)out)[(size_t)dst * d_idx + o] = enc_bf16(y);
        }
    }
    return 0;
}

/* Encodings alone (for pinning them): n float32 values to e4m3fn or bf16. */
int oracle_encode(int n, int out_dtype, const float* v, void* out) {
    if (n < 0 || (out_dtype != ORACLE_FP8_E4M3FN && out_dtype != ORACLE_BF16)) return -1;
    for (int i = 0; i < n; ++i) {
        if (out_dtype == ORACLE_FP8_E4M3FN) ((uint8_t*)out)[i] = enc_e4m3fn_sat(v[i]);
        else ((uint16_t*)out)[i] = enc_bf16(v[i]);
    }
    return 0;
}

/* oracle_topk in threshold mode (thresh_row): the keys scoring above tau, at
 * most k per row. */
int oracle_select_threshold(int B, int rows, int n_k, int pos_begin, int k, float tau,
                            const float* scores, int32_t* idx) {
    if (B < 0 || rows < 0 || n_k < 0 || k < 1 || pos_begin < 0) return -1;
    const long total = (long)B * rows;
    int fail = 0;
#pragma omp parallel
    {
        cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n_k > 0 ? n_k : 1));
        if (!buf) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long t = 0; t < total; ++t) {
            if (!buf) continue;
            int r = (int)(t % rows);
            thresh_row(scores + (size_t)t * n_k, n_k, (long)pos_begin + r, k, tau, buf,
                       idx + (size_t)t * k);
        }
        free(buf);
    }
    return fail ? -2 : 0;
}

/* Attention of one query (DSA page sections 3.3 and 4.2): for each head h,
 * ordinary softmax attention over the selected keys only, with the K/V rows
 * shared by all heads. z_j = Q_h . K_j / sqrt(D); O_h = sum_j w_j V_j / sum w,
 * w_j = exp(z_j - max z); lse_h = max z + log(sum w). An empty selection
 * gives O = 0 and lse = -inf. */
static void attn_row(int H, int D, int n_k, int k, const uint16_t* q,
                     const uint16_t* Kb, const uint16_t* Vb, const int32_t* sel,
                     double* z, double* acc, float* o, float* lse) {
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int h = 0; h < H; ++h) {
        const uint16_t* qh = q + (size_t)h * D;
        double m = -INFINITY;
        int n = 0;
        for (int t = 0; t < k; ++t) {
            int j = sel[t];
            if (j < 0 || j >= n_k) continue;
            double dot = 0.0;
            for (int c = 0; c < D; ++c)
                dot += dec_bf16(qh[c]) * dec_bf16(Kb[(size_t)j * D + c]);
            z[n] = dot * inv_sqrt_d;
            if (z[n] > m) m = z[n];
            ++n;
        }
        for (int c = 0; c < D; ++c) acc[c] = 0.0;
        if (n == 0) {
            for (int c = 0; c < D; ++c) o[(size_t)h * D + c] = 0.0f;
            if (lse) lse[h] = -INFINITY;
            continue;
        }
        double l = 0.0;
        n = 0;
        for (int t = 0; t < k; ++t) {
            int j = sel[t];
            if (j < 0 || j >= n_k) continue;
            double w = exp(z[n++] - m);
            l += w;
            for (int c = 0; c < D; ++c) acc[c] += w * dec_bf16(Vb[(size_t)j * D + c]);
        }
        for (int c = 0; c < D; ++c) o[(size_t)h * D + c] = (float)(acc[c] / l);
        if (lse) lse[h] = (float)(m + log(l));
    }
}

/* O[b][i][h][0..D) and lse[b][i][h] (lse may be NULL) from Q [B][n_q][H][D],
 * K, V [B][n_k][D] (bfloat16 bit patterns) and idx [B][n_q][k]; entries of
 * idx outside [0, n_k) (the -1 padding) are skipped. */
int oracle_sparse_attn(int B, int n_q, int n_k, int H, int D, int k,
                       const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                       const int32_t* idx, float* O, float* lse) {
    if (B < 0 || n_q < 0 || n_k < 0 || H < 1 || D < 1 || k < 1) return -1;
    const long total = (long)B * n_q;
    int fail = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)k);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (!z || !acc) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long t = 0; t < total; ++t) {
            if (!z || !acc) continue;
            int b = (int)(t / n_q);
            attn_row(H, D, n_k, k, Q + (size_t)t * H * D, K + (size_t)b * n_k * D,
                     V + (size_t)b * n_k * D, idx + (size_t)t * k, z, acc,
                     O + (size_t)t * H * D, lse ? lse + (size_t)t * H : NULL);
        }
        free(z);
        free(acc);
    }
    return fail ? -2 : 0;
}

/* The three stages back to back, one query row at a time (the fused chain of
 * the DSA page, section 4.3: index, select, attend), without materialising
 * the full score matrix. Only query rows [q_begin, q_end) of each sequence are
 * computed; idx/O/lse are laid out [B][q_end-q_begin][...]. idx and lse may be
 * NULL. A non-NULL tau selects in threshold mode (thresh_row). */
static int forward_rows(int B, int n_q, int n_k, int q_pos0, const int32_t* seq_pos, int d,
                        int dtype, int k, const float* tau, int H, int D, const void* q_idx,
                        const void* k_idx,
                        const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                        int q_begin, int q_end, const int32_t* row_list, int32_t* idx, float* O,
                        float* lse) {
    if (B < 0 || n_q < 0 || n_k < 0 || d <= 0 || k < 1 || H < 1 || D < 1 ||
        q_begin < 0 || q_begin > q_end || (!row_list && q_end > n_q) ||
        (dtype != ORACLE_FP8_E4M3FN && dtype != ORACLE_BF16))
        return -1;
    if (row_list)
        for (int r = q_begin; r < q_end; ++r)
            if (row_list[r] < 0 || row_list[r] >= n_q) return -1;
    const float scale = oracle_index_scale(d);
    const int rows = q_end - q_begin;
    const long total = (long)B * rows;
    int fail = 0;
#pragma omp parallel
    {
        float* srow = (float*)malloc(sizeof(float) * (size_t)(n_k > 0 ? n_k : 1));
        cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n_k > 0 ? n_k : 1));
        int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        double* z = (double*)malloc(sizeof(double) * (size_t)k);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        int ok = srow && buf && sel && z && acc;
        if (!ok) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < total; ++t) {
            if (!ok) continue;
            int b = (int)(t / rows), i = row_list ? row_list[q_begin + (int)(t % rows)]
                                                  : q_begin + (int)(t % rows);
            long pos = (long)(seq_pos ? seq_pos[b] : q_pos0) + i;
            size_t qoff = ((size_t)b * n_q + i) * d;
            for (int j = 0; j < n_k; ++j)
                srow[j] = j > pos ? -INFINITY
                                  : index_score(q_idx, k_idx, dtype, qoff,
                                                ((size_t)b * n_k + j) * d, d, scale);
            if (tau) thresh_row(srow, n_k, pos, k, *tau, buf, sel);
            else topk_row(srow, n_k, pos, k, buf, sel);
            if (idx) memcpy(idx + (size_t)t * k, sel, sizeof(int32_t) * (size_t)k);
            attn_row(H, D, n_k, k, Q + (((size_t)b * n_q + i) * H) * D,
                     K + (size_t)b * n_k * D, V + (size_t)b * n_k * D, sel, z, acc,
                     O + (size_t)t * H * D, lse ? lse + (size_t)t * H : NULL);
        }
        free(srow); free(buf); free(sel); free(z); free(acc);
    }
    return fail ? -2 : 0;
}

int oracle_forward(int B, int n_q, int n_k, int q_pos0, int d, int dtype, int k,
                   int H, int D, const void* q_idx, const void* k_idx,
                   const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                   int q_begin, int q_end, int32_t* idx, float* O, float* lse) {
    return forward_rows(B, n_q, n_k, q_pos0, NULL, d, dtype, k, NULL, H, D, q_idx, k_idx, Q,
                        K, V, q_begin, q_end, NULL, idx, O, lse);
}

/* oracle_forward over a list of query rows: entry t of the outputs is query
 * row rows[t] of its sequence (the same per-row chain; rows may repeat or come
 * in any order), so sampled rows of a long prefill run as one parallel call. */
int oracle_forward_rowlist(int B, int n_q, int n_k, int q_pos0, int d, int dtype, int k,
                           int H, int D, const void* q_idx, const void* k_idx,
                           const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                           const int32_t* rows, int n_rows, int32_t* idx, float* O, float* lse) {
    if (!rows || n_rows < 0) return -1;
    return forward_rows(B, n_q, n_k, q_pos0, NULL, d, dtype, k, NULL, H, D, q_idx, k_idx, Q,
                        K, V, 0, n_rows, rows, idx, O, lse);
}

/* oracle_forward with threshold-mode selection: each query attends to the
 * keys whose indexer score exceeds tau, at most k of them (thresh_row). */
int oracle_forward_threshold(int B, int n_q, int n_k, int q_pos0, int d, int dtype, int k,
                             float tau, int H, int D, const void* q_idx, const void* k_idx,
                             const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                             int q_begin, int q_end, int32_t* idx, float* O, float* lse) {
    return forward_rows(B, n_q, n_k, q_pos0, NULL, d, dtype, k, &tau, H, D, q_idx, k_idx, Q,
                        K, V, q_begin, q_end, NULL, idx, O, lse);
}

/* oracle_forward for a batch whose sequences sit at different positions:
 * query i of sequence b is at seq_pos[b] + i (sequences of different lengths
 * in one padded [B][n_k] layout; keys past a query's position are not
 * candidates). */
int oracle_forward_seqpos(int B, int n_q, int n_k, const int32_t* seq_pos, int d, int dtype,
                          int k, int H, int D, const void* q_idx, const void* k_idx,
                          const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                          int q_begin, int q_end, int32_t* idx, float* O, float* lse) {
    if (!seq_pos) return -1;
    return forward_rows(B, n_q, n_k, 0, seq_pos, d, dtype, k, NULL, H, D, q_idx, k_idx, Q, K,
                        V, q_begin, q_end, NULL, idx, O, lse);
}

/* oracle_forward_seqpos with threshold-mode selection (thresh_row). */
int oracle_forward_seqpos_threshold(int B, int n_q, int n_k, const int32_t* seq_pos, int d,
                                    int dtype, int k, float tau, int H, int D, const void* q_idx,
                                    const void* k_idx, const uint16_t* Q, const uint16_t* K,
                                    const uint16_t* V, int q_begin, int q_end, int32_t* idx,
                                    float* O, float* lse) {
    if (!seq_pos) return -1;
    return forward_rows(B, n_q, n_k, 0, seq_pos, d, dtype, k, &tau, H, D, q_idx, k_idx, Q, K, V,
                        q_begin, q_end, NULL, idx, O, lse);
}

/* Threads an OpenMP parallel region of this library runs with. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
