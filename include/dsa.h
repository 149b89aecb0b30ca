/*
 * dsa.h - C ABI of the MI355X (gfx950) DSA library: lightning indexer ->
 * top-k selection -> sparse MQA attention.
 *
 * The method is the one on the DeepSeek-V3.2 DSA page (kwkr.cn/news/60693):
 *   section 3.2  indexer score relu(q_idx . k_idx * d_idx^-0.5) per query/key
 *   section 3.3  each query keeps its top_k highest-scoring keys; ordinary
 *                softmax attention then runs over those keys only
 *   section 4.1  FP8 indexer inputs (BF16 also accepted, section 7.3), a
 *                comparison-based selection, BF16 attention
 *   section 4.2  every query head shares one K/V set (MQA)
 *   section 4.3  the whole chain as one call (dsa_forward)
 *   section 7.2  top_k / index_dim / precision are per-workload parameters
 *
 * Conventions for every call:
 *   - Tensors are caller-owned DEVICE memory, row-major and contiguous, each
 *     pointer 16-byte aligned. The library never allocates, frees or keeps a
 *     pointer after the call returns; all work is enqueued on `stream` (a
 *     hipStream_t; NULL is the default stream) and is complete when that
 *     stream is synchronised.
 *   - Query i (0-based) of a sequence sits at position pos(i) = q_pos0 + i and
 *     sees keys 0..pos(i) (itself included). Prefill is q_pos0 = 0 with
 *     n_q = n_k; one decode token is n_q = 1, q_pos0 = n_k - 1.
 *   - All arguments are validated on the host before anything is enqueued; on
 *     any error nothing is enqueued and a negative dsa_status is returned,
 *     with a sentence in dsa_last_error(). A failed HIP launch returns
 *     DSA_E_HIP. Device faults surface at the caller's synchronisation.
 *   - No call blocks the host or synchronises the stream, except the
 *     profiling variants (dsa_forward_timed and the other *_timed calls).
 *   - With the environment variable DSA_LOG set (to anything but "" or "0"),
 *     every forward call prints one line to stderr: the problem, the
 *     selection path it takes (many-row selection, score rows, or the decode
 *     selection) and the workspace bytes it uses.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_E_NULL = -1,        /* a required pointer is NULL */
    DSA_E_SHAPE = -2,       /* sizes out of range or inconsistent */
    DSA_E_UNSUPPORTED = -3, /* a valid problem this library does not handle */
    DSA_E_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    DSA_E_WORKSPACE = -5,   /* workspace missing or smaller than required */
    DSA_E_HIP = -6          /* the HIP runtime reported an error */
} dsa_status;

/* Element type of q_idx / k_idx (the "precision" parameter). */
typedef enum {
    DSA_IDX_FP8_E4M3FN = 0, /* OCP float8 e4m3fn, 1 byte */
    DSA_IDX_BF16 = 1        /* bfloat16, 2 bytes */
} dsa_idx_dtype;

/* Which call a workspace size is asked for. */
typedef enum { DSA_OP_TOPK = 1, DSA_OP_ATTN = 2, DSA_OP_FORWARD = 3 } dsa_op;

/* Problem description shared by every call.
 *   batch     B >= 1 independent sequences
 *   n_q       queries per sequence, 1 <= n_q, q_pos0 + n_q <= n_k
 *   n_k       keys per sequence, 1 <= n_k <= 4194304
 *   q_pos0    position of query 0 (>= 0)
 *   d_idx     indexer dimension ("index_dim"): a multiple of 32, 32..256
 *   idx_dtype a dsa_idx_dtype
 *   top_k     keys kept per query, 1..4096
 *   n_heads   H query heads sharing one K/V row set, 1..16
 *   head_dim  must be 128 */
typedef struct {
    int32_t batch, n_q, n_k, q_pos0;
    int32_t d_idx, idx_dtype;
    int32_t top_k;
    int32_t n_heads, head_dim;
} dsa_problem;

/* Bytes of device workspace `op` needs for problem `p` (written to *bytes;
 * 0 means no workspace). Pure host function. */
dsa_status dsa_workspace_size(const dsa_problem* p, int32_t op, size_t* bytes);

/* Indexer scores (DSA page, section 3.2) for query rows [q_begin, q_end) of
 * every sequence:
 *   scores[b][r][j] = relu(fl32(q_idx[b][q_begin+r] . k_idx[b][j]) * s),
 *   s = dim^-0.5 rounded to float32, for j <= pos(q_begin+r);
 *   scores[b][r][j] = -inf for j > pos(q_begin+r).
 * q_idx [B][n_q][d_idx], k_idx [B][n_k][d_idx] in idx_dtype;
 * scores float32 [B][q_end-q_begin][n_k]. The dot product is accumulated in
 * float32 on matrix cores, exact whenever every partial sum is (for example
 * for the small-integer inputs of the benchmarks). Needs 0 <= q_begin < q_end
 * <= n_q. */
dsa_status dsa_index_scores(const dsa_problem* p, const void* q_idx,
                            const void* k_idx, int32_t q_begin, int32_t q_end,
                            float* scores, void* stream);

/* Top-k selection (DSA page, section 3.3) over score rows produced as above:
 * row r of sequence b belongs to query q_begin + r and its candidates are keys
 * 0..pos(q_begin+r). Keeps the min(top_k, pos+1) candidates ranked first by
 * (score descending, key index ascending) - ties go to the lower index - and
 * writes them in ascending key order, padding the row with -1:
 * idx int32 [B][q_end-q_begin][top_k]. Scores must be >= +0.0 or -inf (as the
 * indexer writes them); ranking compares float32 bit patterns. */
dsa_status dsa_topk(const dsa_problem* p, const float* scores, int32_t q_begin,
                    int32_t q_end, int32_t* idx, void* ws, size_t ws_bytes,
                    void* stream);

/* Sparse MQA attention (DSA page, sections 3.3 and 4.2) for all n_q queries:
 *   O[b][i][h] = sum_{j in sel} softmax_j(Q[b][i][h] . K[b][j] / sqrt(128)) V[b][j]
 * where sel is the set of entries of idx[b][i][0..top_k) inside [0, n_k)
 * (entries outside, such as the -1 padding, are ignored; an empty set gives
 * O = 0 and lse = -inf). Q [B][n_q][H][128], K, V [B][n_k][128] bfloat16;
 * idx int32 [B][n_q][top_k]; O bfloat16 [B][n_q][H][128]; lse (optional,
 * NULL to skip) float32 [B][n_q][H], natural-log sum of exp of the scaled
 * scores. Accumulation is float32; probabilities enter the PV product as
 * bfloat16. */
dsa_status dsa_sparse_attn(const dsa_problem* p, const void* Q, const void* K,
                           const void* V, const int32_t* idx, void* O,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

/* The whole chain (DSA page, section 4.3): indexer scores, top-k, sparse
 * attention, with the same definitions and layouts as the three calls above.
 * idx_out (optional) receives the selection [B][n_q][top_k]; lse optional.
 * Intermediate scores live in the workspace. */
dsa_status dsa_forward(const dsa_problem* p, const void* q_idx,
                       const void* k_idx, const void* Q, const void* K,
                       const void* V, int32_t* idx_out, void* O, float* lse,
                       void* ws, size_t ws_bytes, void* stream);

/* dsa_forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). The same work and results as dsa_forward, with the
 * workspace in a static device array of DSA_NOALLOC_SCRATCH_BYTES (128 MiB)
 * that the library holds on every GPU it runs on until the process ends; the
 * call itself allocates nothing. Problems whose forward workspace
 * (dsa_workspace_size with DSA_OP_FORWARD) exceeds that size are refused with
 * DSA_E_WORKSPACE before anything is enqueued: every decode batch up to
 * 64 x 128K keys with top_k 2048 fits, long prefills do not. Every call on
 * a GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be ordered by
 * the caller. The stream must belong to the current device (else
 * DSA_E_UNSUPPORTED). Other errors: those of dsa_forward. */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dsa_status dsa_forward_noalloc(const dsa_problem* p, const void* q_idx,
                               const void* k_idx, const void* Q, const void* K,
                               const void* V, int32_t* idx_out, void* O,
                               float* lse, void* stream);

/* dsa_forward for a ragged decode batch (DSA page, sections 3.3 and 4.3, per
 * sequence): one query per sequence (n_q = 1, and q_pos0 = 0 in *p), the
 * query of sequence b at position seq_pos[b], seeing keys 0..seq_pos[b] of its
 * row of n_k keys. Sequences of different lengths share the padded
 * [B][n_k] layouts of dsa_forward; keys past a sequence's position are never
 * read for it. seq_pos: int32 [B], device memory, 16-byte aligned; a value
 * >= n_k acts as n_k - 1, and a value < 0 leaves the sequence's row empty
 * (idx all -1, O = 0, lse = -inf). Results per sequence equal dsa_forward on
 * that sequence alone with q_pos0 = seq_pos[b]. Same workspace as
 * dsa_forward (dsa_workspace_size with DSA_OP_FORWARD). Errors: DSA_E_NULL
 * (seq_pos NULL), DSA_E_SHAPE (q_pos0 != 0), DSA_E_UNSUPPORTED (n_q != 1),
 * and those of dsa_forward. */
dsa_status dsa_forward_ragged(const dsa_problem* p, const int32_t* seq_pos,
                              const void* q_idx, const void* k_idx,
                              const void* Q, const void* K, const void* V,
                              int32_t* idx_out, void* O, float* lse, void* ws,
                              size_t ws_bytes, void* stream);

/* dsa_forward_ragged for profiling: the same work and results, plus the
 * device time of each stage, as dsa_forward_timed reports it (blocks until
 * the stream has finished; stage_ms must not be NULL). */
dsa_status dsa_forward_ragged_timed(const dsa_problem* p, const int32_t* seq_pos,
                                    const void* q_idx, const void* k_idx,
                                    const void* Q, const void* K, const void* V,
                                    int32_t* idx_out, void* O, float* lse,
                                    void* ws, size_t ws_bytes, void* stream,
                                    float* stage_ms, int32_t* n_slabs);

/* A paged key layout: the keys of every sequence live in pages of page_size
 * rows inside shared pools, logical key j of sequence b in row
 * block_table[b][j / page_size] * page_size + j % page_size of a pool.
 *   block_table  int32 [batch][pages_per_seq], device memory, 16-byte aligned
 *                (ids outside [0, n_pages) are clamped into it)
 *   page_size    keys per page (>= 1; multiples of 256 let the indexer stream
 *                whole pages, other sizes translate key by key)
 *   pages_per_seq  logical pages per sequence; n_k = pages_per_seq * page_size
 *   n_pages      pages in each pool (n_pages * page_size * 256 < 4 GiB) */
typedef struct {
    const int32_t* block_table;
    int32_t page_size, pages_per_seq, n_pages;
} dsa_pages;

/* dsa_forward_ragged over a paged layout (same definitions): k_pool
 * [n_pages][page_size][d_idx] in idx_dtype, K_pool and V_pool
 * [n_pages][page_size][128] bfloat16 replace k_idx, K and V; idx_out holds
 * logical key indices as for dsa_forward. Same workspace as dsa_forward.
 * Errors: those of dsa_forward_ragged; DSA_E_NULL (pages or its table
 * NULL); DSA_E_SHAPE (page sizes as above). */
dsa_status dsa_forward_paged(const dsa_problem* p, const int32_t* seq_pos,
                             const dsa_pages* pages, const void* q_idx,
                             const void* k_pool, const void* Q,
                             const void* K_pool, const void* V_pool,
                             int32_t* idx_out, void* O, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* dsa_forward_paged for profiling, as dsa_forward_timed (blocks until the
 * stream has finished; stage_ms must not be NULL). */
dsa_status dsa_forward_paged_timed(const dsa_problem* p, const int32_t* seq_pos,
                                   const dsa_pages* pages, const void* q_idx,
                                   const void* k_pool, const void* Q,
                                   const void* K_pool, const void* V_pool,
                                   int32_t* idx_out, void* O, float* lse,
                                   void* ws, size_t ws_bytes, void* stream,
                                   float* stage_ms, int32_t* n_slabs);

/* dsa_forward with threshold-mode selection. The sparse-attention explainer
 * page (yunthe.com/news/469461.html), section 2.2, keeps for each query the
 * keys whose similarity exceeds a threshold; here the similarity is the
 * indexer score S (DSA page, section 3.2) and top_k bounds the kept set:
 * query i keeps {j <= pos(i) : S_j > tau} (a float32 comparison, strict), and
 * when more than top_k keys pass, the top_k highest of them (ties to the lower
 * key index), which is the top-k selection of dsa_forward with the entries
 * scoring <= tau removed. idx_out rows list the kept keys in ascending order,
 * -1 padded (a query may keep none: O = 0, lse = -inf). Since S >= 0, a
 * negative tau gives dsa_forward's results; a NaN tau keeps nothing. Same
 * layouts, workspace and errors as dsa_forward. */
dsa_status dsa_forward_threshold(const dsa_problem* p, float tau,
                                 const void* q_idx, const void* k_idx,
                                 const void* Q, const void* K, const void* V,
                                 int32_t* idx_out, void* O, float* lse,
                                 void* ws, size_t ws_bytes, void* stream);

/* dsa_forward_threshold for profiling, as dsa_forward_timed (the threshold
 * pass counts as top-k time; blocks until the stream has finished; stage_ms
 * must not be NULL). */
dsa_status dsa_forward_threshold_timed(const dsa_problem* p, float tau,
                                       const void* q_idx, const void* k_idx,
                                       const void* Q, const void* K,
                                       const void* V, int32_t* idx_out, void* O,
                                       float* lse, void* ws, size_t ws_bytes,
                                       void* stream, float* stage_ms,
                                       int32_t* n_slabs);

/* dsa_forward for profiling: the same work and results, plus the device time
 * of each stage. HIP events are recorded on `stream` around the indexer
 * kernel, the top-k kernels and the attention kernels of every row slab; the
 * call then waits for the stream (it blocks the calling thread, unlike
 * dsa_forward) and writes the milliseconds spent in each stage, summed over
 * slabs, to stage_ms[0] (indexer), stage_ms[1] (top-k) and stage_ms[2]
 * (attention), and the number of row slabs (indexer launches) to *n_slabs
 * (optional). stage_ms must not be NULL. */
dsa_status dsa_forward_timed(const dsa_problem* p, const void* q_idx,
                             const void* k_idx, const void* Q, const void* K,
                             const void* V, int32_t* idx_out, void* O,
                             float* lse, void* ws, size_t ws_bytes,
                             void* stream, float* stage_ms, int32_t* n_slabs);

/* Layout and mode of dsa_forward_ext (any combination):
 *   seq_pos         optional: a ragged decode batch, as dsa_forward_ragged
 *   pages           optional: a paged key layout, as dsa_forward_paged (needs
 *                   seq_pos; k_idx, K and V are then the pools)
 *   threshold_mode  nonzero: threshold-mode selection at tau, as
 *                   dsa_forward_threshold */
typedef struct {
    const int32_t* seq_pos;
    const dsa_pages* pages;
    int32_t threshold_mode;
    float tau;
} dsa_forward_options;

/* dsa_forward with the options above (NULL options: dsa_forward itself). The
 * definitions, layouts, workspace and errors are those of the entry points
 * each option stands for; results equal theirs bit for bit. */
dsa_status dsa_forward_ext(const dsa_problem* p, const dsa_forward_options* options,
                           const void* q_idx, const void* k_idx, const void* Q,
                           const void* K, const void* V, int32_t* idx_out, void* O,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

/* dsa_forward_ext for profiling, as dsa_forward_timed (blocks until the
 * stream has finished; stage_ms must not be NULL). */
dsa_status dsa_forward_ext_timed(const dsa_problem* p,
                                 const dsa_forward_options* options,
                                 const void* q_idx, const void* k_idx,
                                 const void* Q, const void* K, const void* V,
                                 int32_t* idx_out, void* O, float* lse,
                                 void* ws, size_t ws_bytes, void* stream,
                                 float* stage_ms, int32_t* n_slabs);

/* The indexer projections (DSA page, section 3.2: query_proj and key_proj
 * are bias-free linear maps from the model width d_model to the indexer
 * width d_idx; section 4.1: the index stage runs in FP8). For each input row
 * r of X and output feature o,
 *   y = fl32(sum_c X[r][c] * W[o][c])   (fp32 accumulation)
 * is encoded in out_dtype into row out_rows[r] of out (row r when out_rows is
 * NULL):
 *   DSA_IDX_FP8_E4M3FN  round to nearest, ties to even; |y| >= 448 gives
 *                       +-448 (saturating), NaN the NaN code
 *   DSA_IDX_BF16        round to nearest, ties to even
 * X bfloat16 [rows][d_model]; W bfloat16 [d_idx][d_model] (nn.Linear's weight
 * layout); out [n_out][d_idx] in out_dtype; other rows of out are not
 * touched, so out_rows = b * n_k + pos appends a decode step's new keys to a
 * k_idx cache [B][n_k][d_idx]. out_rows: optional int32 [rows], device
 * memory, 16-byte aligned; entries outside [0, n_out) are skipped; two input
 * rows sent to one output row leave either. d_model: a multiple of 32 in
 * [32, 65536]; d_idx: a multiple of 32 in [32, 256]. Sums over d_model are
 * exact (order-independent) when the products and partial sums are
 * integers below 2^24; otherwise the fp32 summation order is fixed, so
 * results repeat bit for bit. No workspace. Errors: DSA_E_NULL,
 * DSA_E_ALIGN (pointers), DSA_E_SHAPE (rows < 1, n_out < 1, or n_out < rows
 * without out_rows), DSA_E_UNSUPPORTED (widths, dtype). */
dsa_status dsa_index_project(int32_t rows, int32_t d_model, int32_t d_idx,
                             int32_t out_dtype, const void* X, const void* W,
                             void* out, const int32_t* out_rows, int32_t n_out,
                             void* stream);

/* Static name of a status code. */
const char* dsa_status_str(int32_t status);

/* Detail of the last error reported on the calling thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
