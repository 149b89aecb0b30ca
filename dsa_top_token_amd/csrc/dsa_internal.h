// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Key rows of a sequence either follow one another ([B][n_k] rows) or sit in
// pages of a shared pool: logical key j of sequence b is then row
// table[b][j / page] * page + j % page of the pool. With page a multiple of
// 256 every 256-key run that starts at a multiple of 256 lies in one page
// (run_contiguous); other page sizes translate key by key (RunRows).
struct KeyPages {
    const int32_t* table;   // [B][per_seq] physical page ids; null: [B][n_k] rows
    int page, per_seq, n_pages;
};

// Row holding key j (0 <= j < n_k) of sequence b; page ids are clamped into
// the pool.
__device__ __forceinline__ long long key_row(const KeyPages& pg, int b, int n_k, int j) {
    if (!pg.table) return (long long)b * n_k + j;
    const int lp = j / pg.page;
    const int pp = min(max(pg.table[(size_t)b * pg.per_seq + lp], 0), pg.n_pages - 1);
    return (long long)pp * pg.page + (j - lp * pg.page);
}

__host__ __device__ __forceinline__ bool run_contiguous(const KeyPages& pg) {
    return !pg.table || pg.page % 256 == 0;
}

// Pool rows of the 256-key run that starts at key kw0 (a multiple of 256),
// for layouts whose runs are not contiguous: lane l holds the rows of keys
// kw0 + 64 q + l (q = 0..3, clamped to the last key), so the streaming loops
// read a row with one lane shuffle instead of waiting on the page table.
// Pool rows fit 32 bits (pools hold under 4 GiB).
struct RunRows {
    uint32_t r[4] = {0u, 0u, 0u, 0u};
    __device__ __forceinline__ void load(const KeyPages& pg, int b, int n_k, int kw0) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = (uint32_t)key_row(pg, b, n_k, min(kw0 + 64 * q + lane, n_k - 1));
    }
    // Row of key kw0 + 64 q + l (q a compile-time constant after unrolling;
    // every lane of the wave must call it).
    __device__ __forceinline__ uint32_t row(int q, int l) const {
        return (uint32_t)__shfl((int)r[q], l);
    }
};

// Address of key j = min(kw0 + 64 q + l, n_k - 1) of a wave's run: from the
// run's first row when runs are contiguous, else from the run's pool rows.
__device__ __forceinline__ const uint8_t* run_key(bool contig, const uint8_t* pool,
                                                  const uint8_t* run, const RunRows& rr, int kw0,
                                                  int j, int q, int l, int rb) {
    return contig ? run + (size_t)(j - kw0) * rb : pool + (size_t)rr.row(q, l) * rb;
}

// Indexer scores for query rows [q_begin, q_end) of every sequence.
struct IndexArgs {
    const void* q;          // [B][n_q][d] fp8 e4m3fn or bf16
    const void* k;          // [B][n_k][d]
    float* scores;          // [B][q_end-q_begin][n_k]
    int B, n_q, n_k, q_pos0, d, dtype;
    int q_begin, q_end;
    float scale;            // fl32(d^-0.5)
    int write_masked;       // 1: write -inf past each query's position
    const int32_t* seq_pos; // optional [B] (one query row per sequence only): each
                            // sequence's positions are offset by seq_pos[b]
    KeyPages pages;         // k rows (one query row per sequence only)
    uint32_t* hist;         // optional (one query row per sequence only):
                            // per-row digit-1 histograms of the top-k schedule
};

// Top-k over score rows; row r of sequence b belongs to position pos_begin + r
// and is written to idx row idx_row0 + r of an [B][idx_rows][k] array.
struct TopkArgs {
    const float* scores;    // [B][rows][n_k]
    int32_t* idx;           // [B][idx_rows][k]
    int B, rows, n_k, k;
    long long pos_begin;
    const int32_t* seq_pos; // optional [B]: row r of sequence b sits at
                            // pos_begin + seq_pos[b] + r
    int idx_rows, idx_row0;
    void* ws;               // chunked schedule workspace (topk_ws_bytes)
    int hist_ready;         // 1: the indexer already built the row histograms
};

// Sparse MQA attention. With few query rows each (row, split) workgroup
// writes an unnormalised partial to `part` and a combine kernel merges them.
struct AttnArgs {
    const uint16_t* Q;      // [B][n_q][H][128] bf16
    const uint16_t* K;      // [B][n_k][128] bf16
    const uint16_t* V;      // [B][n_k][128] bf16
    const int32_t* idx;     // [B][n_q][k]
    uint16_t* O;            // [B][n_q][H][128] bf16
    float* lse;             // [B][n_q][H] or nullptr
    float* part;            // [B*n_q][n_split][16][128 + 4] fp32 partials
    int B, n_q, n_k, H, k;
    // K/V rows of sequence b start at row b * kv_bstride; idx entries index
    // rows [0, kv_rows) from there (n_k and n_k, or 0 and the pool's rows
    // when idx holds pool rows of a paged layout).
    long long kv_bstride;
    int kv_rows;
    int n_split, split_len; // entries of idx handled per split (multiple of 128)
    // Key-range schedule (idx rows sorted ascending, causal, -1 padded at the
    // end): set by attn_set_ranged.
    int ranged, q_pos0, n_range;
    long long parts_per_seq;
    float* part_lse;        // [parts][16][2] log2-domain lse and scale 2^e of each partial
    uint16_t* part_o;       // [parts][16][128] fp16 (O / l) * 2^-e of each partial
};

// One query row per sequence, selection without a materialised score row
// (sampled threshold, filtered candidates, exact select).
// Threshold mode inside a select kernel: keep only keys whose order key is
// above `key` (the order key of tau; 0xffffffff keeps nothing). A select
// kernel that finishes a row this way (its exact path) sets done[row]
// (row = b * n_q + query row), so the rescoring pass skips that row.
struct ScoreFloor {
    int on;
    uint32_t key;
    uint32_t* done;  // [B][n_q]
};

struct DecodeArgs {
    const void* q;          // [B][n_q][d]
    const void* k;          // [B][n_k][d]
    int32_t* idx;           // [B][idx_rows][top_k]; row idx_row0 is written
    int B, n_q, n_k, q_pos0, d, dtype, top_k;
    int q_row;              // the query row of every sequence (0 <= q_row < n_q)
    int idx_rows, idx_row0;
    float scale;            // fl32(d^-0.5)
    float* fallback;        // [B][n_k] score rows for rows the threshold misses
    const int32_t* seq_pos; // optional [B]: the query of sequence b sits at
                            // q_pos0 + seq_pos[b] + q_row
    KeyPages pages;         // k rows
    uint32_t* tau;          // set by launch_decode_select from its workspace
    uint32_t* cnt;
    uint2* cand;
    uint32_t* samp;         // [B][8192] sample order keys (set by launch_decode_select)
    ScoreFloor floor;       // threshold mode (optional)
};

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Chunked top-k schedule (few long rows): whether it is used, its workspace,
// where its row histograms live inside that workspace, and the kernel that
// clears them before an indexer call that builds them.
bool topk_use_chunked(int B, int rows, int n_k);
size_t topk_ws_bytes(int B, int rows, int n_k);
uint32_t* topk_hist_ptr(void* ws);
hipError_t launch_topk_prepare(const TopkArgs& a, void* ws, hipStream_t s);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s);
// prow[b][s] = pool row of idx[b][s] (or -1) for per_seq entries per sequence.
hipError_t launch_page_rows(const int32_t* idx, int32_t* prow, int B, int per_seq, int n_k,
                            const KeyPages& pg, hipStream_t s);

// Many query rows per sequence: sampled threshold, indexer sweep that keeps
// only candidates, one-wave-per-row exact select, fallback for missed rows.
// A slab holds the query rows row0 + i * rstride, i in [0, rows).
struct PrefillArgs {
    const void* q;          // [B][n_q][d]
    const void* k;          // [B][n_k][d]
    int32_t* idx;           // [B][n_q][top_k]; slab row i -> query row row0 + i * rstride
    int B, n_q, n_k, q_pos0, d, dtype, top_k;
    int row0, rstride, rows;
    float scale;
    int cap;                // candidates kept per (row, key range) (set by launch_prefill_select)
    int rk, nr;             // keys per range (set by launch_prefill_select), ranges per row (caller)
    float* tau_acc;         // workspace pointers (set by launch_prefill_select)
    uint32_t* cnt;          // [rows][nr] sub-list lengths
    uint2* cand;            // [nr][rows][cap] sub-lists (accumulator - threshold, key index)
    uint32_t* fb_list;
    uint32_t* fb_count;
    float* fb_scores;
    ScoreFloor floor;       // threshold mode (optional)
};

int prefill_cap(int top_k);
// Key ranges per row of the many-row filter for a problem of `rows` query
// rows (all sequences) of at most maxlen keys; every slab of the problem
// uses this count (PrefillArgs::nr, prefill_ws_bytes).
int prefill_nranges(int maxlen, long long rows);
size_t prefill_ws_bytes(int B, int rows, int n_k, int top_k, int nr);
// Keys per range for rows of up to maxlen keys in nr ranges (a multiple of
// 128; nr ranges cover maxlen keys).
int prefill_range_len(int maxlen, int nr);
// part 0: threshold, 1: indexer sweep, 2: select, 3: fallback.
hipError_t launch_prefill_select(PrefillArgs a, void* ws, int part, hipStream_t s);
// Selection statistics read back from a many-row slab's workspace after its
// select ran (blocking copies): out = {rows longer than top_k, candidates on
// their lists, rows recomputed by the fallback, rows whose lists overflowed}.
hipError_t prefill_stats(const PrefillArgs& a, const void* ws, long long out[4]);

bool decode_select_applies(int rows, int n_k, int top_k);
size_t decode_select_ws_bytes(int B, int n_k, int top_k);
// part 0: sampled threshold, 1: indexer + filter, 2: exact select.
hipError_t launch_decode_select(DecodeArgs a, void* ws, int part, hipStream_t s);
// The same for the decode select (seq_pos_host: per-sequence positions or
// NULL, added to q_pos); fallback rows are those with fewer than top_k
// candidates or more than the select holds.
hipError_t decode_stats(int B, int n_k, long long q_pos, const int32_t* seq_pos_host, int top_k,
                        const void* ws, long long out[4]);

// Threshold mode: removes from finished top-k lists [B][n_q][top_k] (one row
// per query, ascending, -1 padded) every key whose indexer score is not above
// tau, keeping the survivors in order and padding with -1.
constexpr int kFloorMaxK = 4096;
struct FloorArgs {
    const void* q;      // [B][n_q][d] fp8 e4m3fn or bf16
    const void* k;      // [B][n_k][d]
    int32_t* idx;       // [B][n_q][top_k], rewritten in place
    int B, n_q, n_k, d, dtype, top_k;
    float scale;        // fl32(d^-0.5)
    float tau;
    const uint32_t* done;  // optional [B][n_q]: rows a select kernel already finished
    KeyPages pages;        // k rows (a paged layout's pool when pages.table is set)
};
hipError_t launch_threshold_floor(const FloorArgs& a, hipStream_t s);
// Clears the done flags of rows [0, rows) before the selection.
hipError_t launch_floor_reset(uint32_t* done, long long rows, hipStream_t s);

// Indexer projection: out row out_rows[r] (r when null) of [n_out][d_idx] =
// encode(fl32(X[r] . W[o])) for X [rows][d_model], W [d_idx][d_model] bf16;
// e4m3fn (out_dtype 0, nearest even, saturating) or bf16 (1).
struct ProjectArgs {
    const uint16_t* X;
    const uint16_t* W;
    void* out;
    const int32_t* out_rows;  // optional [rows]; destinations outside [0, n_out) are skipped
    int rows, d_model, d_idx, out_dtype, n_out;
};
hipError_t launch_project(const ProjectArgs& a, hipStream_t s);

// Split plan of the attention: splits per query and entries per split.
void attn_split_plan(int B, int n_q, int k, int* n_split, int* split_len);

// Key-range schedule of the many-row attention (sorted causal idx rows):
// whether it applies, the workspace its partials need, and setting it up
// on AttnArgs from a workspace pointer.
bool attn_ranged_applies(int B, int n_q, int n_k);
size_t attn_ranged_ws_bytes(int B, int n_q, int n_k, int q_pos0);
void attn_set_ranged(AttnArgs& a, int q_pos0, void* ws);

}  // namespace dsa
