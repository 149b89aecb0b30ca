// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Indexer scores for query rows [q_begin, q_end) of every sequence.
struct IndexArgs {
    const void* q;          // [B][n_q][d] fp8 e4m3fn or bf16
    const void* k;          // [B][n_k][d]
    float* scores;          // [B][q_end-q_begin][n_k]
    int B, n_q, n_k, q_pos0, d, dtype;
    int q_begin, q_end;
    float scale;            // fl32(d^-0.5)
    int write_masked;       // 1: write -inf past each query's position
};

// Top-k over score rows; row r of sequence b belongs to position pos_begin + r
// and is written to idx row idx_row0 + r of an [B][idx_rows][k] array.
struct TopkArgs {
    const float* scores;    // [B][rows][n_k]
    int32_t* idx;           // [B][idx_rows][k]
    int B, rows, n_k, k;
    long long pos_begin;
    int idx_rows, idx_row0;
};

// Sparse MQA attention. When n_split > 1 the kernel writes unnormalised
// partials to `part` and a combine kernel finishes O / lse.
struct AttnArgs {
    const uint16_t* Q;      // [B][n_q][H][128] bf16
    const uint16_t* K;      // [B][n_k][128] bf16
    const uint16_t* V;      // [B][n_k][128] bf16
    const int32_t* idx;     // [B][n_q][k]
    uint16_t* O;            // [B][n_q][H][128] bf16
    float* lse;             // [B][n_q][H] or nullptr
    float* part;            // [B*n_q][n_split][16][128 + 2] fp32 partials
    int B, n_q, n_k, H, k;
    int n_split, split_len; // entries of idx handled per split (multiple of 32)
};

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s);

// Split plan of the attention: splits per query and entries per split.
void attn_split_plan(int B, int n_q, int k, int* n_split, int* split_len);

}  // namespace dsa
