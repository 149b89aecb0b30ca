/*
 * Host-side checks run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by build.sh in this folder; no GPU is needed and none is touched).
 *
 * Part 1: the C ABI of include/dsa.h on its validation paths -- problems
 * out of range, NULL and misaligned pointers, workspaces too small, the
 * allocation-free call beyond its scratch -- where every call returns an
 * error before anything is enqueued, plus the workspace sizes and many-row
 * plans of valid problems (host arithmetic only).
 * Part 2: the CPU oracle (test infrastructure) on the hand-worked d = 4 case
 * (indexer scores relu(q.k * d^-0.5) with keys past the query excluded,
 * top-k with ties to the lower index, attention with Q = 0 as the mean of the
 * kept V rows: the DeepSeek-V3.2 DSA page, sections 3.2 and 3.3) and on
 * random integer inputs against a brute-force dot product.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/dsa.h"

/* internal, non-ABI calls of the library */
int32_t dsa_internal_prefill_plan(const dsa_problem* p, int64_t* out);

/* the oracle (oracle/dsa_oracle.c) */
float oracle_index_scale(int d);
int oracle_index_scores(int B, int n_q, int n_k, int q_pos0, int d, int dtype, const void* q_idx,
                        const void* k_idx, int q_begin, int q_end, float* scores);
int oracle_topk(int B, int rows, int n_k, int pos_begin, int k, const float* scores, int32_t* idx);
int oracle_sparse_attn(int B, int n_q, int n_k, int H, int D, int k, const uint16_t* Q,
                       const uint16_t* K, const uint16_t* V, const int32_t* idx, float* O,
                       float* lse);

static int failures = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static dsa_problem prob(int batch, int n_q, int n_k, int q_pos0, int d, int dt, int k, int h) {
    dsa_problem p = {batch, n_q, n_k, q_pos0, d, (dsa_idx_dtype)dt, k, h, 128};
    return p;
}

static void abi_checks(void) {
    for (int s = 0; s >= -6; --s) CHECK(dsa_status_str(s) && strlen(dsa_status_str(s)) > 0);
    size_t n = 0;
    dsa_problem bad[] = {
        prob(0, 64, 64, 0, 128, 0, 8, 8),   prob(1, 0, 64, 0, 128, 0, 8, 8),
        prob(1, 64, 0, 0, 128, 0, 8, 8),    prob(1, 64, 64, -1, 128, 0, 8, 8),
        prob(1, 64, 64, 1, 128, 0, 8, 8),   prob(1, 1, 1 << 23, 0, 128, 0, 8, 8),
        prob(1, 64, 64, 0, 100, 0, 8, 8),   prob(1, 64, 64, 0, 288, 0, 8, 8),
        prob(1, 64, 64, 0, 128, 2, 8, 8),   prob(1, 64, 64, 0, 128, 0, 0, 8),
        prob(1, 64, 64, 0, 128, 0, 4097, 8), prob(1, 64, 64, 0, 128, 0, 8, 0),
        prob(1, 64, 64, 0, 128, 0, 8, 17),
    };
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
        CHECK(dsa_workspace_size(&bad[i], DSA_OP_FORWARD, &n) < 0);
        CHECK(strlen(dsa_last_error()) > 0);
    }
    CHECK(dsa_workspace_size(NULL, DSA_OP_FORWARD, &n) == DSA_E_NULL);
    dsa_problem p = prob(1, 64, 64, 0, 128, 0, 8, 8);
    CHECK(dsa_workspace_size(&p, DSA_OP_FORWARD, NULL) == DSA_E_NULL);
    CHECK(dsa_workspace_size(&p, 99, &n) == DSA_E_UNSUPPORTED);
    void* fake = (void*)(uintptr_t)0x100000; /* never dereferenced */
    void* odd = (void*)(uintptr_t)0x100008;
    CHECK(dsa_index_scores(NULL, fake, fake, 0, 1, (float*)fake, NULL) == DSA_E_NULL);
    CHECK(dsa_index_scores(&p, odd, fake, 0, 1, (float*)fake, NULL) == DSA_E_ALIGN);
    CHECK(dsa_index_scores(&p, fake, fake, 1, 1, (float*)fake, NULL) == DSA_E_SHAPE);
    CHECK(dsa_topk(&p, NULL, 0, 1, (int32_t*)fake, NULL, 0, NULL) == DSA_E_NULL);
    CHECK(dsa_sparse_attn(&p, fake, fake, NULL, fake, fake, NULL, NULL, 0, NULL) == DSA_E_NULL);
    CHECK(dsa_forward(&p, fake, fake, fake, fake, fake, NULL, fake, NULL, NULL, 0, NULL) ==
          DSA_E_WORKSPACE);
    size_t need = 0;
    CHECK(dsa_workspace_size(&p, DSA_OP_FORWARD, &need) == DSA_OK && need > 0);
    CHECK(dsa_forward(&p, fake, fake, fake, fake, fake, NULL, fake, NULL, fake, need - 1, NULL) ==
          DSA_E_WORKSPACE);
    CHECK(dsa_forward(&p, fake, fake, fake, fake, fake, (int32_t*)odd, fake, NULL, fake, need,
                      NULL) == DSA_E_ALIGN);
    dsa_problem dec = prob(2, 1, 64, 0, 128, 0, 8, 8);
    CHECK(dsa_workspace_size(&dec, DSA_OP_FORWARD, &need) == DSA_OK);
    CHECK(dsa_forward_ragged(&dec, NULL, fake, fake, fake, fake, fake, NULL, fake, NULL, fake,
                             need, NULL) == DSA_E_NULL);
    dsa_problem big = prob(1, 65536, 65536, 0, 128, 0, 1536, 16);
    CHECK(dsa_forward_noalloc(&big, fake, fake, fake, fake, fake, NULL, fake, NULL, NULL) ==
          DSA_E_WORKSPACE);
    CHECK(dsa_index_project(0, 64, 32, 0, fake, fake, fake, NULL, 1, NULL) == DSA_E_SHAPE);
    CHECK(dsa_index_project(4, 64, 32, 0, NULL, fake, fake, NULL, 4, NULL) == DSA_E_NULL);
    /* workspace sizes and many-row plans of valid problems */
    const int shapes[][5] = {{1, 1024, 1024, 0, 64},       {1, 65536, 65536, 0, 1536},
                             {1, 131072, 131072, 0, 2048}, {2, 700, 50000, 49300, 512},
                             {64, 1, 131072, 131071, 2048}, {3, 17, 4194304, 4194287, 4096}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        const int* s = shapes[i];
        dsa_problem q = prob(s[0], s[1], s[2], s[3], 128, 0, s[4], 16);
        for (int op = DSA_OP_TOPK; op <= DSA_OP_FORWARD; ++op)
            CHECK(dsa_workspace_size(&q, op, &n) == DSA_OK);
        int64_t plan[6];
        CHECK(dsa_internal_prefill_plan(&q, plan) == DSA_OK);
        const long long maxlen = s[2] < (long long)s[3] + s[1] ? s[2] : (long long)s[3] + s[1];
        CHECK(plan[2] >= 1 && plan[3] % 128 == 0 && plan[2] * plan[3] >= maxlen);
        CHECK(plan[0] * plan[1] >= s[1]);
    }
}

/* e4m3fn code of a small integer v in [-8, 8] (exact) */
static uint8_t e4m3(int v) {
    if (v == 0) return 0;
    const int s = v < 0, a = v < 0 ? -v : v;
    int e = 0;
    while ((1 << (e + 1)) <= a) ++e;
    const int m = (a - (1 << e)) * 8 / (1 << e);
    return (uint8_t)((s << 7) | ((e + 7) << 3) | m);
}

static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16); /* exact for the small values used here */
}

static void oracle_checks(void) {
    /* the hand-worked case: d = 4 (scale exactly 0.5), L = 4, prefill */
    const int qv[4][4] = {{1, 0, 0, 0}, {1, -1, 2, 0}, {0, 1, 1, -1}, {2, 0, -3, 3}};
    const int kv[4][4] = {{1, 1, 0, 0}, {0, 1, 1, 0}, {1, 0, 1, 1}, {1, 0, 0, -1}};
    uint8_t q[16], k[16];
    for (int i = 0; i < 4; ++i)
        for (int c = 0; c < 4; ++c) {
            q[4 * i + c] = e4m3(qv[i][c]);
            k[4 * i + c] = e4m3(kv[i][c]);
        }
    CHECK(oracle_index_scale(4) == 0.5f);
    float s[16];
    CHECK(oracle_index_scores(1, 4, 4, 0, 4, 0, q, k, 0, 4, s) == 0);
    const float want[4][4] = {{0.5f, -INFINITY, -INFINITY, -INFINITY},
                              {0.f, 0.5f, -INFINITY, -INFINITY},
                              {0.5f, 1.f, 0.f, -INFINITY},
                              {1.f, 0.f, 1.f, 0.f}};
    for (int i = 0; i < 16; ++i) CHECK(s[i] == want[i / 4][i % 4]);
    int32_t idx[12];
    CHECK(oracle_topk(1, 4, 4, 0, 1, s, idx) == 0);
    const int32_t k1[4] = {0, 1, 1, 0};
    for (int i = 0; i < 4; ++i) CHECK(idx[i] == k1[i]);
    CHECK(oracle_topk(1, 4, 4, 0, 3, s, idx) == 0);
    const int32_t k3[12] = {0, -1, -1, 0, 1, -1, 0, 1, 2, 0, 1, 2};
    for (int i = 0; i < 12; ++i) CHECK(idx[i] == k3[i]);
    /* attention with Q = 0, k = 2: the mean of the kept V rows */
    int32_t sel[8];
    CHECK(oracle_topk(1, 4, 4, 0, 2, s, sel) == 0);
    uint16_t Q[4 * 128], K[4 * 128], V[4 * 128];
    memset(Q, 0, sizeof Q);
    memset(K, 0, sizeof K);
    memset(V, 0, sizeof V);
    const float v2[4][2] = {{1, 0}, {0, 1}, {2, 2}, {4, -4}};
    for (int j = 0; j < 4; ++j) {
        V[128 * j] = bf16(v2[j][0]);
        V[128 * j + 1] = bf16(v2[j][1]);
    }
    float O[4 * 128], lse[4];
    CHECK(oracle_sparse_attn(1, 4, 4, 1, 128, 2, Q, K, V, sel, O, lse) == 0);
    const float ow[4][2] = {{1, 0}, {0.5f, 0.5f}, {0.5f, 0.5f}, {1.5f, 1.f}};
    for (int i = 0; i < 4; ++i) {
        CHECK(fabsf(O[128 * i] - ow[i][0]) < 1e-6f && fabsf(O[128 * i + 1] - ow[i][1]) < 1e-6f);
        CHECK(fabsf(lse[i] - logf(i == 0 ? 1.f : 2.f)) < 1e-6f);
    }
    /* random integer inputs against a brute-force dot product */
    enum { NQ = 37, NK = 300, D = 64 };
    static uint8_t rq[NQ * D], rk[NK * D];
    static int iq[NQ * D], ik[NK * D];
    unsigned st = 12345u;
    for (int i = 0; i < NQ * D; ++i) {
        st = st * 1103515245u + 12345u;
        iq[i] = (int)((st >> 16) % 9) - 4;
        rq[i] = e4m3(iq[i]);
    }
    for (int i = 0; i < NK * D; ++i) {
        st = st * 1103515245u + 12345u;
        ik[i] = (int)((st >> 16) % 9) - 4;
        rk[i] = e4m3(ik[i]);
    }
    static float rs[NQ * NK];
    const int pos0 = NK - NQ;
    CHECK(oracle_index_scores(1, NQ, NK, pos0, D, 0, rq, rk, 0, NQ, rs) == 0);
    const float sc = oracle_index_scale(D);
    for (int i = 0; i < NQ; ++i)
        for (int j = 0; j < NK; ++j) {
            long dot = 0;
            for (int c = 0; c < D; ++c) dot += (long)iq[i * D + c] * ik[j * D + c];
            const float x = (float)dot * sc;
            const float w = j > pos0 + i ? -INFINITY : (x > 0.f ? x : 0.f);
            CHECK(rs[i * NK + j] == w);
        }
    static int32_t ri[NQ * 50];
    CHECK(oracle_topk(1, NQ, NK, pos0, 50, rs, ri) == 0);
    for (int i = 0; i < NQ; ++i)
        for (int e = 1; e < 50; ++e) CHECK(ri[i * 50 + e] > ri[i * 50 + e - 1]);
}

int main(void) {
    abi_checks();
    oracle_checks();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ALL CHECKS PASSED\n");
    return 0;
}
