// Lightning-indexer scores on gfx950 matrix cores.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), section 3.2: the score of a
// query/key pair is relu(q_idx . k_idx * dim^-0.5) over a small indexer
// dimension, computed as an FP8 matrix product (section 4.1); bf16 inputs are
// the page's fallback precision (section 7.3).
//
// Each wave owns a 16-query x 64-key block: four 16x16 output tiles, each the
// sum of d/128 v_mfma_scale_f32_16x16x128_f8f6f4 (+ (d%128)/32
// v_mfma_f32_16x16x32_fp8) or d/32 v_mfma_f32_16x16x32_bf16 products. The
// fp32 accumulator is scaled by fl32(d^-0.5) once, passed through ReLU and
// masked past the query's position in the epilogue.
//
// Contraction order: both operands of an MFMA place the same contraction
// index k in the same (lane group, register) slot, so any fixed assignment of
// row bytes to slots yields the full dot product. Each lane therefore loads
// contiguous bytes of its row: [128c + 32g, +32) for fp8 chunk c, lane group
// g = lane / 16. For the integer-valued inputs the sum is exact in fp32, so
// the result does not depend on the order.
#include "frag.h"
#include "topk_common.h"

namespace dsa {
namespace {

using namespace frag;

// Workgroup = 4 waves arranged WM (queries) x WN (keys); each wave computes
// 16 queries x 64 keys per iteration and ITER iterations.
// With HIST (one query row per sequence), the workgroup also histograms the
// digit-1 radix of its scores' order keys in LDS and adds the counts to the
// sequence's row histogram, which the top-k selection starts from.
template <int DT, int D, int WM, int WN, int ITER, bool HIST>
__global__ __launch_bounds__(256) void index_scores_kernel(IndexArgs a) {
    __shared__ uint32_t lhist[HIST ? topk::BINS : 1];
    if (HIST) {
        for (int i = threadIdx.x; i < topk::BINS; i += 256) lhist[i] = 0u;
        __syncthreads();
    }
    constexpr int ES = DT == 0 ? 1 : 2;
    constexpr int RB = D * ES;  // bytes per indexer row
    constexpr int QB = 16 * WM;
    constexpr int KB = 64 * WN * ITER;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int m = lane & 15, g = lane >> 4;
    const int rows = a.q_end - a.q_begin;
    const int n_kb = (a.n_k + KB - 1) / KB;
    const int n_qb = (rows + QB - 1) / QB;
    unsigned bid = blockIdx.x;
    const int kb = bid % n_kb;
    bid /= n_kb;
    const int qb = bid % n_qb;
    const int b = bid / n_qb;
    const int wrow0 = qb * QB + wm * 16;
    if (wrow0 >= rows) return;  // never taken when HIST (WM == 1)
    const long long pos0 = (long long)a.q_pos0 + a.q_begin;
    const long long wmaxpos = pos0 + min(wrow0 + 16, rows) - 1;
    const float ninf = -__builtin_inff();
    float* const out = a.scores + (size_t)b * rows * (size_t)a.n_k;

    Frag<DT, D> fa;
    {
        const int ra = min(wrow0 + m, rows - 1);
        fa.load(static_cast<const uint8_t*>(a.q) +
                    ((size_t)b * a.n_q + a.q_begin + ra) * RB, g);
    }
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;

    for (int it = 0; it < ITER; ++it) {
        const int k0 = kb * KB + (it * WN + wn) * 64;
        if (k0 >= a.n_k) break;
        if (k0 > wmaxpos) {  // every key of the block lies past every query
            if (a.write_masked) {
                for (int e = lane; e < 16 * 64; e += 64) {
                    const int row = wrow0 + (e >> 6), key = k0 + (e & 63);
                    if (row < rows && key < a.n_k) out[(size_t)row * a.n_k + key] = ninf;
                }
            }
            continue;
        }
        // All four key fragments are in registers before the first MFMA: a
        // load issued between the MFMAs could return into an A or B operand
        // register of an MFMA still queued behind a dependent accumulate
        // (the operands are read when it starts, not when it issues), and
        // neither the hardware nor the compiler orders that write after the
        // read. The epilogue consumes every accumulator before the next
        // iteration's loads are issued.
        Frag<DT, D> fb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int kr = min(k0 + 16 * t + m, a.n_k - 1);
            fb[t].load(kbase + (size_t)kr * RB, g);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = tile_dot<D>(fa, fb[t]);
        __builtin_amdgcn_sched_barrier(0);
        // Output tile layout: lane holds rows 4g + r, key column m.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wrow0 + 4 * g + r;
            if (row >= rows) continue;
            const long long pos = pos0 + row;
            float* orow = out + (size_t)row * a.n_k;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int key = k0 + 16 * t + m;
                if (key >= a.n_k) continue;
                if (key > pos) {
                    if (a.write_masked) orow[key] = ninf;
                } else {
                    orow[key] = relu_scaled(acc[t][r], a.scale);
                }
            }
        }
        if (HIST) {
            // Row 0 sits in register 0 of lanes 0..15.
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int key = k0 + 16 * t + m;
                const bool act = g == 0 && key < a.n_k && key <= pos0;
                const float s = relu_scaled(acc[t][0], a.scale);
                topk::hist_add(lhist, topk::rank_key(s) >> topk::SHIFT1, act);
            }
        }
    }
    if (HIST) {
        __syncthreads();
        uint32_t* gh = a.hist + (size_t)b * topk::BINS;
        for (int i = threadIdx.x; i < topk::BINS; i += 256)
            if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
    }
}

// One query row per sequence (decode). The 16 keys of a tile are the MFMA's
// row operand and the query is broadcast to all 16 columns, so every lane
// (column n, lane group g) ends up with the scores of keys 4g..4g+3 of the
// tile. A wave loads all TILES key tiles of a step before its first MFMA
// (TILES x 2 KiB in flight for d = 128 fp8), then lanes n < TILES pick tile
// n's four scores and store them as one float4: the step's 16*TILES scores
// leave as one contiguous store. With HIST the same lanes add the scores'
// digit-1 radix to an LDS histogram that is flushed into the sequence's row
// histogram at the end.
// CONTIG: 256-key runs are contiguous (whole-run address arithmetic); else
// per-key pool rows.
template <int DT, int D, int TILES, int STEPS, bool HIST, bool CONTIG>
__global__ __launch_bounds__(256) void index_decode_kernel(IndexArgs a) {
    static_assert(TILES == 8, "the tile pick below assumes 8 tiles per step");
    __shared__ uint32_t lhist[HIST ? topk::BINS : 1];
    if (HIST) {
        for (int i = threadIdx.x; i < topk::BINS; i += 256) lhist[i] = 0u;
        __syncthreads();
    }
    constexpr int ES = DT == 0 ? 1 : 2;
    constexpr int RB = D * ES;
    constexpr int KW = 16 * TILES * STEPS;  // keys per wave
    constexpr int KB = 4 * KW;              // keys per workgroup
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_kb = (a.n_k + KB - 1) / KB;
    const int kb = blockIdx.x % n_kb, b = blockIdx.x / n_kb;
    // The one row of this sequence: query q_begin at position pos.
    const long long pos = (long long)a.q_pos0 + a.q_begin + (a.seq_pos ? a.seq_pos[b] : 0);
    const int lim = (int)max(0LL, min((long long)a.n_k, pos + 1));  // keys < lim are scored
    const float ninf = -__builtin_inff();
    float* const out = a.scores + (size_t)b * a.n_k;

    Frag<DT, D> fq;
    fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.q_begin) * RB, g);
    // the wave's KW keys (contiguous unless pages are smaller)
    const int kw0 = min(kb * KB + wave * KW, a.n_k - 1);
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
    constexpr bool contig = CONTIG;
    const uint8_t* __restrict__ kbase = kpool + (size_t)key_row(a.pages, b, a.n_k, kw0) * RB;
    static_assert(KW == 256, "one 256-key run per wave");
    RunRows rr;
    if constexpr (!contig) rr.load(a.pages, b, a.n_k, kw0);
    const int sel = n & (TILES - 1);
    const bool writer = n < TILES;

    // Scores of every step stay in registers until the wave has issued its
    // last load: on this hardware stores share the load counter, so a store
    // issued between steps would make the next step's load waits also wait
    // for the store to complete.
    float sc[STEPS][4];
    int key0s[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int k0 = kb * KB + wave * KW + st * 16 * TILES;
        key0s[st] = k0 + 16 * sel + 4 * g;
        if (k0 >= a.n_k) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[st][r] = ninf;
            continue;
        }
        Frag<DT, D> fk[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t)
            fk[t].template load<true>(run_key(contig, kpool, kbase, rr, kw0,
                                              min(k0 + 16 * t + n, a.n_k - 1), 2 * st + t / 4,
                                              16 * (t % 4) + n, RB), g);
        // Keep every load of the step ahead of the first MFMA (the scheduler
        // would otherwise recycle two fragments and expose the latency).
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t) acc[t] = tile_dot_k32<D>(fk[t], fq);
        // Lane picks tile `sel` (three levels of selects on n's bits).
        f32x4 v01 = (sel & 1) ? acc[1] : acc[0];
        f32x4 v23 = (sel & 1) ? acc[3] : acc[2];
        f32x4 v45 = (sel & 1) ? acc[5] : acc[4];
        f32x4 v67 = (sel & 1) ? acc[7] : acc[6];
        f32x4 v03 = (sel & 2) ? v23 : v01;
        f32x4 v47 = (sel & 2) ? v67 : v45;
        f32x4 v = (sel & 4) ? v47 : v03;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sc[st][r] = key0s[st] + r < lim ? relu_scaled(v[r], a.scale) : ninf;
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int key0 = key0s[st];
        if (writer && key0 + 3 < a.n_k && (a.write_masked || key0 + 3 < lim)) {
            *reinterpret_cast<float4*>(out + key0) =
                make_float4(sc[st][0], sc[st][1], sc[st][2], sc[st][3]);
        } else if (writer) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (key0 + r < a.n_k && (a.write_masked || key0 + r < lim)) out[key0 + r] = sc[st][r];
        }
        if (HIST) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                topk::hist_add(lhist, topk::rank_key(sc[st][r]) >> topk::SHIFT1,
                               writer && key0 + r < lim);
        }
    }
    if (HIST) {
        __syncthreads();
        uint32_t* gh = a.hist + (size_t)b * topk::BINS;
        for (int i = threadIdx.x; i < topk::BINS; i += 256)
            if (lhist[i]) atomicAdd(&gh[i], lhist[i]);
    }
}

template <int DT, int D>
hipError_t launch_dt_d(const IndexArgs& a, hipStream_t s) {
    const int rows = a.q_end - a.q_begin;
    if ((a.hist || a.seq_pos || a.pages.table) && rows != 1) return hipErrorInvalidValue;
    if (rows == 1) {
        constexpr int TILES = 8, STEPS = 2, KB = 4 * 16 * TILES * STEPS;
        const long long nb = (long long)a.B * ((a.n_k + KB - 1) / KB);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const bool contig = run_contiguous(a.pages);
        if (a.hist && contig)
            hipLaunchKernelGGL((index_decode_kernel<DT, D, TILES, STEPS, true, true>),
                               dim3((unsigned)nb), dim3(256), 0, s, a);
        else if (a.hist)
            hipLaunchKernelGGL((index_decode_kernel<DT, D, TILES, STEPS, true, false>),
                               dim3((unsigned)nb), dim3(256), 0, s, a);
        else if (contig)
            hipLaunchKernelGGL((index_decode_kernel<DT, D, TILES, STEPS, false, true>),
                               dim3((unsigned)nb), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((index_decode_kernel<DT, D, TILES, STEPS, false, false>),
                               dim3((unsigned)nb), dim3(256), 0, s, a);
    } else if (rows <= 16) {
        // Few queries per sequence (decode): the 4 waves split the keys.
        constexpr int QB = 16, KB = 1024;
        const long long nb = (long long)a.B * ((rows + QB - 1) / QB) * ((a.n_k + KB - 1) / KB);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        if (a.hist)
            hipLaunchKernelGGL((index_scores_kernel<DT, D, 1, 4, 4, true>), dim3((unsigned)nb),
                               dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((index_scores_kernel<DT, D, 1, 4, 4, false>), dim3((unsigned)nb),
                               dim3(256), 0, s, a);
    } else {
        if (a.hist) return hipErrorInvalidValue;
        constexpr int QB = 64, KB = 256;
        const long long nb = (long long)a.B * ((rows + QB - 1) / QB) * ((a.n_k + KB - 1) / KB);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        // Few blocks (1024 x 1024 scores: 64 of 256 CUs): one 64-key step per
        // wave, four times the workgroups. Not for fp8 rows wider than 128
        // values: their tiles chain a scaled 16x16x128 MFMA with further
        // MFMAs, and without the loop the register holding the scale
        // exponent is free after the last tile, so it was reused for an
        // accumulator read while the last scaled MFMA still sat behind the
        // previous tile's chain (d = 192 returned wrong scores). In the loop
        // the scale register stays live across iterations.
        constexpr bool one_step_ok = DT == 1 || D <= 128;
        if (one_step_ok && nb < 1024) {
            const long long nb1 = (long long)a.B * ((rows + QB - 1) / QB) * ((a.n_k + 63) / 64);
            hipLaunchKernelGGL((index_scores_kernel<DT, D, 4, 1, (one_step_ok ? 1 : 4), false>),
                               dim3((unsigned)nb1), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((index_scores_kernel<DT, D, 4, 1, 4, false>), dim3((unsigned)nb),
                               dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const IndexArgs& a, hipStream_t s) {
    switch (a.d) {
        case 32: return launch_dt_d<DT, 32>(a, s);
        case 64: return launch_dt_d<DT, 64>(a, s);
        case 96: return launch_dt_d<DT, 96>(a, s);
        case 128: return launch_dt_d<DT, 128>(a, s);
        case 160: return launch_dt_d<DT, 160>(a, s);
        case 192: return launch_dt_d<DT, 192>(a, s);
        case 224: return launch_dt_d<DT, 224>(a, s);
        case 256: return launch_dt_d<DT, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s) {
    if (a.q_end <= a.q_begin || a.B <= 0) return hipSuccess;
    return a.dtype == 0 ? launch_dt<0>(a, s) : launch_dt<1>(a, s);
}

}  // namespace dsa
