// Threshold-mode selection on gfx950: of a finished top-k list, keep only the
// keys whose indexer score exceeds tau.
//
// The sparse-attention explainer page (yunthe.com/news/469461.html), section
// 2.2, keeps for each query the keys whose similarity exceeds a threshold.
// With the indexer score as the similarity and top_k output slots, the kept
// set is {j <= pos : S_j > tau} when it fits and its top_k highest (ties to
// the lower index) otherwise. That is the top-k set with the entries scoring
// <= tau removed: every key above tau outranks every key at or below it. So
// this kernel runs after the selection: one workgroup per query row rescores
// the row's listed keys with the indexer's own arithmetic (the MFMA dot and
// fp32 scale of the decode indexer, so every decision sees the score the
// selection ranked), then compacts the survivors in list order (ascending
// key index) and pads the row with -1.
#include "frag.h"
#include "topk_common.h"

namespace dsa {
namespace {

using namespace frag;

constexpr int TF_NT = 1024;  // threads per row
constexpr int TF_W = TF_NT / 64;
constexpr long long TF_GRID = 1024;  // workgroups of the row loop (four per CU)

// One row: rescore its listed keys, keep those above tau, compact in list
// order, pad with -1. Every thread of the workgroup calls it.
template <int DT, int D, int U>
__device__ __forceinline__ void floor_row(const FloorArgs& a, long long row, int32_t* kept,
                                          uint32_t* wsum, int wave, int n, int g, int K) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    const int b = (int)(row / a.n_q);
    int32_t* list = a.idx + row * K;
    Frag<DT, D> fq;  // the query, in every column of the tile
    fq.load(static_cast<const uint8_t*>(a.q) + (size_t)row * RB, g);
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
    // Tile t holds entries 16 t .. 16 t + 15 as the MFMA's key rows: lane
    // (n, g) loads entry 16 t + n and gets the scores of entries
    // 16 t + 4 g + r (r = 0..3). A wave takes tiles t0 + TF_W u, u < U, at a
    // time: all list reads, then all key loads, then the MFMAs (two memory
    // latencies per pass; a row has only a few passes).
    for (int t0 = wave; 16 * t0 < K; t0 += TF_W * U) {
        int j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = 16 * (t0 + TF_W * u) + n;
            j[u] = e < K ? list[e] : -1;
        }
        bool any[U];
        Frag<DT, D> fk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            any[u] = __ballot(j[u] >= 0) != 0ull;  // lists are -1 padded at the end
            if (any[u])
                fk[u].load(kpool + (size_t)key_row(a.pages, b, a.n_k, j[u] >= 0 ? j[u] : 0) * RB, g);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!any[u]) continue;  // wave-uniform; such tiles get -1 below
            const f32x4 acc = tile_dot_k32<D>(fk[u], fq);
            const int t = t0 + TF_W * u;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int er = 16 * t + 4 * g + r;
                const int jr = __shfl(j[u], 4 * g + r);
                if (n == 0 && er < K)
                    kept[er] = jr >= 0 && relu_scaled(acc[r], a.scale) > a.tau ? jr : -1;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + TF_W * u;
            if (!any[u] && n == 0)
                for (int r = 0; r < 4; ++r)
                    if (16 * t + 4 * g + r < K) kept[16 * t + 4 * g + r] = -1;
        }
    }
    __syncthreads();
    // Compaction in list order: thread t takes entries [t P, t P + P).
    const int P = (K + TF_NT - 1) / TF_NT;
    const int e0 = (int)threadIdx.x * P;
    uint32_t c = 0;
    for (int e = e0; e < e0 + P && e < K; ++e) c += kept[e] >= 0 ? 1u : 0u;
    uint32_t total;
    uint32_t o = topk::block_excl_scan<TF_NT>(c, wsum, &total);
    for (int e = e0; e < e0 + P && e < K; ++e)
        if (kept[e] >= 0) list[o++] = kept[e];
    for (int e = (int)total + (int)threadIdx.x; e < K; e += TF_NT) list[e] = -1;
}

template <int DT, int D>
__global__ __launch_bounds__(TF_NT) void threshold_floor_kernel(FloorArgs a) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    constexpr int U = RB <= 192 ? 4 : 2;  // tiles a wave loads before its first MFMA
    __shared__ int32_t kept[kFloorMaxK];  // entry e: its key if kept, else -1
    __shared__ uint32_t wsum[TF_W];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    __shared__ uint32_t todo[TF_NT];
    const int K = a.top_k;
    // Workgroup w takes rows w, w + G, w + 2G, ... (G workgroups; the rows
    // left to finish, such as the short first rows of a prefill, spread over
    // all of them). Most rows are usually done: each pass reads TF_NT flags
    // at once and compacts the rest into an LDS list, then finishes those
    // rows one by one.
    const long long rows = (long long)a.B * a.n_q;
    const long long G = gridDim.x;
    for (long long c0 = blockIdx.x; c0 < rows; c0 += G * TF_NT) {
        const long long r = c0 + G * threadIdx.x;
        const bool need = r < rows && !(a.done && a.done[r]);  // done: a select kernel applied tau
        uint32_t total;
        const uint32_t pos = topk::block_excl_scan<TF_NT>(need ? 1u : 0u, wsum, &total);
        if (need) todo[pos] = (uint32_t)threadIdx.x;
        __syncthreads();
        for (uint32_t q = 0; q < total; ++q) {
            floor_row<DT, D, U>(a, c0 + G * todo[q], kept, wsum, wave, n, g, K);
            __syncthreads();  // kept[] and wsum are reused by the next row
        }
    }
}

__global__ __launch_bounds__(256) void floor_reset_kernel(uint32_t* done, long long rows) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < rows) done[i] = 0u;
}

template <int DT, int D>
hipError_t launch_d(const FloorArgs& a, hipStream_t s) {
    const long long rows = (long long)a.B * a.n_q;
    const unsigned grid = (unsigned)(rows < TF_GRID ? rows : TF_GRID);
    hipLaunchKernelGGL((threshold_floor_kernel<DT, D>), dim3(grid), dim3(TF_NT), 0, s, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const FloorArgs& a, hipStream_t s) {
    switch (a.d) {
        case 32: return launch_d<DT, 32>(a, s);
        case 64: return launch_d<DT, 64>(a, s);
        case 96: return launch_d<DT, 96>(a, s);
        case 128: return launch_d<DT, 128>(a, s);
        case 160: return launch_d<DT, 160>(a, s);
        case 192: return launch_d<DT, 192>(a, s);
        case 224: return launch_d<DT, 224>(a, s);
        case 256: return launch_d<DT, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_floor_reset(uint32_t* done, long long rows, hipStream_t s) {
    if (rows < 1 || (rows + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(floor_reset_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                       done, rows);
    return hipGetLastError();
}

hipError_t launch_threshold_floor(const FloorArgs& a, hipStream_t s) {
    if (a.top_k < 1 || a.top_k > kFloorMaxK || a.B < 1 || a.n_q < 1) return hipErrorInvalidValue;
    return a.dtype == 0 ? launch_dt<0>(a, s) : launch_dt<1>(a, s);
}

}  // namespace dsa
