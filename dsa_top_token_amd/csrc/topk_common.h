// Device helpers of the top-k selection: order keys, wave-aggregated
// histogram updates, workgroup scans and the threshold-bin search.
#pragma once

#include "dsa_internal.h"

namespace dsa {
namespace topk {

constexpr int BINS = 2048;   // 11-bit radix digits
constexpr int SHIFT1 = 21;   // digit 1: key bits 31..21
constexpr int SHIFT2 = 10;   // digit 2: key bits 20..10; digit 3: bits 9..0

// Order key: float order mapped to unsigned order; -0.0 ranks with +0.0.
__device__ __forceinline__ uint32_t rank_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histogram increment issued by a whole wave (every lane must call it).
// Lanes that share the first active lane's bin add with one atomic, which
// keeps large tie classes (such as ReLU zeros) from serialising.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int leader = __ffsll((long long)act) - 1;
    const uint32_t lead_bin = __shfl(bin, leader);
    const bool same = active && bin == lead_bin;
    const unsigned long long same_mask = __ballot(same);
    if ((int)__lane_id() == leader) atomicAdd(&hist[lead_bin], (uint32_t)__popcll(same_mask));
    if (active && !same) atomicAdd(&hist[bin], 1u);
}

// Exclusive prefix sum over an NT-thread workgroup; *total gets the sum.
// wsum needs NT/64 words of LDS. Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t s = wsum[i];
        pre += i < w ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return pre + x - v;
}

// Bin holding the rem-th largest counted key of a BINS-bin histogram:
// res[0] = bin, res[1] = keys in higher bins (res[1] < rem <= res[1] + hist[bin]).
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t rem, uint32_t* wsum,
                                         uint32_t* res) {
    constexpr int PER = BINS / NT;
    const int hi = BINS - 1 - (int)threadIdx.x * PER;
    uint32_t c[PER], loc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = hist[hi - i];
        loc += c[i];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(loc, wsum, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (above < rem && above + c[i] >= rem) {
            res[0] = (uint32_t)(hi - i);
            res[1] = above;
        }
        above += c[i];
    }
    __syncthreads();
}

}  // namespace topk
}  // namespace dsa
