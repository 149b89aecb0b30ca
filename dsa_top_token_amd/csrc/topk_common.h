// Device helpers of the top-k selection: order keys, wave-aggregated
// histogram updates, workgroup scans and the threshold-bin search.
#pragma once

#include "dsa_internal.h"
#include "lanes.h"

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
    const uint32_t lead_bin = __builtin_amdgcn_readlane(bin, leader);
    const bool same = active && bin == lead_bin;
    const unsigned long long same_mask = __ballot(same);
    if ((int)__lane_id() == leader) atomicAdd(&hist[lead_bin], (uint32_t)__popcll(same_mask));
    if (active && !same) atomicAdd(&hist[bin], 1u);
}

// Plain per-key LDS atomic add. In the latency-bound selection rounds it
// times faster than hist_add's vote chain (per-row kernel over 4096 x 4096
// causal rows 54.5 -> 46.1 us); hist_add stays where many keys of a wave
// share a bin and the kernel has waves to spare.
__device__ __forceinline__ void hist_inc(uint32_t* hist, uint32_t bin, bool active) {
    if (active) atomicAdd(&hist[bin], 1u);
}

// Slot of this lane's item in an LDS list whose length is *count, for the
// lanes that pass `take`: one atomic per wave (lanes of a wave take
// consecutive slots), so a long list does not serialise on the counter.
// Called by every lane of the wave; the result is meaningful where take holds.
__device__ __forceinline__ uint32_t wave_append(bool take, uint32_t* count) {
    const unsigned long long m = __ballot(take);
    if (m == 0ull) return 0u;
    const int leader = __ffsll((long long)m) - 1;
    uint32_t base = 0u;
    if ((int)__lane_id() == leader) base = atomicAdd(count, (uint32_t)__popcll(m));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
    return base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum across the 64 lanes of a wave: DPP row shifts within
// each 16-lane row, then the row totals (read from lanes 15, 31, 47).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    // row_shr:n = 0x110 + n; lanes shifted in from outside the row read 0
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = (int)(threadIdx.x & 63) >> 4;
    x += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
    return x;
}

// Minimum / maximum across the 64 lanes of a wave (bits 5 and 4 of the lane
// index on VALU permutes, the rest on swizzles).
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    x = min(x, lane_partner32(x));
    x = min(x, lane_partner16(x));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, m));
    return x;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max(x, lane_partner32(x));
    x = max(x, lane_partner16(x));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, m));
    return x;
}

// Exclusive prefix sum over an NT-thread workgroup; *total gets the sum.
// wsum needs NT/64 words of LDS. Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
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

// Four consecutive order keys starting at element j (j % 4 == 0), valid
// below n.
template <bool VEC>
__device__ __forceinline__ void load4(const float* row, int j, int n, uint32_t key[4], bool ok[4]) {
    if (VEC && j + 3 < n) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        key[0] = rank_key(v.x);
        key[1] = rank_key(v.y);
        key[2] = rank_key(v.z);
        key[3] = rank_key(v.w);
        ok[0] = ok[1] = ok[2] = ok[3] = true;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[e] = j + e < n;
            key[e] = ok[e] ? rank_key(row[j + e]) : 0u;
        }
    }
}

// Exact top-k of one score row of n > k candidates, run by an NT-thread
// workgroup: three histogram rounds find the k-th order key T and the number
// `rem` of T-ties to keep, then an ordered compaction writes every key above
// T plus the first `rem` keys equal to T, in ascending index order.
// LDS: hist[BINS], cand[CAP] (keys of the digit-1 threshold bin, when they
// fit), wsum[NT/64], res[4].
template <int NT, int CAP, bool VEC>
__device__ __forceinline__ void row_topk(const float* row, int n, int k, int32_t* out, uint32_t* hist,
                         uint32_t* cand, uint32_t* wsum, uint32_t* res) {
    const int tid = threadIdx.x;
    // Digit 1.
    for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
    if (tid == 0) res[2] = 0u;
    __syncthreads();
    for (int base = 0; base < n; base += 4 * NT) {
        uint32_t key[4];
        bool ok[4];
        load4<VEC>(row, base + 4 * tid, n, key, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) hist_inc(hist, key[e] >> SHIFT1, ok[e]);
    }
    __syncthreads();
    find_bin<NT>(hist, (uint32_t)k, wsum, res);
    const uint32_t b1 = res[0];
    uint32_t rem = (uint32_t)k - res[1];
    const uint32_t cnt1 = hist[b1];
    const bool gather = cnt1 <= (uint32_t)CAP;
    __syncthreads();
    // Digit 2 among keys in b1 (gathered into LDS when they fit).
    for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < n; base += 4 * NT) {
        uint32_t key[4];
        bool ok[4];
        load4<VEC>(row, base + 4 * tid, n, key, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = ok[e] && (key[e] >> SHIFT1) == b1;
            hist_inc(hist, (key[e] >> SHIFT2) & (BINS - 1), in);
            if (gather && in) cand[atomicAdd(&res[2], 1u)] = key[e];
        }
    }
    __syncthreads();
    find_bin<NT>(hist, rem, wsum, res);
    const uint32_t pre22 = (b1 << 11) | res[0];
    rem -= res[1];
    __syncthreads();
    // Digit 3 among keys in (b1, b2).
    for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
    __syncthreads();
    if (gather) {
        for (int base = 0; base < (int)cnt1; base += NT) {
            const int c = base + tid;
            const bool ok = c < (int)cnt1;
            const uint32_t key = ok ? cand[c] : 0u;
            hist_inc(hist, key & 1023u, ok && (key >> SHIFT2) == pre22);
        }
    } else {
        for (int base = 0; base < n; base += 4 * NT) {
            uint32_t key[4];
            bool ok[4];
            load4<VEC>(row, base + 4 * tid, n, key, ok);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hist_inc(hist, key[e] & 1023u, ok[e] && (key[e] >> SHIFT2) == pre22);
        }
    }
    __syncthreads();
    find_bin<NT>(hist, rem, wsum, res);
    const uint32_t T = (pre22 << 10) | res[0];
    rem -= res[1];
    const uint32_t n_gt = (uint32_t)k - rem;

    // Ordered compaction: 8 consecutive keys per thread per pass.
    uint32_t gt_run = 0, eq_run = 0;
    for (int base = 0; base < n; base += 8 * NT) {
        const int j0 = base + 8 * tid;
        uint32_t key[8];
        bool ok[8];
        load4<VEC>(row, j0, n, key, ok);
        load4<VEC>(row, j0 + 4, n, key + 4, ok + 4);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gt += (ok[e] && key[e] > T) ? 1u : 0u;
            eq += (ok[e] && key[e] == T) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t pk = block_excl_scan<NT>((gt << 16) | eq, wsum, &tot);
        uint32_t gb = gt_run + (pk >> 16), eb = eq_run + (pk & 0xffffu);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!ok[e]) continue;
            if (key[e] > T) {
                const uint32_t o = gb + min(eb, rem);
                if (o < (uint32_t)k) out[o] = j0 + e;
                ++gb;
            } else if (key[e] == T) {
                if (eb < rem && gb + eb < (uint32_t)k) out[gb + eb] = j0 + e;
                ++eb;
            }
        }
        gt_run += tot >> 16;
        eq_run += tot & 0xffffu;
        if (gt_run >= n_gt && eq_run >= rem) break;
    }
}

__device__ __forceinline__ void fill_prefix(int32_t* out, int n, int k, int tid, int nt) {
    for (int j = tid; j < k; j += nt) out[j] = j < n ? j : -1;
}

}  // namespace topk
}  // namespace dsa
