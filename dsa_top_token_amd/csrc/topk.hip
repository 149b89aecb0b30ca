// Exact per-query top-k of indexer scores on gfx950.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), section 3.3: each query keeps
// the top_k keys by indexer score; section 4.1 describes the selection stage
// as plain comparisons. Here the comparisons are on 32-bit order keys (the
// float32 bit pattern made monotone), resolved by a three-round radix select
// (11 + 11 + 10 bits) and an ordered compaction:
//   round 1  histogram of key bits 31..21 over the row -> threshold bin b1
//   round 2  histogram of bits 20..10 among keys in b1 -> bin b2; the keys
//            of b1 are also gathered into LDS when they fit
//   round 3  histogram of bits 9..0 among keys in (b1, b2) -> exact value T
//   output   every key above T, plus the `rem` lowest-index keys equal to T,
//            written in ascending key order via a block-wide prefix scan.
// Ties at T therefore go to the lower key index. One 512-thread workgroup
// owns one score row; histograms live in LDS, and lanes of a wave that fall
// in the same bin add to it once (ReLU zeros are one large tie class).
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int NT = 512;
constexpr int NW = NT / 64;
constexpr int BINS = 2048;
constexpr int CAP = 8192;

// Order key: float order mapped to unsigned order (-0.0 ranks with +0.0).
__device__ __forceinline__ uint32_t rank_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histogram increment for the whole wave (call with every lane present).
// Lanes that share the first active lane's bin add with one atomic.
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

// Exclusive prefix sum over the workgroup; *total receives the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
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

// The bin holding the rem-th largest counted key: res[0] = bin, res[1] = keys
// in higher bins (so res[1] < rem <= res[1] + hist[bin]).
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
    uint32_t above = block_excl_scan(loc, wsum, &tot);
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

// Four consecutive order keys starting at element j (j % 4 == 0); lanes past
// n get valid = false.
template <bool VEC>
__device__ __forceinline__ void load4(const float* row, int j, int n, uint32_t key[4], bool ok[4]) {
    if (VEC && j + 3 < n) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        key[0] = rank_key(v.x); key[1] = rank_key(v.y);
        key[2] = rank_key(v.z); key[3] = rank_key(v.w);
        ok[0] = ok[1] = ok[2] = ok[3] = true;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ok[e] = j + e < n;
            key[e] = ok[e] ? rank_key(row[j + e]) : 0u;
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t cand[CAP];
    __shared__ uint32_t wsum[NW];
    __shared__ uint32_t res[4];
    const int tid = threadIdx.x;
    const unsigned rid = blockIdx.x;
    const int b = (int)(rid / (unsigned)a.rows), r = (int)(rid % (unsigned)a.rows);
    const long long pos = a.pos_begin + r;
    const int n = (int)min((long long)a.n_k, pos + 1);
    const float* row = a.scores + (size_t)rid * a.n_k;
    int32_t* out = a.idx + ((size_t)b * a.idx_rows + a.idx_row0 + r) * a.k;
    const int k = a.k;
    if (n <= k) {
        for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
        return;
    }

    // Round 1: bits 31..21.
    for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
    if (tid == 0) res[2] = 0u;
    __syncthreads();
    for (int base = 0; base < n; base += 4 * NT) {
        uint32_t key[4];
        bool ok[4];
        load4<VEC>(row, base + 4 * tid, n, key, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) hist_add(hist, key[e] >> 21, ok[e]);
    }
    __syncthreads();
    find_bin(hist, (uint32_t)k, wsum, res);
    const uint32_t b1 = res[0];
    uint32_t rem = (uint32_t)k - res[1];
    const uint32_t cnt1 = hist[b1];
    const bool gather = cnt1 <= (uint32_t)CAP;
    __syncthreads();

    // Round 2: bits 20..10 of the keys in bin b1.
    for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < n; base += 4 * NT) {
        uint32_t key[4];
        bool ok[4];
        load4<VEC>(row, base + 4 * tid, n, key, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = ok[e] && (key[e] >> 21) == b1;
            hist_add(hist, (key[e] >> 10) & 2047u, in);
            if (gather && in) cand[atomicAdd(&res[2], 1u)] = key[e];
        }
    }
    __syncthreads();
    find_bin(hist, rem, wsum, res);
    const uint32_t pre22 = (b1 << 11) | res[0];
    rem -= res[1];
    __syncthreads();

    // Round 3: bits 9..0 of the keys in (b1, b2).
    for (int i = tid; i < BINS; i += NT) hist[i] = 0u;
    __syncthreads();
    if (gather) {
        for (int base = 0; base < (int)cnt1; base += NT) {
            const int c = base + tid;
            const bool ok = c < (int)cnt1;
            const uint32_t key = ok ? cand[c] : 0u;
            hist_add(hist, key & 1023u, ok && (key >> 10) == pre22);
        }
    } else {
        for (int base = 0; base < n; base += 4 * NT) {
            uint32_t key[4];
            bool ok[4];
            load4<VEC>(row, base + 4 * tid, n, key, ok);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                hist_add(hist, key[e] & 1023u, ok[e] && (key[e] >> 10) == pre22);
        }
    }
    __syncthreads();
    find_bin(hist, rem, wsum, res);
    const uint32_t T = (pre22 << 10) | res[0];
    rem -= res[1];
    const uint32_t n_gt = (uint32_t)k - rem;

    // Ordered compaction: 8 consecutive keys per thread per chunk.
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
        const uint32_t pk = block_excl_scan((gt << 16) | eq, wsum, &tot);
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

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
    const long long nb = (long long)a.B * a.rows;
    if (nb <= 0) return hipSuccess;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const bool vec = (a.n_k % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.scores) & 15) == 0);
    if (vec)
        hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)nb), dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)nb), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa
