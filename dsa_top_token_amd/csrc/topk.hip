// Exact per-query top-k of indexer scores on gfx950.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), section 3.3: each query keeps
// the top_k keys by indexer score; section 4.1 describes the selection stage
// as plain comparisons. Comparisons here are on 32-bit order keys (the
// float32 bit pattern made monotone) and ties go to the lower key index.
//
// Two schedules share the same radix digits (key bits 31..21, 20..10, 9..0):
//
// Per-row (many rows, as in prefill): one 512-thread workgroup per row runs
//   three histogram rounds to find the exact k-th key T and the number `rem`
//   of T-ties to keep, then an ordered compaction writes every key above T
//   plus the first `rem` keys equal to T, in ascending index order.
//
// Chunked (few long rows, as in decode): a row is split into 2048-key chunks
//   so the whole chip works on it.
//     hist     per-row histogram of digit 1 (or built by the indexer kernel)
//     select_a per chunk: count keys above the threshold bin b1 and write
//              the keys inside b1 to the chunk's own candidate slot (an LDS
//              counter, no device-wide atomics)
//     select_b per row: finish digits 2 and 3 on the candidates (-> T), pick
//              the tie cut-off index j_T by a radix select on indices, and
//              turn per-chunk counts into output offsets
//     out      per chunk: ordered compaction of keys > T or (= T and j <= j_T)
//   A row whose candidates overflow (a chunk slot, or the LDS list of
//   select_b) falls back to the per-row schedule inside select_b.
#include "topk_common.h"

namespace dsa {
namespace {

using namespace topk;

constexpr int ROW_NT = 512;       // per-row schedule threads
constexpr int ROW_CAP = 8192;     // per-row LDS candidate capacity (digit-2 keys)
constexpr int CHUNK = 2048;       // chunked schedule: keys per chunk
constexpr int CH_NT = 256;        // chunked schedule: threads of hist/select_a/out
constexpr int SB_NT = 512;        // select_b threads
constexpr int CAND_CAP = 12288;   // chunked schedule: candidates per row
constexpr int CH_CAP = 512;       // chunked schedule: candidates kept per chunk
constexpr int MAX_CHUNKS = 2048;  // 4M keys / CHUNK
constexpr int MULTI_MAX_ROWS = 256;
constexpr int MULTI_MIN_KEYS = 4 * CHUNK;


template <bool VEC>
__global__ __launch_bounds__(ROW_NT) void topk_row_kernel(TopkArgs a) {
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t cand[ROW_CAP];
    __shared__ uint32_t wsum[ROW_NT / 64];
    __shared__ uint32_t res[4];
    const unsigned rid = blockIdx.x;
    const int b = (int)(rid / (unsigned)a.rows), r = (int)(rid % (unsigned)a.rows);
    const long long pos = a.pos_begin + r + (a.seq_pos ? a.seq_pos[b] : 0);
    const int n = (int)max(0LL, min((long long)a.n_k, pos + 1));
    const float* row = a.scores + (size_t)rid * a.n_k;
    int32_t* out = a.idx + ((size_t)b * a.idx_rows + a.idx_row0 + r) * a.k;
    if (n <= a.k) {
        fill_prefix(out, n, a.k, threadIdx.x, ROW_NT);
        return;
    }
    row_topk<ROW_NT, ROW_CAP, VEC>(row, n, a.k, out, hist, cand, wsum, res);
}

// ---------------------------------------------------------------------------
// Short rows (at most WV_MAXN keys): each row split over NWV waves of one
// workgroup, lane l of wave h holding keys 64 E h + E l + i, i < E (E =
// WV_MAXN / (64 NWV) keys per lane), so waves of several rows share a SIMD
// and hide each other's latency. The bits above the highest one where
// the row's smallest and largest keys differ are common to every key, so the
// search starts there; 8-bit radix rounds over a shared 256-bin LDS histogram
// filled by plain LDS atomics then find the k-th key. A round whose chosen
// bin is taken whole ends the search early (every key of that bin is then
// kept), and once the chosen bin holds at most 64 keys they are gathered, one
// per lane, and the k-th key is found among them by comparing every pair.
// Wave scans of the per-lane counts, offset by the earlier waves' totals,
// give each kept key its place in ascending index order. Every decision
// comes from shared values, so all waves take the same path through the
// barriers.
constexpr int WV_MAXN = 1024;          // keys per row at most
constexpr int WV_NWV = 2;              // waves per row

template <bool VEC, int NWV>
__global__ __launch_bounds__(64 * NWV) void topk_wave_kernel(TopkArgs a) {
    constexpr int NT = 64 * NWV;
    constexpr int KPL = WV_MAXN / NT;  // keys per lane
    static_assert(KPL % 4 == 0 && KPL * NT == WV_MAXN, "lane layout");
    __shared__ uint32_t hist[256];
    __shared__ uint32_t gath[64];
    __shared__ uint32_t xmm[2 * NWV];  // per-wave key minimum and maximum
    __shared__ uint32_t xg[NWV];       // per-wave counts of gathered keys
    __shared__ uint32_t xc[NWV];       // per-wave packed kept counts
    const int tid = threadIdx.x, lane = tid & 63, h = tid >> 6;
    const long long rid = blockIdx.x;
    const int b = (int)(rid / a.rows), r = (int)(rid % a.rows);
    const long long pos = a.pos_begin + r + (a.seq_pos ? a.seq_pos[b] : 0);
    const int n = (int)max(0LL, min((long long)a.n_k, pos + 1));
    const float* row = a.scores + (size_t)rid * a.n_k;
    int32_t* out = a.idx + ((size_t)b * a.idx_rows + a.idx_row0 + r) * a.k;
    if (n <= a.k) {  // the whole workgroup
        fill_prefix(out, n, a.k, tid, NT);
        return;
    }
    const int j0 = 64 * KPL * h + KPL * lane;
    uint32_t key[KPL];
    bool ok[KPL];
#pragma unroll
    for (int q = 0; q < KPL; q += 4) load4<VEC>(row, j0 + q, n, key + q, ok + q);
    uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        kmin = ok[i] ? min(kmin, key[i]) : kmin;
        kmax = ok[i] ? max(kmax, key[i]) : kmax;
    }
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) {
        xmm[2 * h] = kmin;
        xmm[2 * h + 1] = kmax;
    }
    __syncthreads();
    kmin = ~0u;
    kmax = 0u;
#pragma unroll
    for (int x = 0; x < NWV; ++x) {
        kmin = min(kmin, xmm[2 * x]);
        kmax = max(kmax, xmm[2 * x + 1]);
    }
    kmin = (uint32_t)__builtin_amdgcn_readfirstlane((int)kmin);
    kmax = (uint32_t)__builtin_amdgcn_readfirstlane((int)kmax);
    const uint32_t dif = kmin ^ kmax;
    int sh = dif == 0u ? 0 : 32 - __builtin_clz(dif);
    uint32_t pre = sh >= 32 ? 0u : (kmin >> sh) << sh;
    uint32_t rem = (uint32_t)a.k;
#pragma unroll 1
    while (sh > 0) {
        const int s = max(sh - 8, 0);
        const uint32_t ph = sh >= 32 ? 0u : pre >> sh;
        for (int x = tid; x < 256; x += NT) hist[x] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const bool in = ok[i] && (sh >= 32 || (key[i] >> sh) == ph);
            if (in) atomicAdd(&hist[(key[i] >> s) & 255u], 1u);
        }
        __syncthreads();
        // both waves find the same bin (lanes own bins top-down)
        const int hi = 255 - 4 * lane;
        uint32_t c[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c[q] = hist[hi - q];
            loc += c[q];
        }
        uint32_t above = wave_incl_scan(loc) - loc;
        int fb = -1;
        uint32_t fa = 0, fc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (above < rem && above + c[q] >= rem) {
                fb = hi - q;
                fa = above;
                fc = c[q];
            }
            above += c[q];
        }
        const unsigned long long mk = __ballot(fb >= 0);
        const int src = __ffsll((long long)mk) - 1;
        const uint32_t bin = (uint32_t)__builtin_amdgcn_readlane(fb, src);
        const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)fa, src);
        const uint32_t cb = (uint32_t)__builtin_amdgcn_readlane((int)fc, src);
        pre |= bin << s;
        rem -= ab;
        sh = s;
        if (rem == cb) break;
        if (cb <= 64u && s > 0) {
            const uint32_t ps = pre >> s;
            uint32_t cnt = 0;
#pragma unroll
            for (int i = 0; i < KPL; ++i) cnt += ok[i] && (key[i] >> s) == ps ? 1u : 0u;
            const uint32_t inc = wave_incl_scan(cnt);
            if (lane == 63) xg[h] = inc;
            __syncthreads();
            uint32_t slot = inc - cnt;
#pragma unroll
            for (int x = 0; x < NWV - 1; ++x) slot += x < h ? xg[x] : 0u;
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                if (ok[i] && (key[i] >> s) == ps) gath[slot++] = key[i];
            }
            __syncthreads();
            const uint32_t mine = lane < (int)cb ? gath[lane] : 0u;
            uint32_t ngt = 0, nge = 0;
            for (uint32_t x = 0; x < cb; ++x) {
                const uint32_t o = gath[x];
                ngt += o > mine ? 1u : 0u;
                nge += o >= mine ? 1u : 0u;
            }
            const unsigned long long hit = __ballot(lane < (int)cb && ngt < rem && rem <= nge);
            const int hl = __ffsll((long long)hit) - 1;
            pre = (uint32_t)__builtin_amdgcn_readlane((int)mine, hl);
            rem -= (uint32_t)__builtin_amdgcn_readlane((int)ngt, hl);
            sh = 0;
            break;
        }
        __syncthreads();  // the next round clears the histogram
    }
    const uint32_t th = pre >> sh;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint32_t kh = key[i] >> sh;
        gt += ok[i] && kh > th ? 1u : 0u;
        eq += ok[i] && kh == th ? 1u : 0u;
    }
    const uint32_t pk = (gt << 16) | eq;
    const uint32_t inc = wave_incl_scan(pk);
    if (lane == 63) xc[h] = inc;
    __syncthreads();
    uint32_t ex = inc - pk;
#pragma unroll
    for (int x = 0; x < NWV - 1; ++x) ex += x < h ? xc[x] : 0u;
    uint32_t gb = ex >> 16, eb = ex & 0xffffu;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        if (!ok[i]) continue;
        const uint32_t kh = key[i] >> sh;
        if (kh > th) {
            out[gb + min(eb, rem)] = j0 + i;
            ++gb;
        } else if (kh == th) {
            if (eb < rem) out[gb + eb] = j0 + i;
            ++eb;
        }
    }
}

// ---------------------------------------------------------------------------
// Chunked schedule.

struct MultiWs {
    uint32_t* hist;      // [slots][BINS]
    uint32_t* cnt;       // [slots][n_chunks] candidates found per chunk
    uint2* cand;         // [slots][n_chunks][CH_CAP] (key, index)
    uint32_t* chunk_gt;  // [slots][n_chunks] keys above bin b1 per chunk
    uint32_t* chunk_off; // [slots][n_chunks] output offset per chunk
    uint32_t* state;     // [slots][4]: T, j_T, fallback-done flag
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

MultiWs carve(void* ws, int slots, int n_chunks, size_t* total) {
    char* p = static_cast<char*>(ws);
    size_t off = 0;
    MultiWs w;
    w.hist = reinterpret_cast<uint32_t*>(p + off);
    off += align256((size_t)slots * BINS * 4);
    w.cnt = reinterpret_cast<uint32_t*>(p + off);
    off += align256((size_t)slots * n_chunks * 4);
    w.cand = reinterpret_cast<uint2*>(p + off);
    off += align256((size_t)slots * n_chunks * CH_CAP * 8);
    w.chunk_gt = reinterpret_cast<uint32_t*>(p + off);
    off += align256((size_t)slots * n_chunks * 4);
    w.chunk_off = reinterpret_cast<uint32_t*>(p + off);
    off += align256((size_t)slots * n_chunks * 4);
    w.state = reinterpret_cast<uint32_t*>(p + off);
    off += align256((size_t)slots * 16);
    if (total) *total = off;
    return w;
}

struct MultiArgs {
    TopkArgs t;
    MultiWs w;
    int n_chunks;
};

__device__ __forceinline__ void slot_info(const MultiArgs& a, int slot, int* b, int* r, int* n) {
    *b = slot / a.t.rows;
    *r = slot % a.t.rows;
    const long long pos = a.t.pos_begin + *r + (a.t.seq_pos ? a.t.seq_pos[*b] : 0);
    *n = (int)max(0LL, min((long long)a.t.n_k, pos + 1));
}

// Zero the per-row histograms (a kernel rather than a memset so the sequence
// can be captured in a graph).
__global__ __launch_bounds__(256) void topk_prepare_kernel(MultiArgs a) {
    const long long total = (long long)a.t.B * a.t.rows * BINS;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (long long)gridDim.x * 256)
        a.w.hist[i] = 0u;
}

// Digit-1 histogram of every chunk, flushed into the row's histogram.
template <bool VEC>
__global__ __launch_bounds__(CH_NT) void topk_hist_kernel(MultiArgs a) {
    __shared__ uint32_t hist[BINS];
    const int slot = blockIdx.x / a.n_chunks, c = blockIdx.x % a.n_chunks;
    int b, r, n;
    slot_info(a, slot, &b, &r, &n);
    const int j0 = c * CHUNK;
    if (n <= a.t.k || j0 >= n) return;
    const int j1 = min(n, j0 + CHUNK);
    for (int i = threadIdx.x; i < BINS; i += CH_NT) hist[i] = 0u;
    __syncthreads();
    const float* row = a.t.scores + (size_t)slot * a.t.n_k;
    for (int base = j0; base < j1; base += 4 * CH_NT) {
        uint32_t key[4];
        bool ok[4];
        load4<VEC>(row, base + 4 * threadIdx.x, j1, key, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) hist_inc(hist, key[e] >> SHIFT1, ok[e]);
    }
    __syncthreads();
    uint32_t* g = a.w.hist + (size_t)slot * BINS;
    for (int i = threadIdx.x; i < BINS; i += CH_NT)
        if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// Per chunk: count keys above bin b1; store the keys inside b1 (with their
// indices) in the chunk's candidate slot, in any order.
template <bool VEC>
__global__ __launch_bounds__(CH_NT) void topk_select_a_kernel(MultiArgs a) {
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t wsum[CH_NT / 64];
    __shared__ uint32_t res[4];
    const int slot = blockIdx.x / a.n_chunks, c = blockIdx.x % a.n_chunks;
    int b, r, n;
    slot_info(a, slot, &b, &r, &n);
    if (n <= a.t.k) return;
    const size_t sc = (size_t)slot * a.n_chunks + c;
    const int j0 = c * CHUNK;
    if (j0 >= n) {
        if (threadIdx.x == 0) {
            a.w.chunk_gt[sc] = 0u;
            a.w.cnt[sc] = 0u;
        }
        return;
    }
    const int j1 = min(n, j0 + CHUNK);
    const uint32_t* g = a.w.hist + (size_t)slot * BINS;
    for (int i = threadIdx.x; i < BINS; i += CH_NT) hist[i] = g[i];
    if (threadIdx.x == 0) res[2] = 0u;
    __syncthreads();
    find_bin<CH_NT>(hist, (uint32_t)a.t.k, wsum, res);
    const uint32_t b1 = res[0];
    const float* row = a.t.scores + (size_t)slot * a.t.n_k;
    uint2* cand = a.w.cand + sc * CH_CAP;
    const int lane = threadIdx.x & 63;
    uint32_t gt = 0;
    for (int base = j0; base < j1; base += 4 * CH_NT) {
        const int j = base + 4 * threadIdx.x;
        uint32_t key[4];
        bool ok[4];
        load4<VEC>(row, j, j1, key, ok);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t bin = key[e] >> SHIFT1;
            gt += (ok[e] && bin > b1) ? 1u : 0u;
            const bool in = ok[e] && bin == b1;
            const unsigned long long m = __ballot(in);
            if (m) {
                const int leader = __ffsll((long long)m) - 1;
                uint32_t p0 = 0;
                if (lane == leader) p0 = atomicAdd(&res[2], (uint32_t)__popcll(m));
                p0 = __shfl(p0, leader);
                if (in) {
                    const uint32_t p = p0 + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
                    if (p < (uint32_t)CH_CAP) cand[p] = make_uint2(key[e], (uint32_t)(j + e));
                }
            }
        }
    }
    uint32_t tot;
    block_excl_scan<CH_NT>(gt, wsum, &tot);
    if (threadIdx.x == 0) {
        a.w.chunk_gt[sc] = tot;
        a.w.cnt[sc] = res[2];
    }
}

// Per row: exact threshold T and tie cut-off j_T from the candidates, and the
// output offset of every chunk.
template <bool VEC>
__global__ __launch_bounds__(SB_NT) void topk_select_b_kernel(MultiArgs a) {
    // LDS: hist[BINS] | keys[CAND_CAP] | idx[CAND_CAP] | cs[MAX_CHUNKS] | wsum | res
    __shared__ uint32_t smem[BINS + 2 * CAND_CAP + MAX_CHUNKS + SB_NT / 64 + 4];
    uint32_t* hist = smem;
    uint32_t* keys = smem + BINS;
    uint32_t* jj = keys + CAND_CAP;
    uint32_t* cs = jj + CAND_CAP;
    uint32_t* wsum = cs + MAX_CHUNKS;
    uint32_t* res = wsum + SB_NT / 64;
    const int tid = threadIdx.x;
    const int slot = blockIdx.x;
    int b, r, n;
    slot_info(a, slot, &b, &r, &n);
    const int k = a.t.k;
    int32_t* out = a.t.idx + ((size_t)b * a.t.idx_rows + a.t.idx_row0 + r) * k;
    uint32_t* st = a.w.state + (size_t)slot * 4;
    if (n <= k) {
        fill_prefix(out, n, k, tid, SB_NT);
        return;
    }
    // Candidate counts per chunk -> offsets in the LDS list (cs holds them).
    const int nch = a.n_chunks;
    constexpr int PER = MAX_CHUNKS / SB_NT;
    const uint32_t* ccnt = a.w.cnt + (size_t)slot * nch;
    uint32_t cv[PER], cloc = 0, cmax = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int c = tid * PER + e;
        cv[e] = c < nch ? ccnt[c] : 0u;
        cloc += cv[e];
        cmax = max(cmax, cv[e]);
    }
    if (tid == 0) res[3] = 0u;
    uint32_t cnt;
    uint32_t coff = block_excl_scan<SB_NT>(cloc, wsum, &cnt);  // has barriers
    if (cmax > (uint32_t)CH_CAP || cnt > (uint32_t)CAND_CAP) res[3] = 1u;
    __syncthreads();
    const bool overflow = res[3] != 0u;
    __syncthreads();
    if (overflow) {
        // A candidate slot overflowed: resolve the row on its own.
        row_topk<SB_NT, ROW_CAP, VEC>(a.t.scores + (size_t)slot * a.t.n_k, n, k, out, hist, keys, wsum,
                                      res);
        if (tid == 0) st[2] = 1u;
        return;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int c = tid * PER + e;
        if (c < nch) cs[c] = coff;
        coff += cv[e];
    }
    const uint32_t* g = a.w.hist + (size_t)slot * BINS;
    for (int i = tid; i < BINS; i += SB_NT) hist[i] = g[i];
    __syncthreads();
    // Copy every chunk's candidates: one wave per chunk at a time.
    {
        const int wv = tid >> 6, ln = tid & 63;
        for (int c = wv; c < nch; c += SB_NT / 64) {
            const uint32_t nc = ccnt[c], o = cs[c];
            const uint2* src = a.w.cand + ((size_t)slot * nch + c) * CH_CAP;
            for (uint32_t i = ln; i < nc; i += 64) {
                const uint2 v = src[i];
                keys[o + i] = v.x;
                jj[o + i] = v.y;
            }
        }
    }
    __syncthreads();
    find_bin<SB_NT>(hist, (uint32_t)k, wsum, res);
    const uint32_t b1 = res[0];
    uint32_t rem = (uint32_t)k - res[1];
    __syncthreads();
    // Digit 2.
    for (int i = tid; i < BINS; i += SB_NT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < (int)cnt; base += SB_NT) {
        const int i = base + tid;
        const bool ok = i < (int)cnt;
        hist_inc(hist, ok ? (keys[i] >> SHIFT2) & (BINS - 1) : 0u, ok);
    }
    __syncthreads();
    find_bin<SB_NT>(hist, rem, wsum, res);
    const uint32_t pre22 = (b1 << 11) | res[0];
    rem -= res[1];
    __syncthreads();
    // Digit 3.
    for (int i = tid; i < BINS; i += SB_NT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < (int)cnt; base += SB_NT) {
        const int i = base + tid;
        const bool ok = i < (int)cnt && (keys[i] >> SHIFT2) == pre22;
        hist_inc(hist, ok ? keys[i] & 1023u : 0u, ok);
    }
    __syncthreads();
    find_bin<SB_NT>(hist, rem, wsum, res);
    const uint32_t T = (pre22 << 10) | res[0];
    rem -= res[1];
    __syncthreads();
    // Tie cut-off: the rem-th smallest index among keys equal to T, found as
    // the rem-th largest of (2^22 - 1 - j) in two 11-bit digits.
    constexpr uint32_t JMAX = (1u << 22) - 1u;
    for (int i = tid; i < BINS; i += SB_NT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < (int)cnt; base += SB_NT) {
        const int i = base + tid;
        const bool ok = i < (int)cnt && keys[i] == T;
        hist_inc(hist, ok ? (JMAX - jj[i]) >> 11 : 0u, ok);
    }
    __syncthreads();
    find_bin<SB_NT>(hist, rem, wsum, res);
    const uint32_t a1 = res[0];
    const uint32_t remj = rem - res[1];
    __syncthreads();
    for (int i = tid; i < BINS; i += SB_NT) hist[i] = 0u;
    __syncthreads();
    for (int base = 0; base < (int)cnt; base += SB_NT) {
        const int i = base + tid;
        const bool ok = i < (int)cnt && keys[i] == T && ((JMAX - jj[i]) >> 11) == a1;
        hist_inc(hist, ok ? (JMAX - jj[i]) & 2047u : 0u, ok);
    }
    __syncthreads();
    find_bin<SB_NT>(hist, remj, wsum, res);
    const uint32_t jT = JMAX - ((a1 << 11) | res[0]);
    __syncthreads();
    // Selected candidates per chunk, then chunk offsets.
    for (int i = tid; i < nch; i += SB_NT) cs[i] = 0u;
    __syncthreads();
    for (int i = tid; i < (int)cnt; i += SB_NT) {
        const uint32_t key = keys[i], j = jj[i];
        if (key > T || (key == T && j <= jT)) atomicAdd(&cs[j / CHUNK], 1u);
    }
    __syncthreads();
    uint32_t v[PER], loc = 0;
    const uint32_t* cg = a.w.chunk_gt + (size_t)slot * nch;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int c = tid * PER + e;
        v[e] = c < nch ? cg[c] + cs[c] : 0u;
        loc += v[e];
    }
    uint32_t tot;
    uint32_t off = block_excl_scan<SB_NT>(loc, wsum, &tot);
    uint32_t* co = a.w.chunk_off + (size_t)slot * nch;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int c = tid * PER + e;
        if (c < nch) co[c] = off;
        off += v[e];
    }
    if (tid == 0) {
        st[0] = T;
        st[1] = jT;
        st[2] = 0u;
    }
}

// Per chunk: ordered compaction of the selected keys into the output row.
template <bool VEC>
__global__ __launch_bounds__(CH_NT) void topk_out_kernel(MultiArgs a) {
    __shared__ uint32_t wsum[CH_NT / 64];
    constexpr int E = CHUNK / CH_NT;  // 8 consecutive keys per thread
    const int slot = blockIdx.x / a.n_chunks, c = blockIdx.x % a.n_chunks;
    int b, r, n;
    slot_info(a, slot, &b, &r, &n);
    const int k = a.t.k;
    const int j0 = c * CHUNK;
    if (n <= k || j0 >= n) return;
    const uint32_t* st = a.w.state + (size_t)slot * 4;
    if (st[2]) return;
    const uint32_t T = st[0], jT = st[1];
    const uint32_t off = a.w.chunk_off[(size_t)slot * a.n_chunks + c];
    const int j1 = min(n, j0 + CHUNK);
    const float* row = a.t.scores + (size_t)slot * a.t.n_k;
    int32_t* out = a.t.idx + ((size_t)b * a.t.idx_rows + a.t.idx_row0 + r) * k;
    const int jt = j0 + E * threadIdx.x;
    uint32_t key[E];
    bool ok[E];
#pragma unroll
    for (int e = 0; e < E; e += 4) load4<VEC>(row, jt + e, j1, key + e, ok + e);
    uint32_t cntl = 0;
    bool sel[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        sel[e] = ok[e] && (key[e] > T || (key[e] == T && (uint32_t)(jt + e) <= jT));
        cntl += sel[e] ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t o = off + block_excl_scan<CH_NT>(cntl, wsum, &tot);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (sel[e]) {
            if (o < (uint32_t)k) out[o] = jt + e;
            ++o;
        }
}

}  // namespace

bool topk_use_chunked(int B, int rows, int n_k) {
    return (long long)B * rows <= MULTI_MAX_ROWS && n_k >= MULTI_MIN_KEYS;
}

size_t topk_ws_bytes(int B, int rows, int n_k) {
    if (!topk_use_chunked(B, rows, n_k)) return 0;
    size_t total = 0;
    carve(nullptr, B * rows, (n_k + CHUNK - 1) / CHUNK, &total);
    return total;
}

uint32_t* topk_hist_ptr(void* ws) { return static_cast<uint32_t*>(ws); }

hipError_t launch_topk_prepare(const TopkArgs& t, void* ws, hipStream_t s) {
    MultiArgs a{t, carve(ws, t.B * t.rows, (t.n_k + CHUNK - 1) / CHUNK, nullptr),
                (t.n_k + CHUNK - 1) / CHUNK};
    const long long total = (long long)t.B * t.rows * BINS;
    const unsigned nb = (unsigned)min(1024LL, (total + 255) / 256);
    hipLaunchKernelGGL(topk_prepare_kernel, dim3(nb), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& t, hipStream_t s) {
    const long long rows = (long long)t.B * t.rows;
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const bool vec = (t.n_k % 4 == 0) && ((reinterpret_cast<uintptr_t>(t.scores) & 15) == 0);
    if (!topk_use_chunked(t.B, t.rows, t.n_k)) {
        if (t.n_k <= WV_MAXN) {
            if (vec)
                hipLaunchKernelGGL((topk_wave_kernel<true, WV_NWV>), dim3((unsigned)rows),
                                   dim3(64 * WV_NWV), 0, s, t);
            else
                hipLaunchKernelGGL((topk_wave_kernel<false, WV_NWV>), dim3((unsigned)rows),
                                   dim3(64 * WV_NWV), 0, s, t);
            return hipGetLastError();
        }
        if (vec)
            hipLaunchKernelGGL(topk_row_kernel<true>, dim3((unsigned)rows), dim3(ROW_NT), 0, s, t);
        else
            hipLaunchKernelGGL(topk_row_kernel<false>, dim3((unsigned)rows), dim3(ROW_NT), 0, s, t);
        return hipGetLastError();
    }
    if (!t.ws) return hipErrorInvalidValue;
    const int nch = (t.n_k + CHUNK - 1) / CHUNK;
    MultiArgs a{t, carve(t.ws, t.B * t.rows, nch, nullptr), nch};
    hipError_t e;
    if (!t.hist_ready) {
        if ((e = launch_topk_prepare(t, t.ws, s)) != hipSuccess) return e;
        if (vec)
            hipLaunchKernelGGL(topk_hist_kernel<true>, dim3((unsigned)(rows * nch)), dim3(CH_NT),
                               0, s, a);
        else
            hipLaunchKernelGGL(topk_hist_kernel<false>, dim3((unsigned)(rows * nch)), dim3(CH_NT),
                               0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (vec) {
        hipLaunchKernelGGL(topk_select_a_kernel<true>, dim3((unsigned)(rows * nch)), dim3(CH_NT),
                           0, s, a);
        hipLaunchKernelGGL(topk_select_b_kernel<true>, dim3((unsigned)rows), dim3(SB_NT), 0, s, a);
        hipLaunchKernelGGL(topk_out_kernel<true>, dim3((unsigned)(rows * nch)), dim3(CH_NT), 0, s,
                           a);
    } else {
        hipLaunchKernelGGL(topk_select_a_kernel<false>, dim3((unsigned)(rows * nch)), dim3(CH_NT),
                           0, s, a);
        hipLaunchKernelGGL(topk_select_b_kernel<false>, dim3((unsigned)rows), dim3(SB_NT), 0, s,
                           a);
        hipLaunchKernelGGL(topk_out_kernel<false>, dim3((unsigned)(rows * nch)), dim3(CH_NT), 0,
                           s, a);
    }
    return hipGetLastError();
}

}  // namespace dsa
