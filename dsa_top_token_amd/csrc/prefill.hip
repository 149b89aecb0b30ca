// Many-row (prefill-shaped) selection with a sampled threshold on gfx950:
// the indexer sweep keeps only candidate keys, so no score matrix is written.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), sections 3.2-3.3 and 4.3: the
// indexer scores each query's causal prefix and the query keeps its top_k
// keys; the page fuses indexing, selection and masking to avoid writing the
// intermediates. Kernels, per slab of query rows:
//   threshold  per 16-row block: scores every S-th key of each row's prefix
//              (MFMA), two 10-bit radix rounds over those samples give tau,
//              the lower edge of the 20-bit bin holding the m-th largest
//              sample (m = ceil(1.5 k / S)); tau is turned into the smallest
//              fp32 accumulator value whose scaled score reaches it.
//   filter     per 256-row block (4 waves x 64 rows): sweeps the block's
//              causal keys in 64-key chunks staged in LDS, computes the
//              scores on MFMA and keeps every (order key, index) whose
//              accumulator reaches the row's threshold, appended to the row's
//              list in ascending index order (per-row counts live in the
//              registers of the row's lane group; no atomics).
//   select     one wave per row: the candidates' order keys sit in registers,
//              three radix rounds find the exact k-th key T, a radix select
//              on indices cuts the T-ties at the lowest indices, and an
//              ordered compaction writes the row. Rows with k or fewer keys
//              are filled directly. A row whose threshold kept fewer than k
//              keys, or more than its list holds, is queued.
//   fallback   a persistent kernel recomputes each queued row's scores into
//              the workspace and selects on them with the per-row radix
//              schedule.
#include "frag.h"
#include "topk_common.h"

namespace dsa {
namespace {

using namespace frag;
using namespace topk;

constexpr int TH_ROWS = 16;       // rows per threshold workgroup
constexpr int TH_BINS = 1024;     // 10-bit digits of the threshold rounds
constexpr int TH_MAX_SAMPLES = 4096;
constexpr int FL_CHUNK = 64;      // keys per staged chunk of the filter
constexpr int FL_ROWS_W = 64;     // rows per filter wave
constexpr int FL_ROWS = 4 * FL_ROWS_W;
constexpr int FB_WGS = 256;       // fallback workgroups

__device__ __forceinline__ int row_len(const PrefillArgs& a, int r) {
    const long long pos = (long long)a.q_pos0 + a.row0 + r;
    return (int)min((long long)a.n_k, pos + 1);
}

// Smallest fp32 accumulator a with relu(fl(a * scale)) >= tau (tau > 0).
__device__ float raw_threshold(float tau, float scale) {
    float x = tau / scale;
    // fl(x * scale) is non-decreasing in x; step to the boundary.
    for (int it = 0; it < 64 && x * scale >= tau; ++it)
        x = __uint_as_float(__float_as_uint(x) - 1u);
    for (int it = 0; it < 64 && x * scale < tau; ++it)
        x = __uint_as_float(__float_as_uint(x) + 1u);
    return x;
}

// The bin of a wave-private histogram (nbins, bins owned top-down by lanes)
// holding the rem-th largest counted key: returns bin, *above = count of
// keys in higher bins. Every lane of the wave calls it.
template <int NBINS>
__device__ __forceinline__ uint32_t wave_find_bin(const uint32_t* hist, uint32_t rem,
                                                  uint32_t* above_out) {
    constexpr int PER = NBINS / 64;
    const int lane = threadIdx.x & 63;
    const int hi = NBINS - 1 - lane * PER;
    uint32_t loc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) loc += hist[hi - i];
    uint32_t above = wave_incl_scan(loc) - loc;
    uint32_t bin = 0, ab = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint32_t c = hist[hi - i];
        if (!found && above < rem && above + c >= rem) {
            found = true;
            bin = (uint32_t)(hi - i);
            ab = above;
        }
        above += c;
    }
    const unsigned long long f = __ballot(found);
    const int src = f ? __ffsll((long long)f) - 1 : 0;
    *above_out = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
    return (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
}

// ---------------------------------------------------------------- threshold

template <int DT, int D>
__global__ __launch_bounds__(256) void prefill_threshold_kernel(PrefillArgs a) {
    __shared__ uint32_t hist[TH_ROWS][TH_BINS];
    __shared__ uint32_t digit1[TH_ROWS];
    __shared__ uint32_t rem1[TH_ROWS];
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_blk = (a.rows + TH_ROWS - 1) / TH_ROWS;
    const int blk = blockIdx.x % n_blk, b = blockIdx.x / n_blk;
    const int r0 = blk * TH_ROWS;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.fb_count = 0u;
    // Sampling plan of the block (shared stride, per-row sample counts).
    const int nmax = row_len(a, min(r0 + TH_ROWS, a.rows) - 1);
    const int S = max(32, (nmax + TH_MAX_SAMPLES - 1) / TH_MAX_SAMPLES);
    const uint32_t m = (uint32_t)((3 * a.top_k + 2 * S - 1) / (2 * S));
    const int ns_max = (nmax + S - 1) / S;

    Frag<DT, D> fq;  // A operand: the block's 16 query rows
    fq.load(static_cast<const uint8_t*>(a.q) +
                ((size_t)b * a.n_q + a.row0 + min(r0 + n, a.rows - 1)) * RB, g);
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;
    // Sample count of the rows this lane's scores belong to (rows 4g + r).
    int ns_r[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = r0 + 4 * g + r;
        ns_r[r] = row < a.rows ? (row_len(a, row) + S - 1) / S : 0;
    }

#pragma unroll 1
    for (int round = 0; round < 2; ++round) {
        for (int i = threadIdx.x; i < TH_ROWS * TH_BINS; i += 256) (&hist[0][0])[i] = 0u;
        __syncthreads();
        for (int t0 = wave * 16; t0 < ns_max; t0 += 4 * 16) {
            Frag<DT, D> fk;
            fk.load(kbase + (size_t)(min(t0 + n, ns_max - 1) * S) * RB, g);
            const f32x4 acc = tile_dot_k32<D>(fq, fk);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                const uint32_t key = rank_key(relu_scaled(acc[r], a.scale));
                const bool ok = t0 + n < ns_r[r];
                const bool in = round == 0 ? ok : ok && (key >> 22) == digit1[row];
                const uint32_t bin = round == 0 ? (key >> 22) : ((key >> 12) & 1023u);
                hist_add(&hist[0][0], (uint32_t)row * TH_BINS + bin, in);
            }
        }
        __syncthreads();
        // Each wave resolves 4 rows.
        for (int rr = 0; rr < 4; ++rr) {
            const int row = wave * 4 + rr;
            uint32_t above;
            const uint32_t want = round == 0 ? m : rem1[row];
            const uint32_t bin = wave_find_bin<TH_BINS>(hist[row], want, &above);
            if (lane == 0) {
                if (round == 0) {
                    digit1[row] = bin;
                    rem1[row] = m - above;
                } else {
                    const int grow = r0 + row;
                    if (grow < a.rows) {
                        const int len = row_len(a, grow);
                        const int ns = (len + S - 1) / S;
                        float tacc;
                        if (len <= a.top_k) {
                            tacc = __builtin_inff();  // trivial row: no candidates
                        } else if ((uint32_t)ns <= m) {
                            tacc = -__builtin_inff();  // every key is a candidate
                        } else {
                            const uint32_t tkey = (digit1[row] << 22) | (bin << 12);
                            if (tkey <= 0x80000000u) {
                                tacc = -__builtin_inff();
                            } else {
                                const float tau = __uint_as_float(tkey & 0x7fffffffu);
                                tacc = raw_threshold(tau, a.scale);
                            }
                        }
                        a.tau_acc[(size_t)b * a.rows + grow] = tacc;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------- filter

template <int DT, int D>
__global__ __launch_bounds__(256) void prefill_filter_kernel(PrefillArgs a) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    constexpr int PITCH = RB + 16;
    constexpr int CHUNK_BYTES = FL_CHUNK * RB;
    constexpr int LD_PER_THREAD = (CHUNK_BYTES + 256 * 16 - 1) / (256 * 16);
    __shared__ __attribute__((aligned(16))) uint8_t kt[2][FL_CHUNK * PITCH];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_blk = (a.rows + FL_ROWS - 1) / FL_ROWS;
    // largest blocks (latest rows) first
    const int blk = n_blk - 1 - (int)(blockIdx.x / (unsigned)a.B);
    const int b = blockIdx.x % a.B;
    const int r0 = blk * FL_ROWS;
    const int wr0 = r0 + wave * FL_ROWS_W;
    const long long pos_base = (long long)a.q_pos0 + a.row0;
    const int blk_last = min(r0 + FL_ROWS, a.rows) - 1;
    const int kend = (int)min((long long)a.n_k, pos_base + blk_last + 1);
    const int n_chunks = (kend + FL_CHUNK - 1) / FL_CHUNK;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;

    // A fragments (4 row tiles) and per-row thresholds of this lane's rows.
    Frag<DT, D> fa[4];
    float tacc[4][4];
    int pos_r[4][4];
    uint32_t cnt[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int qr = min(wr0 + 16 * t + n, a.rows - 1);
        fa[t].load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.row0 + qr) * RB, g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wr0 + 16 * t + 4 * g + r;
            tacc[t][r] = row < a.rows ? a.tau_acc[(size_t)b * a.rows + row] : __builtin_inff();
            pos_r[t][r] = (int)(pos_base + row);
            cnt[t][r] = 0u;
        }
    }
    const int wave_last = min(wr0 + FL_ROWS_W, a.rows) - 1;
    const long long wave_maxpos = pos_base + wave_last;
    const long long wave_minpos = pos_base + wr0;
    const bool wave_live = wr0 < a.rows;

    auto load_chunk = [&](int c, i32x4* stg) {
        const uint8_t* src = kbase + (size_t)c * CHUNK_BYTES;
        const size_t lim = (size_t)(a.n_k - c * FL_CHUNK) * RB;  // bytes of valid keys
#pragma unroll
        for (int i = 0; i < LD_PER_THREAD; ++i) {
            const size_t off = (size_t)(threadIdx.x + 256 * i) * 16;
            stg[i] = off < (size_t)CHUNK_BYTES && off < lim
                         ? *reinterpret_cast<const i32x4*>(src + off)
                         : i32x4{0, 0, 0, 0};
        }
    };
    auto store_chunk = [&](int buf, const i32x4* stg) {
#pragma unroll
        for (int i = 0; i < LD_PER_THREAD; ++i) {
            const int off = (threadIdx.x + 256 * i) * 16;
            if (off < CHUNK_BYTES) {
                const int row = off / RB, col = off % RB;
                *reinterpret_cast<i32x4*>(&kt[buf][row * PITCH + col]) = stg[i];
            }
        }
    };

    i32x4 stg[LD_PER_THREAD];
    if (n_chunks > 0) {
        load_chunk(0, stg);
        store_chunk(0, stg);
    }
    __syncthreads();
    uint2* cand_rows = a.cand + ((size_t)b * a.rows) * a.cap;
    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < n_chunks) load_chunk(c + 1, stg);
        const int k0 = c * FL_CHUNK;
        if (wave_live && k0 <= wave_maxpos) {
            f32x4 acc[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                Frag<DT, D> fb;
                fb.load(&kt[buf][(16 * u + n) * PITCH], g);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[t][u] = tile_dot<D>(fa[t], fb);
            }
            if constexpr (DT == 0) {
                if constexpr (Frag<0, D>::NB > 0) mfma_drain();
            }
            const bool diag = k0 + FL_CHUNK - 1 > wave_minpos || k0 + FL_CHUNK > a.n_k;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int key = k0 + 16 * u + n;
                    bool cr[4];
                    bool any = false;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        cr[r] = acc[t][u][r] >= tacc[t][r];
                        if (diag) cr[r] = cr[r] && key <= pos_r[t][r] && key < a.n_k;
                        any = any || cr[r];
                    }
                    if (__ballot(any) == 0ull) continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const unsigned long long msk = __ballot(cr[r]);
                        if (msk == 0ull) continue;
                        const uint32_t seg = (uint32_t)(msk >> (16 * g)) & 0xffffu;
                        if (cr[r]) {
                            const uint32_t o = cnt[t][r] + (uint32_t)__popc(seg & ((1u << n) - 1u));
                            if (o < (uint32_t)a.cap) {
                                const int row = wr0 + 16 * t + 4 * g + r;
                                cand_rows[(size_t)row * a.cap + o] =
                                    make_uint2(rank_key(relu_scaled(acc[t][u][r], a.scale)),
                                               (uint32_t)key);
                            }
                        }
                        cnt[t][r] += (uint32_t)__popc(seg);
                    }
                }
            }
        }
        if (c + 1 < n_chunks) store_chunk(buf ^ 1, stg);
        __syncthreads();
    }
    if (n == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wr0 + 16 * t + 4 * g + r;
                if (row < a.rows) a.cnt[(size_t)b * a.rows + row] = cnt[t][r];
            }
    }
}

// ------------------------------------------------------------------- select

// One 64-thread workgroup (one wave) per row. Dynamic LDS: the row's order
// keys (cap words) then a 2048-bin histogram.
__global__ __launch_bounds__(64) void prefill_select_kernel(PrefillArgs a) {
    extern __shared__ uint32_t smem[];
    uint32_t* keys = smem;
    uint32_t* hist = smem + a.cap;
    const int lane = threadIdx.x;
    const long long task = blockIdx.x;
    const int b = (int)(task / a.rows), row = (int)(task % a.rows);
    const int n = row_len(a, row);
    const int k = a.top_k;
    int32_t* out = a.idx + ((size_t)b * a.idx_rows + a.idx_row0 + row) * k;
    if (n <= k) {
        fill_prefix(out, n, k, lane, 64);
        return;
    }
    const uint32_t cnt = a.cnt[task];
    if (cnt < (uint32_t)k || cnt > (uint32_t)a.cap) {
        if (lane == 0) a.fb_list[atomicAdd(a.fb_count, 1u)] = (uint32_t)task;
        return;
    }
    const uint2* cl = a.cand + (size_t)task * a.cap;
    const int cn = (int)cnt;
    for (int c = lane; c < cn; c += 64) keys[c] = cl[c].x;
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    wave_sync();
    // Exact k-th key: digits 31..21, 20..10, 9..0.
    uint32_t rem = (uint32_t)k, prefix = 0;
#pragma unroll 1
    for (int round = 0; round < 3; ++round) {
        const int sh = round == 0 ? 21 : (round == 1 ? 10 : 0);
        const int psh = round == 1 ? 21 : 10;  // prefix bits of the earlier rounds
        const uint32_t msk = round == 2 ? 1023u : 2047u;
        for (int i = lane; i < BINS; i += 64) hist[i] = 0u;
        wave_sync();
        for (int c0 = 0; c0 < cn; c0 += 64) {
            const int c = c0 + lane;
            const uint32_t key = c < cn ? keys[c] : 0u;
            const bool in = c < cn && (round == 0 || (key >> psh) == prefix);
            hist_add(hist, (key >> sh) & msk, in);
        }
        wave_sync();
        uint32_t above;
        const uint32_t bin = wave_find_bin<BINS>(hist, rem, &above);
        prefix = round == 0 ? bin : ((prefix << (round == 1 ? 11 : 10)) | bin);
        rem -= above;
        wave_sync();
    }
    const uint32_t T = prefix;
    uint32_t gt = 0, eq = 0;
    for (int c = lane; c < cn; c += 64) {
        gt += keys[c] > T ? 1u : 0u;
        eq += keys[c] == T ? 1u : 0u;
    }
    const uint32_t pk = wave_incl_scan((gt << 16) | eq);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)pk, 63);
    const uint32_t n_gt = tot >> 16, n_eq = tot & 0xffffu;
    const uint32_t keep = (uint32_t)k - n_gt;  // ties to keep (>= 1)
    // Tie cut-off: keep the `keep` lowest indices among keys equal to T.
    constexpr uint32_t JMAX = (1u << 22) - 1u;
    uint32_t jT = JMAX;
    if (n_eq > keep) {
        uint32_t r2 = keep, pre = 0;
#pragma unroll 1
        for (int round = 0; round < 2; ++round) {
            for (int i = lane; i < BINS; i += 64) hist[i] = 0u;
            wave_sync();
            for (int c0 = 0; c0 < cn; c0 += 64) {
                const int c = c0 + lane;
                const bool tie = c < cn && keys[c] == T;
                const uint32_t kj = tie ? JMAX - cl[c].y : 0u;
                const bool in = tie && (round == 0 || (kj >> 11) == pre);
                hist_add(hist, round == 0 ? (kj >> 11) : (kj & 2047u), in);
            }
            wave_sync();
            uint32_t above;
            const uint32_t bin = wave_find_bin<BINS>(hist, r2, &above);
            pre = round == 0 ? bin : ((pre << 11) | bin);
            r2 -= above;
            wave_sync();
        }
        jT = JMAX - pre;
    }
    // Ordered compaction over the index-sorted list, 64 candidates at a time.
    uint32_t base = 0;
    for (int c0 = 0; c0 < cn; c0 += 64) {
        const int c = c0 + lane;
        bool s = false;
        uint32_t j = 0;
        if (c < cn && keys[c] >= T) {
            j = cl[c].y;
            s = keys[c] > T || j <= jT;
        }
        const unsigned long long msk = __ballot(s);
        const uint32_t o = base + (uint32_t)__popcll(msk & ((1ull << lane) - 1ull));
        if (s && o < (uint32_t)k) out[o] = (int32_t)j;
        base += (uint32_t)__popcll(msk);
    }
}

// ----------------------------------------------------------------- fallback

template <int DT, int D>
__global__ __launch_bounds__(512) void prefill_fallback_kernel(PrefillArgs a) {
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t cand[8192];
    __shared__ uint32_t wsum[8];
    __shared__ uint32_t res[4];
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const uint32_t total = *a.fb_count;
    float* srow = a.fb_scores + (size_t)blockIdx.x * a.n_k;
    for (uint32_t f = blockIdx.x; f < total; f += gridDim.x) {
        const uint32_t task = a.fb_list[f];
        const int b = (int)(task / a.rows), row = (int)(task % a.rows);
        const int len = row_len(a, row);
        Frag<DT, D> fq;  // the query row, broadcast to all 16 B columns
        fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.row0 + row) * RB, g);
        const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;
        for (int t0 = wave * 16; t0 < len; t0 += 8 * 16) {
            Frag<DT, D> fk;
            fk.load(kbase + (size_t)min(t0 + n, len - 1) * RB, g);
            const f32x4 acc = tile_dot_k32<D>(fk, fq);
            if (n == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (t0 + 4 * g + r < len) srow[t0 + 4 * g + r] = relu_scaled(acc[r], a.scale);
            }
        }
        __threadfence();
        __syncthreads();
        int32_t* out = a.idx + ((size_t)b * a.idx_rows + a.idx_row0 + row) * a.top_k;
        row_topk<512, 8192, false>(srow, len, a.top_k, out, hist, cand, wsum, res);
        __syncthreads();
    }
}

template <int DT, int D>
hipError_t launch_d(const PrefillArgs& a, int part, hipStream_t s) {
    const long long rows = (long long)a.B * a.rows;
    if (part == 0) {
        const long long nb = (long long)a.B * ((a.rows + TH_ROWS - 1) / TH_ROWS);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_threshold_kernel<DT, D>), dim3((unsigned)nb), dim3(256), 0, s,
                           a);
    } else if (part == 1) {
        const long long nb = (long long)a.B * ((a.rows + FL_ROWS - 1) / FL_ROWS);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_filter_kernel<DT, D>), dim3((unsigned)nb), dim3(256), 0, s, a);
    } else if (part == 2) {
        if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const size_t lds = ((size_t)a.cap + BINS) * 4;
        hipLaunchKernelGGL(prefill_select_kernel, dim3((unsigned)rows), dim3(64), lds, s, a);
    } else {
        hipLaunchKernelGGL((prefill_fallback_kernel<DT, D>), dim3(FB_WGS), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const PrefillArgs& a, int part, hipStream_t s) {
    switch (a.d) {
        case 32: return launch_d<DT, 32>(a, part, s);
        case 64: return launch_d<DT, 64>(a, part, s);
        case 96: return launch_d<DT, 96>(a, part, s);
        case 128: return launch_d<DT, 128>(a, part, s);
        case 160: return launch_d<DT, 160>(a, part, s);
        case 192: return launch_d<DT, 192>(a, part, s);
        case 224: return launch_d<DT, 224>(a, part, s);
        case 256: return launch_d<DT, 256>(a, part, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int prefill_cap(int top_k) {
    // candidate list per row: about 2.5 k plus room for ties, whole waves
    const int c = (5 * top_k / 2 + 512 + 63) / 64 * 64;
    return c;
}

size_t prefill_ws_bytes(int B, int rows, int n_k, int top_k) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t r = (size_t)B * rows;
    return al(r * 4) + al(r * 4) + al(r * (size_t)prefill_cap(top_k) * 8) + al(r * 4) + al(4) +
           al((size_t)FB_WGS * n_k * 4);
}

hipError_t launch_prefill_select(PrefillArgs a, void* ws, int part, hipStream_t s) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t r = (size_t)a.B * a.rows;
    a.cap = prefill_cap(a.top_k);
    char* p = static_cast<char*>(ws);
    a.tau_acc = reinterpret_cast<float*>(p);
    p += al(r * 4);
    a.cnt = reinterpret_cast<uint32_t*>(p);
    p += al(r * 4);
    a.cand = reinterpret_cast<uint2*>(p);
    p += al(r * (size_t)a.cap * 8);
    a.fb_list = reinterpret_cast<uint32_t*>(p);
    p += al(r * 4);
    a.fb_count = reinterpret_cast<uint32_t*>(p);
    p += al(4);
    a.fb_scores = reinterpret_cast<float*>(p);
    return a.dtype == 0 ? launch_dt<0>(a, part, s) : launch_dt<1>(a, part, s);
}

}  // namespace dsa
