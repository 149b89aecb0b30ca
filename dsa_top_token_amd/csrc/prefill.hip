// Many-row (prefill-shaped) selection with a sampled threshold on gfx950:
// the indexer sweep keeps only candidate keys, so no score matrix is written.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), sections 3.2-3.3 and 4.3: the
// indexer scores each query's causal prefix and the query keeps its top_k
// keys; the page fuses indexing, selection and masking to avoid writing the
// intermediates. Kernels, per slab of query rows:
//   threshold  per 16-row block: scores every S-th key of each row's prefix
//              (MFMA), two 9-bit radix rounds over those samples give tau,
//              the lower edge of the 18-bit bin holding the m-th largest
//              sample (m S ~ 2 top_k); tau becomes the smallest fp32
//              accumulator whose scaled score reaches it. A row whose sample
//              threshold is not positive keeps every non-negative
//              accumulator instead ("zero mode").
//   filter     per 64- or 128-row block: a producer wave streams the block's causal
//              keys into an LDS ring of 64-key chunks with global->LDS copies
//              (several chunks in flight); four
//              consumer waves of 16 or 32 rows each score every chunk on MFMA.
//              Keys are the MFMA row operand, so each lane holds 16
//              consecutive keys of one query; a subtract and a funnel shift
//              per score build the lane's accept mask, and the accepted
//              (accumulator, index) pairs go to the row's list in ascending
//              index order.
//   select     one 256-thread workgroup per row with its list in registers:
//              radix rounds of 12-bit digits over the order keys relative to
//              the row's smallest (as many rounds as the key range needs)
//              give the exact k-th key T; the T-ties are cut in list (=
//              index) order. A zero-mode row with fewer than top_k positive
//              scores takes its positives plus the lowest-index zero scores.
//              A row whose threshold kept fewer than top_k keys, or more than
//              its list holds, is queued.
//   fallback   a persistent kernel recomputes each queued row's scores into
//              the workspace and selects on them with the per-row radix
//              schedule.
#include "frag.h"
#include "topk_common.h"
#include "lanes.h"

#include <type_traits>

namespace dsa {
namespace {

using namespace frag;
using namespace topk;

constexpr int TH_ROWS = 16;       // rows per threshold workgroup
constexpr int TH_DIG = 9;         // bits per digit of the two threshold rounds (the
                                  // 16 x 512-bin histogram fits four workgroups per CU)
constexpr int TH_BINS = 1 << TH_DIG;
constexpr int TH_MAX_SAMPLES = 4096;
constexpr int TH_TARGET = 64;     // samples expected above tau
constexpr int TH_UN = 4;          // sampled-key tiles loaded together per pass
constexpr int FL_CHUNK = 64;      // keys per staged chunk of the filter
constexpr int FB_WGS = 256;       // fallback workgroups
constexpr int kBufWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int qrow(const PrefillArgs& a, int i) { return a.row0 + i * a.rstride; }

__device__ __forceinline__ int row_len(const PrefillArgs& a, int i) {
    const long long pos = (long long)a.q_pos0 + qrow(a, i);
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

// Fragment of row position rp from a granule-major LDS tile: byte b of row
// rp sits at tile + (b / 16) * COLB + 16 rp + b % 16 (the same bytes, in the
// same register slots, as Frag::load takes from a contiguous row).
template <int COLB, int D>
__device__ __forceinline__ void load_cm(Frag<0, D>& f, const uint8_t* tile, int rp, int g) {
    const uint8_t* t = tile + 16 * rp;
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NB; ++c) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(t + (8 * c + g) * COLB);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(t + (8 * c + 4 + g) * COLB);
        f.big[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NS; ++c)
        f.small[c] = *reinterpret_cast<const long*>(
            t + (8 * Frag<0, D>::NB + 2 * c + (g >> 1)) * COLB + 8 * (g & 1));
}

template <int COLB, int D>
__device__ __forceinline__ void load_cm(Frag<1, D>& f, const uint8_t* tile, int rp, int g) {
    const uint8_t* t = tile + 16 * rp;
#pragma unroll
    for (int c = 0; c < Frag<1, D>::NC; ++c)
        f.v[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(t + (4 * c + g) * COLB));
}

// Row-major key chunks in LDS: chunk key r occupies RB contiguous bytes at
// tile + r RB, its 16-byte granule q at granule slot q ^ sw(r). The chunk is
// contiguous in global memory too, so each 1 KB global->LDS copy reads 1 KB
// of consecutive bytes (every 4 lanes one 64-byte segment: XOR keeps aligned
// groups of four granules together). A fragment read touches chunk keys
// r = 16 a + 4 u + b (a, b = 0..3) for one tile u; the row pitch already
// separates some values of b in the LDS banks, so sw takes a and the bits of
// b that the pitch leaves together, as far as q ^ sw stays below GPR.
constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }

template <int RB>
struct RingSw {
    static constexpr int GPR = RB / 16;             // granules per key row
    static constexpr int P2 = GPR & -GPR;           // largest power of two dividing GPR
    static constexpr int SWM = (P2 < 16 ? P2 : 16) - 1;
    static constexpr int SB = (RB / 4) % 64 == 32 ? 1 : 0;  // pitch separates b & 1 only
    __device__ static __forceinline__ int sw(int r) {
        return (((r >> 4) & 3) | (((r & 3) >> SB) << 2)) & SWM;
    }
    // byte b of chunk key r
    __device__ static __forceinline__ const uint8_t* at(const uint8_t* tile, int r, int b) {
        return tile + r * RB + 16 * ((b >> 4) ^ sw(r)) + (b & 15);
    }
};

// Fragment of chunk key r from a row-major ring slot (the same bytes, in the
// same register slots, as Frag::load takes from a contiguous row). The XOR
// only touches the low bits of the granule index, so each read is a
// per-lane base plus a constant offset.
template <int RB, int D>
__device__ __forceinline__ void load_rm(Frag<0, D>& f, const uint8_t* tile, int r, int g) {
    using W = RingSw<RB>;
    const int sw = W::sw(r);
    const uint8_t* row = tile + r * RB;
    // granule 8c + h ^ sw = 8 (c ^ (sw >> 3)) + (h ^ (sw & 7))
    const uint8_t* lo = row + 16 * (g ^ (sw & 7));
    const uint8_t* hi = row + 16 * ((4 + g) ^ (sw & 7));
    const int sc = sw >> 3;
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NB; ++c) {
        const int cc = W::SWM <= 7 ? c : (c ^ sc);
        const i32x4 l = *reinterpret_cast<const i32x4*>(lo + 128 * cc);
        const i32x4 h = *reinterpret_cast<const i32x4*>(hi + 128 * cc);
        f.big[c] = i32x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    }
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NS; ++c)
        f.small[c] = *reinterpret_cast<const long*>(
            W::at(tile, r, 128 * Frag<0, D>::NB + 32 * c + 8 * g));
}

template <int RB, int D>
__device__ __forceinline__ void load_rm(Frag<1, D>& f, const uint8_t* tile, int r, int g) {
    using W = RingSw<RB>;
    const int sw = W::sw(r);
    // granule 4c + g ^ sw = 4 (c ^ (sw >> 2)) + (g ^ (sw & 3))
    const uint8_t* base = tile + r * RB + 16 * (g ^ (sw & 3));
    const int sc = sw >> 2;
#pragma unroll
    for (int c = 0; c < Frag<1, D>::NC; ++c) {
        const int cc = W::SWM <= 3 ? c : (c ^ sc);
        f.v[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(base + 64 * cc));
    }
}

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
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
    const int S = max(max(1, 2 * a.top_k / TH_TARGET), (nmax + TH_MAX_SAMPLES - 1) / TH_MAX_SAMPLES);
    const uint32_t m = (uint32_t)((2 * a.top_k + S - 1) / S);
    const int ns_max = (nmax + S - 1) / S;

    Frag<DT, D> fq;  // A operand: the block's 16 query rows
    fq.load(static_cast<const uint8_t*>(a.q) +
                ((size_t)b * a.n_q + qrow(a, min(r0 + n, a.rows - 1))) * RB, g);
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
        // TH_UN tiles per pass: their sampled key rows are loaded together
        // (one memory latency per pass, not per tile).
        for (int t00 = wave * 16; t00 < ns_max; t00 += TH_UN * 4 * 16) {
            Frag<DT, D> fk[TH_UN];
#pragma unroll
            for (int u = 0; u < TH_UN; ++u)
                fk[u].load(kbase + (size_t)(min(t00 + 64 * u + n, ns_max - 1) * S) * RB, g);
#pragma unroll
            for (int u = 0; u < TH_UN; ++u) {
                const int t0 = t00 + 64 * u;
                const f32x4 acc = tile_dot_k32<D>(fq, fk[u]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * g + r;
                    const uint32_t key = rank_key(relu_scaled(acc[r], a.scale));
                    const bool ok = t0 + n < ns_r[r];
                    const bool in = round == 0 ? ok : ok && (key >> (32 - TH_DIG)) == digit1[row];
                    const uint32_t bin = round == 0 ? (key >> (32 - TH_DIG))
                                                    : ((key >> (32 - 2 * TH_DIG)) & (TH_BINS - 1u));
                    hist_add(&hist[0][0], (uint32_t)row * TH_BINS + bin, in);
                }
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
                            tacc = 0.0f;  // zero mode
                        } else {
                            const uint32_t tkey = (digit1[row] << (32 - TH_DIG)) | (bin << (32 - 2 * TH_DIG));
                            if (tkey <= 0x80000000u) {
                                tacc = 0.0f;  // zero mode
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

// Ring depth of the key-chunk pipeline (chunks in flight ahead of the one
// being consumed is FL_NBUF - 1).
template <int RB>
constexpr int fl_nbuf() { return FL_CHUNK * RB <= 8192 || RB <= 320 ? 3 : 2; }

// Query tiles per consumer wave of the filter. Two tiles halve the ring
// traffic and fragment reads per row (bf16 128K: 7.7 -> 6.4 ms); fp8 keys
// are cheap to stream and there one tile keeps the longest workgroup's
// chunk chain (which sets the kernel time at 64K) short.
template <int DT, int D>
constexpr int filter_qt() { return DT == 1 ? 2 : 1; }

// Waits until at most `ahead` chunks of GPR copies each are in flight
// (0 <= ahead <= A).
template <int A, int GPR>
__device__ __forceinline__ void wait_chunks(int ahead) {
    if constexpr (A > 0) {
        if (ahead >= A) {
            wait_vmcnt<A * GPR>();
            return;
        }
        wait_chunks<A - 1, GPR>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}
static_assert(FL_CHUNK == 64, "the producer's lane -> key map covers 64 keys");

// QT query tiles of 16 rows per consumer wave share every key fragment read
// from the ring (the workgroup covers 64 QT rows).
template <int DT, int D, int QT>
__global__ __launch_bounds__(320) void prefill_filter_kernel(PrefillArgs a) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    // Ring layout: row-major for fp8 keys (timed 1.31 -> 1.20 ms at 64K),
    // granule-major for bf16 (row-major timed 6.4 -> 6.9 ms at 128K).
    constexpr bool RM = DT == 0;
    constexpr int WROWS = 16 * QT;   // rows per consumer wave
    constexpr int ROWS = 4 * WROWS;  // rows per workgroup
    constexpr int GPR = RB / 16;            // 16-byte granules per key row
    constexpr int NBUF = fl_nbuf<RB>();
    static_assert(RB % 16 == 0 && (NBUF - 1) * GPR < 64, "chunk pipeline");
    // Key chunks: row-major with swizzled granules (RingSw), or granule-major
    // (granule j of the key at row position rp at slot + j * 1024 + 16 rp).
    __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF][FL_CHUNK * RB];
    // per-wave copy of each lane's 16 accumulators: [wave][u][lane] x 4
    __shared__ f32x4 stage[4][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_blk = (a.rows + ROWS - 1) / ROWS;
    // largest blocks (latest rows) first
    const int blk = n_blk - 1 - (int)(blockIdx.x / (unsigned)a.B);
    const int b = blockIdx.x % a.B;
    const int i0 = blk * ROWS;
    const int kend = row_len(a, min(i0 + ROWS, a.rows) - 1);
    const int n_chunks = (kend + FL_CHUNK - 1) / FL_CHUNK;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;

    if (wave == 4) {
        // Producer: global -> LDS copies, NBUF - 1 chunks ahead.
        //   row-major (RM): copy i moves granules 64 i .. 64 i + 63 of the
        //     chunk: lane l fills granule slot s = P % GPR of chunk key
        //     r = P / GPR (P = 64 i + l) with the key's granule s ^ sw(r);
        //   granule-major: copy j moves granule j of every key, lane l taking
        //     the key at row position l (chunk key 16 ((l / 4) % 4) + 4 (l / 16)
        //     + l % 4).
        const int kr = 16 * ((lane >> 2) & 3) + 4 * (lane >> 4) + (lane & 3);
        auto issue = [&](int c) {
            uint8_t* dst = ring[c % NBUF];
#pragma unroll
            for (int i = 0; i < GPR; ++i) {
                if constexpr (RM) {
                    const int P = 64 * i + lane, r = P / GPR, q = (P % GPR) ^ RingSw<RB>::sw(r);
                    const int key = min(c * FL_CHUNK + r, a.n_k - 1);
                    __builtin_amdgcn_global_load_lds(kbase + (size_t)key * RB + 16 * q,
                                                     dst + 1024 * i, 16, 0, 0);
                } else {
                    const int key = min(c * FL_CHUNK + kr, a.n_k - 1);
                    __builtin_amdgcn_global_load_lds(kbase + (size_t)key * RB + 16 * i,
                                                     dst + i * (FL_CHUNK * 16), 16, 0, 0);
                }
            }
        };
        const int pre = min(NBUF - 1, n_chunks);
        for (int c = 0; c < pre; ++c) issue(c);
        for (int c = 0; c < n_chunks; ++c) {
            // chunk c has landed once at most `ahead` later chunks are in flight
            const int ahead = min(c + NBUF - 1, n_chunks) - c - 1;
            wait_chunks<NBUF - 2, GPR>(ahead);
            // A workgroup barrier without the release fence of __syncthreads
            // (that fence would wait for every copy in flight); the wait
            // above has already made chunk c visible in LDS.
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (c + NBUF - 1 < n_chunks) issue(c + NBUF - 1);
        }
        wait_vmcnt<0>();
        return;
    }

    // Consumers: wave w scores rows [i0 + WROWS w, +WROWS) against each chunk,
    // query tile t holding rows i0 + WROWS w + 16 t + n.
    const int wi0 = i0 + wave * WROWS;
    int my_i[QT], my_len[QT];
    bool live[QT];
    float tau[QT];
    Frag<DT, D> fq[QT];
    int row_vo[QT];    // byte offset of the row's list in the wave's list block
    uint32_t cnt[QT];  // each row's list length (same in the row's 4 lanes)
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int r = wi0 + 16 * t + n;
        live[t] = r < a.rows;
        my_i[t] = min(r, a.rows - 1);
        my_len[t] = live[t] ? row_len(a, my_i[t]) : 0;
        tau[t] = live[t] ? a.tau_acc[(size_t)b * a.rows + my_i[t]] : __builtin_inff();
        fq[t].load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + qrow(a, my_i[t])) * RB, g);
        row_vo[t] = (16 * t + n) * a.cap * 8;
        cnt[t] = 0;
    }
    // Wave-uniform bounds (scalar registers, so the tail test is a branch).
    const int wi0s = __builtin_amdgcn_readfirstlane(wi0);
    const bool wave_live = wi0s < a.rows;
    const int w_kend = wave_live ? row_len(a, min(wi0s + WROWS - 1, a.rows - 1)) : 0;
    const int w_kmin = wave_live ? row_len(a, wi0s) : 0;
    // The wave's WROWS lists are consecutive: one buffer descriptor covers
    // them, and a store takes a 32-bit byte offset.
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.cand + ((size_t)b * a.rows + (wave_live ? wi0s : 0)) * a.cap), (short)0,
        WROWS * a.cap * 8, kBufWord3);
    wait_vmcnt<0>();  // the query fragments are in registers before the chunk loop
    const uint32_t cap = (uint32_t)a.cap;

    // A operand row n of key tile u is chunk key 16 (n / 4) + 4 u + n % 4
    // (row position 16 u + n), so output row 4 g + r of tile u is key
    // 16 g + 4 u + r: lane (n, g) holds keys [16 g, 16 g + 16) of the chunk.
    // Chunks below w_kmin lie inside every row's causal range; only the
    // later ones (TAIL) mask keys past a row's end.
    auto chunk = [&](const int c, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        __syncthreads();
        const int k0 = c * FL_CHUNK;
        if (k0 < w_kend) {
            const uint8_t* tile = ring[c % NBUF];
            // Every fragment load of the chunk completes before the first
            // MFMA, so no load can overwrite an operand register of an MFMA
            // still queued behind a dependent accumulate chain.
            // A operand row n of key tile u: chunk key 16 (n / 4) + 4 u + n % 4
            // (row position 16 u + n in the granule-major layout)
            Frag<DT, D> fk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if constexpr (RM) load_rm<RB>(fk[u], tile, 16 * (n >> 2) + 4 * u + (n & 3), g);
                else load_cm<FL_CHUNK * 16>(fk[u], tile, 16 * u + n, g);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc[QT][4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int t = 0; t < QT; ++t) acc[t][u] = tile_dot<D>(fk[u], fq[t]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                // bit i of rej: sign of (accumulator of key 16 g + i) - tau
                uint32_t rej = 0;
#pragma unroll
                for (int i = 15; i >= 0; --i)
                    rej = __builtin_amdgcn_alignbit(
                        rej, __float_as_uint(acc[t][i >> 2][i & 3] - tau[t]), 31);
                uint32_t bits = ~rej & 0xffffu;
                if constexpr (TAIL) {
                    const int v = my_len[t] - (k0 + 16 * g);
                    bits &= v >= 16 ? 0xffffu : (v <= 0 ? 0u : (1u << v) - 1u);
                }
                // The row's lanes g = 0..3 hold consecutive key ranges:
                // exclusive prefix of their counts.
                const uint32_t lc = (uint32_t)__popc(bits);
                const uint32_t x1 = lane_partner16(lc);
                const uint32_t s01 = lc + x1;
                const uint32_t x2 = lane_partner32(s01);
                const uint32_t tot = s01 + x2;
                const uint32_t o = cnt[t] + ((g & 1) ? x1 : 0u) + ((g & 2) ? x2 : 0u);
                // An overflowing row's list is abandoned (the row is
                // recomputed by the fallback); nothing is stored at or past cap.
                const uint32_t ne = cnt[t] + tot > cap ? 0u : lc;
                if (ne == 0u) bits = 0u;
                cnt[t] += tot;
                if (__ballot(bits != 0u) != 0ull) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) stage[wave][u][lane] = acc[t][u];
                    // accumulator i of this lane: byte (i / 4) * 1024 + (i % 4) * 4
                    // of its stage column, = (260 i) & 0xC0C
                    const uint8_t* sb = reinterpret_cast<const uint8_t*>(&stage[wave][0][lane]);
                    const uint32_t kb = (uint32_t)(k0 + 16 * g);
                    int vo = row_vo[t] + (int)o * 8;
                    while (bits != 0u) {
                        const int i = __builtin_ctz(bits);
                        bits &= bits - 1u;
                        const uint32_t v = *reinterpret_cast<const uint32_t*>(sb + ((i * 260) & 0xC0C));
                        const u32x2 e = {v, kb + (uint32_t)i};
                        __builtin_amdgcn_raw_buffer_store_b64(e, lrs, vo, 0, 0);
                        vo += 8;
                    }
                }
            }
        }
    };
    const int c_full = min(n_chunks, w_kmin / FL_CHUNK);
    int c = 0;
    for (; c < c_full; ++c) chunk(c, std::false_type{});
    for (; c < n_chunks; ++c) chunk(c, std::true_type{});
#pragma unroll
    for (int t = 0; t < QT; ++t)
        if (g == 0 && live[t]) a.cnt[(size_t)b * a.rows + my_i[t]] = cnt[t];
}

// ------------------------------------------------------------------- select

__device__ __forceinline__ uint32_t cand_key(uint32_t acc_bits, float scale) {
    return rank_key(relu_scaled(__uint_as_float(acc_bits), scale));
}

constexpr int SL_NT = 512;      // threads per select workgroup (one row each)
constexpr int SL_GMAX = 1024;   // keys of a radix bin gathered for the refinement rounds


// Bin of a 256-bin histogram holding the rem-th largest counted key, found
// by wave 0: res[0] = bin, res[1] = keys in higher bins. Called by wave 0.
__device__ __forceinline__ void wave_find_bin8(const uint32_t* hist, uint32_t rem, uint32_t* res) {
    const int lane = threadIdx.x & 63;
    const int hi = 255 - 4 * lane;
    uint32_t c[4], loc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        c[q] = hist[hi - q];
        loc += c[q];
    }
    uint32_t above = wave_incl_scan(loc) - loc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (above < rem && above + c[q] >= rem) {
            res[0] = (uint32_t)(hi - q);
            res[1] = above;
        }
        above += c[q];
    }
}

// Orders one wave's LDS accesses across lanes (its histogram updates before
// the reads that follow them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One SL_NT-thread workgroup per row. Thread t holds list entries
// t, t + SL_NT, t + 2 SL_NT, ... in registers, so every load instruction of a
// wave reads 64 consecutive entries (a lane-per-slice layout made the address
// unit the bottleneck). The k-th key T is found by 8-bit radix rounds over
// the keys relative to the row's smallest: block-wide while the current bin
// holds many keys, then by wave 0 alone over the keys of that bin gathered
// into LDS. Positions in list (= index) order come from ballots within a
// wave and one table of per-(slot, wave) counts scanned by wave 0.
template <int PER>
struct SelRow {
    uint32_t cnt;
    float tau;
    uint2 raw[PER];
};

// Entries below this bound are fetched before the count is known; a row's
// list almost always holds about 2 top_k entries or more.
__device__ __forceinline__ int sel_spec(const PrefillArgs& a) { return min(a.cap, 2 * a.top_k); }

template <int PER>
__device__ __forceinline__ void sel_fetch(const PrefillArgs& a, long long task, SelRow<PER>& r) {
    if (task >= (long long)a.B * a.rows) return;
    r.cnt = a.cnt[task];
    r.tau = a.tau_acc[task];
    const uint2* cl = a.cand + (size_t)task * a.cap;
    const int spec = sel_spec(a);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int j = e * SL_NT + (int)threadIdx.x;
        r.raw[e] = j < spec ? cl[j] : make_uint2(0u, 0u);
    }
}

// The rest of the thread's entries, once the count is known (entries past
// the count are not read).
template <int PER>
__device__ __forceinline__ void sel_fetch_rest(const PrefillArgs& a, long long task, int cn,
                                               SelRow<PER>& r) {
    const uint2* cl = a.cand + (size_t)task * a.cap;
    const int spec = sel_spec(a);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int j = e * SL_NT + (int)threadIdx.x;
        if (j >= spec && j < cn) r.raw[e] = cl[j];
    }
}

// Exclusive prefix, in list order, of two flags per entry packed as
// (count of fa) << 16 | (count of fb): pre[e] for this thread's entry e
// (list index e SL_NT + tid), *total for the row. tbl needs
// PER * SL_NT / 64 + 1 words. Two workgroup barriers; call from every thread.
template <int PER>
__device__ __forceinline__ void list_prefix2(const bool fa[PER], const bool fb[PER], uint32_t* tbl,
                                             uint32_t pre[PER], uint32_t* total) {
    constexpr int NW = SL_NT / 64, NE = PER * NW;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const unsigned long long ma = __ballot(fa[e]), mb = __ballot(fb[e]);
        pre[e] = (__builtin_amdgcn_mbcnt_hi((uint32_t)(ma >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ma, 0u)) << 16) |
                 __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u));
        if (lane == 0) tbl[e * NW + w] = ((uint32_t)__popcll(ma) << 16) | (uint32_t)__popcll(mb);
    }
    __syncthreads();
    if (w == 0) {
        // (slot, wave) order is list order: slot e's 512 entries precede slot e + 1's
        uint32_t carry = 0;
#pragma unroll
        for (int b0 = 0; b0 < NE; b0 += 64) {
            const uint32_t v = b0 + lane < NE ? tbl[b0 + lane] : 0u;
            const uint32_t inc = wave_incl_scan(v) + carry;
            if (b0 + lane < NE) tbl[b0 + lane] = inc - v;
            carry = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        }
        if (lane == 0) tbl[NE] = carry;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) pre[e] += tbl[e * NW + w];
    *total = tbl[NE];
}

template <int PER>
__device__ __forceinline__ void select_row(const PrefillArgs& a, long long task, SelRow<PER> rw,
                                           uint32_t* hist, uint32_t* gk, uint32_t* tbl,
                                           uint32_t* res) {
    const int tid = threadIdx.x;
    const int b = (int)(task / a.rows), i = (int)(task % a.rows);
    const int n = row_len(a, i);
    const int k = a.top_k;
    int32_t* out = a.idx + ((size_t)b * a.n_q + qrow(a, i)) * k;
    if (n <= k) {
        fill_prefix(out, n, k, tid, SL_NT);
        return;
    }
    const uint32_t cnt = rw.cnt;
    const bool zero_mode = __float_as_uint(rw.tau) == 0u;
    if (cnt > (uint32_t)a.cap || (!zero_mode && cnt < (uint32_t)k)) {
        if (tid == 0) a.fb_list[atomicAdd(a.fb_count, 1u)] = (uint32_t)task;
        return;
    }
    const int cn = (int)cnt;
    sel_fetch_rest<PER>(a, task, cn, rw);
    const float scale = a.scale;
    constexpr uint32_t ZERO_KEY = 0x80000000u;  // order key of a zero score
    // An entry past the count holds key 0, below every candidate's order key
    // (scores are >= +0.0, so keys are >= ZERO_KEY): such entries never pass a
    // comparison against ZERO_KEY or T, and the radix rounds place them in
    // digit 0 (d = max(key, kmin) - kmin = 0), below the k-th key.
    uint32_t key[PER], ix[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        key[e] = e * SL_NT + tid < cn ? cand_key(rw.raw[e].x, scale) : 0u;
        ix[e] = rw.raw[e].y;
    }

    if (zero_mode) {
        // The list holds every key with a positive score (plus some zeros);
        // every key off the list scores zero.
        bool pos[PER], none[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            pos[e] = key[e] > ZERO_KEY;
            none[e] = false;
        }
        uint32_t rk[PER], np;
        list_prefix2<PER>(pos, none, tbl, rk, &np);
        np >>= 16;
        if (np < (uint32_t)k) {
            // Positives plus the lowest-index zeros. With P the positives in
            // index order, P[r] - r zeros precede P[r]; the first cs
            // positives (P[r] - r < Z) come before the Z-th zero.
            const uint32_t Z = (uint32_t)k - np;
            bool early[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) early[e] = pos[e] && ix[e] - (rk[e] >> 16) < Z;
            uint32_t dummy[PER], cs;
            list_prefix2<PER>(early, none, tbl, dummy, &cs);
            cs >>= 16;
            const uint32_t head = Z + cs;  // out[0, head) = 0 .. head - 1
            for (uint32_t o = tid; o < head; o += SL_NT) out[o] = (int32_t)o;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const uint32_t r = rk[e] >> 16;
                if (pos[e] && r >= cs) out[Z + r] = (int32_t)ix[e];
            }
            return;
        }
    }

    // Range of the row's order keys; digits are taken relative to the smallest.
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        lo = min(lo, key[e] - 1u);  // an entry past the count wraps to the top
        hi = max(hi, key[e]);
    }
    lo += 1u;
    if (tid == 0) {
        res[2] = 0xffffffffu;
        res[3] = 0u;
        res[4] = 0u;
    }
    __syncthreads();
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((tid & 63) == 0 && lo <= hi) {
        atomicMin(&res[2], lo);
        atomicMax(&res[3], hi);
    }
    __syncthreads();
    const uint32_t kmin = res[2];
    const uint32_t range = res[3] - kmin;
    // Radix rounds over bits [sh, hsh) of d = key - kmin, from the top.
    uint32_t rem = (uint32_t)k, prefix = 0;
    int sh = 32 - __clz((int)range);
    bool first = true, gathered = false;
    uint32_t G = 0;
    while (sh > 0 && !gathered) {
        const int hsh = sh;
        sh = sh > 8 ? sh - 8 : 0;
        const uint32_t mask = (1u << (hsh - sh)) - 1u;
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (e * SL_NT >= cn) continue;  // workgroup-uniform
            const uint32_t d = max(key[e], kmin) - kmin;
            hist_add(hist, (d >> sh) & mask, first || (d >> hsh) == prefix);
        }
        __syncthreads();
        if (tid < 64) wave_find_bin8(hist, rem, res);
        __syncthreads();
        const uint32_t bin = res[0];
        prefix = (prefix << (hsh - sh)) | bin;
        rem -= res[1];
        first = false;
        // Few keys left in the bin: gather them for wave 0.
        if (sh > 0 && hist[bin] <= (uint32_t)SL_GMAX) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                if (e * SL_NT >= cn) continue;
                const uint32_t d = max(key[e], kmin) - kmin;
                if ((d >> sh) == prefix) gk[atomicAdd(&res[4], 1u)] = d;
            }
            gathered = true;
        }
        __syncthreads();
    }
    if (gathered) {
        G = res[4];
        if (tid < 64) {
            // wave 0 alone: the remaining rounds over the gathered keys
            while (sh > 0) {
                const int hsh = sh;
                sh = sh > 8 ? sh - 8 : 0;
                const uint32_t mask = (1u << (hsh - sh)) - 1u;
#pragma unroll
                for (int q = 0; q < 4; ++q) hist[tid + 64 * q] = 0u;
                wave_lds_sync();
                for (uint32_t g0 = 0; g0 < G; g0 += 64) {
                    const uint32_t gi = g0 + tid;
                    const uint32_t d = gi < G ? gk[gi] : 0u;
                    hist_add(hist, (d >> sh) & mask, gi < G && (d >> hsh) == prefix);
                }
                wave_lds_sync();
                wave_find_bin8(hist, rem, res);
                wave_lds_sync();
                const uint32_t bin = (uint32_t)__builtin_amdgcn_readfirstlane((int)res[0]);
                const uint32_t above = (uint32_t)__builtin_amdgcn_readfirstlane((int)res[1]);
                prefix = (prefix << (hsh - sh)) | bin;
                rem -= above;
                wave_lds_sync();  // res and hist are rewritten by the next round
            }
            if (tid == 0) {
                res[5] = prefix;
                res[6] = rem;
            }
        }
        __syncthreads();
        prefix = res[5];
        rem = res[6];
    }
    uint32_t T = kmin + prefix;  // keep every key above T and the first rem keys equal to T
    // Threshold mode: when the k-th key is not above the floor, the kept set
    // is every key above the floor (all on the list, since they outrank the
    // k-th key); otherwise the top-k set is already above it.
    const bool floored = a.floor.on && T <= a.floor.key;
    if (floored) {
        T = a.floor.key;
        rem = 0;
    }
    // Ordered compaction: every key above T, and the T-ties in list order.
    bool gt[PER], eq[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        gt[e] = key[e] > T;
        eq[e] = key[e] == T;
    }
    uint32_t pk[PER], tot;
    list_prefix2<PER>(gt, eq, tbl, pk, &tot);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const uint32_t gb = pk[e] >> 16, eb = pk[e] & 0xffffu;
        if (gt[e]) out[gb + min(eb, rem)] = (int32_t)ix[e];
        else if (eq[e] && eb < rem) out[gb + eb] = (int32_t)ix[e];
    }
    if (floored)
        for (int j = (int)(tot >> 16) + tid; j < k; j += SL_NT) out[j] = -1;
    if (a.floor.on && tid == 0) a.floor.done[(size_t)b * a.n_q + qrow(a, i)] = 1u;
}
template <int PER>
__global__ __launch_bounds__(SL_NT) void prefill_select_kernel(PrefillArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t gk[SL_GMAX];
    __shared__ uint32_t tbl[PER * SL_NT / 64 + 1];
    __shared__ uint32_t res[8];
    SelRow<PER> rw;
    sel_fetch<PER>(a, blockIdx.x, rw);
    select_row<PER>(a, blockIdx.x, rw, hist, gk, tbl, res);
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
        const int b = (int)(task / a.rows), i = (int)(task % a.rows);
        const int len = row_len(a, i);
        Frag<DT, D> fq;  // the query row, broadcast to all 16 B columns
        fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + qrow(a, i)) * RB, g);
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
        int32_t* out = a.idx + ((size_t)b * a.n_q + qrow(a, i)) * a.top_k;
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
        constexpr int QT = filter_qt<DT, D>();
        const long long nb = (long long)a.B * ((a.rows + 64 * QT - 1) / (64 * QT));
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_filter_kernel<DT, D, QT>), dim3((unsigned)nb), dim3(320), 0, s,
                           a);
    } else if (part == 2) {
        if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)rows), blk(SL_NT);
        // PER = ceil(cap / SL_NT) entries per thread at most
        const int per = (a.cap + SL_NT - 1) / SL_NT;
        if (per <= 2) hipLaunchKernelGGL(prefill_select_kernel<2>, grid, blk, 0, s, a);
        else if (per <= 4) hipLaunchKernelGGL(prefill_select_kernel<4>, grid, blk, 0, s, a);
        else if (per <= 8) hipLaunchKernelGGL(prefill_select_kernel<8>, grid, blk, 0, s, a);
        else if (per <= 11) hipLaunchKernelGGL(prefill_select_kernel<11>, grid, blk, 0, s, a);
        else if (per <= 14) hipLaunchKernelGGL(prefill_select_kernel<14>, grid, blk, 0, s, a);
        else if (per <= 18) hipLaunchKernelGGL(prefill_select_kernel<18>, grid, blk, 0, s, a);
        else if (per <= 26) hipLaunchKernelGGL(prefill_select_kernel<26>, grid, blk, 0, s, a);
        else return hipErrorInvalidValue;
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
    // expected list length is about 2 top_k; room for sampling spread and ties
    return (3 * top_k + 768 + 63) / 64 * 64;
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
