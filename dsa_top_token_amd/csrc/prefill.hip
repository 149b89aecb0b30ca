// Many-row (prefill-shaped) selection with a sampled threshold on gfx950:
// the indexer sweep keeps only candidate keys, so no score matrix is written.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), sections 3.2-3.3 and 4.3: the
// indexer scores each query's causal prefix and the query keeps its top_k
// keys; the page fuses indexing, selection and masking to avoid writing the
// intermediates. Kernels, per slab of query rows:
//   threshold  per 16- or 32-row block: scores every S-th key of each row's prefix
//              (MFMA), two 9-bit radix rounds over those samples give tau,
//              the lower edge of the 18-bit bin holding the m-th largest
//              sample (m S ~ 2 top_k); tau becomes tau', the smallest fp32
//              accumulator whose scaled score reaches it, rounded toward zero
//              to 8 significant bits. A row whose sample threshold is not
//              positive keeps every non-negative accumulator instead ("zero
//              mode").
//   filter     per block of 64 to 352 rows: a producer wave streams the
//              block's causal keys into an LDS ring of key slots (128 keys
//              for narrow fp8 rows, else 64) with global->LDS copies, several
//              slots in flight; consumer waves (eleven of 16 rows for narrow
//              fp8 rows, else four, eleven or three of 16 or 32) score
//              every slot on MFMA, starting each accumulator at -tau', so a
//              score's accept bit is its sign bit. Keys are the MFMA row
//              operand, so each lane holds consecutive keys of one query and
//              one funnel shift per score builds the lane's accept mask; the
//              accepted (acc - tau', index) pairs go to the row's list in
//              ascending index order. Problems with few rows cut the keys
//              into up to four ranges, each with its own sub-list per row.
//   select     one 512-thread workgroup per row with its list in registers:
//              8-bit radix rounds over the order keys relative to the key of
//              tau' give the exact k-th key T (wave 0 finishes once T's bin
//              is small); the T-ties are cut in list (= index) order. A
//              zero-mode row with fewer than top_k positive scores takes its
//              positives plus the lowest-index zero scores. A row whose
//              threshold kept fewer than top_k keys, or more than its list
//              holds, is queued.
//   fallback   a persistent kernel recomputes each queued row's scores into
//              the workspace and selects on them with the per-row radix
//              schedule.
#include "frag.h"
#include "topk_common.h"
#include "lanes.h"

#include <type_traits>
#include <vector>

namespace dsa {
namespace {

using namespace frag;
using namespace topk;

constexpr int TH_ROWS_MAX = 32;   // rows per threshold workgroup (at most)
constexpr int TH_DIG = 9;         // bits per digit of the two threshold rounds (the
                                  // 16 x 512-word histogram fits four workgroups per CU)
constexpr int TH_BINS = 1 << TH_DIG;
constexpr int TH_MAX_SAMPLES = 4096;
constexpr int TH_TARGET = 64;     // samples expected above tau
constexpr int FL_CHUNK = 64;      // keys per staged chunk of the filter
constexpr int FB_WGS = 256;       // fallback workgroups
// Key ranges of the many-row filter: a row longer than kRangeMin keys is cut
// into at most kRangesMax ranges of rk keys (a multiple of every slot width),
// each scored by workgroups of its own into a sub-list of its own, so that no
// workgroup streams more than rk keys and the longest rows no longer set the
// kernel time by themselves.
constexpr int kRangeMin = 16384;
constexpr int kRangesMax = 4;
constexpr long long kRangeRowsMin = 16384;  // B x rows from which rows are not split
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

// The filter's accumulator threshold tau': t rounded toward zero to 8
// significant bits when t >= 1/16 (then acc - tau' is exact for integer
// indexer inputs: see the filter), smaller thresholds unchanged. Keys with
// acc >= t all have acc >= tau', so the lists keep at least those keys.
__device__ __forceinline__ float snap_tau(float t) {
    return t >= 0.0625f ? __uint_as_float(__float_as_uint(t) & 0xFFFF0000u) : t;
}

// The bin of a wave-private histogram (nbins, bins owned top-down by lanes)
// holding the rem-th largest counted key: returns bin, *above = count of
// keys in higher bins. Every lane of the wave calls it.
// The counts are the 16-bit fields at bit sh of the histogram words.
template <int NBINS>
__device__ __forceinline__ uint32_t wave_find_bin(const uint32_t* hist, int sh, uint32_t rem,
                                                  uint32_t* above_out) {
    constexpr int PER = NBINS / 64;
    const int lane = threadIdx.x & 63;
    const int hi = NBINS - 1 - lane * PER;
    uint32_t loc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) loc += (hist[hi - i] >> sh) & 0xffffu;
    uint32_t above = wave_incl_scan(loc) - loc;
    uint32_t bin = 0, ab = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint32_t c = (hist[hi - i] >> sh) & 0xffffu;
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

// Row-major key slots in LDS: slot key r occupies RB contiguous bytes at
// tile + r RB, its 16-byte granule q at granule slot q ^ sw(r). The slot is
// contiguous in global memory too, so each 1 KB global->LDS copy reads 1 KB
// of consecutive bytes (every 4 lanes one 64-byte segment: XOR keeps aligned
// groups of four granules together). A fragment read touches slot keys
// r = 16 G a + 4 u + b (a, b = 0..3) for one tile u of a 64 G-key slot; the
// row pitch already separates some values of b in the LDS banks, so sw takes
// a and the bits of b that the pitch leaves together, as far as q ^ sw stays
// below GPR.
constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }
constexpr int log2_c(int x) { return x <= 1 ? 0 : 1 + log2_c(x / 2); }

template <int RB, int G>
struct RingSw {
    static constexpr int GPR = RB / 16;             // granules per key row
    static constexpr int P2 = GPR & -GPR;           // largest power of two dividing GPR
    static constexpr int SWM = (P2 < 16 ? P2 : 16) - 1;
    static constexpr int SB = (RB / 4) % 64 == 32 ? 1 : 0;  // pitch separates b & 1 only
    static constexpr int AS = 4 + log2_c(G);        // r >> AS = a
    __device__ static __forceinline__ int sw(int r) {
        return (((r >> AS) & 3) | (((r & 3) >> SB) << 2)) & SWM;
    }
    // byte b of slot key r
    __device__ static __forceinline__ const uint8_t* at(const uint8_t* tile, int r, int b) {
        return tile + r * RB + 16 * ((b >> 4) ^ sw(r)) + (b & 15);
    }
};

// Fragment of slot key r from a row-major ring slot (the same bytes, in the
// same register slots, as Frag::load takes from a contiguous row). The XOR
// only touches the low bits of the granule index, so each read is a
// per-lane base plus a constant offset.
template <int RB, int G, int D>
__device__ __forceinline__ void load_rm(Frag<0, D>& f, const uint8_t* tile, int r, int g) {
    using W = RingSw<RB, G>;
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

template <int RB, int G, int D>
__device__ __forceinline__ void load_rm(Frag<1, D>& f, const uint8_t* tile, int r, int g) {
    using W = RingSw<RB, G>;
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

// Query tiles of 16 rows per threshold workgroup, and sampled-key tiles
// loaded together per pass. Every sampled key row is loaded once per
// workgroup and scored against all its query tiles; the sampled rows are the
// same for every workgroup of a slab, so these loads are L2 reads whose volume
// the rows per workgroup set. bf16 d = 160 at 131072 rows: two tiles of
// 16 rows with two key tiles per pass took the threshold and select from
// 2.36 to 2.18 ms (one tile with four key tiles: 2.36; two with four, more
// registers: 2.42); fp8 d = 128 at 65536 rows gained nothing from two tiles.
template <int DT>
constexpr int th_qt() { return DT == 1 ? 2 : 1; }
template <int DT>
constexpr int th_un() { return DT == 1 ? 2 : 4; }

// Each workgroup covers 16 th_qt rows with one sample stride S. Row 16 t + j
// counts in the 16-bit field 16 t of word [j][bin] (at most 4096 samples per
// row).
template <int DT, int D>
__global__ __launch_bounds__(256) void prefill_threshold_kernel(PrefillArgs a) {
    constexpr int TH_QT = th_qt<DT>(), TH_UN = th_un<DT>(), TH_ROWS = 16 * TH_QT;
    __shared__ uint32_t hist[16][TH_BINS];
    __shared__ uint32_t digit1[TH_ROWS];
    __shared__ uint32_t rem1[TH_ROWS];
    static_assert(TH_ROWS <= TH_ROWS_MAX && TH_MAX_SAMPLES < 65536, "at most two 16-bit counts per word");
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

    Frag<DT, D> fq[TH_QT];  // A operands: query tile t holds rows r0 + 16 t + n
#pragma unroll
    for (int t = 0; t < TH_QT; ++t)
        fq[t].load(static_cast<const uint8_t*>(a.q) +
                       ((size_t)b * a.n_q + qrow(a, min(r0 + 16 * t + n, a.rows - 1))) * RB, g);
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;
    // Sample count of the rows this lane's scores belong to (rows 16 t + 4g + r).
    int ns_r[TH_QT][4];
#pragma unroll
    for (int t = 0; t < TH_QT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + 16 * t + 4 * g + r;
            ns_r[t][r] = row < a.rows ? (row_len(a, row) + S - 1) / S : 0;
        }

#pragma unroll 1
    for (int round = 0; round < 2; ++round) {
        for (int i = threadIdx.x; i < 16 * TH_BINS; i += 256) (&hist[0][0])[i] = 0u;
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
#pragma unroll
                for (int t = 0; t < TH_QT; ++t) {
                    const f32x4 acc = tile_dot_k32<D>(fq[t], fk[u]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 4 * g + r, row = 16 * t + j;
                        const uint32_t key = rank_key(relu_scaled(acc[r], a.scale));
                        const bool ok = t0 + n < ns_r[t][r];
                        const bool in = round == 0 ? ok : ok && (key >> (32 - TH_DIG)) == digit1[row];
                        const uint32_t bin = round == 0 ? (key >> (32 - TH_DIG))
                                                        : ((key >> (32 - 2 * TH_DIG)) & (TH_BINS - 1u));
                        // packed 16-bit counts (query tile t in half t of the word), by
                        // plain LDS atomics: first merging the lanes that add to the
                        // same word as the wave's first active lane (a vote and two
                        // read-lanes per key) timed 203 against 167 us at 64K rows
                        if (in) atomicAdd(&(&hist[0][0])[(uint32_t)j * TH_BINS + bin], 1u << (16 * t));
                    }
                }
            }
        }
        __syncthreads();
        // Each wave resolves TH_ROWS / 4 rows.
        for (int rr = 0; rr < TH_ROWS / 4; ++rr) {
            const int row = wave * (TH_ROWS / 4) + rr;
            uint32_t above;
            const uint32_t want = round == 0 ? m : rem1[row];
            const uint32_t bin = wave_find_bin<TH_BINS>(hist[row & 15], 16 * (row >> 4), want, &above);
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
                                tacc = snap_tau(raw_threshold(tau, a.scale));
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

// Slot width of the filter's key ring, in 64-key units: lane (n, g) of a
// consumer wave scores keys [16 G g, 16 G g + 16 G) of a 64 G-key slot for
// its query n, so one accept mask covers 16 G consecutive keys of one row and
// a row's four lanes hold the slot in index order. Two units halve the
// per-row prefix and emission passes per score; wide rows keep one (the
// fragments of all 4 G key tiles of a slot sit in registers at once).
template <int DT, int D>
constexpr int filter_g() { return DT == 0 && D <= 128 ? 2 : 1; }

// Query tiles per consumer wave of the filter. Two tiles halve the ring
// traffic and fragment reads per row (bf16 128K: 7.7 -> 6.4 ms).
template <int DT, int D>
constexpr int filter_qt() { return DT == 1 ? 2 : 1; }

// Consumer waves per filter workgroup. Every workgroup streams its rows'
// causal keys through the ring once, so the rows per workgroup set how often
// each key row is read: 96-row workgroups re-read the 320-byte keys of a
// 131072-row bf16 d = 160 prefill 28.6 GB worth, and the address and data
// units were the filter's busiest. Eleven consumer waves and the producer
// (three waves per SIMD, their registers fit in 170) cover 352 rows, one
// workgroup per CU: 5.0 -> 4.2 ms. The narrow fp8 rows (128-key slots) also
// take eleven consumer waves of 16 rows: 0.99 against 1.02 ms with eight at
// 65536 rows (fifteen, four per SIMD: 1.22). Other fp8 widths keep four, and
// wider bf16 rows three (their waves need more than 170 registers).
template <int DT, int D>
constexpr int filter_nw() {
    return filter_g<DT, D>() == 2 ? 11 : (DT == 1 && D > 128 ? (D <= 160 ? 11 : 3) : 4);
}

// Ring depth of the key-slot pipeline, and key slots consumed between two
// workgroup barriers (fl_sb): the consumers score and emit fl_sb slots per
// barrier while the producer fills the next NBUF - fl_sb. Fewer barriers per
// key, and each consumer's emission work evened out between them: the
// 65536-row fp8 filter took 0.995 ms with one slot per barrier, 0.914 with
// two (5-slot ring) and 0.883 with three (6 slots of 16 KB); the 131072-row
// bf16 d = 160 filter 4.29 -> 4.23 ms with two (4 slots of 20 KB).
template <int RB, int G>
constexpr int fl_nbuf() {
    return FL_CHUNK * G * RB <= 16384 ? 6 : (FL_CHUNK * G * RB <= 20480 ? 4 : 2);
}
template <int RB, int G>
constexpr int fl_sb() { return fl_nbuf<RB, G>() == 6 ? 3 : (fl_nbuf<RB, G>() >= 4 ? 2 : 1); }

// Waits until at most `ahead` slots of CPS copies each are in flight
// (0 <= ahead <= A).
template <int A, int CPS>
__device__ __forceinline__ void wait_chunks(int ahead) {
    if constexpr (A > 0) {
        if (ahead >= A) {
            wait_vmcnt<A * CPS>();
            return;
        }
        wait_chunks<A - 1, CPS>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}
static_assert(FL_CHUNK == 64, "the producer's lane -> key map covers 64-key units");

// The threshold enters the MFMA as its initial accumulator: the product of a
// key tile with a query tile starting from -tau' leaves acc - tau' for every
// pair, so the accept bit of a key is the sign bit of its accumulator
// (+0.0 when acc == tau' is accepted). tau' is the row's accumulator
// threshold rounded toward zero to 8 significant bits, so with integer
// indexer inputs (exact products and sums, |acc| < 2^13) every partial sum is
// a multiple of ulp(tau') >= 2^-11 below 2^13 and acc - tau' is exact. The
// lists hold acc - tau'; the select adds tau' back (exact for the same
// reason).
//
// QT query tiles of 16 rows per consumer wave share every key fragment read
// from the ring (the workgroup covers 64 QT rows).
template <int DT, int D, int QT, int G, int NW>
__global__ __launch_bounds__(64 * (NW + 1)) void prefill_filter_kernel(PrefillArgs a) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    // Ring layout: row-major for fp8 keys (timed 1.31 -> 1.20 ms at 64K),
    // granule-major for bf16 (row-major timed 6.4 -> 6.9 ms at 128K).
    constexpr bool RM = DT == 0;
    static_assert(RM || G == 1, "granule-major slots hold 64 keys");
    constexpr int SK = FL_CHUNK * G;       // keys per slot
    constexpr int LK = 16 * G;             // keys per lane per slot
    constexpr int NU = 4 * G;              // 16-key tiles per slot
    constexpr int WROWS = 16 * QT;         // rows per consumer wave
    constexpr int ROWS = NW * WROWS;       // rows per workgroup (NW consumer waves)
    constexpr int LKH = LK < 16 ? LK : 16; // accumulators staged per lane at a time
    constexpr int GPR = RB / 16;           // 16-byte granules per key row
    constexpr int CPS = G * GPR;           // 1 KB copies per slot
    constexpr int NBUF = fl_nbuf<RB, G>();
    constexpr int SB = fl_sb<RB, G>();
    // copies in flight stay below the 6-bit vmcnt limit
    static_assert(RB % 16 == 0 && (NBUF - SB) * CPS < 64 && NBUF >= 2 * SB, "slot pipeline");
    // Key slots: row-major with swizzled granules (RingSw), or granule-major
    // (granule j of the key at row position rp at slot + j * 1024 + 16 rp).
    __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF][SK * RB];
    // per-wave stage of 16 of a lane's accumulators at a time: value i of
    // lane l at [i][l] (a lane's reads of different i hit different banks)
    __shared__ float stage[NW][LKH * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_blk = (a.rows + ROWS - 1) / ROWS;
    // Work item (sequence b, row block blk, key range rg): the block's rows
    // against keys [rg rk, (rg + 1) rk), into sub-list rg of each row. Largest
    // blocks (latest rows) first; ranges past the block's last key are empty.
    // Consecutive workgroups are dealt in turn to the 8 XCDs and, within an
    // XCD, to its 4 shader engines, so each run of 32 consecutive workgroups
    // takes one range of 32 blocks: every shader engine gets every range
    // (later ranges are shorter or empty).
    const int b = blockIdx.x % a.B;
    const int j = (int)(blockIdx.x / (unsigned)a.B);
    const int rg = (j >> 5) % a.nr;
    const int bj = (j >> 5) / a.nr * 32 + (j & 31);
    if (bj >= n_blk) return;  // the grid covers whole runs of 32
    const int blk = n_blk - 1 - bj;
    const int i0 = blk * ROWS;
    const int kend = row_len(a, min(i0 + ROWS, a.rows) - 1);
    const int kr0 = rg * a.rk;
    if (kr0 >= kend) return;  // the whole workgroup
    const int kr1 = min(kr0 + a.rk, kend);
    const int c0 = kr0 / SK;              // rk is a multiple of SK
    const int c1 = (kr1 + SK - 1) / SK;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;

    if (wave == NW) {
        // Producer: global -> LDS copies, NBUF - SB slots ahead.
        //   row-major (RM): copy i moves granules 64 i .. 64 i + 63 of the
        //     slot: lane l fills granule slot s = P % GPR of slot key
        //     r = P / GPR (P = 64 i + l) with the key's granule s ^ sw(r);
        //   granule-major: copy j moves granule j of every key, lane l taking
        //     the key at row position l (slot key 16 ((l / 4) % 4) + 4 (l / 16)
        //     + l % 4).
        const int kr = 16 * ((lane >> 2) & 3) + 4 * (lane >> 4) + (lane & 3);
        auto issue = [&](int c) {
            uint8_t* dst = ring[c % NBUF];
#pragma unroll
            for (int i = 0; i < CPS; ++i) {
                if constexpr (RM) {
                    const int P = 64 * i + lane, r = P / GPR,
                              q = (P % GPR) ^ RingSw<RB, G>::sw(r);
                    const int key = min(c * SK + r, a.n_k - 1);
                    __builtin_amdgcn_global_load_lds(kbase + (size_t)key * RB + 16 * q,
                                                     dst + 1024 * i, 16, 0, 0);
                } else {
                    const int key = min(c * SK + kr, a.n_k - 1);
                    __builtin_amdgcn_global_load_lds(kbase + (size_t)key * RB + 16 * i,
                                                     dst + i * (FL_CHUNK * 16), 16, 0, 0);
                }
            }
        };
        const int pre = min(c0 + NBUF - SB, c1);
        for (int c = c0; c < pre; ++c) issue(c);
        for (int c = c0; c < c1; c += SB) {
            // slots c .. c + SB - 1 have landed once at most `ahead` later
            // slots are in flight
            const int ahead = min(c + NBUF - SB, c1) - min(c + SB, c1);
            wait_chunks<NBUF - 2 * SB, CPS>(ahead);
            // A workgroup barrier without the release fence of __syncthreads
            // (that fence would wait for every copy in flight); the wait
            // above has already made the slots visible in LDS.
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            // into the buffers of slots c - SB .. c - 1, consumed before this barrier
            for (int u = 0; u < SB; ++u)
                if (c + NBUF - SB + u < c1) issue(c + NBUF - SB + u);
        }
        wait_vmcnt<0>();
        return;
    }

    // Consumers: wave w scores rows [i0 + WROWS w, +WROWS) against each slot,
    // query tile t holding rows i0 + WROWS w + 16 t + n.
    const int wi0 = i0 + wave * WROWS;
    int my_i[QT], my_len[QT];
    bool live[QT];
    f32x4 cinit[QT];   // -tau' of the lane's query, the MFMAs' initial accumulator
    Frag<DT, D> fq[QT];
    int row_vo[QT];    // byte offset of the row's sub-list rg in the wave's list block
    uint32_t cnt[QT];  // each row's sub-list length (same in the row's 4 lanes)
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int r = wi0 + 16 * t + n;
        live[t] = r < a.rows;
        my_i[t] = min(r, a.rows - 1);
        my_len[t] = live[t] ? row_len(a, my_i[t]) : 0;
        const float tau = live[t] ? a.tau_acc[(size_t)b * a.rows + my_i[t]] : __builtin_inff();
        cinit[t] = f32x4{-tau, -tau, -tau, -tau};
        fq[t].load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + qrow(a, my_i[t])) * RB, g);
        row_vo[t] = (16 * t + n) * a.cap * 8;
        cnt[t] = 0;
    }
    // Wave-uniform bounds (scalar registers, so the tail test is a branch).
    const int wi0s = __builtin_amdgcn_readfirstlane(wi0);
    const bool wave_live = wi0s < a.rows;
    const int w_kend = wave_live ? row_len(a, min(wi0s + WROWS - 1, a.rows - 1)) : 0;
    const int w_kmin = wave_live ? row_len(a, wi0s) : 0;
    // Sub-lists are stored range-major ([range][row][cap]), so the wave's
    // WROWS sub-lists of range rg are consecutive: one buffer descriptor
    // covers them, and a store takes a 32-bit byte offset.
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.cand + ((size_t)rg * a.B * a.rows + (size_t)b * a.rows + (wave_live ? wi0s : 0)) *
                             a.cap),
        (short)0, WROWS * a.cap * 8, kBufWord3);
    wait_vmcnt<0>();  // the query fragments are in registers before the slot loop
    const uint32_t cap = (uint32_t)a.cap;
    float* stg = &stage[wave][0];
    // value i of this lane in the stage: byte 256 i + 4 lane
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(stg + lane);
    constexpr uint32_t LMASK = LK == 32 ? 0xffffffffu : (1u << LK) - 1u;

    // A operand row n of key tile u is slot key 16 G (n / 4) + 4 u + n % 4
    // (row position 16 u + n in the granule-major layout), so output row
    // 4 g + r of tile u is key 16 G g + 4 u + r: lane (n, g) holds keys
    // [16 G g, 16 G g + 16 G) of the slot, value i = 4 u + r.
    // Slots below w_kmin lie inside every row's causal range; only the
    // later ones (TAIL) mask keys past a row's end.
    auto slot = [&](const int c, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int k0 = c * SK;
        if (k0 < w_kend) {
            const uint8_t* tile = ring[c % NBUF];
            // Every fragment load of the slot completes before the first
            // MFMA, so no load can overwrite an operand register of an MFMA
            // still queued behind a dependent accumulate chain.
            Frag<DT, D> fk[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if constexpr (RM) load_rm<RB, G>(fk[u], tile, LK * (n >> 2) + 4 * u + (n & 3), g);
                else load_cm<FL_CHUNK * 16>(fk[u], tile, 16 * u + n, g);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc[QT][NU];
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int t = 0; t < QT; ++t) acc[t][u] = tile_dot_c<D>(fk[u], fq[t], cinit[t]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < QT; ++t) {
                // bit i of rej: sign of acc - tau' for key 16 G g + i
                uint32_t rej = 0;
#pragma unroll
                for (int i = LK - 1; i >= 0; --i)
                    rej = __builtin_amdgcn_alignbit(rej, __float_as_uint(acc[t][i >> 2][i & 3]), 31);
                uint32_t bits = ~rej & LMASK;
                if constexpr (TAIL) {
                    const int v = my_len[t] - (k0 + LK * g);
                    bits &= v >= LK ? LMASK : (v <= 0 ? 0u : (1u << v) - 1u);
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
                if (cnt[t] + tot > cap) bits = 0u;
                cnt[t] += tot;
                const int vo0 = row_vo[t] + (int)o * 8;
                // 16 accumulators at a time go through the stage; a lane's
                // lower 16 keys precede its upper 16, so order is kept.
#pragma unroll
                for (int h = 0; h < LK / LKH; ++h) {
                    uint32_t hb = LK == LKH ? bits : ((bits >> (LKH * h)) & 0xffffu);
                    if (__ballot(hb != 0u) == 0ull) continue;
                    int vo = h == 0 ? vo0 : vo0 + 8 * __popc(bits & 0xffffu);
#pragma unroll
                    for (int i = 0; i < LKH; ++i) {
                        const int v = LKH * h + i;
                        stg[64 * i + lane] = acc[t][v >> 2][v & 3];
                    }
                    const uint32_t kb = (uint32_t)(k0 + LK * g + LKH * h);
                    // Four entries per round: their stage reads are issued
                    // together, so a round waits for one LDS latency. Past a
                    // lane's last entry, ctz(hb | 2^31) keeps the read inside
                    // the stage (bit 31 only exists when LKH is 32) and the
                    // store is skipped.
                    while (hb != 0u) {
                        uint32_t ix[4];
                        bool has[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            has[j] = hb != 0u;
                            ix[j] = (uint32_t)__builtin_ctz(hb | (1u << (LKH - 1)));
                            hb &= hb - 1u;
                        }
                        uint32_t v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            v[j] = *reinterpret_cast<const uint32_t*>(sb + 256 * ix[j]);
                        // all four reads complete here (one wait), none sunk
                        // into its conditional store
                        asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
                        // consecutive entries of the lane leave in pairs (16-byte stores)
#pragma unroll
                        for (int j = 0; j < 4; j += 2) {
                            if (has[j + 1])
                                __builtin_amdgcn_raw_buffer_store_b128(
                                    i32x4{(int)v[j], (int)(kb + ix[j]), (int)v[j + 1],
                                          (int)(kb + ix[j + 1])},
                                    lrs, vo + 8 * j, 0, 0);
                            else if (j == 0 || has[j])
                                __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[j], kb + ix[j]}, lrs,
                                                                      vo + 8 * j, 0, 0);
                        }
                        vo += 32;
                    }
                }
            }
        }
    };
    const int c_full = max(c0, min(c1, w_kmin / SK));
    // One barrier per SB slots, matching the producer's. A bare barrier: a
    // consumer's ring reads have completed (lgkmcnt(0)) before its MFMAs, its
    // stage is its own, and its list stores need no order with other waves,
    // so the release fence of __syncthreads would only wait for those stores.
    for (int c = c0; c < c1; c += SB) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        for (int u = 0; u < SB; ++u) {
            const int cc = c + u;
            if (cc >= c1) break;
            if (cc < c_full) slot(cc, std::false_type{});
            else slot(cc, std::true_type{});
        }
    }
#pragma unroll
    for (int t = 0; t < QT; ++t)
        if (g == 0 && live[t]) a.cnt[((size_t)b * a.rows + my_i[t]) * a.nr + rg] = cnt[t];
}

// ------------------------------------------------------------------- select

// Order key of a list entry: the filter stores acc - tau' (tau' the row's
// threshold, exact for integer indexer inputs), so acc = entry + tau'.
__device__ __forceinline__ uint32_t cand_key(uint32_t d_bits, float tau, float scale) {
    return rank_key(relu_scaled(__uint_as_float(d_bits) + tau, scale));
}

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

// One NT-thread workgroup per row. Thread t holds list entries t, t + NT,
// t + 2 NT, ... in registers, so every load instruction of a wave reads 64
// consecutive entries (a lane-per-slice layout made the address unit the
// bottleneck). Each row is a chain of dependent steps, so the kernel is
// bound by how many rows a CU holds at once: two registers per entry (the
// key relative to a lower bound, and the index), ballots taken again after
// a scan rather than kept per entry, and eight waves per SIMD where that fits
// without spilling (128 threads per row with four times the entries per
// thread held more rows but ran each 2.6 times longer). The k-th key T is
// found by 8-bit radix rounds: workgroup-wide while the current bin holds
// many keys, then by wave 0 alone over the keys of that bin gathered into
// LDS. Positions in list (= index) order come from ballots within a wave and
// one table of per-(slot, wave) counts scanned by wave 0.
template <int PER>
struct SelRow {
    uint32_t cnt;
    float tau;
    uint2 raw[PER];
};

// The row's list: its sub-lists (one per key range) concatenated in range
// order, which is index order, so entry j of the list is entry j - pre[q] of
// sub-list q (pre: the exclusive prefix of the sub-list lengths). cnt > cap
// marks a row whose sub-lists overflowed or together exceed cap. Trivial rows
// (at most top_k keys) read nothing.
template <int NT, int PER>
__device__ __forceinline__ void sel_fetch(const PrefillArgs& a, long long task, SelRow<PER>& r) {
    if (task >= (long long)a.B * a.rows) return;
    r.cnt = 0;
    r.tau = a.tau_acc[task];
    const int n = row_len(a, (int)(task % a.rows));
    if (n <= a.top_k) return;
    const int nr = min((n + a.rk - 1) / a.rk, a.nr);  // ranges holding the row's keys
    const uint32_t cap = (uint32_t)a.cap;
    const uint32_t* cp = a.cnt + task * a.nr;
    uint32_t pre[kRangesMax + 1];
    pre[0] = 0;
    bool over = false;
#pragma unroll
    for (int q = 0; q < kRangesMax; ++q) {
        const uint32_t c = q < nr ? cp[q] : 0u;
        over |= c > cap;
        pre[q + 1] = pre[q] + min(c, cap + 1u);
    }
    r.cnt = over || pre[kRangesMax] > cap ? cap + 1u : pre[kRangesMax];
    if (r.cnt > cap) return;
    const uint2* cl = a.cand + (size_t)task * a.cap;
    if (nr == 1) {  // one sub-list (workgroup-uniform)
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t j = (uint32_t)(e * NT) + threadIdx.x;
            r.raw[e] = j < r.cnt ? cl[j] : make_uint2(0u, 0u);
        }
        return;
    }
    const size_t rstep = (size_t)a.B * a.rows * a.cap;  // sub-list q at cl + q rstep
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const uint32_t j = (uint32_t)(e * NT) + threadIdx.x;
        uint2 v = make_uint2(0u, 0u);
        if (j < r.cnt) {
            uint32_t q = 0, o = j;
#pragma unroll
            for (int x = 1; x < kRangesMax; ++x)
                if (j >= pre[x]) {
                    q = (uint32_t)x;
                    o = j - pre[x];
                }
            v = cl[q * rstep + o];
        }
        r.raw[e] = v;
    }
}

// Counts of two flags per (entry slot e, wave), packed (count of fa) << 16 |
// (count of fb), into tbl, then their exclusive scan in list order by wave 0
// ((slot, wave) order is list order: slot e's NT entries precede slot
// e + 1's). Returns the row totals, packed the same way. tbl needs
// PER * NT / 64 + 1 words. Two workgroup barriers; call from every thread.
template <int NT, int PER, typename Flags>
__device__ __forceinline__ uint32_t list_scan2(Flags flags, uint32_t* tbl) {
    constexpr int NW = NT / 64, NE = PER * NW;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        bool fa, fb;
        flags(e, fa, fb);
        const unsigned long long ma = __ballot(fa), mb = __ballot(fb);
        if (lane == 0) tbl[e * NW + w] = ((uint32_t)__popcll(ma) << 16) | (uint32_t)__popcll(mb);
        __builtin_amdgcn_sched_barrier(0);  // one entry at a time: short live ranges
    }
    __syncthreads();
    if (w == 0) {
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
    return tbl[NE];
}

// Packed position of this thread's entry among the flagged entries before it
// in list order, from the scanned table entry of its (slot, wave).
__device__ __forceinline__ uint32_t list_pos2(bool fa, bool fb, uint32_t base) {
    const unsigned long long ma = __ballot(fa), mb = __ballot(fb);
    return base +
           ((__builtin_amdgcn_mbcnt_hi((uint32_t)(ma >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ma, 0u)) << 16) |
            __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u)));
}

template <int NT, int PER>
__device__ __forceinline__ void select_row(const PrefillArgs& a, long long task, const SelRow<PER>& rw,
                                           uint32_t* hist, uint32_t* gk, uint32_t* tbl,
                                           uint32_t* wmax, uint32_t* res) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, w = tid >> 6;
    const int b = (int)(task / a.rows), i = (int)(task % a.rows);
    const int n = row_len(a, i);
    const int k = a.top_k;
    int32_t* out = a.idx + ((size_t)b * a.n_q + qrow(a, i)) * k;
    if (n <= k) {
        fill_prefix(out, n, k, tid, NT);
        return;
    }
    const uint32_t cnt = rw.cnt;
    const bool zero_mode = __float_as_uint(rw.tau) == 0u;
    if (cnt > (uint32_t)a.cap || (!zero_mode && cnt < (uint32_t)k)) {
        if (tid == 0) a.fb_list[atomicAdd(a.fb_count, 1u)] = (uint32_t)task;
        return;
    }
    const int cn = (int)cnt;
    const float scale = a.scale;
    // Keys are held as dk = key - kmin + 1, kmin being the order key of a
    // score of exactly tau' (every entry holds acc - tau' >= +0.0, so every
    // listed key is at least kmin and its dk at least 1). An entry past the
    // count holds dk = 0: below every listed key, so it never reaches the k-th
    // key, and never equal to it.
    const uint32_t kmin = cand_key(0u, rw.tau, scale);
    uint32_t dk[PER], ix[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        dk[e] = e * NT + tid < cn ? cand_key(rw.raw[e].x, rw.tau, scale) - kmin + 1u : 0u;
        ix[e] = rw.raw[e].y;
    }
    if (tid == 0) res[4] = 0u;

    if (zero_mode) {
        // The list holds every key with a positive score (plus some zeros);
        // every key off the list scores zero. With tau' = 0, kmin is the key
        // of a zero score, so an entry is positive when its dk exceeds 1.
        const uint32_t np = list_scan2<NT, PER>(
            [&](int e, bool& fa, bool& fb) {
                fa = dk[e] > 1u;
                fb = false;
            },
            tbl) >> 16;
        if (np < (uint32_t)k) {
            // Positives plus the lowest-index zeros. With P the positives in
            // index order, P[r] - r zeros precede P[r]; P[r] - r does not
            // decrease with r, so the positives with P[r] - r < Z (those
            // before the Z-th zero) are the first cs of them.
            const uint32_t Z = (uint32_t)k - np;
            uint32_t early = 0;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const bool pos = dk[e] > 1u;
                const uint32_t r = list_pos2(pos, false, tbl[e * NW + w]) >> 16;
                early += pos && ix[e] - r < Z ? 1u : 0u;
                __builtin_amdgcn_sched_barrier(0);
            }
            early = wave_incl_scan(early);
            if ((tid & 63) == 63) atomicAdd(&res[4], early);
            __syncthreads();
            const uint32_t cs = res[4];
            const uint32_t head = Z + cs;  // out[0, head) = 0 .. head - 1
            for (uint32_t o = tid; o < head; o += NT) out[o] = (int32_t)o;
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const bool pos = dk[e] > 1u;
                const uint32_t r = list_pos2(pos, false, tbl[e * NW + w]) >> 16;
                if (pos && r >= cs) out[Z + r] = (int32_t)ix[e];
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
    }

    // Radix digits of dk, from the top bit of the row's largest dk.
    uint32_t hi = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) hi = max(hi, dk[e]);
    hi = wave_max(hi);
    if ((tid & 63) == 0) wmax[w] = hi;
    __syncthreads();
    uint32_t range = 0u;
#pragma unroll
    for (int x = 0; x < NW; ++x) range = max(range, wmax[x]);
    // Radix rounds over bits [sh, hsh) of dk, from the top. Counts go in by
    // plain LDS atomics, here and in wave 0's rounds below: aggregating the
    // lanes of a wave that share a bin first (a vote, a first-lane pick and a
    // read-lane per key) timed 744 against 669 us at 65536 rows.
    uint32_t rem = (uint32_t)k, prefix = 0;
    int sh = 32 - __clz((int)range);
    bool first = true, gathered = false;
    while (sh > 0 && !gathered) {
        const int hsh = sh;
        sh = sh > 8 ? sh - 8 : 0;
        const uint32_t mask = (1u << (hsh - sh)) - 1u;
        for (int x = tid; x < 256; x += NT) hist[x] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (e * NT >= cn) continue;  // workgroup-uniform
            if (first || (dk[e] >> hsh) == prefix) atomicAdd(&hist[(dk[e] >> sh) & mask], 1u);
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
            // Independent per-key atomics: the entries' appends overlap in
            // the LDS pipeline. Appends chained through one wave-wide
            // reservation per entry (ballot, atomic, broadcast) timed 2.28
            // against 1.63 ms at 131072 rows, and one reservation for all of
            // a wave's entries 1.95.
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                if (e * NT >= cn) continue;  // workgroup-uniform
                if ((dk[e] >> sh) == prefix) gk[atomicAdd(&res[4], 1u)] = dk[e];
            }
            gathered = true;
        }
        __syncthreads();
    }
    if (gathered) {
        const uint32_t G = res[4];
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
                    if (gi < G && (d >> hsh) == prefix) atomicAdd(&hist[(d >> sh) & mask], 1u);
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
    // The k-th key T = kmin + prefix - 1: keep every key above T and the
    // first rem keys equal to it (in dk terms: above, or equal to, prefix).
    uint32_t Td = prefix;
    // Threshold mode: when the k-th key is not above the floor, the kept set
    // is every key above the floor (all on the list, since they outrank the
    // k-th key); otherwise the top-k set is already above it. A floor below
    // kmin keeps every listed key (dk above 0).
    const bool floored = a.floor.on && kmin + prefix - 1u <= a.floor.key;
    if (floored) {
        Td = a.floor.key >= kmin ? a.floor.key - kmin + 1u : 0u;
        rem = 0;
    }
    // Ordered compaction: every key above T, and the T-ties in list order.
    const uint32_t tot = list_scan2<NT, PER>(
        [&](int e, bool& fa, bool& fb) {
            fa = dk[e] > Td;
            fb = dk[e] == Td;
        },
        tbl);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const bool gt = dk[e] > Td, eq = dk[e] == Td;
        const uint32_t pk = list_pos2(gt, eq, tbl[e * NW + w]);
        const uint32_t gb = pk >> 16, eb = pk & 0xffffu;
        if (gt) out[gb + min(eb, rem)] = (int32_t)ix[e];
        else if (eq && eb < rem) out[gb + eb] = (int32_t)ix[e];
        __builtin_amdgcn_sched_barrier(0);
    }
    if (floored)
        for (int j = (int)(tot >> 16) + tid; j < k; j += NT) out[j] = -1;
    if (a.floor.on && tid == 0) a.floor.done[(size_t)b * a.n_q + qrow(a, i)] = 1u;
}

template <int NT, int PER>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(PER <= 14 ? 8 : 1))) void prefill_select_kernel(PrefillArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t gk[SL_GMAX];
    __shared__ uint32_t tbl[PER * NT / 64 + 1];
    __shared__ uint32_t wmax[NT / 64];
    __shared__ uint32_t res[8];
    SelRow<PER> rw;
    sel_fetch<NT, PER>(a, blockIdx.x, rw);
    select_row<NT, PER>(a, blockIdx.x, rw, hist, gk, tbl, wmax, res);
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
        constexpr int TH_ROWS = 16 * th_qt<DT>();
        const long long nb = (long long)a.B * ((a.rows + TH_ROWS - 1) / TH_ROWS);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_threshold_kernel<DT, D>), dim3((unsigned)nb), dim3(256), 0, s,
                           a);
    } else if (part == 1) {
        constexpr int QT = filter_qt<DT, D>();
        constexpr int G = filter_g<DT, D>();
        constexpr int NW = filter_nw<DT, D>();
        constexpr int ROWS = 16 * QT * NW;
        const long long nb =
            (long long)a.B * a.nr * (((a.rows + ROWS - 1) / ROWS + 31) / 32 * 32);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_filter_kernel<DT, D, QT, G, NW>), dim3((unsigned)nb),
                           dim3(64 * (NW + 1)), 0, s, a);
    } else if (part == 2) {
        if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)rows), blk(512);
        // PER = ceil(cap / 512) entries per thread at most
        const int per = (a.cap + 511) / 512;
        if (per <= 2) hipLaunchKernelGGL((prefill_select_kernel<512, 2>), grid, blk, 0, s, a);
        else if (per <= 4) hipLaunchKernelGGL((prefill_select_kernel<512, 4>), grid, blk, 0, s, a);
        else if (per <= 8) hipLaunchKernelGGL((prefill_select_kernel<512, 8>), grid, blk, 0, s, a);
        else if (per <= 11) hipLaunchKernelGGL((prefill_select_kernel<512, 11>), grid, blk, 0, s, a);
        else if (per <= 14) hipLaunchKernelGGL((prefill_select_kernel<512, 14>), grid, blk, 0, s, a);
        else if (per <= 18) hipLaunchKernelGGL((prefill_select_kernel<512, 18>), grid, blk, 0, s, a);
        else if (per <= 26) hipLaunchKernelGGL((prefill_select_kernel<512, 26>), grid, blk, 0, s, a);
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

namespace {
int range_keys(int maxlen) {
    int rk = (maxlen + kRangesMax - 1) / kRangesMax;
    rk = (rk + 127) / 128 * 128;
    return rk < kRangeMin ? kRangeMin : rk;
}
}  // namespace

// Keys per range when a row of up to maxlen keys is cut into nr ranges: a
// multiple of every slot width (128 keys), nr ranges covering maxlen keys.
int prefill_range_len(int maxlen, int nr) {
    const long long rk = ((long long)maxlen + nr - 1) / nr;
    return (int)((rk + 127) / 128 * 128);
}

int prefill_nranges(int maxlen, long long rows) {
    // Ranges pay off when few row blocks would otherwise leave CUs idle
    // (few long rows, e.g. a chunk of queries at the end of a long context).
    // With many rows every CU already holds whole blocks, and the extra
    // sub-lists would only cost memory (more slabs).
    if (rows >= kRangeRowsMin) return 1;
    const int rk = range_keys(maxlen);
    const int nr = (maxlen + rk - 1) / rk;
    return nr < 1 ? 1 : nr;
}

size_t prefill_ws_bytes(int B, int rows, int n_k, int top_k, int nr_) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t r = (size_t)B * rows, nr = (size_t)nr_;
    return al(r * 4) + al(r * nr * 4) + al(r * nr * (size_t)prefill_cap(top_k) * 8) + al(r * 4) +
           al(4) + al((size_t)FB_WGS * n_k * 4);
}

hipError_t prefill_stats(const PrefillArgs& a0, const void* ws, long long out[4]) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t r = (size_t)a0.B * a0.rows;
    const int cap = prefill_cap(a0.top_k);
    const long long ml = (long long)a0.q_pos0 + a0.n_q;
    const int maxlen = (int)(ml < a0.n_k ? ml : a0.n_k);
    const int nr = a0.nr, rk = prefill_range_len(maxlen, nr);
    const char* p = static_cast<const char*>(ws) + al(r * 4);
    std::vector<uint32_t> cnt(r * nr);
    hipError_t e = hipMemcpy(cnt.data(), p, cnt.size() * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    p += al(r * nr * 4) + al(r * nr * (size_t)cap * 8) + al(r * 4);
    uint32_t fb = 0;
    if ((e = hipMemcpy(&fb, p, 4, hipMemcpyDeviceToHost)) != hipSuccess) return e;
    long long rows = 0, cand = 0, over = 0;
    for (size_t t = 0; t < r; ++t) {
        const long long pos = (long long)a0.q_pos0 + a0.row0 + (long long)(t % a0.rows) * a0.rstride;
        const long long n = pos + 1 < a0.n_k ? pos + 1 : a0.n_k;
        if (n <= a0.top_k) continue;
        const int q = (int)std::min<long long>((n + rk - 1) / rk, nr);
        long long tot = 0;
        bool ov = false;
        for (int x = 0; x < q; ++x) {
            tot += cnt[t * nr + x];
            ov |= cnt[t * nr + x] > (uint32_t)cap;
        }
        ++rows;
        cand += tot;
        over += ov || tot > cap;
    }
    out[0] = rows;
    out[1] = cand;
    out[2] = fb;
    out[3] = over;
    return hipSuccess;
}

hipError_t launch_prefill_select(PrefillArgs a, void* ws, int part, hipStream_t s) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t r = (size_t)a.B * a.rows;
    a.cap = prefill_cap(a.top_k);
    const long long ml = (long long)a.q_pos0 + a.n_q;
    const int maxlen = (int)(ml < a.n_k ? ml : a.n_k);
    a.rk = prefill_range_len(maxlen, a.nr);  // a.nr: set by the caller (prefill_nranges)
    char* p = static_cast<char*>(ws);
    a.tau_acc = reinterpret_cast<float*>(p);
    p += al(r * 4);
    a.cnt = reinterpret_cast<uint32_t*>(p);
    p += al(r * a.nr * 4);
    a.cand = reinterpret_cast<uint2*>(p);
    p += al(r * a.nr * (size_t)a.cap * 8);
    a.fb_list = reinterpret_cast<uint32_t*>(p);
    p += al(r * 4);
    a.fb_count = reinterpret_cast<uint32_t*>(p);
    p += al(4);
    a.fb_scores = reinterpret_cast<float*>(p);
    return a.dtype == 0 ? launch_dt<0>(a, part, s) : launch_dt<1>(a, part, s);
}

}  // namespace dsa
