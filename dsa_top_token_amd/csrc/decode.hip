// Decode-shaped selection (one query row per sequence, long key rows) with a
// sampled threshold, on gfx950.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), sections 3.2-3.3: the indexer
// scores every key of the query's prefix and the query keeps its top_k keys.
// Here the full score row never reaches memory:
//   threshold  every S-th key of the row (S = max(top_k / 32, ceil(n/8192)))
//              is scored with fp32 VALU dot products over coalesced row loads
//              by several small workgroups per sequence (a sampled row is a
//              scattered read, and one CU alone pulls them at a fraction of
//              the chip's rate); then one workgroup per sequence takes as tau
//              the lower edge of the bin (two 8-bit radix rounds over the
//              sample keys relative to the smallest) holding the m-th largest
//              sample, m = ceil(2 * top_k / S). About 2 * top_k keys of the
//              row are expected to reach tau.
//   filter     the streaming indexer kernel scores every key and keeps only
//              those whose order key is >= tau, each wave writing its own
//              (order key, index) list for its 256 keys in ascending index
//              order (no device atomics). Key rows of up to 160 bytes are
//              streamed by contiguous nontemporal global->LDS copies into a
//              two-buffer ring per wave; wider rows load MFMA fragments
//              directly.
//   select     one workgroup per sequence loads the candidates into LDS and
//              finds the exact k-th key T from the keys relative to tau: a
//              12-bit radix round over the workgroup, then wave 0 alone over
//              the keys of T's bin once it is small (further workgroup rounds
//              otherwise); it writes the selection in ascending index order,
//              cutting the T-ties in list (= index) order.
// The result is exact whenever at least top_k keys reach tau, which select
// checks; otherwise (or when the candidates exceed its LDS list) select
// recomputes the row's scores into the workspace and runs the per-row radix
// selection on them.
#include "frag.h"

#include <algorithm>
#include <vector>
#include "topk_common.h"

namespace dsa {
namespace {

using namespace frag;
using namespace topk;

constexpr int TH_MAX_SAMPLES = 8192;
constexpr int SLOT = 256;          // keys per filter wave = one candidate list
constexpr int SEL_NT = 1024;         // select threads per row (1024 timed 12.8 us against 16.6 with 512)
constexpr int SEL_CAP = 12288;     // candidates select can hold in LDS
constexpr int SEL_MAX_SLOTS = 4096;
constexpr int SEL_GMAX = 1024;     // keys of a radix bin gathered for wave 0
struct Plan {
    int n, S, ns, m;
};

// Most samples any row of a problem with n_k keys can take: ns = ceil(n / S)
// with S >= max(1, top_k / 32) and S >= ceil(n / TH_MAX_SAMPLES). The sample
// keys of sequence b sit at a.samp[b * sample_cap(n_k, top_k) + i].
__host__ __device__ inline int sample_cap(int n_k, int top_k) {
    const long long smin = top_k / 32 > 1 ? top_k / 32 : 1;
    const long long c = ((long long)n_k + smin - 1) / smin;
    return (int)(c < TH_MAX_SAMPLES ? c : TH_MAX_SAMPLES);
}

__device__ __forceinline__ Plan plan_row(const DecodeArgs& a, int b) {
    Plan p;
    const long long pos = (long long)a.q_pos0 + a.q_row + (a.seq_pos ? a.seq_pos[b] : 0);
    p.n = (int)max(0LL, min((long long)a.n_k, pos + 1));
    // about 64 samples are expected above tau (sd ~ S sqrt(m)): the miss
    // margin (k of the expected 2k candidates) is sqrt(k / (2 S)) = 4 sd
    p.S = max(max(1, a.top_k / 32), (p.n + TH_MAX_SAMPLES - 1) / TH_MAX_SAMPLES);
    p.ns = (p.n + p.S - 1) / p.S;
    p.m = (2 * a.top_k + p.S - 1) / p.S;  // ceil(2 k / S)
    return p;
}

// Scores of keys t0 + 16*0.., as order keys, for the 16 keys of one tile whose
// row index is key(i) for tile row i; lanes with column 0 hold rows 4g..4g+3.
template <int DT, int D>
__device__ __forceinline__ f32x4 key_tile(const uint8_t* kpool, long long row, const Frag<DT, D>& fq,
                                          int g) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    Frag<DT, D> fk;
    fk.load(kpool + (size_t)row * RB, g);
    return tile_dot_k32<D>(fk, fq);
}

constexpr int TH_NT = 1024;   // threads of the threshold workgroup (one per row)
constexpr int RB12 = 4096;    // 12-bit digits of the select rounds

// Orders one wave's LDS accesses across its lanes.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bin of a 256-bin histogram holding the rem-th largest counted key, found
// by one whole wave: bin and the number of keys in higher bins, in every lane.
__device__ __forceinline__ void find_bin8_wave(const uint32_t* hist, uint32_t rem, uint32_t& bin,
                                               uint32_t& above_bin) {
    const int lane = threadIdx.x & 63;
    const int hi = 255 - 4 * lane;
    uint32_t c[4], loc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        c[q] = hist[hi - q];
        loc += c[q];
    }
    uint32_t above = wave_incl_scan(loc) - loc;
    int fb = -1;
    uint32_t fa = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (above < rem && above + c[q] >= rem) {
            fb = hi - q;
            fa = above;
        }
        above += c[q];
    }
    const unsigned long long mk = __ballot(fb >= 0);
    const int src = mk ? __ffsll((long long)mk) - 1 : 0;
    bin = mk ? (uint32_t)__builtin_amdgcn_readlane(fb, src) : 0u;
    above_bin = mk ? (uint32_t)__builtin_amdgcn_readlane((int)fa, src) : 0u;
}

// Sample rows are read with LPR consecutive lanes per row (GPL 16-byte
// granules per lane), so each load instruction covers whole contiguous rows:
// reads in the MFMA fragment layout, where consecutive lanes fall in
// different rows, cost the address unit about one cycle per lane.
template <int RB> struct SampleShape {
    static constexpr int NG = RB / 16;  // granules per row
    static constexpr int LPR = NG <= 2 ? 2 : NG <= 4 ? 4 : NG <= 8 ? 8 : 16;
    static constexpr int GPL = (NG + LPR - 1) / LPR;
    static constexpr int RPI = 64 / LPR;        // rows per load instruction
    static constexpr int NB = GPL == 1 ? 16 : 8;  // load instructions in flight
};

// The 16 fp8 e4m3fn (DT 0) or 8 bf16 (DT 1) values of a granule as float.
template <int DT>
__device__ __forceinline__ void granule_values(i32x4 w, float* v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if constexpr (DT == 0) {
            const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[c], 1.0f, false);
            const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[c], 1.0f, true);
            v[4 * c] = lo[0];
            v[4 * c + 1] = lo[1];
            v[4 * c + 2] = hi[0];
            v[4 * c + 3] = hi[1];
        } else {
            v[2 * c] = __uint_as_float((uint32_t)w[c] << 16);
            v[2 * c + 1] = __uint_as_float((uint32_t)w[c] & 0xffff0000u);
        }
    }
}

constexpr int SP_NT = 256;  // threads of a sampling workgroup
// Sample load instructions in flight per lane: 8, or 4 (twice the sampling
// workgroups) when 8 would leave fewer than 512 of them: 32 rows of 32K keys
// 24.8 -> 23.9 us for the threshold and select; 64 rows of 128K keys keep 8
// (512 workgroups), where 4 made the sampling kernel 0.4 us slower.
constexpr int SP_NB_MAX = 8;
constexpr int SP_MIN_WGS = 512;

// Samples scored by one sampling workgroup.
template <int RB, int NB>
constexpr int sample_chunk() { return (SP_NT / 64) * NB * SampleShape<RB>::RPI; }

// Sample scores of each row: sampling workgroup (b, part) scores samples
// [part C, part C + C) of row b (C = sample_chunk<RB, SP_NB>) and writes their order
// keys to a.samp[b][i]. tau only steers how many candidates the filter keeps;
// the selection is exact for any tau, so the sample scores are fp32 VALU dot
// products (summation order of their own) rather than the filter's MFMAs.
template <int DT, int D, int SP_NB>
__global__ __launch_bounds__(SP_NT) void decode_sample_kernel(DecodeArgs a, int per_row) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    constexpr int WAVES = SP_NT / 64;
    constexpr int EPG = DT == 0 ? 16 : 8;  // values per granule
    using SS = SampleShape<RB>;
    const int b = (int)(blockIdx.x / (unsigned)per_row);
    const int i_lo = (int)(blockIdx.x % (unsigned)per_row) * sample_chunk<RB, SP_NB>();
    const Plan p = plan_row(a, b);
    if (p.n <= a.top_k || p.ns <= p.m || i_lo >= p.ns) return;  // (the threshold kernel's cases)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pl = lane % SS::LPR, rl = lane / SS::LPR;
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.q_row) * RB;
    float qv[SS::GPL][EPG];
#pragma unroll
    for (int g = 0; g < SS::GPL; ++g) {
        const int gi = pl + SS::LPR * g;
        const i32x4 w = gi < SS::NG ? *reinterpret_cast<const i32x4*>(qrow + 16 * gi)
                                    : i32x4{0, 0, 0, 0};
        granule_values<DT>(w, qv[g]);
    }
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
    uint32_t* out = a.samp + (size_t)b * sample_cap(a.n_k, a.top_k);
    // Sample i_lo + (u WAVES + wave) RPI + rl: SP_NB instructions per lane in
    // flight, then their dot products.
    i32x4 w[SP_NB][SS::GPL];
#pragma unroll
    for (int u = 0; u < SP_NB; ++u) {
        const int i = min(i_lo + (u * WAVES + wave) * SS::RPI + rl, p.ns - 1);
        const uint8_t* row = kpool + (size_t)key_row(a.pages, b, a.n_k, i * p.S) * RB;
#pragma unroll
        for (int g = 0; g < SS::GPL; ++g) {
            const int gi = pl + SS::LPR * g;
            w[u][g] = gi < SS::NG ? *reinterpret_cast<const i32x4*>(row + 16 * gi)
                                  : i32x4{0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int u = 0; u < SP_NB; ++u) {
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < SS::GPL; ++g) {
            float kv[EPG];
            granule_values<DT>(w[u][g], kv);
#pragma unroll
            for (int e = 0; e < EPG; ++e) s = fmaf(kv[e], qv[g][e], s);
        }
#pragma unroll
        for (int off = SS::LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
        const int i = i_lo + (u * WAVES + wave) * SS::RPI + rl;
        if (pl == 0 && i < p.ns) out[i] = rank_key(relu_scaled(s, a.scale));
    }
}

// Sampled threshold of each row (one workgroup per sequence): the row's
// sample keys into LDS, then two 8-bit radix rounds over the keys relative to
// the smallest sample give the lower edge of the bin holding the m-th largest
// sample (at least m samples reach it). The histograms here, and those of
// the select kernel's one-wave rounds, take plain LDS atomics: aggregating
// the lanes of a wave that share a bin first (a vote, a first-lane pick and a
// read-lane per key) timed slower on these short latency-bound rounds. The
// select kernel's workgroup-wide 12-bit rounds keep the aggregated add: on
// ragged batches many candidates share a bin there, and plain atomics on them
// timed slower.
template <int DT, int D>
__global__ __launch_bounds__(TH_NT) void decode_threshold_kernel(DecodeArgs a) {
    constexpr int WAVES = TH_NT / 64;
    __shared__ uint32_t samp[TH_MAX_SAMPLES];
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t wlo[WAVES], whi[WAVES];
    __shared__ uint32_t res[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const Plan p = plan_row(a, b);
    if (p.n <= a.top_k || p.ns <= p.m) {
        if (tid == 0) a.tau[b] = 0u;  // every key is a candidate
        return;
    }
    const uint32_t* in = a.samp + (size_t)b * sample_cap(a.n_k, a.top_k);
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int i = tid; i < p.ns; i += TH_NT) {
        const uint32_t key = in[i];
        samp[i] = key;
        lo = min(lo, key);
        hi = max(hi, key);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
        wlo[wave] = lo;
        whi[wave] = hi;
    }
    if (tid < 512) (&hist[0][0])[tid] = 0u;
    __syncthreads();
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        kmin = min(kmin, wlo[w]);
        kmax = max(kmax, whi[w]);
    }
    // order keys of non-negative scores: the range is below 2^31
    const int bits = 32 - __clz((int)(kmax - kmin));
    if (bits == 0) {  // every sample has the same key
        if (tid == 0) a.tau[b] = kmin;
        return;
    }
    const int sh0 = bits > 8 ? bits - 8 : 0;
    for (int i0 = 0; i0 < p.ns; i0 += TH_NT) {
        const int i = i0 + tid;
        if (i < p.ns) atomicAdd(&hist[0][(samp[i] - kmin) >> sh0], 1u);
    }
    __syncthreads();
    if (wave == 0) {
        uint32_t bin, above;
        find_bin8_wave(hist[0], (uint32_t)p.m, bin, above);
        if (lane == 0) {
            res[0] = bin;
            res[1] = above;
        }
    }
    __syncthreads();
    const uint32_t b0 = res[0];
    const uint32_t rem = (uint32_t)p.m - res[1];
    if (sh0 == 0) {
        if (tid == 0) a.tau[b] = kmin + b0;
        return;
    }
    const int sh1 = sh0 > 8 ? sh0 - 8 : 0;
    const uint32_t dmask = (1u << (sh0 - sh1)) - 1u;
    for (int i0 = 0; i0 < p.ns; i0 += TH_NT) {
        const int i = i0 + tid;
        const uint32_t d = i < p.ns ? samp[i] - kmin : 0u;
        if (i < p.ns && (d >> sh0) == b0) atomicAdd(&hist[1][(d >> sh1) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
        uint32_t bin, above;
        find_bin8_wave(hist[1], rem, bin, above);
        if (lane == 0) a.tau[b] = kmin + ((((b0 << (sh0 - sh1)) | bin)) << sh1);
    }
}

// Bin of an RB12-bin histogram holding the rem-th largest counted key over
// an NT-thread workgroup: res[0] = bin, res[1] = keys in higher bins.
template <int NT>
__device__ __forceinline__ void find_bin12(const uint32_t* hist, uint32_t rem, uint32_t* wsum,
                                           uint32_t* res) {
    constexpr int PER = RB12 / NT;
    const int hi = RB12 - 1 - (int)threadIdx.x * PER;
    uint32_t c[PER], loc = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        c[q] = hist[hi - q];
        loc += c[q];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(loc, wsum, &tot);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (above < rem && above + c[q] >= rem) {
            res[0] = (uint32_t)(hi - q);
            res[1] = above;
        }
        above += c[q];
    }
    __syncthreads();
}

// The streaming indexer of one query row per sequence (see index_decode_kernel
// in indexer.hip for the tile layout), keeping only keys at or above tau.
// CONTIG: 256-key runs are contiguous (whole-run address arithmetic); else
// per-key pool rows.
template <int DT, int D, bool CONTIG>
__global__ __launch_bounds__(256) void decode_filter_kernel(DecodeArgs a) {
    constexpr int TILES = 8, STEPS = 2;
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    constexpr int KW = 16 * TILES * STEPS;  // = SLOT
    constexpr int KB = 4 * KW;
    static_assert(KW == SLOT, "one candidate list per wave");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_kb = (a.n_k + KB - 1) / KB;
    const int kb = blockIdx.x % n_kb, b = blockIdx.x / n_kb;
    const Plan p = plan_row(a, b);
    const int lim = p.n;
    const uint32_t tau = a.tau[b];
    const int slot = kb * 4 + wave;
    const int n_slots = (a.n_k + SLOT - 1) / SLOT;

    Frag<DT, D> fq;
    fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.q_row) * RB, g);
    // the wave's 256 keys (contiguous unless pages are smaller)
    const int kw0 = min(kb * KB + wave * KW, a.n_k - 1);
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
    constexpr bool contig = CONTIG;
    const uint8_t* __restrict__ kbase = kpool + (size_t)key_row(a.pages, b, a.n_k, kw0) * RB;
    RunRows rr;
    if constexpr (!contig) rr.load(a.pages, b, a.n_k, kw0);
    const int sel = n & (TILES - 1);
    const bool writer = n < TILES;
    uint32_t sk[STEPS][4];
    int key0s[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int k0 = kb * KB + wave * KW + st * 16 * TILES;
        key0s[st] = k0 + 16 * sel + 4 * g;
        if (k0 >= lim) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sk[st][r] = 0u;
            continue;
        }
        Frag<DT, D> fk[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t)
            fk[t].template load<true>(run_key(contig, kpool, kbase, rr, kw0,
                                              min(k0 + 16 * t + n, a.n_k - 1), 2 * st + t / 4,
                                              16 * (t % 4) + n, RB), g);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t) acc[t] = tile_dot_k32<D>(fk[t], fq);
        f32x4 v01 = (sel & 1) ? acc[1] : acc[0];
        f32x4 v23 = (sel & 1) ? acc[3] : acc[2];
        f32x4 v45 = (sel & 1) ? acc[5] : acc[4];
        f32x4 v67 = (sel & 1) ? acc[7] : acc[6];
        f32x4 v03 = (sel & 2) ? v23 : v01;
        f32x4 v47 = (sel & 2) ? v67 : v45;
        f32x4 v = (sel & 4) ? v47 : v03;
#pragma unroll
        for (int r = 0; r < 4; ++r) sk[st][r] = rank_key(relu_scaled(v[r], a.scale));
    }
    // Candidates of this wave into its list in ascending index order. In a
    // step, writer lane (sel, g) holds keys k0 + 16*sel + 4*g + r, so its place
    // in index order is p = 4*sel + g: counts are gathered into position order
    // (lane p takes lane 16*(p%4) + p/4), scanned, and scattered back.
    uint2* list = a.cand + ((size_t)b * n_slots + slot) * SLOT;
    uint32_t count = 0;
    const int src = 16 * (lane & 3) + ((lane >> 2) & 7);
    const int myp = 4 * sel + g;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        bool c[4];
        uint32_t cl = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = key0s[st] + r;
            c[r] = writer && j < lim && sk[st][r] >= tau;
            cl += c[r] ? 1u : 0u;
        }
        uint32_t cp = (uint32_t)__shfl((int)cl, src);
        if (lane >= 32) cp = 0u;
        const uint32_t incl = wave_incl_scan(cp);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 31);
        uint32_t o = count + (uint32_t)__shfl((int)(incl - cp), myp);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (c[r]) list[o++] = make_uint2(sk[st][r], (uint32_t)(key0s[st] + r));
        count += tot;
    }
    if (lane == 0 && slot < n_slots) a.cnt[(size_t)b * n_slots + slot] = count;
}

// Cache-policy operand of a global->LDS copy: nontemporal (keys are streamed
// once).
constexpr int kNontemporal = 2;

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// 128-byte key rows staged in LDS by contiguous 1 KB global->LDS copies.
// Granule j (16 bytes) of row r of a 64-row buffer sits at 16-byte slot
// 8 r + (j ^ f(r)), f(r) = (r mod 8) ^ ((r / 8) mod 2): each copy
// instruction still covers 8 whole rows of global memory, and the 16 rows a
// fragment read touches (fixed j) land in 16 distinct bank groups.
__device__ __forceinline__ int sw_slot(int r, int j) { return 8 * r + (j ^ ((r & 7) ^ ((r >> 3) & 1))); }

template <int DT, int D>
__device__ __forceinline__ void load_sw(Frag<DT, D>& f, const uint8_t* buf, int r, int g) {
    static_assert(D * (DT == 0 ? 1 : 2) == 128, "128-byte rows");
    const i32x4 lo = *reinterpret_cast<const i32x4*>(buf + 16 * sw_slot(r, g));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(buf + 16 * sw_slot(r, g + 4));
    if constexpr (DT == 0) {
        f.big[0] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
        f.v[0] = __builtin_bit_cast(bf16x8, lo);
        f.v[1] = __builtin_bit_cast(bf16x8, hi);
    }
}

// Key rows of at most LDS_RB_MAX bytes take the LDS-staged filter.
constexpr int LDS_RB_MAX = 160;

// The filter for key rows of up to LDS_RB_MAX bytes: each wave streams its
// 256 keys in four 64-key steps through a two-buffer LDS ring of contiguous
// 1 KB copies (128-byte rows: swizzled per row as sw_slot gives; other
// widths: the step's bytes in order), the same scores and candidate lists as
// decode_filter_kernel.
template <int DT, int D, bool CONTIG>
__global__ __launch_bounds__(256) void decode_filter_lds_kernel(DecodeArgs a) {
    constexpr int TILES = 4, STEPS = 4;
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    constexpr bool SW = RB == 128;
    constexpr int KW = 16 * TILES * STEPS;  // = SLOT
    constexpr int KB = 4 * KW;
    constexpr int STEP_BYTES = 16 * TILES * RB;  // RB / 16 copies of 1 KB
    constexpr int CPS = STEP_BYTES / 1024;       // copies per step
    static_assert(KW == SLOT && RB % 16 == 0 && RB <= LDS_RB_MAX, "one candidate list per wave");
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][2][STEP_BYTES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_kb = (a.n_k + KB - 1) / KB;
    const int kb = blockIdx.x % n_kb, b = blockIdx.x / n_kb;
    const Plan p = plan_row(a, b);
    const int lim = p.n;
    const int slot = kb * 4 + wave;
    const int n_slots = (a.n_k + SLOT - 1) / SLOT;
    const int kw0 = kb * KB + wave * KW;
    if (kw0 >= lim) {  // no key of this wave is in the row (wave-uniform)
        if (lane == 0 && slot < n_slots) a.cnt[(size_t)b * n_slots + slot] = 0u;
        return;
    }
    const uint32_t tau = a.tau[b];
    // the wave's 256 keys (contiguous unless pages are smaller)
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
    constexpr bool contig = CONTIG;
    const uint8_t* __restrict__ kbase = kpool + (size_t)key_row(a.pages, b, a.n_k, kw0) * RB;
    RunRows rr;
    if constexpr (!contig) rr.load(a.pages, b, a.n_k, kw0);
    // 128-byte rows: copy lane l of instruction i moves granule
    // ((l % 8) ^ f(r)) of row r = 8 i + l / 8 into slot 64 i + l. Other
    // widths: copy i moves bytes [1024 i, 1024 i + 1024) of the step (rows
    // past the sequence read its last 16 bytes; they are masked later).
    const size_t seq_bytes = (size_t)(a.n_k - kw0) * RB;  // from the wave's first key
    auto issue = [&](int st) {
        const int k0 = kw0 + st * 16 * TILES;
        uint8_t* dst = ring[wave][st & 1];
#pragma unroll
        for (int i = 0; i < CPS; ++i) {
            const uint8_t* src;
            if constexpr (SW) {
                const int r = 8 * i + (lane >> 3);
                const int j = (lane & 7) ^ ((r & 7) ^ ((r >> 3) & 1));
                src = run_key(contig, kpool, kbase, rr, kw0, min(k0 + r, a.n_k - 1), st, r, RB) +
                      16 * j;
            } else if constexpr (contig) {
                src = kbase + min((size_t)(k0 - kw0) * RB + 1024 * i + 16 * lane, seq_bytes - 16);
            } else {
                // byte o of the step: column o % RB of chunk key o / RB
                const int o = 1024 * i + 16 * lane, r = o / RB;
                src = kpool + (size_t)rr.row(st, r) * RB + (o - r * RB);
            }
            __builtin_amdgcn_global_load_lds(src, dst + 1024 * i, 16, 0, kNontemporal);
        }
    };
    Frag<DT, D> fq;
    fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.q_row) * RB, g);
    issue(0);
    issue(1);
    const int sel = n & (TILES - 1);
    const bool writer = n < TILES;
    uint32_t sk[STEPS][4];
    int key0s[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int k0 = kw0 + st * 16 * TILES;
        key0s[st] = k0 + 16 * sel + 4 * g;
        // step st has landed once only the copies issued after it remain
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < STEPS) wait_vmcnt<CPS>();
        else wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* buf = ring[wave][st & 1];
        Frag<DT, D> fk[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            if constexpr (SW) load_sw(fk[t], buf, 16 * t + n, g);
            else fk[t].load(buf + (16 * t + n) * RB, g);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the buffer may be refilled
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if (st + 2 < STEPS) issue(st + 2);
        f32x4 acc[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t) acc[t] = tile_dot_k32<D>(fk[t], fq);
        const f32x4 v01 = (sel & 1) ? acc[1] : acc[0];
        const f32x4 v23 = (sel & 1) ? acc[3] : acc[2];
        const f32x4 v = (sel & 2) ? v23 : v01;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sk[st][r] = k0 < lim ? rank_key(relu_scaled(v[r], a.scale)) : 0u;
    }
    // Candidates of this wave into its list in ascending index order. In a
    // step, writer lane (sel, g) holds keys k0 + 16*sel + 4*g + r, so its place
    // in index order is p = 4*sel + g: counts are gathered into position order
    // (lane p takes lane 16*(p%4) + p/4), scanned, and scattered back.
    uint2* list = a.cand + ((size_t)b * n_slots + slot) * SLOT;
    uint32_t count = 0;
    const int src = 16 * (lane & 3) + ((lane >> 2) & 3);
    const int myp = 4 * sel + g;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        bool c[4];
        uint32_t cl = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = key0s[st] + r;
            c[r] = writer && j < lim && sk[st][r] >= tau;
            cl += c[r] ? 1u : 0u;
        }
        uint32_t cp = (uint32_t)__shfl((int)cl, src);
        if (lane >= 16) cp = 0u;
        const uint32_t incl = wave_incl_scan(cp);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 15);
        uint32_t o = count + (uint32_t)__shfl((int)(incl - cp), myp);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (c[r]) list[o++] = make_uint2(sk[st][r], (uint32_t)(key0s[st] + r));
        count += tot;
    }
    if (lane == 0 && slot < n_slots) a.cnt[(size_t)b * n_slots + slot] = count;
}

// Every score of the row (order keys) into `row` (fallback path of select).
template <int DT, int D>
__device__ void row_scores(const DecodeArgs& a, int b, int nkeys, float* row) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    Frag<DT, D> fq;
    fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + a.q_row) * RB, g);
    const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
    for (int t0 = wave * 16; t0 < nkeys; t0 += (SEL_NT / 64) * 16) {
        const f32x4 acc =
            key_tile<DT, D>(kpool, key_row(a.pages, b, a.n_k, min(t0 + n, nkeys - 1)), fq, g);
        if (n == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (t0 + 4 * g + r < nkeys) row[t0 + 4 * g + r] = relu_scaled(acc[r], a.scale);
        }
    }
}

template <int DT, int D>
__global__ __launch_bounds__(SEL_NT) void decode_select_kernel(DecodeArgs a) {
    // LDS: keys | idx (candidates), hist, per-slot candidate offsets, scan
    // scratch.
    __shared__ uint32_t keys[SEL_CAP];
    __shared__ uint32_t jj[SEL_CAP];
    __shared__ uint32_t hist[RB12];
    __shared__ uint32_t soff[SEL_MAX_SLOTS + 1];
    __shared__ uint32_t wsum[SEL_NT / 64];
    __shared__ uint32_t res[4];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const Plan p = plan_row(a, b);
    const int k = a.top_k;
    int32_t* out = a.idx + ((size_t)b * a.idx_rows + a.idx_row0) * k;
    if (p.n <= k) {
        fill_prefix(out, p.n, k, tid, SEL_NT);
        return;
    }
    const int n_slots = (a.n_k + SLOT - 1) / SLOT;
    const int used = (p.n + SLOT - 1) / SLOT;  // slots holding keys < n
    // Candidate offsets per slot.
    constexpr int PER = SEL_MAX_SLOTS / SEL_NT;
    const uint32_t* gcnt = a.cnt + (size_t)b * n_slots;
    uint32_t cv[PER], loc = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int s = tid * PER + e;
        cv[e] = s < used ? gcnt[s] : 0u;
        loc += cv[e];
    }
    uint32_t total;
    uint32_t off = block_excl_scan<SEL_NT>(loc, wsum, &total);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int s = tid * PER + e;
        if (s <= SEL_MAX_SLOTS - 1) soff[s] = off;
        off += cv[e];
    }
    if (tid == 0) soff[SEL_MAX_SLOTS] = total;
    __syncthreads();
    if (total < (uint32_t)k || total > (uint32_t)SEL_CAP) {
        // tau kept fewer than k keys, or more than the LDS list holds:
        // recompute the whole row and select on it directly.
        float* row = a.fallback + (size_t)b * a.n_k;
        row_scores<DT, D>(a, b, p.n, row);
        __threadfence();
        __syncthreads();
        row_topk<SEL_NT, SEL_CAP, false>(row, p.n, k, out, hist, keys, wsum, res);
        return;
    }
    // Load every candidate (lists are in index order, slots in key order, so
    // the LDS list is sorted by index). Thread t copies a contiguous block,
    // eight loads in flight at a time.
    {
        const int E = ((int)total + SEL_NT - 1) / SEL_NT;
        const int c0 = tid * E, c1 = min((int)total, c0 + E);
        if (c0 < c1) {
            int s = 0, hi = used - 1;  // last slot with soff[s] <= c0
            while (s < hi) {
                const int mid = (s + hi + 1) >> 1;
                if (soff[mid] <= (uint32_t)c0) s = mid;
                else hi = mid - 1;
            }
            for (int c = c0; c < c1; c += 8) {
                uint2 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int cc = c + u;
                    if (cc < c1) {
                        while (soff[s + 1] <= (uint32_t)cc) ++s;
                        v[u] = a.cand[((size_t)b * n_slots + s) * SLOT + (cc - soff[s])];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (c + u < c1) {
                        keys[c + u] = v[u].x;
                        jj[c + u] = v[u].y;
                    }
            }
        }
    }
    __syncthreads();
    const int cnt = (int)total;
    // Exact k-th key T from the order keys relative to tau (every listed key
    // reached it): 12-bit radix rounds over the workgroup from the top bit of
    // the largest, until the bin holding the k-th key is small enough to be
    // gathered into LDS (soff is free by now); wave 0 alone then takes 8-bit
    // rounds over the gathered keys' remaining bits.
    const uint32_t kmin = a.tau[b];
    uint32_t hi = 0u;
    for (int i = tid; i < cnt; i += SEL_NT) hi = max(hi, keys[i]);
    hi = wave_max(hi);
    if ((tid & 63) == 0) wsum[tid >> 6] = hi;
    if (tid == 0) res[2] = 0u;
    __syncthreads();
    uint32_t kmax = 0u;
#pragma unroll
    for (int x = 0; x < SEL_NT / 64; ++x) kmax = max(kmax, wsum[x]);
    __syncthreads();  // wsum is rewritten by the scans below
    const uint32_t range = kmax - kmin;
    const int R = (32 - __clz((int)range) + 11) / 12;
    uint32_t rem = (uint32_t)k, prefix = 0;
    uint32_t* gk = soff;
    int cur_sh = 0;
    bool gathered = false;
    for (int r = 0; r < R && !gathered; ++r) {
        const int sh = 12 * (R - 1 - r);
        const int hsh = sh + 12;
        cur_sh = sh;
        for (int q = tid; q < RB12; q += SEL_NT) hist[q] = 0u;
        __syncthreads();
        for (int i0 = 0; i0 < cnt; i0 += SEL_NT) {
            const int i = i0 + tid;
            const uint32_t d = i < cnt ? keys[i] - kmin : 0u;
            hist_add(hist, (d >> sh) & (RB12 - 1), i < cnt && (r == 0 || (d >> hsh) == prefix));
        }
        __syncthreads();
        find_bin12<SEL_NT>(hist, rem, wsum, res);
        prefix = (prefix << 12) | res[0];
        rem -= res[1];
        if (sh > 0 && hist[res[0]] <= (uint32_t)SEL_GMAX) {
            const uint32_t low = (1u << sh) - 1u;
            for (int i0 = 0; i0 < cnt; i0 += SEL_NT) {
                const int i = i0 + tid;
                const uint32_t d = i < cnt ? keys[i] - kmin : 0u;
                const bool take = i < cnt && (d >> sh) == prefix;
                const uint32_t slot = wave_append(take, &res[2]);
                if (take) gk[slot] = d & low;
            }
            gathered = true;
        }
        __syncthreads();
    }
    if (gathered) {
        if (tid < 64) {
            const uint32_t G = res[2];
            uint32_t sp = 0, rm = rem;  // bits [s2, cur_sh) found so far
            int s2 = cur_sh;
            while (s2 > 0) {
                const int h2 = s2;
                s2 = s2 > 8 ? s2 - 8 : 0;
                const uint32_t mask = (1u << (h2 - s2)) - 1u;
#pragma unroll
                for (int q = 0; q < 4; ++q) hist[tid + 64 * q] = 0u;
                wave_lds_fence();
                for (uint32_t g0 = 0; g0 < G; g0 += 64) {
                    const uint32_t gi = g0 + tid;
                    const uint32_t v = gi < G ? gk[gi] : 0u;
                    if (gi < G && (v >> h2) == sp) atomicAdd(&hist[(v >> s2) & mask], 1u);
                }
                wave_lds_fence();
                uint32_t bin, above;
                find_bin8_wave(hist, rm, bin, above);
                sp = (sp << (h2 - s2)) | bin;
                rm -= above;
                wave_lds_fence();  // hist is cleared again by the next round
            }
            if (tid == 0) {
                res[0] = (prefix << cur_sh) | sp;
                res[1] = rm;
            }
        }
        __syncthreads();
        prefix = res[0];
        rem = res[1];
    }
    uint32_t T = kmin + prefix;  // keep every key above T and the first rem keys equal to T
    // Threshold mode: when the k-th key is not above the floor, the kept set
    // is every key above the floor (all candidates, since they outrank the
    // k-th key); otherwise the top-k set is already above it.
    const bool floored = a.floor.on && T <= a.floor.key;
    if (floored) {
        T = a.floor.key;
        rem = 0;
    }
    // Ordered compaction (the list is sorted by index): thread t takes a
    // contiguous block; the T-ties are cut in list order.
    const int E = (cnt + SEL_NT - 1) / SEL_NT;
    const int c0 = tid * E, c1 = min(cnt, c0 + E);
    uint32_t gtl = 0, eql = 0;
    for (int i = c0; i < c1; ++i) {
        gtl += keys[i] > T ? 1u : 0u;
        eql += keys[i] == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pk = block_excl_scan<SEL_NT>((gtl << 16) | eql, wsum, &tot);
    uint32_t gb = pk >> 16, eb = pk & 0xffffu;
    for (int i = c0; i < c1; ++i) {
        if (keys[i] > T) {
            out[gb + min(eb, rem)] = (int32_t)jj[i];
            ++gb;
        } else if (keys[i] == T) {
            if (eb < rem) out[gb + eb] = (int32_t)jj[i];
            ++eb;
        }
    }
    if (floored)
        for (int j = (int)(tot >> 16) + tid; j < k; j += SEL_NT) out[j] = -1;
    if (a.floor.on && tid == 0)
        a.floor.done[(size_t)b * a.n_q + a.q_row] = 1u;
}

template <int DT, int D>
hipError_t launch_d(const DecodeArgs& a, int part, hipStream_t s) {
    if (part == 0) {
        // sampling workgroups per row: enough for the most samples any row
        // of the problem can take
        constexpr int RB = D * (DT == 0 ? 1 : 2);
        const long long ns_max = sample_cap(a.n_k, a.top_k);
        constexpr int CH8 = sample_chunk<RB, SP_NB_MAX>(), CH4 = sample_chunk<RB, SP_NB_MAX / 2>();
        const long long nb8 = (long long)a.B * ((ns_max + CH8 - 1) / CH8);
        const bool half = nb8 < SP_MIN_WGS;
        const int CH = half ? CH4 : CH8;
        const int per_row = (int)((ns_max + CH - 1) / CH);
        const long long nb = (long long)a.B * per_row;
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        if (nb > 0 && half)
            hipLaunchKernelGGL((decode_sample_kernel<DT, D, SP_NB_MAX / 2>), dim3((unsigned)nb),
                               dim3(SP_NT), 0, s, a, per_row);
        else if (nb > 0)
            hipLaunchKernelGGL((decode_sample_kernel<DT, D, SP_NB_MAX>), dim3((unsigned)nb),
                               dim3(SP_NT), 0, s, a, per_row);
        hipLaunchKernelGGL((decode_threshold_kernel<DT, D>), dim3(a.B), dim3(TH_NT), 0, s, a);
    } else if (part == 1) {
        const int KB = 4 * SLOT;
        const long long nb = (long long)a.B * ((a.n_k + KB - 1) / KB);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const bool contig = run_contiguous(a.pages);
        if constexpr (D * (DT == 0 ? 1 : 2) <= LDS_RB_MAX) {
            if (contig)
                hipLaunchKernelGGL((decode_filter_lds_kernel<DT, D, true>), dim3((unsigned)nb),
                                   dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((decode_filter_lds_kernel<DT, D, false>), dim3((unsigned)nb),
                                   dim3(256), 0, s, a);
        } else {
            if (contig)
                hipLaunchKernelGGL((decode_filter_kernel<DT, D, true>), dim3((unsigned)nb),
                                   dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((decode_filter_kernel<DT, D, false>), dim3((unsigned)nb),
                                   dim3(256), 0, s, a);
        }
    } else {
        hipLaunchKernelGGL((decode_select_kernel<DT, D>), dim3(a.B), dim3(SEL_NT), 0, s, a);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const DecodeArgs& a, int part, hipStream_t s) {
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

bool decode_select_applies(int rows, int n_k, int top_k) {
    return rows == 1 && n_k >= 8192 && (long long)n_k <= (long long)SEL_MAX_SLOTS * SLOT &&
           top_k <= SEL_CAP;
}

size_t decode_select_ws_bytes(int B, int n_k, int top_k) {
    const size_t n_slots = (n_k + SLOT - 1) / SLOT;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    return al((size_t)B * 4) + al((size_t)B * n_slots * 4) + al((size_t)B * n_slots * SLOT * 8) +
           al((size_t)B * sample_cap(n_k, top_k) * 4);
}

hipError_t decode_stats(int B, int n_k, long long q_pos, const int32_t* seq_pos_host, int top_k,
                        const void* ws, long long out[4]) {
    const size_t n_slots = (n_k + SLOT - 1) / SLOT;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    std::vector<uint32_t> cnt((size_t)B * n_slots);
    hipError_t e = hipMemcpy(cnt.data(), static_cast<const char*>(ws) + al((size_t)B * 4),
                             cnt.size() * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    long long rows = 0, cand = 0, fb = 0, over = 0;
    for (int b = 0; b < B; ++b) {
        const long long pos = seq_pos_host ? (long long)seq_pos_host[b] + q_pos : q_pos;
        const long long n = pos + 1 < n_k ? pos + 1 : n_k;
        if (n <= top_k) continue;
        const size_t used = (size_t)((n + SLOT - 1) / SLOT);
        long long tot = 0;
        for (size_t x = 0; x < used; ++x) tot += cnt[(size_t)b * n_slots + x];
        ++rows;
        cand += tot;
        fb += tot < top_k || tot > SEL_CAP;
        over += tot > SEL_CAP;
    }
    out[0] = rows;
    out[1] = cand;
    out[2] = fb;
    out[3] = over;
    return hipSuccess;
}

hipError_t launch_decode_select(DecodeArgs a, void* ws, int part, hipStream_t s) {
    const size_t n_slots = (a.n_k + SLOT - 1) / SLOT;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    char* p = static_cast<char*>(ws);
    a.tau = reinterpret_cast<uint32_t*>(p);
    p += al((size_t)a.B * 4);
    a.cnt = reinterpret_cast<uint32_t*>(p);
    p += al((size_t)a.B * n_slots * 4);
    a.cand = reinterpret_cast<uint2*>(p);
    p += al((size_t)a.B * n_slots * SLOT * 8);
    a.samp = reinterpret_cast<uint32_t*>(p);
    return a.dtype == 0 ? launch_dt<0>(a, part, s) : launch_dt<1>(a, part, s);
}

}  // namespace dsa
