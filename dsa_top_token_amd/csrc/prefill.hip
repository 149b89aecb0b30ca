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
//              sample (m S ~ 2 top_k); tau becomes the smallest fp32
//              accumulator whose scaled score reaches it. A row whose sample
//              threshold is not positive keeps every non-negative
//              accumulator instead ("zero mode").
//   filter     per 64-row block (4 waves x 16 rows): sweeps the block's
//              causal keys in 64-key chunks staged in LDS. Keys are the MFMA
//              row operand, so each lane holds 16 consecutive keys of one
//              query; a subtract and a funnel shift per score build the
//              lane's accept mask, and the accepted (accumulator, index)
//              pairs go to the row's list in ascending index order.
//   select     one wave per row over its list: three radix rounds give the
//              exact k-th key T, the T-ties are cut in list (= index) order.
//              A zero-mode row with fewer than top_k positive scores takes
//              its positives plus the lowest-index zero scores. A row whose
//              threshold kept fewer than top_k keys, or more than its list
//              holds, is queued.
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
constexpr int TH_TARGET = 64;     // samples expected above tau
constexpr int FL_CHUNK = 64;      // keys per staged chunk of the filter
constexpr int FL_ROWS = 64;       // rows per filter workgroup (16 per wave)
constexpr int FB_WGS = 256;       // fallback workgroups

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

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

__device__ __forceinline__ unsigned long long lanes_below() {
    return (1ull << (threadIdx.x & 63)) - 1ull;
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
                            tacc = 0.0f;  // zero mode
                        } else {
                            const uint32_t tkey = (digit1[row] << 22) | (bin << 12);
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

template <int DT, int D>
__global__ __launch_bounds__(256) void prefill_filter_kernel(PrefillArgs a) {
    constexpr int RB = D * (DT == 0 ? 1 : 2);
    constexpr int PITCH = RB + 16;
    constexpr int CHUNK_BYTES = FL_CHUNK * RB;
    constexpr int LD_PER_THREAD = (CHUNK_BYTES + 256 * 16 - 1) / (256 * 16);
    __shared__ __attribute__((aligned(16))) uint8_t kt[2][FL_CHUNK * PITCH];
    // per-wave copy of each lane's 16 accumulators: [wave][u][lane] x 4
    __shared__ f32x4 stage[4][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int n_blk = (a.rows + FL_ROWS - 1) / FL_ROWS;
    // largest blocks (latest rows) first
    const int blk = n_blk - 1 - (int)(blockIdx.x / (unsigned)a.B);
    const int b = blockIdx.x % a.B;
    const int i0 = blk * FL_ROWS;
    const int wi0 = i0 + wave * 16;
    const int kend = row_len(a, min(i0 + FL_ROWS, a.rows) - 1);
    const int n_chunks = (kend + FL_CHUNK - 1) / FL_CHUNK;
    const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (size_t)b * a.n_k * RB;

    // This lane's query (column n of the B operand) and its row state.
    const int my_i = min(wi0 + n, a.rows - 1);
    const bool live = wi0 + n < a.rows;
    const int my_len = live ? row_len(a, my_i) : 0;
    const float tau = live ? a.tau_acc[(size_t)b * a.rows + my_i] : __builtin_inff();
    const bool wave_live = wi0 < a.rows;
    const int w_kend = wave_live ? row_len(a, min(wi0 + 15, a.rows - 1)) : 0;
    const int w_kmin = wave_live ? row_len(a, wi0) : 0;
    Frag<DT, D> fq;
    fq.load(static_cast<const uint8_t*>(a.q) + ((size_t)b * a.n_q + qrow(a, my_i)) * RB, g);
    uint2* list = a.cand + ((size_t)b * a.rows + my_i) * a.cap;
    const uint32_t cap = (uint32_t)a.cap;
    uint32_t cnt = 0;  // the row's list length (same in the row's 4 lanes)

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

    // A operand row n of key tile u is key 16 (n / 4) + 4 u + n % 4 of the
    // chunk, so output row 4 g + r of tile u is key 16 g + 4 u + r: lane
    // (n, g) holds keys [16 g, 16 g + 16) of the chunk for query n.
    const int krow = 16 * (n >> 2) + (n & 3);

    i32x4 stg[LD_PER_THREAD];
    if (n_chunks > 0) {
        load_chunk(0, stg);
        store_chunk(0, stg);
    }
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < n_chunks) load_chunk(c + 1, stg);
        const int k0 = c * FL_CHUNK;
        if (k0 < w_kend) {
            f32x4 acc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                Frag<DT, D> fk;
                fk.load(&kt[buf][(krow + 4 * u) * PITCH], g);
                acc[u] = tile_dot<D>(fk, fq);
            }
            if constexpr (DT == 0) {
                if constexpr (Frag<0, D>::NB > 0) mfma_drain();
            }
            // bit i of rej: sign of (accumulator of key 16 g + i) - tau
            uint32_t rej = 0;
#pragma unroll
            for (int i = 15; i >= 0; --i)
                rej = __builtin_amdgcn_alignbit(rej, __float_as_uint(acc[i >> 2][i & 3] - tau), 31);
            uint32_t bits = ~rej & 0xffffu;
            if (k0 + FL_CHUNK > w_kmin) {
                const int v = my_len - (k0 + 16 * g);
                bits &= v >= 16 ? 0xffffu : (v <= 0 ? 0u : (1u << v) - 1u);
            }
            // The row's lanes g = 0..3 hold consecutive key ranges: exclusive
            // prefix of their counts.
            const uint32_t lc = (uint32_t)__popc(bits);
            const uint32_t x1 = (uint32_t)__shfl_xor((int)lc, 16);
            const uint32_t s01 = lc + x1;
            const uint32_t x2 = (uint32_t)__shfl_xor((int)s01, 32);
            const uint32_t tot = s01 + x2;
            uint32_t o = cnt + ((g & 1) ? x1 : 0u) + ((g & 2) ? x2 : 0u);
            if (cnt + tot > cap) bits = 0u;  // overflowing row: its list is abandoned
            cnt += tot;
            if (__ballot(bits != 0u) != 0ull) {
#pragma unroll
                for (int u = 0; u < 4; ++u) stage[wave][u][lane] = acc[u];
                const uint32_t kb = (uint32_t)(k0 + 16 * g);
                while (bits != 0u) {
                    const int i = __builtin_ctz(bits);
                    bits &= bits - 1u;
                    const float v = reinterpret_cast<const float*>(&stage[wave][i >> 2][lane])[i & 3];
                    list[o] = make_uint2(__float_as_uint(v), kb + (uint32_t)i);
                    ++o;
                }
            }
        }
        if (c + 1 < n_chunks) store_chunk(buf ^ 1, stg);
        __syncthreads();
    }
    if (g == 0 && live) a.cnt[(size_t)b * a.rows + my_i] = cnt;
}

// ------------------------------------------------------------------- select

__device__ __forceinline__ uint32_t cand_key(uint32_t acc_bits, float scale) {
    return rank_key(relu_scaled(__uint_as_float(acc_bits), scale));
}

// One 64-thread workgroup (one wave) per row; the list is read from global
// memory on every pass.
__global__ __launch_bounds__(64) void prefill_select_kernel(PrefillArgs a) {
    __shared__ uint32_t hist[BINS];
    const int lane = threadIdx.x;
    const long long task = blockIdx.x;
    const int b = (int)(task / a.rows), i = (int)(task % a.rows);
    const int n = row_len(a, i);
    const int k = a.top_k;
    int32_t* out = a.idx + ((size_t)b * a.n_q + qrow(a, i)) * k;
    if (n <= k) {
        fill_prefix(out, n, k, lane, 64);
        return;
    }
    const uint32_t cnt = a.cnt[task];
    const bool zero_mode = __float_as_uint(a.tau_acc[task]) == 0u;
    if (cnt > (uint32_t)a.cap || (!zero_mode && cnt < (uint32_t)k)) {
        if (lane == 0) a.fb_list[atomicAdd(a.fb_count, 1u)] = (uint32_t)task;
        return;
    }
    const uint2* cl = a.cand + (size_t)task * a.cap;
    const int cn = (int)cnt;
    const float scale = a.scale;
    constexpr uint32_t ZERO_KEY = 0x80000000u;  // order key of a zero score

    if (zero_mode) {
        // The list holds every key with a positive score (plus some zeros);
        // every key off the list scores zero.
        uint32_t np = 0;
        for (int c = lane; c < cn; c += 64) np += cand_key(cl[c].x, scale) > ZERO_KEY ? 1u : 0u;
        np = wave_sum(np);
        if (np < (uint32_t)k) {
            // Positives plus the lowest-index zeros. With P the positives in
            // index order, P[r] - r zeros precede P[r]; the first cs
            // positives (P[r] - r < Z) come before the Z-th zero.
            const uint32_t Z = (uint32_t)k - np;
            uint32_t run = 0, cs = 0;
            for (int c0 = 0; c0 < cn; c0 += 64) {
                const int c = c0 + lane;
                bool pos = false;
                uint32_t j = 0;
                if (c < cn) {
                    const uint2 e = cl[c];
                    pos = cand_key(e.x, scale) > ZERO_KEY;
                    j = e.y;
                }
                const unsigned long long pm = __ballot(pos);
                const uint32_t r = run + (uint32_t)__popcll(pm & lanes_below());
                cs += (uint32_t)__popcll(__ballot(pos && j - r < Z));
                run += (uint32_t)__popcll(pm);
            }
            const uint32_t head = Z + cs;  // out[0, head) = 0 .. head - 1
            for (uint32_t o = lane; o < head; o += 64) out[o] = (int32_t)o;
            run = 0;
            for (int c0 = 0; c0 < cn; c0 += 64) {
                const int c = c0 + lane;
                bool pos = false;
                uint32_t j = 0;
                if (c < cn) {
                    const uint2 e = cl[c];
                    pos = cand_key(e.x, scale) > ZERO_KEY;
                    j = e.y;
                }
                const unsigned long long pm = __ballot(pos);
                const uint32_t r = run + (uint32_t)__popcll(pm & lanes_below());
                if (pos && r >= cs) out[Z + r] = (int32_t)j;
                run += (uint32_t)__popcll(pm);
            }
            return;
        }
    }

    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    // Exact k-th key: digits 31..21, 20..10, 9..0.
    uint32_t rem = (uint32_t)k, prefix = 0;
#pragma unroll 1
    for (int round = 0; round < 3; ++round) {
        const int sh = round == 0 ? 21 : (round == 1 ? 10 : 0);
        const int psh = round == 1 ? 21 : 10;  // prefix bits of the earlier rounds
        const uint32_t msk = round == 2 ? 1023u : 2047u;
        for (int t = lane; t < BINS; t += 64) hist[t] = 0u;
        wave_sync();
        for (int c0 = 0; c0 < cn; c0 += 256) {
            uint32_t key[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + 64 * u + lane;
                ok[u] = c < cn;
                key[u] = ok[u] ? cand_key(cl[c].x, scale) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool in = ok[u] && (round == 0 || (key[u] >> psh) == prefix);
                hist_add(hist, (key[u] >> sh) & msk, in);
            }
        }
        wave_sync();
        uint32_t above;
        const uint32_t bin = wave_find_bin<BINS>(hist, rem, &above);
        prefix = round == 0 ? bin : ((prefix << (round == 1 ? 11 : 10)) | bin);
        rem -= above;
        wave_sync();
    }
    const uint32_t T = prefix;  // keep every key above T and the first rem keys equal to T
    // Ordered compaction over the index-ordered list.
    uint32_t base = 0, eq_run = 0;
    for (int c0 = 0; c0 < cn && base < (uint32_t)k; c0 += 64) {
        const int c = c0 + lane;
        uint32_t key = 0, j = 0;
        if (c < cn) {
            const uint2 e = cl[c];
            key = cand_key(e.x, scale);
            j = e.y;
        }
        const bool gt = c < cn && key > T;
        const bool eq = c < cn && key == T;
        const unsigned long long me = __ballot(eq);
        const bool keep = gt || (eq && eq_run + (uint32_t)__popcll(me & lanes_below()) < rem);
        const unsigned long long mk = __ballot(keep);
        if (keep) out[base + (uint32_t)__popcll(mk & lanes_below())] = (int32_t)j;
        base += (uint32_t)__popcll(mk);
        eq_run += (uint32_t)__popcll(me);
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
        const long long nb = (long long)a.B * ((a.rows + FL_ROWS - 1) / FL_ROWS);
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((prefill_filter_kernel<DT, D>), dim3((unsigned)nb), dim3(256), 0, s, a);
    } else if (part == 2) {
        if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(prefill_select_kernel, dim3((unsigned)rows), dim3(64), 0, s, a);
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
