// Sparse MQA attention over the selected keys on gfx950.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693): section 3.3 runs ordinary
// softmax attention over each query's selected keys only; section 4.2 has all
// query heads share one K/V set (MQA), so one gathered K/V row serves every
// head; section 4.1 runs this stage in BF16.
//
// One wave owns one (query, split) or (query, key range) task: up to 16
// heads against the task's selected keys, 32 keys per step.
//   S^T (keys x heads) = K_sel (keys x 128) . Q^T    4+4 bf16 16x16x32 MFMAs
//   online softmax per head (log2 domain, fp32)
//   O^T (dims x heads) += V_sel^T . P^T              8 bf16 16x16x32 MFMAs
// With S^T as the MFMA output, lane (head h = lane%16, group g = lane/16)
// holds scores of keys 4g..4g+3 and 16+4g..16+4g+3, which is exactly the
// 8-key slice of P^T the PV product wants from that lane (the contraction
// order over keys is free). Selected K and V rows are gathered with 16 lanes
// per row, written to the wave's LDS slice and read back as fragments (K) and
// with transposed reads (V^T).
// Partials of split or key-range tasks are merged by log-sum-exp rescaling.
#include "dsa_internal.h"
#include "lanes.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int HD = 128;          // head dim
constexpr int PART = HD + 4;     // floats per (task, head) partial: O[128], m, l, pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float wave_xor_max(float v) { return lanes4_max(v); }

__device__ __forceinline__ float wave_xor_sum(float v) { return lanes4_sum(v); }

// One wave's pass over selected-key slots e = e_first, e_first + e_step, ...
// (32 slots each, all below e_end) of query row qrow: online softmax state
// (running max in the log2 domain, this lane's partial sum) and the
// unnormalised O^T tiles: lane (head m, group g) holds dims 16d + 4g + r.
struct WaveState {
    f32x4 o[8];
    float mrun, lpart;
};

// The K and V rows of a step are gathered into registers with loads in which
// every 16 consecutive lanes read one row's 256 contiguous bytes (one cache
// line pair per 16 lanes; a lane-per-row layout costs the address unit four
// times as many cycles), then written to the wave's LDS slice, from which the
// MFMA fragments are read. Slice: 32 K rows then 32 V rows of 256 bytes, then
// the 16 Q rows. Granule (16 bytes) q of row rho sits at granule slot
// q ^ (rho % 16) of that row, so fragment reads and transposed reads meet
// every bank once per 16 lanes.
constexpr int ROWB = HD * 2;             // bytes of one K, V or Q row
constexpr int KVB = 32 * ROWB;           // the K (or V) rows of one step: 8 KB
// 16 KB per wave (the prologue stages Q through the K rows' space): eight
// waves per CU fit in 128 KB of LDS.
constexpr int WAVE_LDS = 2 * KVB;

typedef short i16x4 __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format

// idx entry of slot e + lane % 32, clamped into the row so every load is in
// bounds (slots at or past e_end are masked out by slot_mask).
__device__ __forceinline__ int load_slot(const int32_t* sel, int e, int e_end, int lane) {
    return sel[min(e + (lane & 31), e_end - 1)];
}

// Bit s: slot e + s exists and holds a key inside [0, n_k).
__device__ __forceinline__ uint32_t slot_mask(int j, int e, int e_end, int n_k, int lane) {
    const bool ok = e + (lane & 31) < e_end && j >= 0 && j < n_k;
    return (uint32_t)__ballot(ok);  // lanes 32..63 repeat lanes 0..31
}

// One step's rows in registers: lane l holds granule l % 16 of the K and V
// rows of slots 8(l / 16) + c, c = 0..7.
struct StepRows {
    u16x8 k[8], v[8];
};

// Buffer loads through descriptors that cover the sequence's n_k rows: an
// entry outside [0, n_k) (the -1 padding, for one) lands past the end and
// reads zeros, and slot_mask keeps it out of the softmax.
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int j, int lane, StepRows& R) {
    const int q = lane >> 4, p = lane & 15;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t off = ((uint32_t)__shfl(j, 8 * q + c) << 8) + 16 * p;
        R.k[c] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
        R.v[c] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
}

__device__ __forceinline__ void store_rows(uint8_t* buf, const StepRows& R, int lane) {
    const int q = lane >> 4, p = lane & 15;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int rho = 8 * q + c;
        uint8_t* d = buf + rho * ROWB + 16 * (p ^ (rho & 15));
        *reinterpret_cast<u16x8*>(d) = R.k[c];
        *reinterpret_cast<u16x8*>(d + KVB) = R.v[c];
    }
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight transposed V reads (ds_read_b64_tr_b16) for four dim blocks, rows
// 16 + ... being 4096 bytes further, waited for inside the block (results of
// loads written in inline asm are taken as available at once).
__device__ __forceinline__ void tr_reads4(const uint32_t ad[4], i16x4 lo[4], i16x4 hi[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:4096\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:4096\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:4096\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
}

// Scores, online softmax update and PV product of one staged step; vm marks
// its valid slots.
__device__ __forceinline__ void attend_step(const uint8_t* buf, uint32_t vm, const bf16x8 qf[4],
                                            int m, int g, WaveState& ws) {
    const float ninf = -__builtin_inff();
    const float sl2 = 0.08838834764831845f * kLog2e;  // 128^-0.5 * log2(e)
    // K fragment (t, s): lane (m, g) takes dims 32s + 8g .. +8 (granule 4s + g)
    // of row 16t + m, matching the Q fragment.
    u16x8 kf[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            kf[t][s] = *reinterpret_cast<const u16x8*>(buf + (16 * t + m) * ROWB +
                                                       16 * ((4 * s + g) ^ m));
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[t][s]), qf[s], st[t],
                                                            0, 0, 0);
    }
    // This lane holds the scores of slots 16t + 4g + r.
    float z[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            z[4 * t + r] = ((vm >> (16 * t + 4 * g + r)) & 1u) ? st[t][r] * sl2 : ninf;
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = wave_xor_max(mx);
    // The reference maximum moves only when a head's maximum exceeds it by
    // more than 8 (so p <= 2^8 in between); O and l are rescaled only then.
    const bool grow = mx > ws.mrun + 8.f;
    if (__ballot(grow) != 0ull) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(ws.mrun - mx) : 1.f;
        ws.lpart *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) ws.o[d] *= alpha;
        ws.mrun = grow ? mx : ws.mrun;
    }
    const float base = ws.mrun == ninf ? 0.f : ws.mrun;  // every z is -inf while mrun is
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(z[i] - base);
        psum += p[i];
    }
    ws.lpart += psum;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (__bf16)p[i];
    // V^T fragment d by transposed LDS reads: in each 16-lane group, output
    // lane i element q comes from source lane 4q + i/4, element i % 4. Source
    // lane (m, g) points at dims 16d + 4(m % 4) .. +4 of V row 16t + 4g + m/4,
    // so lane (m, g) receives V[16t + 4g + q][16d + m] - keys 4g..4g+3 (t = 0)
    // and 16+4g..16+4g+3 (t = 1), the same slots as pb.
    const uint32_t vb = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)(buf + KVB);
    const int row = 4 * g + (m >> 2);  // t = 0; t = 1 is 16 rows further
#pragma unroll
    for (int d0 = 0; d0 < 8; d0 += 4) {
        uint32_t ad[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            ad[d] = vb + row * ROWB + 16 * ((2 * (d0 + d) + ((m & 3) >> 1)) ^ row) + 8 * (m & 1);
        i16x4 lo[4], hi[4];
        tr_reads4(ad, lo, hi);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u16x8 va = __builtin_bit_cast(
                u16x8, (short __attribute__((ext_vector_type(8)))){lo[d][0], lo[d][1], lo[d][2],
                                                                   lo[d][3], hi[d][0], hi[d][1],
                                                                   hi[d][2], hi[d][3]});
            ws.o[d0 + d] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, ws.o[d0 + d], 0, 0, 0);
        }
    }
}

// Software pipeline over the steps: while step i computes from LDS, the rows
// of step i + 1 are in flight to registers and the idx entries of step i + 2
// have been loaded. Unrolled by two so that the idx registers alternate
// instead of being copied while their loads are outstanding.
__device__ __forceinline__ void wave_attend(const AttnArgs& a, long long qrow, int e_first,
                                            int e_end, int e_step, uint8_t* lds,
                                            WaveState& ws) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int b = (int)(qrow / a.n_q);
    const int32_t* sel = a.idx + qrow * (long long)a.k;
    const int n_k = a.kv_rows;
    const int nrec = (int)((uint32_t)n_k * (uint32_t)ROWB);  // < 2^32 bytes (checked by the host)
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.K + (size_t)b * a.kv_bstride * HD), (short)0, nrec, kBufWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.V + (size_t)b * a.kv_bstride * HD), (short)0, nrec, kBufWord3);
#pragma unroll
    for (int d = 0; d < 8; ++d) ws.o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws.mrun = -__builtin_inff();
    ws.lpart = 0.f;
    if (e_first >= e_end) return;

    int jA = load_slot(sel, e_first, e_end, lane);
    int jB = load_slot(sel, e_first + e_step, e_end, lane);
    // Q rows: lane l holds granule l % 16 of head rows 4c + l / 16 (heads
    // past H repeat head H - 1; their fragments are zeroed below).
    u16x8 qv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int h = min(4 * c + (lane >> 4), a.H - 1);
        qv[c] = *reinterpret_cast<const u16x8*>(a.Q + (qrow * a.H + h) * HD + 8 * (lane & 15));
    }
    StepRows R;
    uint32_t vc = slot_mask(jA, e_first, e_end, n_k, lane);
    load_rows(rk, rv, jA, lane, R);
    // Q goes through the K rows' space first (its fragments are read back
    // before the first step's rows are stored there).
    uint8_t* qs = lds;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int rho = 4 * c + (lane >> 4);
        *reinterpret_cast<u16x8*>(qs + rho * ROWB + 16 * ((lane & 15) ^ rho)) = qv[c];
    }
    wave_lds_fence();
    // Q^T fragment: lane (head m, group g) holds Q[m][32s + 8g .. +8] for s = 0..3.
    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const u16x8 v = *reinterpret_cast<const u16x8*>(qs + m * ROWB + 16 * ((4 * s + g) ^ m));
        qf[s] = as_bf16x8(m < a.H ? v : u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }
    wave_lds_fence();
    store_rows(lds, R, lane);
    uint32_t vn = slot_mask(jB, e_first + e_step, e_end, n_k, lane);
    if (e_first + e_step < e_end) load_rows(rk, rv, jB, lane, R);
    jA = load_slot(sel, e_first + 2 * e_step, e_end, lane);
    wave_lds_fence();
    int e = e_first;
    for (;;) {
        // LDS: step e; R: step e + 1 (in flight); jA: idx of step e + 2.
        attend_step(lds, vc, qf, m, g, ws);
        if (e + e_step >= e_end) break;
        wave_lds_fence();
        store_rows(lds, R, lane);
        vc = vn;
        vn = slot_mask(jA, e + 2 * e_step, e_end, n_k, lane);
        if (e + 2 * e_step < e_end) load_rows(rk, rv, jA, lane, R);
        jB = load_slot(sel, e + 3 * e_step, e_end, lane);
        e += e_step;
        wave_lds_fence();
        // LDS: step e; R: step e + 1; jB: idx of step e + 2.
        attend_step(lds, vc, qf, m, g, ws);
        if (e + e_step >= e_end) break;
        wave_lds_fence();
        store_rows(lds, R, lane);
        vc = vn;
        vn = slot_mask(jB, e + 2 * e_step, e_end, n_k, lane);
        if (e + 2 * e_step < e_end) load_rows(rk, rv, jB, lane, R);
        jA = load_slot(sel, e + 3 * e_step, e_end, lane);
        e += e_step;
        wave_lds_fence();
    }
}

// One wave per query row (many queries): normalised O and lse directly.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[WAVE_LDS];
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const long long qrow = blockIdx.x;
    WaveState ws;
    wave_attend(a, qrow, 0, a.k, 32, lds, ws);
    const float l = wave_xor_sum(ws.lpart);
    if (m >= a.H) return;
    const float ninf = -__builtin_inff();
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = a.O + (qrow * a.H + m) * HD;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        bf16x4 h4;
#pragma unroll
        for (int r = 0; r < 4; ++r) h4[r] = (__bf16)(ws.o[d][r] * inv);
        *reinterpret_cast<uint2*>(op + 16 * d + 4 * g) = __builtin_bit_cast(uint2, h4);
    }
    if (a.lse && g == 0) a.lse[qrow * a.H + m] = l > 0.f ? (ws.mrun + log2f(l)) * kLn2 : ninf;
}

// Few query rows: a 4-wave workgroup per (query, split). Waves take every
// fourth 32-slot step of the split and merge in LDS; each workgroup writes its
// split's partial (max, sum, unnormalised O per head) for the combine kernel.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_split_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * WAVE_LDS];  // rows, then merge
    static_assert(4 * 16 * PART * sizeof(float) <= 4 * WAVE_LDS, "merge buffer fits");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int split = (int)(blockIdx.x % (unsigned)a.n_split);
    const long long qrow = blockIdx.x / (unsigned)a.n_split;
    const int e0 = split * a.split_len;
    const int e1 = min(a.k, e0 + a.split_len);
    const float ninf = -__builtin_inff();
    WaveState ws;
    wave_attend(a, qrow, e0 + 32 * wave, e1, 128, lds + wave * WAVE_LDS, ws);
    const float lw = wave_xor_sum(ws.lpart);
    __syncthreads();  // staged rows no longer needed
    // merge buffer: [wave][head][PART] with O[128], max, sum
    float* mb = reinterpret_cast<float*>(lds);
    float* mine = mb + ((size_t)wave * 16 + m) * PART;
#pragma unroll
    for (int d = 0; d < 8; ++d)
        *reinterpret_cast<float4*>(mine + 16 * d + 4 * g) =
            make_float4(ws.o[d][0], ws.o[d][1], ws.o[d][2], ws.o[d][3]);
    if (g == 0) {
        mine[HD] = ws.mrun;
        mine[HD + 1] = lw;
    }
    __syncthreads();
    // thread t: head h = t / 16, dims 8c .. 8c + 7 with c = t % 16
    const int h = threadIdx.x >> 4, c = threadIdx.x & 15;
    float M = ninf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mb[((size_t)w * 16 + h) * PART + HD]);
    float L = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (M != ninf) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float* src = mb + ((size_t)w * 16 + h) * PART;
            const float sc = exp2f(src[HD] - M);
            L += sc * src[HD + 1];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += sc * src[8 * c + i];
        }
    }
    float* pp = a.part + ((size_t)blockIdx.x * 16 + h) * PART;
#pragma unroll
    for (int i = 0; i < 8; i += 4)
        *reinterpret_cast<float4*>(pp + 8 * c + i) =
            make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    if (c == 0) {
        pp[HD] = M;
        pp[HD + 1] = L;
    }
}

// Merge of the split partials: a 64-thread workgroup per (query row, group of
// four heads); thread t takes head 4 * blockIdx.y + t / 16 and dims
// 8 * (t % 16) .. +8. One online pass (running maximum, earlier sums rescaled
// when it grows) with sixteen splits' partials in flight at a time.
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
    constexpr int G = 16;
    const long long qrow = blockIdx.x;
    const int h = 4 * (int)blockIdx.y + (threadIdx.x >> 4), c = threadIdx.x & 15;
    if (h >= a.H) return;
    const float ninf = -__builtin_inff();
    const float* base = a.part + ((size_t)qrow * a.n_split * 16 + h) * PART;
    const size_t stride = (size_t)16 * PART;
    float MM = ninf, LL = 0.f, o8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o8[i] = 0.f;
    for (int s0 = 0; s0 < a.n_split; s0 += G) {
        float mg[G], lg[G];
        float4 v0[G], v1[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
            mg[q] = ninf;
            lg[q] = 0.f;
            v0[q] = v1[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s0 + q < a.n_split) {
                const float* ps = base + (size_t)(s0 + q) * stride;
                mg[q] = ps[HD];
                lg[q] = ps[HD + 1];
                v0[q] = *reinterpret_cast<const float4*>(ps + 8 * c);
                v1[q] = *reinterpret_cast<const float4*>(ps + 8 * c + 4);
            }
        }
        float cm = ninf;
#pragma unroll
        for (int q = 0; q < G; ++q) cm = fmaxf(cm, mg[q]);
        const float nm = fmaxf(MM, cm);
        if (nm == ninf) continue;
        const float so = MM == ninf ? 0.f : exp2f(MM - nm);
        LL *= so;
#pragma unroll
        for (int i = 0; i < 8; ++i) o8[i] *= so;
#pragma unroll
        for (int q = 0; q < G; ++q) {
            if (mg[q] == ninf) continue;
            const float sc = exp2f(mg[q] - nm);
            LL += sc * lg[q];
            o8[0] += sc * v0[q].x; o8[1] += sc * v0[q].y; o8[2] += sc * v0[q].z; o8[3] += sc * v0[q].w;
            o8[4] += sc * v1[q].x; o8[5] += sc * v1[q].y; o8[6] += sc * v1[q].z; o8[7] += sc * v1[q].w;
        }
        MM = nm;
    }
    const float inv = LL > 0.f ? 1.f / LL : 0.f;
    bf16x8 h8;
#pragma unroll
    for (int i = 0; i < 8; ++i) h8[i] = (__bf16)(o8[i] * inv);
    *reinterpret_cast<uint4*>(a.O + (qrow * a.H + h) * HD + 8 * c) = __builtin_bit_cast(uint4, h8);
    if (a.lse && c == 0) a.lse[qrow * a.H + h] = LL > 0.f ? (MM + log2f(LL)) * kLn2 : ninf;
}

// ------------------------------------------------------------ key ranges
//
// Many query rows whose idx rows are sorted and causal: the work is cut into
// (key range of RK keys, row) items taken in range order. Workgroups are
// dealt to the XCDs round robin, so every XCD works on the same range at a
// time and its L2 (backed by the MALL) holds most of that range's K and V
// rows while they are gathered. Each wave writes the partial softmax of its row over the range
// (O / l in fp16, log2-domain lse in fp32); a merge kernel combines a row's
// partials. Rows that reach one range only are finished directly.

constexpr int RK = 12288;  // keys per range: 6 MiB of bf16 K and V rows (measured best)

// sum over t in [0, x) of min(nr - 1, floor(t / RK))
__host__ __device__ inline long long range_floor_sum(long long x, int nr) {
    const long long cap = (long long)(nr - 1) * RK;
    const long long y = x < cap ? x : cap;
    const long long m = y / RK;
    long long s = RK * (m * (m - 1) / 2) + m * (y - m * RK);
    if (x > cap) s += (long long)(nr - 1) * (x - cap);
    return s;
}

// Ranges that row `row` of a sequence reaches, and where its partials start
// within the sequence's partials.
__host__ __device__ inline int row_ranges(long long pos, int nr) {
    const long long r = pos / RK + 1;
    return (int)(r < nr ? r : nr);
}

__host__ __device__ inline long long row_part_base(int q_pos0, int row, int nr) {
    return range_floor_sum((long long)q_pos0 + row, nr) - range_floor_sum(q_pos0, nr) + row;
}

// First row of a sequence whose position reaches range r (n_q if none).
__host__ __device__ inline int range_first_row(int r, int q_pos0, int n_q) {
    const long long f = (long long)r * RK - q_pos0;
    return f <= 0 ? 0 : (f >= n_q ? n_q : (int)f);
}

// Number of entries of the sorted sel[0, nv) below `bound` (nv <= 4096):
// 64 evenly spaced probes, then the 64 entries of the bracket they leave.
__device__ __forceinline__ int lower_bound_wave(const int32_t* sel, int nv, int bound) {
    const int lane = threadIdx.x & 63;
    const int stride = (nv + 63) / 64;
    const int p1 = lane * stride;
    const int c1 = __popcll(__ballot(p1 < nv && sel[p1] < bound));
    if (c1 == 0) return 0;
    const int base = (c1 - 1) * stride;  // sel[base] < bound
    const int end = min(base + stride, nv);
    const int p2 = base + 1 + lane;
    return base + 1 + __popcll(__ballot(p2 < end && sel[p2] < bound));
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_range_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[WAVE_LDS];
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    long long j = blockIdx.x;
    int r = 0, f = 0;
    for (; r < a.n_range; ++r) {
        f = range_first_row(r, a.q_pos0, a.n_q);
        const long long cnt = (long long)a.B * (a.n_q - f);
        if (j < cnt) break;
        j -= cnt;
    }
    if (r >= a.n_range) return;
    const int per = a.n_q - f;
    const int b = (int)(j / per), row = f + (int)(j % per);
    const long long pos = (long long)a.q_pos0 + row;
    const int R = row_ranges(pos, a.n_range);
    const long long qrow = (long long)b * a.n_q + row;
    const int nv = (int)min((long long)a.k, min((long long)a.n_k, pos + 1));
    const int32_t* sel = a.idx + qrow * a.k;
    const int s0 = r == 0 ? 0 : lower_bound_wave(sel, nv, r * RK);
    const int s1 = r == R - 1 ? nv : lower_bound_wave(sel, nv, (r + 1) * RK);
    WaveState ws;
    wave_attend(a, qrow, s0, s1, 32, lds, ws);
    const float l = wave_xor_sum(ws.lpart);
    if (m >= a.H) return;
    const float ninf = -__builtin_inff();
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (R == 1) {
        uint16_t* op = a.O + (qrow * a.H + m) * HD;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            bf16x4 h4;
#pragma unroll
            for (int q = 0; q < 4; ++q) h4[q] = (__bf16)(ws.o[d][q] * inv);
            *reinterpret_cast<uint2*>(op + 16 * d + 4 * g) = __builtin_bit_cast(uint2, h4);
        }
        if (a.lse && g == 0) a.lse[qrow * a.H + m] = l > 0.f ? (ws.mrun + log2f(l)) * kLn2 : ninf;
        return;
    }
    // Partial of range r: fp16 mantissas u = (O / l) * 2^-e with 2^e above the
    // head's largest |O / l| (so |u| < 1 whatever V's range), 2^e and the
    // log2-domain lse beside them.
    float amax = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fabsf(ws.o[d][q] * inv));
    amax = wave_xor_max(amax);
    int e = 0;
    (void)frexpf(amax, &e);
    const float down = ldexpf(1.f, -e);
    const long long pidx = (long long)b * a.parts_per_seq + row_part_base(a.q_pos0, row, a.n_range) + r;
    _Float16* po = reinterpret_cast<_Float16*>(a.part_o) + (pidx * 16 + m) * HD;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        f16x4 h4;
#pragma unroll
        for (int q = 0; q < 4; ++q) h4[q] = (_Float16)(ws.o[d][q] * inv * down);
        *reinterpret_cast<uint2*>(po + 16 * d + 4 * g) = __builtin_bit_cast(uint2, h4);
    }
    if (g == 0)
        *reinterpret_cast<float2*>(a.part_lse + (pidx * 16 + m) * 2) =
            make_float2(l > 0.f ? ws.mrun + log2f(l) : ninf, ldexpf(1.f, e));
}

// Merge of a row's range partials: thread t takes head t / 16 and dims
// 8 * (t % 16) .. +8; one online pass, eight partials in flight at a time.
__global__ __launch_bounds__(256) void attn_range_merge_kernel(AttnArgs a) {
    constexpr int G = 8;
    const long long qrow = blockIdx.x;
    const int b = (int)(qrow / a.n_q), row = (int)(qrow % a.n_q);
    const long long pos = (long long)a.q_pos0 + row;
    const int R = row_ranges(pos, a.n_range);
    if (R == 1) return;  // finished by the range kernel
    const int h = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (h >= a.H) return;
    const float ninf = -__builtin_inff();
    const long long pb = (long long)b * a.parts_per_seq + row_part_base(a.q_pos0, row, a.n_range);
    float MM = ninf, LL = 0.f, o8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o8[i] = 0.f;
    for (int r0 = 0; r0 < R; r0 += G) {
        float2 lg[G];
        uint4 v[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
            lg[q] = make_float2(ninf, 0.f);
            v[q] = make_uint4(0u, 0u, 0u, 0u);
            if (r0 + q < R) {
                const long long pi = pb + r0 + q;
                lg[q] = *reinterpret_cast<const float2*>(a.part_lse + (pi * 16 + h) * 2);
                v[q] = *reinterpret_cast<const uint4*>(a.part_o + (pi * 16 + h) * HD + 8 * c);
            }
        }
        float cm = ninf;
#pragma unroll
        for (int q = 0; q < G; ++q) cm = fmaxf(cm, lg[q].x);
        const float nm = fmaxf(MM, cm);
        if (nm == ninf) continue;
        const float so = MM == ninf ? 0.f : exp2f(MM - nm);
        LL *= so;
#pragma unroll
        for (int i = 0; i < 8; ++i) o8[i] *= so;
#pragma unroll
        for (int q = 0; q < G; ++q) {
            if (lg[q].x == ninf) continue;
            const float w = exp2f(lg[q].x - nm);
            LL += w;
            const float ws = w * lg[q].y;
            const f16x8 h8 = __builtin_bit_cast(f16x8, v[q]);
#pragma unroll
            for (int i = 0; i < 8; ++i) o8[i] += ws * (float)h8[i];
        }
        MM = nm;
    }
    const float inv = LL > 0.f ? 1.f / LL : 0.f;
    bf16x8 h8;
#pragma unroll
    for (int i = 0; i < 8; ++i) h8[i] = (__bf16)(o8[i] * inv);
    *reinterpret_cast<uint4*>(a.O + (qrow * a.H + h) * HD + 8 * c) = __builtin_bit_cast(uint4, h8);
    if (a.lse && c == 0) a.lse[qrow * a.H + h] = LL > 0.f ? (MM + log2f(LL)) * kLn2 : ninf;
}

}  // namespace

void attn_split_plan(int B, int n_q, int k, int* n_split, int* split_len) {
    // Many rows: one wave per row. Few rows: 4-wave workgroups per (row,
    // split), splits of a multiple of 128 slots, about 256 workgroups in all
    // (one per CU: 512 left the combine with twice the partials to merge and
    // timed 19.6 us against 17.7 for a 128K-key decode batch).
    const long long rows = (long long)B * n_q;
    if (rows >= 2048) {
        *n_split = 1;
        *split_len = k;
        return;
    }
    const int max_split = (k + 127) / 128;
    long long want = (256 + rows - 1) / rows;
    int ns = (int)(want < 1 ? 1 : (want > max_split ? max_split : want));
    int len = (k + ns - 1) / ns;
    len = (len + 127) / 128 * 128;
    ns = (k + len - 1) / len;
    *n_split = ns;
    *split_len = len;
}

bool attn_ranged_applies(int B, int n_q, int n_k) {
    // the range of a workgroup is found by a walk over the ranges: up to 64
    return (long long)B * n_q >= 2048 && n_k > RK && n_k <= 64 * RK;
}

static long long ranged_parts_per_seq(int n_q, int n_k, int q_pos0) {
    const int nr = (n_k + RK - 1) / RK;
    return range_floor_sum((long long)q_pos0 + n_q, nr) - range_floor_sum(q_pos0, nr) + n_q;
}

size_t attn_ranged_ws_bytes(int B, int n_q, int n_k, int q_pos0) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t parts = (size_t)B * (size_t)ranged_parts_per_seq(n_q, n_k, q_pos0);
    return al(parts * 16 * 2 * sizeof(float)) + al(parts * 16 * HD * sizeof(uint16_t));
}

void attn_set_ranged(AttnArgs& a, int q_pos0, void* ws) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    a.ranged = 1;
    a.q_pos0 = q_pos0;
    a.n_range = (a.n_k + RK - 1) / RK;
    a.parts_per_seq = ranged_parts_per_seq(a.n_q, a.n_k, q_pos0);
    const size_t parts = (size_t)a.B * (size_t)a.parts_per_seq;
    a.part_lse = static_cast<float*>(ws);
    a.part_o = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + al(parts * 16 * 2 * sizeof(float)));
}

// Pool rows of the selected keys of a paged layout: prow[t] = key_row of
// entry t of sequence t / per_seq for entries inside [0, n_k), -1 otherwise.
__global__ __launch_bounds__(256) void page_rows_kernel(const int32_t* idx, int32_t* prow,
                                                        long long total, int per_seq, int n_k,
                                                        KeyPages pg) {
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int j = idx[t];
    prow[t] = (j >= 0 && j < n_k) ? (int32_t)key_row(pg, (int)(t / per_seq), n_k, j) : -1;
}

hipError_t launch_page_rows(const int32_t* idx, int32_t* prow, int B, int per_seq, int n_k,
                            const KeyPages& pg, hipStream_t s) {
    const long long total = (long long)B * per_seq;
    if (total <= 0) return hipSuccess;
    const long long nb = (total + 255) / 256;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(page_rows_kernel, dim3((unsigned)nb), dim3(256), 0, s, idx, prow, total,
                       per_seq, n_k, pg);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s) {
    const long long rows = (long long)a.B * a.n_q;
    if (rows <= 0) return hipSuccess;
    if (a.ranged) {
        long long nb = 0;
        for (int r = 0; r < a.n_range; ++r)
            nb += (long long)a.B * (a.n_q - range_first_row(r, a.q_pos0, a.n_q));
        if (nb > 0x7fffffffLL || rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        if (nb > 0)
            hipLaunchKernelGGL(sparse_attn_range_kernel, dim3((unsigned)nb), dim3(64), 0, s, a);
        hipLaunchKernelGGL(attn_range_merge_kernel, dim3((unsigned)rows), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (rows >= 2048 || a.n_split == 1) {
        // one wave per row; also for few rows of one split each, where a
        // combine pass would only copy the split's partial
        if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)rows), dim3(64), 0, s, a);
        return hipGetLastError();
    }
    const long long nb = rows * a.n_split;
    hipLaunchKernelGGL(sparse_attn_split_kernel, dim3((unsigned)nb), dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows, (unsigned)((a.H + 3) / 4)), dim3(64), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace dsa
