// Sparse MQA attention over the selected keys on gfx950.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693): section 3.3 runs ordinary
// softmax attention over each query's selected keys only; section 4.2 has all
// query heads share one K/V set (MQA), so one gathered K/V row serves every
// head; section 4.1 runs this stage in BF16.
//
// One wave owns one (query, split) task: up to 16 heads against the split's
// selected keys, 32 keys per step.
//   S^T (keys x heads) = K_sel (keys x 128) . Q^T    4+4 bf16 16x16x32 MFMAs
//   online softmax per head (log2 domain, fp32)
//   O^T (dims x heads) += V_sel^T . P^T              8 bf16 16x16x32 MFMAs
// With S^T as the MFMA output, lane (head h = lane%16, group g = lane/16)
// holds scores of keys 4g..4g+3 and 16+4g..16+4g+3, which is exactly the
// 8-key slice of P^T the PV product wants from that lane (the contraction
// order over keys is free). V rows are gathered with coalesced 64-byte
// loads, staged in the wave's LDS slice and read back transposed.
// With n_split > 1 each task writes unnormalised partials (O, running max,
// running sum) and a second kernel merges them by log-sum-exp rescaling.
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int HD = 128;          // head dim
constexpr int LROW = HD + 8;     // LDS row pitch in bf16 elements (272 B)
constexpr int PART = HD + 4;     // floats per (task, head) partial: O[128], m, l, pad
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float wave_xor_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

__device__ __forceinline__ float wave_xor_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// One wave's pass over selected-key slots e = e_first, e_first + e_step, ...
// (32 slots each, all below e_end) of query row qrow: online softmax state
// (running max in the log2 domain, this lane's partial sum) and the
// unnormalised O^T tiles: lane (head m, group g) holds dims 16d + 4g + r.
struct WaveState {
    f32x4 o[8];
    float mrun, lpart;
};

__device__ __forceinline__ void wave_attend(const AttnArgs& a, long long qrow, int e_first,
                                            int e_end, int e_step,
                                            unsigned short (*lv)[LROW], WaveState& ws) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, g = lane >> 4;
    const int b = (int)(qrow / a.n_q);
    const int32_t* sel = a.idx + qrow * (long long)a.k;
    const uint16_t* Kb = a.K + (size_t)b * a.n_k * HD;
    const uint16_t* Vb = a.V + (size_t)b * a.n_k * HD;

    // Q^T fragment: lane (head m, group g) holds Q[m][32g + 8s .. +8] for s = 0..3,
    // matching the K fragment's dims below.
    bf16x8 qf[4];
    if (m < a.H) {
        const u16x8* qp = reinterpret_cast<const u16x8*>(a.Q + (qrow * a.H + m) * HD + 32 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(qp[s]);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }

#pragma unroll
    for (int d = 0; d < 8; ++d) ws.o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float ninf = -__builtin_inff();
    ws.mrun = ninf;
    ws.lpart = 0.f;
    const float sl2 = 0.08838834764831845f * kLog2e;  // 128^-0.5 * log2(e)
    const int e1 = e_end;

    for (int e = e_first; e < e1; e += e_step) {
        // Key rows gathered by this lane: slot 16t + m, dims [32g, 32g + 32).
        int jr[2];
        bool vr[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int slot = e + 16 * t + m;
            const int j = slot < e1 ? sel[slot] : -1;
            vr[t] = j >= 0 && j < a.n_k;
            jr[t] = vr[t] ? j : 0;
        }
        if (__ballot(vr[0] || vr[1]) == 0ull) continue;
        u16x8 kf[2][4], vf[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u16x8* kp = reinterpret_cast<const u16x8*>(Kb + (size_t)jr[t] * HD + 32 * g);
            const u16x8* vp = reinterpret_cast<const u16x8*>(Vb + (size_t)jr[t] * HD + 32 * g);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                kf[t][s] = kp[s];
                vf[t][s] = vp[s];
            }
        }
        // Validity of the keys whose scores this lane holds: slots 16t + 4g + r.
        bool vs_ok[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = e + 16 * t + 4 * g + r;
                const int j = slot < e1 ? sel[slot] : -1;
                vs_ok[t][r] = j >= 0 && j < a.n_k;
            }

        f32x4 st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[t][s]), qf[s], st[t],
                                                                0, 0, 0);
        }
        // Stage V rows: LDS row 16t + m, columns [32g, 32g + 32).
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                *reinterpret_cast<u16x8*>(&lv[16 * t + m][32 * g + 8 * s]) = vf[t][s];

        float z[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) z[4 * t + r] = vs_ok[t][r] ? st[t][r] * sl2 : ninf;
        float mx = z[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
        mx = wave_xor_max(mx);
        const float mnew = fmaxf(ws.mrun, mx);
        const bool live = mnew != ninf;
        const float alpha = live ? exp2f(ws.mrun - mnew) : 1.f;
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = live ? exp2f(z[i] - mnew) : 0.f;
            psum += p[i];
        }
        ws.lpart = ws.lpart * alpha + psum;
        ws.mrun = mnew;
#pragma unroll
        for (int d = 0; d < 8; ++d) ws.o[d] *= alpha;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)p[i];

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // V^T fragment: lane (dim 16d + m, group g) holds V[key][16d + m] for
        // keys 4g..4g+3 and 16+4g..16+4g+3, the same key slots as pb.
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            u16x8 va;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int key = i < 4 ? 4 * g + i : 12 + 4 * g + i;
                va[i] = lv[key][16 * d + m];
            }
            ws.o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, ws.o[d], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

}

// One wave per query row (many queries): normalised O and lse directly.
__global__ __launch_bounds__(256) void sparse_attn_kernel(AttnArgs a) {
    __shared__ unsigned short vs[4][32][LROW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const long long qrow = (long long)blockIdx.x * 4 + wave;
    if (qrow >= (long long)a.B * a.n_q) return;  // no workgroup barrier below
    WaveState ws;
    wave_attend(a, qrow, 0, a.k, 32, vs[wave], ws);
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
__global__ __launch_bounds__(256) void sparse_attn_split_kernel(AttnArgs a) {
    __shared__ float lds[4 * 32 * LROW / 2];  // V staging, then the merge buffer
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int split = (int)(blockIdx.x % (unsigned)a.n_split);
    const long long qrow = blockIdx.x / (unsigned)a.n_split;
    const int e0 = split * a.split_len;
    const int e1 = min(a.k, e0 + a.split_len);
    const float ninf = -__builtin_inff();
    unsigned short(*vstage)[32][LROW] = reinterpret_cast<unsigned short(*)[32][LROW]>(lds);
    WaveState ws;
    wave_attend(a, qrow, e0 + 32 * wave, e1, 128, vstage[wave], ws);
    const float lw = wave_xor_sum(ws.lpart);
    __syncthreads();  // V staging no longer needed
    // merge buffer: [wave][head][PART] with O[128], max, sum
    float* mb = lds;
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

}  // namespace

void attn_split_plan(int B, int n_q, int k, int* n_split, int* split_len) {
    // Many rows: one wave per row. Few rows: 4-wave workgroups per (row,
    // split), splits of a multiple of 128 slots, about 2048 waves in all.
    const long long rows = (long long)B * n_q;
    if (rows >= 2048) {
        *n_split = 1;
        *split_len = k;
        return;
    }
    const int max_split = (k + 127) / 128;
    long long want = (512 + rows - 1) / rows;
    int ns = (int)(want < 1 ? 1 : (want > max_split ? max_split : want));
    int len = (k + ns - 1) / ns;
    len = (len + 127) / 128 * 128;
    ns = (k + len - 1) / len;
    *n_split = ns;
    *split_len = len;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s) {
    const long long rows = (long long)a.B * a.n_q;
    if (rows <= 0) return hipSuccess;
    if (rows >= 2048) {
        const long long nb = (rows + 3) / 4;
        if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)nb), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const long long nb = rows * a.n_split;
    hipLaunchKernelGGL(sparse_attn_split_kernel, dim3((unsigned)nb), dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows, (unsigned)((a.H + 3) / 4)), dim3(64), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace dsa
