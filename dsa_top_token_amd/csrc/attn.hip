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

template <bool SPLIT>
__global__ __launch_bounds__(256) void sparse_attn_kernel(AttnArgs a) {
    __shared__ unsigned short vs[4][32][LROW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const long long task = (long long)blockIdx.x * 4 + wave;
    const long long n_tasks = (long long)a.B * a.n_q * a.n_split;
    if (task >= n_tasks) return;  // no workgroup barrier below
    const int split = (int)(task % a.n_split);
    const long long qrow = task / a.n_split;  // b * n_q + i
    const int b = (int)(qrow / a.n_q);
    const int e0 = split * a.split_len;
    const int e1 = min(a.k, e0 + a.split_len);
    const int32_t* sel = a.idx + qrow * (long long)a.k;
    const uint16_t* Kb = a.K + (size_t)b * a.n_k * HD;
    const uint16_t* Vb = a.V + (size_t)b * a.n_k * HD;
    unsigned short(*lv)[LROW] = vs[wave];

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

    f32x4 o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float ninf = -__builtin_inff();
    float mrun = ninf, lpart = 0.f;
    const float sl2 = 0.08838834764831845f * kLog2e;  // 128^-0.5 * log2(e)

    for (int e = e0; e < e1; e += 32) {
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
        const float mnew = fmaxf(mrun, mx);
        const bool live = mnew != ninf;
        const float alpha = live ? exp2f(mrun - mnew) : 1.f;
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = live ? exp2f(z[i] - mnew) : 0.f;
            psum += p[i];
        }
        lpart = lpart * alpha + psum;
        mrun = mnew;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d] *= alpha;
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
            o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, o[d], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    const float l = wave_xor_sum(lpart);
    if (m >= a.H) return;
    if (!SPLIT) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* op = a.O + (qrow * a.H + m) * HD;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            bf16x4 h4;
#pragma unroll
            for (int r = 0; r < 4; ++r) h4[r] = (__bf16)(o[d][r] * inv);
            *reinterpret_cast<uint2*>(op + 16 * d + 4 * g) = __builtin_bit_cast(uint2, h4);
        }
        if (a.lse && g == 0) a.lse[qrow * a.H + m] = l > 0.f ? (mrun + log2f(l)) * kLn2 : ninf;
    } else {
        float* pp = a.part + ((size_t)task * 16 + m) * PART;
#pragma unroll
        for (int d = 0; d < 8; ++d)
            *reinterpret_cast<float4*>(pp + 16 * d + 4 * g) =
                make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
        if (g == 0) {
            pp[HD] = mrun;
            pp[HD + 1] = l;
        }
    }
}

// Merge of split partials: one wave per (query, head); lane l owns dims
// 2l, 2l+1. Every split's (max, sum) pair is read first, then the rescaled
// partial outputs are summed.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63;
    const long long qh = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (qh >= (long long)a.B * a.n_q * a.H) return;
    const int h = (int)(qh % a.H);
    const long long qrow = qh / a.H;
    const float ninf = -__builtin_inff();
    const float* base = a.part + (size_t)qrow * a.n_split * 16 * PART + (size_t)h * PART;
    const size_t stride = (size_t)16 * PART;
    // lanes read the split statistics in parallel (n_split <= 64 per pass)
    float M = ninf;
    for (int s0 = 0; s0 < a.n_split; s0 += 64) {
        const int s = s0 + lane;
        const float ms = s < a.n_split ? base[(size_t)s * stride + HD] : ninf;
        M = fmaxf(M, ms);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != ninf) {
        for (int s = 0; s < a.n_split; ++s) {
            const float* ps = base + (size_t)s * stride;
            const float w = exp2f(ps[HD] - M);
            L += w * ps[HD + 1];
            const float2 v = *reinterpret_cast<const float2*>(ps + 2 * lane);
            o0 += w * v.x;
            o1 += w * v.y;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 h2 = {(__bf16)(o0 * inv), (__bf16)(o1 * inv)};
    *reinterpret_cast<uint32_t*>(a.O + (qrow * a.H + h) * HD + 2 * lane) =
        __builtin_bit_cast(uint32_t, h2);
    if (a.lse && lane == 0) a.lse[qrow * a.H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : ninf;
}

}  // namespace

void attn_split_plan(int B, int n_q, int k, int* n_split, int* split_len) {
    const long long rows = (long long)B * n_q;
    const int max_split = (k + 63) / 64;  // at least 64 entries per split
    long long want = (2048 + rows - 1) / rows;
    int ns = (int)(want < 1 ? 1 : (want > max_split ? max_split : want));
    if (ns < 1) ns = 1;
    int len = (k + ns - 1) / ns;
    len = (len + 31) / 32 * 32;
    ns = (k + len - 1) / len;
    *n_split = ns;
    *split_len = len;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s) {
    const long long tasks = (long long)a.B * a.n_q * a.n_split;
    if (tasks <= 0) return hipSuccess;
    const long long nb = (tasks + 3) / 4;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.n_split == 1) {
        hipLaunchKernelGGL(sparse_attn_kernel<false>, dim3((unsigned)nb), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(sparse_attn_kernel<true>, dim3((unsigned)nb), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long nc = ((long long)a.B * a.n_q * a.H + 3) / 4;
    if (nc > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)nc), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa
