// Indexer projection front-end on gfx950: q_idx = X W_q^T and k_idx = X W_k^T
// in the indexer's input format, written to chosen rows of the output.
//
// DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), section 3.2: the lightning
// indexer maps the model width down to the indexer width with two bias-free
// linear layers (query_proj, key_proj); section 4.1 runs the index stage in
// FP8. For each input row r and output feature o,
//   y = fl32(sum_c X[r][c] W[o][c])     (bf16 inputs, fp32 MFMA accumulation)
// is encoded as e4m3fn (round to nearest even, saturating at +-448) or bf16
// (round to nearest even) into row out_rows[r] of the output; a decode step
// appends each sequence's new key row to the k_idx cache this way.
//
// Layout of the product (many rows): a wave owns RT tiles of 16 input rows
// and all DI / 16 tiles of 16 output features. Per 32-wide step of the model
// width it loads RT X fragments (streamed from HBM once) and DI / 16 W
// fragments (W is in nn.Linear's [d_idx][d_model] layout, so a lane's B
// operand, 8 consecutive elements of one W row, is one 16-byte load; W is
// read from L2, so more row tiles per wave mean less W traffic per row), then
// issues RT * DI / 16 bf16 MFMAs. Few rows (a decode batch) cannot fill the
// chip that way: a 16-wave workgroup then owns 16 rows x 16 features, its
// waves split the model width, and the partial tiles are added through LDS
// in wave order (one launch, deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Many-rows kernel: 4 waves; row tiles per wave and steps of X and W
// fragments in flight, sized so accumulators and fragments stay in registers.
constexpr int PJ_NT = 256;
template <int DI> constexpr int pj_rt() { return DI <= 128 ? 4 : 2; }
constexpr int PJ_PX = 2;
template <int DI> constexpr int pj_pw() { return DI <= 128 ? 2 : 1; }
constexpr int PJ_MIN_WGS = 192;     // fewer row workgroups than this: the split-width kernel
// LDS-staged many-rows kernel (d_idx <= 128, model width a multiple of 64):
// chunks of 64 model-width columns (128 bytes of every X and W row) in a ring
// of pl_nbuf buffers, pl_nbuf - 1 chunks in flight. Measured at 65536 x 4096:
// two workgroups per CU beat a deeper ring (d_idx 128: 2 row tiles per wave,
// 2 buffers, 64 KB; d_idx <= 64: 1 row tile, 3 buffers).
template <int DI> constexpr int pl_rt() { return DI <= 64 ? 1 : 2; }
template <int DI> constexpr int pl_nbuf() { return DI <= 64 ? 3 : 2; }
template <int DI> constexpr int pl_rows() { return 4 * 16 * pl_rt<DI>(); }  // per workgroup
constexpr int kNontemporal = 2;           // cache policy of the X copies (read once)
// Split-width kernel: 16 waves, steps of fragments in flight per wave.
constexpr int PS_NT = 1024;
constexpr int PS_W = PS_NT / 64;
constexpr int PS_PF = 6;

// e4m3fn code of v: nearest value, ties to an even mantissa; |v| >= 448
// saturates (the values in [448, 464] round there anyway); NaN -> 0x7f.
__device__ __forceinline__ uint32_t to_e4m3fn_sat(float v) {
    const uint32_t s = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (!(a == a)) return 0x7fu;
    if (a >= 448.0f) return s | 0x7eu;
    uint32_t c;
    if (a < 0.015625f) {
        // below 2^-6: codes m * 2^-9 (the scaling is exact, rintf rounds
        // half to even; m = 8 is the smallest normal code)
        c = (uint32_t)rintf(a * 512.0f);
    } else {
        // keep 3 mantissa bits, rounding half to even (a carry moves into the
        // exponent); rebias the exponent from 127 to 7
        uint32_t w = __float_as_uint(a);
        w += 0x7ffffu + ((w >> 20) & 1u);
        c = (((w >> 23) - 120u) << 3) | ((w >> 20) & 7u);
        c = min(c, 0x7eu);
    }
    return s | c;
}

// bf16 code of v: round half to even; NaN -> 0x7fc0.
__device__ __forceinline__ uint32_t to_bf16(float v) {
    if (!(v == v)) return 0x7fc0u;
    uint32_t u = __float_as_uint(v);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ void store_code(const ProjectArgs& a, int r, int col, float y) {
    const int dst = a.out_rows ? a.out_rows[r] : r;
    if (dst < 0 || dst >= a.n_out) return;  // destinations outside the output are skipped
    const size_t o = (size_t)dst * a.d_idx + col;
    if (a.out_dtype == 0) static_cast<uint8_t*>(a.out)[o] = (uint8_t)to_e4m3fn_sat(y);
    else static_cast<uint16_t*>(a.out)[o] = (uint16_t)to_bf16(y);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(p));
}

// s_waitcnt with vmcnt = N (expcnt and lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Waits until at most `ahead` chunks of OPS copies each are in flight
// (0 <= ahead <= A).
template <int A, int OPS>
__device__ __forceinline__ void wait_chunks(int ahead) {
    if constexpr (A > 0) {
        if (ahead >= A) {
            wait_vmcnt<A * OPS>();
            return;
        }
        wait_chunks<A - 1, OPS>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}

// Slot of granule j (16 bytes) of row r in a chunk of 128-byte rows: each
// copy instruction still moves 8 whole rows (1 KB) of global memory, and the
// 16 rows a fragment read touches (fixed j) land in 16 distinct bank groups.
__device__ __forceinline__ int pl_slot(int r, int j) {
    return 8 * r + (j ^ ((r & 7) ^ ((r >> 3) & 1)));
}

// Many rows through LDS: wave w of the workgroup owns PL_RT tiles of 16 rows
// and every feature. Per 64-column chunk the wave copies its X rows with
// global->LDS copies of 1 KB (8 whole 128-byte lines each) and a
// quarter of the chunk's W rows (shared by the workgroup), waits for its own
// copies, meets the other waves at a barrier, then reads fragments from LDS
// for two 32-wide MFMA steps.
template <int DI>
__global__ __launch_bounds__(PJ_NT) void project_lds_kernel(ProjectArgs a) {
    constexpr int PL_RT = pl_rt<DI>(), PL_NBUF = pl_nbuf<DI>(), PL_ROWS = pl_rows<DI>();
    constexpr int CT = DI / 16;
    constexpr int WR = 16 * PL_RT;    // rows per wave
    constexpr int XB = 4 * WR * 128;  // X bytes of a chunk (4 waves)
    constexpr int WB = DI * 128;      // W bytes of a chunk
    constexpr int X_OPS = WR / 8;     // X copies per wave per chunk
    constexpr int W_OPS = DI / 32;    // W copies per wave per chunk (DI / 8 over 4 waves)
    constexpr int OPS = X_OPS + W_OPS;
    static_assert(DI % 32 == 0 && DI <= 128 && PL_NBUF * (XB + WB) <= 160 * 1024, "LDS ring");
    static_assert(PL_NBUF >= 2 && (PL_NBUF - 2) * OPS < 64, "copies in flight");
    __shared__ __attribute__((aligned(16))) uint8_t ring[PL_NBUF][XB + WB];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = (int)blockIdx.x * PL_ROWS + WR * wave;  // may pass the last row: clamped
    const int nch = a.d_model / 64;
    const size_t rowb = (size_t)a.d_model * 2;
    const uint8_t* Xb = reinterpret_cast<const uint8_t*>(a.X);
    const uint8_t* Wb = reinterpret_cast<const uint8_t*>(a.W);
    // copy lane l moves granule (l % 8) ^ f(r) of row r = 8 i + l / 8 into slot 64 i + l
    const int cr = lane >> 3, cp = lane & 7;
    auto issue = [&](int c) {
        uint8_t* buf = ring[c % PL_NBUF];
        const size_t kb = (size_t)c * 128;
#pragma unroll
        for (int i = 0; i < X_OPS; ++i) {
            const int r = 8 * i + cr;
            const int j = cp ^ ((r & 7) ^ ((r >> 3) & 1));
            const size_t grow = (size_t)min(r0 + r, a.rows - 1);
            __builtin_amdgcn_global_load_lds(Xb + grow * rowb + kb + 16 * j,
                                             buf + WR * 128 * wave + 1024 * i, 16, 0, kNontemporal);
        }
#pragma unroll
        for (int u = 0; u < W_OPS; ++u) {
            const int i = wave + 4 * u;
            const int r = 8 * i + cr;
            const int j = cp ^ ((r & 7) ^ ((r >> 3) & 1));
            __builtin_amdgcn_global_load_lds(Wb + (size_t)r * rowb + kb + 16 * j,
                                             buf + XB + 1024 * i, 16, 0, 0);
        }
    };
    f32x4 acc[PL_RT][CT];
#pragma unroll
    for (int t = 0; t < PL_RT; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // PL_NBUF - 1 chunks ahead of the one being read
#pragma unroll
    for (int c = 0; c < PL_NBUF - 1; ++c)
        if (c < nch) issue(c);
    for (int c = 0; c < nch; ++c) {
        // chunk c has landed once only the later chunks' copies remain; the
        // barrier (no release fence, which would wait for every copy in
        // flight) also means every wave is done reading chunk c - 1
        __builtin_amdgcn_sched_barrier(0);
        wait_chunks<PL_NBUF - 2, OPS>(min(PL_NBUF - 2, nch - 1 - c));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (c + PL_NBUF - 1 < nch) issue(c + PL_NBUF - 1);  // into chunk c - 1's buffer
        const uint8_t* xs = ring[c % PL_NBUF] + WR * 128 * wave;
        const uint8_t* ws = ring[c % PL_NBUF] + XB;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 af[PL_RT], bf[CT];
#pragma unroll
            for (int t = 0; t < PL_RT; ++t)
                af[t] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const i32x4*>(xs + 16 * pl_slot(16 * t + n, 4 * s + g)));
#pragma unroll
            for (int f = 0; f < CT; ++f)
                bf[f] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const i32x4*>(ws + 16 * pl_slot(16 * f + n, 4 * s + g)));
#pragma unroll
            for (int t = 0; t < PL_RT; ++t)
#pragma unroll
                for (int f = 0; f < CT; ++f)
                    acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t], bf[f], acc[t][f], 0,
                                                                       0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < PL_RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 16 * t + 4 * g + i;
            if (r >= a.rows) continue;
#pragma unroll
            for (int f = 0; f < CT; ++f) store_code(a, r, 16 * f + n, acc[t][f][i]);
        }
}

template <int DI, int RT, int PX, int PW>
__global__ __launch_bounds__(PJ_NT) void project_kernel(ProjectArgs a) {
    static_assert(PX % PW == 0, "static ring slots");
    constexpr int CT = DI / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = __builtin_amdgcn_readfirstlane((blockIdx.x * (PJ_NT / 64) + wave) * 16 * RT);
    if (r0 >= a.rows) return;  // wave-uniform
    const int ke = a.d_model;
    // A operand: lane (n, g) holds elements [k + 8 g, +8) of row r0 + 16 t + n;
    // B operand: the same elements of W row 16 c + n.
    const uint16_t* xr[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        xr[t] = a.X + (size_t)min(r0 + 16 * t + n, a.rows - 1) * a.d_model + 8 * g;
    const uint16_t* wr = a.W + (size_t)n * a.d_model + 8 * g;
    const size_t wstep = (size_t)16 * a.d_model;  // next column tile
    f32x4 acc[RT][CT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Register rings: X fragments (streamed from HBM) PX steps ahead, W
    // fragments (L2 hits) PW steps ahead; step k + 32 p uses X slot p and
    // W slot p % PW, and the loop runs PX steps per pass so every slot index
    // is static.
    bf16x8 xf[PX][RT], wf[PW][CT];
    auto load_x = [&](int p, int k) {
#pragma unroll
        for (int t = 0; t < RT; ++t) xf[p][t] = ld8(xr[t] + k);
    };
    auto load_w = [&](int p, int k) {
#pragma unroll
        for (int c = 0; c < CT; ++c) wf[p][c] = ld8(wr + c * wstep + k);
    };
#pragma unroll
    for (int p = 0; p < PX; ++p)
        if (32 * p < ke) load_x(p, 32 * p);
#pragma unroll
    for (int p = 0; p < PW; ++p)
        if (32 * p < ke) load_w(p, 32 * p);
    for (int k = 0; k < ke; k += 32 * PX) {
#pragma unroll
        for (int p = 0; p < PX; ++p) {
            const int kp = k + 32 * p;
            if (kp >= ke) break;  // uniform
            bf16x8 xc[RT], wc[CT];
#pragma unroll
            for (int t = 0; t < RT; ++t) xc[t] = xf[p][t];
#pragma unroll
            for (int c = 0; c < CT; ++c) wc[c] = wf[p % PW][c];
            // refill both slots; the loads fly under these MFMAs
            if (kp + 32 * PX < ke) load_x(p, kp + 32 * PX);
            if (kp + 32 * PW < ke) load_w(p % PW, kp + 32 * PW);
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int c = 0; c < CT; ++c)
                    acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xc[t], wc[c], acc[t][c],
                                                                       0, 0, 0);
        }
    }
    // lane (n, g), register i of tile (t, c): input row r0 + 16 t + 4 g + i,
    // output feature 16 c + n
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 16 * t + 4 * g + i;
            if (r >= a.rows) continue;
#pragma unroll
            for (int c = 0; c < CT; ++c) store_code(a, r, 16 * c + n, acc[t][c][i]);
        }
}

// Few rows: workgroup (bx, by) owns rows 16 bx .. +16 and features
// 16 by .. +16 (small tiles spread the rows' loads over many CUs); wave w
// takes the w-th of PS_W equal parts of the model width (a multiple of 32
// each), then the PS_W partial tiles are added in wave order through LDS.
template <int PF>
__global__ __launch_bounds__(PS_NT) void project_small_kernel(ProjectArgs a) {
    __shared__ f32x4 red[PS_W][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = blockIdx.x * 16, c0 = blockIdx.y * 16;
    const int part = (a.d_model / 32 + PS_W - 1) / PS_W * 32;
    // scalar bounds: the step loop stays a uniform branch (no reconvergence waits)
    const int kb = __builtin_amdgcn_readfirstlane(min(a.d_model, wave * part));
    const int ke = __builtin_amdgcn_readfirstlane(min(a.d_model, kb + part));
    const uint16_t* xr = a.X + (size_t)min(r0 + n, a.rows - 1) * a.d_model + 8 * g;
    const uint16_t* wr = a.W + (size_t)(c0 + n) * a.d_model + 8 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    bf16x8 xf[PF], wf[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (kb + 32 * p < ke) {
            xf[p] = ld8(xr + kb + 32 * p);
            wf[p] = ld8(wr + kb + 32 * p);
        }
    for (int k = kb; k < ke; k += 32 * PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int kp = k + 32 * p;
            if (kp >= ke) break;  // uniform
            const bf16x8 x = xf[p], w = wf[p];
            if (kp + 32 * PF < ke) {
                xf[p] = ld8(xr + kp + 32 * PF);
                wf[p] = ld8(wr + kp + 32 * PF);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, w, acc, 0, 0, 0);
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    // thread (lane l, register i) adds the waves' values in order
    if (threadIdx.x < 64 * 4) {
        const int l = threadIdx.x >> 2, i = threadIdx.x & 3;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < PS_W; ++w) y += red[w][l][i];
        const int r = r0 + 4 * (l >> 4) + i;
        if (r < a.rows) store_code(a, r, c0 + (l & 15), y);
    }
}

template <int DI>
hipError_t launch_di(const ProjectArgs& a, hipStream_t s) {
    constexpr long long rows_per_wg = (PJ_NT / 64) * 16 * pj_rt<DI>();
    const long long nb = (a.rows + rows_per_wg - 1) / rows_per_wg;
    if (nb < PJ_MIN_WGS) {
        hipLaunchKernelGGL((project_small_kernel<PS_PF>),
                           dim3((unsigned)((a.rows + 15) / 16), DI / 16), dim3(PS_NT), 0, s, a);
        return hipGetLastError();
    }
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if constexpr (DI <= 128) {
        if (a.d_model % 64 == 0) {
            const long long nl = (a.rows + pl_rows<DI>() - 1) / pl_rows<DI>();
            hipLaunchKernelGGL((project_lds_kernel<DI>), dim3((unsigned)nl), dim3(PJ_NT), 0, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((project_kernel<DI, pj_rt<DI>(), PJ_PX, pj_pw<DI>()>),
                       dim3((unsigned)nb), dim3(PJ_NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_project(const ProjectArgs& a, hipStream_t s) {
    switch (a.d_idx) {
        case 32: return launch_di<32>(a, s);
        case 64: return launch_di<64>(a, s);
        case 96: return launch_di<96>(a, s);
        case 128: return launch_di<128>(a, s);
        case 160: return launch_di<160>(a, s);
        case 192: return launch_di<192>(a, s);
        case 224: return launch_di<224>(a, s);
        case 256: return launch_di<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
