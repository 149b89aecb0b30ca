// MFMA operand fragments of indexer rows (query or key) for gfx950 and the
// tile products the indexer kernels are built from.
//
// Both operands of an MFMA put the same contraction index in the same (lane
// group, register byte) slot, so any fixed assignment of row bytes to slots
// yields the full dot product. Lane group g = lane / 16 of an fp8 row takes
// bytes [16g, +16) and [64 + 16g, +16) of every 128-byte chunk, 8 bytes at
// [32c + 8g, +8) of each trailing 32-byte chunk, and a bf16 row's lane group
// takes elements [32c + 8g, +8) of every 32-element chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {
namespace frag {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kE8M0One = 127;  // E8M0 block scale encoding 2^0

template <int DT, int D> struct Frag;

// fp8 e4m3fn row fragment: NB chunks of 128 bytes (32 per lane) and NS
// chunks of 32 bytes (8 per lane).
// NT selects nontemporal loads (rows streamed once from HBM).
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int D> struct Frag<0, D> {
    static constexpr int NB = D / 128, NS = (D % 128) / 32;
    i32x8 big[NB > 0 ? NB : 1];
    long small[NS > 0 ? NS : 1];
    template <bool NT = false>
    __device__ __forceinline__ void load(const uint8_t* row, int g) {
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            // bytes [16g, +16) and [64 + 16g, +16) of the chunk: each load
            // instruction covers one contiguous 64-byte half of 16 rows
            const uint8_t* p = row + 128 * c + 16 * g;
            i32x4 lo = ld<NT>(reinterpret_cast<const i32x4*>(p));
            i32x4 hi = ld<NT>(reinterpret_cast<const i32x4*>(p + 64));
            big[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int c = 0; c < NS; ++c)
            small[c] = ld<NT>(reinterpret_cast<const long*>(row + 128 * NB + 32 * c + 8 * g));
    }
};

// bf16 row fragment: D/32 chunks of 32 elements (8 per lane).
template <int D> struct Frag<1, D> {
    static constexpr int NC = D / 32;
    bf16x8 v[NC];
    template <bool NT = false>
    __device__ __forceinline__ void load(const uint8_t* row, int g) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const i32x4 w = ld<NT>(reinterpret_cast<const i32x4*>(row + 64 * c + 16 * g));
            v[c] = __builtin_bit_cast(bf16x8, w);
        }
    }
};

template <int D>
__device__ __forceinline__ f32x4 tile_dot(const Frag<0, D>& a, const Frag<0, D>& b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NB; ++c)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a.big[c], b.big[c], acc, 0, 0, 0, kE8M0One, 0, kE8M0One);
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NS; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a.small[c], b.small[c], acc, 0, 0, 0);
    return acc;
}

// tile_dot accumulated onto c0 instead of zero: acc = c0 + a . b.
template <int D>
__device__ __forceinline__ f32x4 tile_dot_c(const Frag<0, D>& a, const Frag<0, D>& b, f32x4 acc) {
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NB; ++c)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a.big[c], b.big[c], acc, 0, 0, 0, kE8M0One, 0, kE8M0One);
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NS; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a.small[c], b.small[c], acc, 0, 0, 0);
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 tile_dot_c(const Frag<1, D>& a, const Frag<1, D>& b, f32x4 acc) {
#pragma unroll
    for (int c = 0; c < Frag<1, D>::NC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[c], b.v[c], acc, 0, 0, 0);
    return acc;
}

// The same fp8 product through v_mfma_f32_16x16x32_fp8_fp8 only (the 32-byte
// chunks split into four 8-byte steps, the pairing of bytes unchanged).
template <int D>
__device__ __forceinline__ f32x4 tile_dot_k32(const Frag<0, D>& a, const Frag<0, D>& b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NB; ++c) {
        const long* pa = reinterpret_cast<const long*>(&a.big[c]);
        const long* pb = reinterpret_cast<const long*>(&b.big[c]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pa[s], pb[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < Frag<0, D>::NS; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a.small[c], b.small[c], acc, 0, 0, 0);
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 tile_dot_k32(const Frag<1, D>& a, const Frag<1, D>& b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Frag<1, D>::NC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[c], b.v[c], acc, 0, 0, 0);
    return acc;
}

template <int D>
__device__ __forceinline__ f32x4 tile_dot(const Frag<1, D>& a, const Frag<1, D>& b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < Frag<1, D>::NC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[c], b.v[c], acc, 0, 0, 0);
    return acc;
}

// relu(x * scale) with +0.0 for every non-positive (or NaN) product.
__device__ __forceinline__ float relu_scaled(float x, float scale) {
    const float s = x * scale;
    return s > 0.0f ? s : 0.0f;
}


}  // namespace frag
}  // namespace dsa
