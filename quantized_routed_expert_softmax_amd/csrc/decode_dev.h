// decode_dev.h — device helpers of the one-launch decode kernels (decode.hip,
// decode1.hip): loading a lane's units of a weight row, the P16 activation
// layout in LDS, and the dequantizing row dot product.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dev.h"

namespace moe {

template <int B, int UPL>
struct RowLoad {
    uint32_t w[UPL][B];
    uint32_t sb[UPL];
};

typedef uint32_t u32x2a_t __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x3a_t __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x4a_t __attribute__((ext_vector_type(4), aligned(4)));

// The B dwords of one pack unit with as few vector loads as the size allows.
template <int B>
__device__ __forceinline__ void load_unit(uint32_t (&w)[B], const uint32_t* __restrict__ p)
{
    if constexpr (B == 3) {
        const u32x3a_t v = *(const u32x3a_t*)p;
        w[0] = v.x; w[1] = v.y; w[2] = v.z;
    } else if constexpr (B == 4) {
        const u32x4a_t v = *(const u32x4a_t*)p;
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (B == 6) {
        const u32x4a_t v = *(const u32x4a_t*)p;
        const u32x2a_t u = *(const u32x2a_t*)(p + 4);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; w[4] = u.x; w[5] = u.y;
    } else if constexpr (B == 8) {
        const u32x4a_t v = *(const u32x4a_t*)p;
        const u32x4a_t u = *(const u32x4a_t*)(p + 4);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
    } else {
        static_assert(B == 16, "bits");
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4a_t v = *(const u32x4a_t*)(p + 4 * c);
            w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
        }
    }
}

// One lane's units of a weight row: codes at byte offset `codes` and scale/bias
// at byte offset `sb` from the slot base (32-bit offsets from a wave-uniform
// base, so the loads take the scalar-base form).
template <int B, int UPL>
__device__ __forceinline__ void load_row(RowLoad<B, UPL>& r, const uint8_t* __restrict__ base,
                                         uint32_t codes, uint32_t sb, int seg, int lpr)
{
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
        const uint32_t u = (uint32_t)(seg + lpr * j);
        load_unit<B>(r.w[j], (const uint32_t*)(base + (codes + u * (uint32_t)(4 * B))));
        if constexpr (Code<B>::affine) r.sb[j] = *(const uint32_t*)(base + (sb + (u >> 1) * 4u));
        else r.sb[j] = 0u;  // width 16: bf16 weights, no scale/bias
    }
}

// Row of phase-1 index j of a hit: consecutive indices 2m, 2m+1 are the rows of
// one P16 pair, n and n + 16 of a 32-row chunk.
__device__ __forceinline__ int pair_row(int j) { return (j & ~31) | ((j >> 1) & 15) | ((j & 1) << 4); }

// LDS layout of a row of P16 activations: the 16 dwords of unit u are contiguous
// (dwords 16u..16u+15), in four 16-byte chunks whose order is rotated by an XOR
// with (u >> 2) & 3, so 16 lanes reading chunk c of units u..u+15 touch 64
// distinct banks.  Dword i of unit u sits at swz(u, i).
__device__ __forceinline__ int swz(int u, int i) { return 16 * u + ((((i >> 2) ^ (u >> 2)) & 3) << 2) + (i & 3); }

// a / b for a >= 0, b > 0: a shift when b is a power of two (the usual case for
// the layer's sizes; a general integer division costs tens of instructions)
__device__ __forceinline__ int udiv(int a, int b)
{
    return (b & (b - 1)) == 0 ? (a >> __builtin_ctz(b)) : a / b;
}

// The 16 dwords of unit u, in order, with four 16-byte LDS reads.
__device__ __forceinline__ void load_unit_act(const uint32_t* __restrict__ row, int u, uint32_t (&a)[16])
{
    const uint32_t* base = row + 16 * u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 v = *(const uint4*)(base + (((c ^ (u >> 2)) & 3) << 2));
        a[4 * c] = v.x;
        a[4 * c + 1] = v.y;
        a[4 * c + 2] = v.z;
        a[4 * c + 3] = v.w;
    }
}

// Dot of one row's lane share (UPL units) with a row of activations in LDS
// (layout swz); each unit is unpacked right before its dot product, so only
// one unit's 16 pairs are live at a time.  xs[u] is the activations' sum over
// unit u.  Per unit: s*acc + (z - off*s)*xs.
template <int B, int UPL>
__device__ __forceinline__ float row_dot_raw(const RowLoad<B, UPL>& r, const uint32_t* __restrict__ act,
                                             const float* __restrict__ xs, int seg, int lpr)
{
    constexpr float off = Code<B>::offset;
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
        const int u = seg + lpr * j;
        uint32_t av[16], cp[16];
        load_unit_act(act, u, av);
        unit_pairs<B>(r.w[j], cp);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc = dot2(cp[i], av[i], acc);
        if constexpr (Code<B>::affine) {
            const float s = half_bits_to_f32(r.sb[j] & 0xFFFFu);
            const float z = __builtin_fmaf(-off, s, half_bits_to_f32(r.sb[j] >> 16));
            y = __builtin_fmaf(s, acc, __builtin_fmaf(z, xs[u], y));
        } else {
            y += acc;  // width 16: the pairs are the weights themselves
        }
    }
    return y;
}

// Sum over unit u of a row of P16 activations (bf16 dot2 against ones, i ascending).
__device__ __forceinline__ float unit_sum(const uint32_t* __restrict__ row, int u)
{
    uint32_t av[16];
    load_unit_act(row, u, av);
    float X = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) X = dot2(av[i], MOE_ONES_PAIR, X);
    return X;
}

}  // namespace moe
