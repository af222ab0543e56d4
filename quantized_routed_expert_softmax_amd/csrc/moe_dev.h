// moe_dev.h — device helpers shared by the gfx950 kernels of the routed-expert
// MoE layer: bf16 pair arithmetic, code extraction from the slot format's pack
// units, wave reductions.
//
// Slot format (one expert row; the pages fix only a group-wise affine code and
// a single unbroken row per expert — "RFC: stream MoE experts from disk in
// from_pretrained", How the prototype works): codes are a little-endian bit
// stream in pack units of 32 values held in B uint32 words; scale and bias are
// one fp16 pair per group of 64 inputs.
//
// Pairing used by every kernel ("P16"): the 32 codes of a unit are consumed as
// 16 pairs (c_i, c_{i+16}), i = 0..15.  A pair is packed into one register as
// two bf16 values 128 + c (bf16 bits 0x4300 | c, exact for c < 128), or for
// 8-bit codes as two bf16 values c (exact for c < 256).  Activations are laid
// out to match: within every 32-wide chunk, position 2i+h holds input i+16h.
// A bf16 dot2 then accumulates sum x*(off + c) exactly per product, and the
// affine map is applied per group afterwards:
//     sum_g s_g * sum x*c + z_g * sum x  =  s_g * acc + (z_g - off*s_g) * X_g.
// Width 16 (unquantized bf16 weights) uses the same unit rule with the bf16 bit
// patterns as codes: a unit is 16 words holding the 32 values in order, a pair
// is taken straight from them, and there is no affine step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

#define MOE_MAGIC_PAIR 0x43004300u  // two bf16 128.0
#define MOE_ONES_PAIR 0x3F803F80u   // two bf16 1.0

namespace moe {

template <int B>
struct Code {
    static constexpr uint32_t mask = (1u << B) - 1u;
    static constexpr uint32_t mask2 = mask * 0x10001u;
    static constexpr float offset = (B >= 8) ? 0.0f : 128.0f;  // bf16 value of code 0
    static constexpr bool affine = B != 16;                       // width 16: bf16 weights
    static constexpr int per_t = 16 / B;                          // pairs from one window pair
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    __bf16 b = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// 32-bit window of a unit's bit stream starting at compile-time bit `o`.
template <int B>
__device__ __forceinline__ uint32_t win(const uint32_t (&w)[B], int o)
{
    const int wi = o >> 5, sh = o & 31;
    if (sh == 0) return w[wi];
    if (wi + 1 >= B) return w[wi] >> sh;
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
}

// Pair i of a unit with its low code at bit 0 and high code at bit 16
// (other bits hold neighbouring codes; callers mask).
template <int B>
__device__ __forceinline__ uint32_t pair_window(const uint32_t (&w)[B], int i)
{
    const uint32_t lo = win<B>(w, B * i);
    const uint32_t hi = win<B>(w, B * i + 16 * B - 16);
    return (lo & 0xFFFFu) | (hi & 0xFFFF0000u);
}

// (x & M) | 0x43004300 in one gfx950 three-input bitwise op.  Truth table 0xEA:
// output bit = (a & b) | c, indexed by (a << 2) | (b << 1) | c.
template <uint32_t M>
__device__ __forceinline__ uint32_t bits_or_magic(uint32_t x)
{
    static_assert((M & MOE_MAGIC_PAIR) == 0, "mask and magic overlap");
    return __builtin_amdgcn_bitop3_b32(x, M, MOE_MAGIC_PAIR, 0xEA);
}

// Float of byte N of t (the compiler emits v_cvt_f32_ubyteN).
template <int N>
__device__ __forceinline__ float ubyte_f32(uint32_t t)
{
    return (float)((t >> (8 * N)) & 0xFFu);
}

// Two bf16 values of the codes held at bits 0 and 16 of t (8-bit codes).
__device__ __forceinline__ uint32_t bytes02_to_bf16pair(uint32_t t)
{
    const float f0 = ubyte_f32<0>(t);
    const float f1 = ubyte_f32<2>(t);
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// All 16 P16 pairs of one unit, as bf16 pairs of (offset + code); width 16:
// pair i = (value i, value i + 16), halves of words i/2 and 8 + i/2.
template <int B>
__device__ __forceinline__ void unit_pairs(const uint32_t (&w)[B], uint32_t (&pr)[16])
{
    if constexpr (B == 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            pr[i] = __builtin_amdgcn_perm(w[8 + (i >> 1)], w[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
    } else {
        constexpr int S = Code<B>::per_t;
#pragma unroll
        for (int i = 0; i < 16; i += S) {
            const uint32_t t = pair_window<B>(w, i);
#pragma unroll
            for (int m = 0; m < S; ++m) {
                if (i + m < 16) {
                    const uint32_t tm = t >> (B * m);
                    if constexpr (B == 8)
                        pr[i + m] = bytes02_to_bf16pair(tm);
                    else
                        pr[i + m] = bits_or_magic<Code<B>::mask2>(tm);
                }
            }
        }
    }
}

// DPP lane moves within rows of 16 (gfx9 encodings): 0xB1 quad xor 1, 0x4E quad
// xor 2, 0x141 half-row mirror (lane i <-> 7-i), 0x140 row mirror (i <-> 15-i).
// A lane whose source lies outside its row reads 0; no caller uses such a lane's
// result.  (No old value to keep, so the move folds into the instruction that
// uses it: one v_add_f32_dpp instead of a copy, a move and an add.)
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v + (the same register of lane i ^ 16), resp. i ^ 32, via the gfx950 swaps.
__device__ __forceinline__ float xor16_add(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_add(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned segments of W lanes (W a power of two <= 64); every lane of a
// segment gets the same sum (each step adds a lane to its partner, and the
// partner adds the same two values).  DPP and lane swaps, no LDS traffic.
template <int W>
__device__ __forceinline__ float seg_sum_w(float v)
{
    if constexpr (W >= 2) v += dpp_move<0xB1>(v);
    if constexpr (W >= 4) v += dpp_move<0x4E>(v);
    if constexpr (W >= 8) v += dpp_move<0x141>(v);
    if constexpr (W >= 16) v += dpp_move<0x140>(v);
    if constexpr (W >= 32) v = xor16_add(v);
    if constexpr (W >= 64) v = xor32_add(v);
    return v;
}

__device__ __forceinline__ float seg_sum(float v, int width)
{
    switch (width) {
    case 1: return v;
    case 2: return seg_sum_w<2>(v);
    case 4: return seg_sum_w<4>(v);
    case 8: return seg_sum_w<8>(v);
    case 16: return seg_sum_w<16>(v);
    case 32: return seg_sum_w<32>(v);
    default: return seg_sum_w<64>(v);
    }
}

// silu(g) * u = g / (1 + e^-g) * u, with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Sums of a, b, c, d over the 64 lanes of a wave, as one transposed reduction:
// at the i^32 step a lane keeps two of its four values and trades the other two
// with its partner, at the i^16 step one of two, then a sum within rows of 16.
// On return lanes 0-15 hold sum(a), 16-31 sum(b), 32-47 sum(c), 48-63 sum(d).
__device__ __forceinline__ float wave_sum4(float a, float b, float c, float d, int lane)
{
    const bool lo = lane < 32;
    const float x = lo ? c : a, y = lo ? d : b;  // the values this lane hands over
    const auto rx = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const auto ry = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    const float v0 = (lo ? a : c) + __uint_as_float(lo ? rx[1] : rx[0]);
    const float v1 = (lo ? b : d) + __uint_as_float(lo ? ry[1] : ry[0]);
    const bool even = (lane & 16) == 0;
    const float z = even ? v1 : v0;
    const auto rz = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
    const float w = (even ? v0 : v1) + __uint_as_float(even ? rz[1] : rz[0]);
    return seg_sum_w<16>(w);
}

// Position of input c (0..31) of a chunk in the P16 activation layout.
__device__ __forceinline__ int p16_pos(int c) { return ((c & 15) << 1) | (c >> 4); }

}  // namespace moe
