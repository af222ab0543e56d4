// convert.hip — one-time conversion of expert weights (fp32 or bf16) into slot
// rows of the size class's format.
//
// Source: "RFC: stream MoE experts from disk in from_pretrained", How the
// prototype works, Quantized experts bullet (an offline pass converts the
// experts to the affine quantized format and stores each one as a single
// contiguous row).  The pages give no rule for scale and bias; the one used
// here is min/max affine quantization per group of 64 inputs, stated in
// include/moe.h at moe_quantize_experts.
//
// One wave per (expert, matrix, row, group of 64): lane i holds input 64 g + i.
// Minimum and maximum are wave reductions; scale, bias and codes are computed
// in double (IEEE division, round-to-nearest-even `rint`); the codes of each
// pack unit (32 lanes, one half of the wave) are OR-reduced into its `bits`
// words, which lanes 0 .. bits - 1 of the half store.  A fill kernel zeroes
// the rows first, so the padding between blocks is zero.
#pragma clang fp contract(off)

#include "../../include/moe.h"
#include "moe_internal.h"
#include "moe_dev.h"

namespace moe {
namespace {

// Nearest fp16 pattern to x, ties to the even pattern: |x| is scaled by a power
// of two (exact) so that the fp16 spacing of its binade becomes 1, rounded once
// by rint, and the integer is the pattern's significand.  Finite input; results
// past the largest finite half (65504 plus half a spacing) are infinity.
__device__ uint16_t f64_to_f16_rne(double x)
{
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    const double a = fabs(x);
    if (!(a < 65520.0)) return sign | 0x7C00u;
    if (a < 0x1p-14) {  // subnormal binade: spacing 2^-24; 1024 is the smallest normal
        return sign | (uint16_t)rint(a * 0x1p24);
    }
    int e = ilogb(a);                      // -14 .. 15
    double m = rint(ldexp(a, 10 - e));     // 1024 .. 2048
    if (m == 2048.0) {
        m = 1024.0;
        ++e;
    }
    if (e > 15) return sign | 0x7C00u;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

__device__ double f16_bits_to_f64(uint16_t h) { return (double)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int o = 32; o; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

struct ConvArgs {
    const void* w_gu;      // [n, 2I, H]
    const void* w_d;       // [n, H, I]
    int bf16_in;
    int64_t n;
    int H, I, bits_gu, bits_d;
    int64_t off_gu_codes, off_gu_sb, off_d_codes, off_d_sb, slot_bytes;
    uint8_t* rows;
};

__global__ __launch_bounds__(256) void zero_rows_kernel(uint4* __restrict__ p, int64_t n16)
{
    const uint4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) p[i] = z;
}

__global__ __launch_bounds__(256) void convert_kernel(ConvArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t gu_items = (int64_t)2 * a.I * (a.H / 64);
    const int64_t d_items = (int64_t)a.H * (a.I / 64);
    const int64_t per_expert = gu_items + d_items;
    const int64_t total = a.n * per_expert;
    const int64_t waves = (int64_t)gridDim.x * 4;
    for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < total; it += waves) {
        const int64_t e = it / per_expert;
        int64_t rem = it - e * per_expert;
        const bool gu = rem < gu_items;
        if (!gu) rem -= gu_items;
        const int C = gu ? a.H : a.I;           // inputs per row
        const int R = gu ? 2 * a.I : a.H;       // rows of the matrix
        const int bits = gu ? a.bits_gu : a.bits_d;
        const int64_t r = rem / (C / 64);
        const int g = (int)(rem - r * (C / 64));
        const size_t src = ((size_t)e * R + (size_t)r) * (size_t)C + (size_t)g * 64 + lane;
        const void* wbase = gu ? a.w_gu : a.w_d;
        const float v = a.bf16_in ? __uint_as_float((uint32_t)((const uint16_t*)wbase)[src] << 16)
                                  : ((const float*)wbase)[src];
        uint8_t* row = a.rows + (size_t)e * (size_t)a.slot_bytes;
        uint8_t* codes = row + (gu ? a.off_gu_codes : a.off_d_codes) + (size_t)r * ((size_t)C * bits / 8);
        if (bits == 16) {  // 32 16-bit codes per unit in 16 words: the bf16 values in order
            ((uint16_t*)codes)[g * 64 + lane] = f32_to_bf16(v);
            continue;
        }
        const double qmax = (double)((1 << bits) - 1);
        const float lo = wave_min(v), hi = wave_max(v);
        const uint16_t s16 = f64_to_f16_rne(((double)hi - (double)lo) / qmax);
        const uint16_t z16 = f64_to_f16_rne((double)lo + 0.0);  // a zero minimum as +0
        const double s = f16_bits_to_f64(s16), z = f16_bits_to_f64(z16);
        uint32_t q = 0;
        if (s != 0.0) q = (uint32_t)fmin(fmax(rint(((double)v - z) / s), 0.0), qmax);
        // code of unit position i at bits [bits i, bits i + bits) of the unit
        const int t = bits * (lane & 31), wi = t >> 5, off = t & 31;
        const uint32_t part0 = q << off;
        const uint32_t part1 = (off + bits > 32) ? (q >> (32 - off)) : 0u;
        uint32_t mine = 0;
        for (int j = 0; j < bits; ++j) {
            uint32_t c = (wi == j ? part0 : 0u) | (wi + 1 == j ? part1 : 0u);
#pragma unroll
            for (int o = 16; o; o >>= 1) c |= __shfl_xor(c, o);  // stays within the 32-lane half
            if ((lane & 31) == j) mine = c;
        }
        if ((lane & 31) < bits) ((uint32_t*)codes)[(2 * g + (lane >> 5)) * bits + (lane & 31)] = mine;
        if (lane == 0) {
            uint32_t* sb = (uint32_t*)(row + (gu ? a.off_gu_sb : a.off_d_sb));
            sb[(size_t)r * (C / 64) + g] = (uint32_t)s16 | ((uint32_t)z16 << 16);
        }
    }
}

}  // namespace

hipError_t launch_convert(const void* w_gu, const void* w_d, int bf16_in, int64_t n, const ClassView& d,
                          void* rows, hipStream_t s)
{
    const int64_t n16 = n * d.slot_bytes / 16;
    const int64_t zb = std::min<int64_t>((n16 + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)zb), dim3(256), 0, s, (uint4*)rows, n16);
    ConvArgs a{w_gu, w_d, bf16_in, n, d.H, d.I, d.bits_gu, d.bits_d,
               d.off_gu_codes, d.off_gu_sb, d.off_d_codes, d.off_d_sb, d.slot_bytes, (uint8_t*)rows};
    const int64_t items = n * ((int64_t)2 * d.I * (d.H / 64) + (int64_t)d.H * (d.I / 64));
    const int64_t blocks = std::min<int64_t>((items + 3) / 4, 8192);
    hipLaunchKernelGGL(convert_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
