// router.hip — router logits of several consecutive layers from one hidden state,
// the input of the lookahead guesses: logits[m][t][e] = sum_i x[t][i] * Wr_m[e][i].
//
// Source: "RFC: stream MoE experts from disk in from_pretrained", How the
// prototype works, Reads bullet (the experts of the two following layers are
// predicted by applying their router weights to the present hidden state, and
// fetched while compute goes on).
//
// HBM-bound GEMV: the routers' bf16 rows are read once.  One wave owns one
// (layer, expert) row; its 64 lanes each load 16 bytes (8 values) per step along
// H, so a wave reads 1 KiB per step with fully coalesced loads, and keeps four
// tokens' partial sums in registers (tokens beyond four re-read the row from L2).
// bf16 x bf16 products are exact in fp32; sums are fp32.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTok = 4;

__device__ inline float lo16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float hi16(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ inline float dot8(const uint4& a, const float (&b)[8])
{
    float s = lo16(a.x) * b[0];
    s += hi16(a.x) * b[1];
    s += lo16(a.y) * b[2];
    s += hi16(a.y) * b[3];
    s += lo16(a.z) * b[4];
    s += hi16(a.z) * b[5];
    s += lo16(a.w) * b[6];
    s += hi16(a.w) * b[7];
    return s;
}

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                           const uint16_t* __restrict__ w, int E,
                                                           int n_rows, float* __restrict__ logits)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + wave;  // row = m * E + e
    if (row >= n_rows) return;              // whole wave; the kernel has no barrier
    const int m = row / E, e = row - m * E;
    const uint16_t* wr = w + (size_t)row * H;
    for (int t0 = 0; t0 < T; t0 += kTok) {
        const int nt = min(kTok, T - t0);
        float acc[kTok] = {0.f, 0.f, 0.f, 0.f};
        for (int i = lane * 8; i < H; i += 64 * 8) {
            const uint4 wv = *reinterpret_cast<const uint4*>(wr + i);
            const float wf[8] = {lo16(wv.x), hi16(wv.x), lo16(wv.y), hi16(wv.y),
                                 lo16(wv.z), hi16(wv.z), lo16(wv.w), hi16(wv.w)};
#pragma unroll
            for (int tt = 0; tt < kTok; ++tt)
                if (tt < nt)
                    acc[tt] += dot8(*reinterpret_cast<const uint4*>(x + (size_t)(t0 + tt) * H + i), wf);
        }
#pragma unroll
        for (int tt = 0; tt < kTok; ++tt)
            if (tt < nt) {
                const float s = wave_sum(acc[tt]);
                if (lane == 0) logits[((size_t)m * T + t0 + tt) * E + e] = s;
            }
    }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int n_mats, int E,
                                float* logits, hipStream_t s)
{
    const int rows = n_mats * E;
    router_logits_kernel<<<dim3((rows + 3) / 4), dim3(256), 0, s>>>(x, T, H, w, E, rows, logits);
    return hipGetLastError();
}

}  // namespace moe
