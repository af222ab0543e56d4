// route.hip — router softmax, top-k and renormalised weights, with the optional
// cache-aware substitution, on gfx950.
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", Motivation
// (each token uses k of E experts; only the top-k are read); BigMoeOnEdge commit
// message adding cache-aware substitution (every cached expert's score is
// raised by L times the token's score range, then top-k is taken again; the
// same number of experts runs).
//
// One wavefront per token; lane l holds logits l, l+64, ... (E <= 1024).  The
// arithmetic follows the routing numeric contract of include/moe.h operation by
// operation (no contraction, explicit fma, correctly rounded division, fixed
// summation tree), so ids and weights are bit-reproducible on any implementation
// of that contract.
#pragma clang fp contract(off)

#include <math.h>

#include "../../include/moe.h"
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxPerLane = 16;  // E <= 1024

// e^x for x <= 0: x = n ln2 + r (Cody-Waite, two-part ln2), e^r by its degree-7
// Taylor polynomial in Horner form, times 2^n through the exponent field.
__device__ __forceinline__ float exp_contract(float x)
{
    if (x < -86.0f) return 0.0f;
    const float n = __builtin_rintf(x * 1.44269502f);
    float r = __builtin_fmaf(-n, __uint_as_float(0x3f317218u), x);
    r = __builtin_fmaf(-n, __uint_as_float(0xb102e308u), r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int ni = (int)n;
    return p * __uint_as_float((uint32_t)(ni + 127) << 23);
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_min(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
    return v;
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int mode, float L,
                                                         const int32_t* __restrict__ table,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wout,
                                                         uint32_t* __restrict__ err)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wave
    const float* lr = logits + (size_t)t * E;

    float v[kMaxPerLane];
    bool bad = false;
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        const int i = lane + 64 * j;
        v[j] = -INFINITY;
        if (i < E) {
            v[j] = lr[i];
            bad |= !isfinite(v[j]);
            m = fmaxf(m, v[j]);
        }
    }
    if (__any(bad)) {
        if (lane == 0 && err) atomicOr(err, MOE_ERRW_NONFINITE);
        if (lane < k) {  // defined but meaningless output
            ids[(size_t)t * k + lane] = lane;
            wout[(size_t)t * k + lane] = 0.0f;
        }
        return;
    }
    m = wave_max(m);

    // e_i, lane partial sums in ascending order, then the fixed halving tree
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        const int i = lane + 64 * j;
        v[j] = (i < E) ? exp_contract(v[j] - m) : 0.0f;
        S = S + v[j];
    }
    for (int off = 32; off > 0; off >>= 1) S = S + __shfl_down(S, off, 64);
    const float Z = __shfl(S, 0, 64);

    // probabilities and selection keys
    float key[kMaxPerLane];
    float pmax = -INFINITY, pmin = INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        const int i = lane + 64 * j;
        if (i < E) {
            v[j] = __fdiv_rn(v[j], Z);
            pmax = fmaxf(pmax, v[j]);
            pmin = fminf(pmin, v[j]);
        }
        key[j] = (i < E) ? v[j] : -INFINITY;
    }
    if (mode == MOE_ROUTE_SUBST) {
        pmax = wave_max(pmax);
        pmin = wave_min(pmin);
        const float range = pmax - pmin;
        const float c = L * range;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            const int i = lane + 64 * j;
            if (i < E && table[i] >= 0) key[j] = v[j] + c;
        }
    }

    // top-k by repeated argmax: larger key first, equal keys -> smaller id
    int my_id = 0;
    float my_p = 0.0f;
    for (int r = 0; r < k; ++r) {
        float bk = -INFINITY;
        int bi = 0x7fffffff;
        float bp = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            if (key[j] > bk) {  // ascending j = ascending id within a lane
                bk = key[j];
                bi = lane + 64 * j;
                bp = v[j];
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const float ok = __shfl_xor(bk, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            const float op = __shfl_xor(bp, off, 64);
            if (ok > bk || (ok == bk && oi < bi)) {
                bk = ok;
                bi = oi;
                bp = op;
            }
        }
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (lane + 64 * j == bi) key[j] = -INFINITY;
        if (lane == r) {
            my_id = bi;
            my_p = bp;
        }
    }
    // renormalise over the chosen k, summed left to right
    float s = 0.0f;
    for (int r = 0; r < k; ++r) s = s + __shfl(my_p, r, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        wout[(size_t)t * k + lane] = __fdiv_rn(my_p, s);
    }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int mode, float L,
                        const int32_t* table, int32_t* ids, float* w, uint32_t* err, hipStream_t s)
{
    const int blocks = (T + 3) / 4;
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), 0, s, logits, T, E, k, mode, L,
                       table, ids, w, err);
    return hipGetLastError();
}

}  // namespace moe
