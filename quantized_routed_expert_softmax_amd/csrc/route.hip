// route.hip — router kernel: one wavefront per token (see route_dev.h).
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", Motivation
// (softmax top-k routing); BigMoeOnEdge commit message adding cache-aware
// substitution.
#pragma clang fp contract(off)

#include "../../include/moe.h"
#include "moe_internal.h"
#include "route_dev.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int mode, float L,
                                                         const int32_t* __restrict__ table,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ wout,
                                                         uint32_t* __restrict__ err)
{
    __shared__ RouteScratch sc[4];
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wave
    const bool ok = route_token(logits + (size_t)t * E, E, k, mode, L, table, lane,
                                ids + (size_t)t * k, wout + (size_t)t * k, &sc[threadIdx.x >> 6]);
    if (!ok && lane == 0 && err) atomicOr(err, MOE_ERRW_NONFINITE);
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
