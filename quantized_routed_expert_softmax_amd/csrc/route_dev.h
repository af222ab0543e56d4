// route_dev.h — one wavefront routes one token: softmax over E router logits,
// top-k, renormalised weights, optional cache-aware substitution.
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", Motivation
// (each token uses k of E experts; only the top-k are read); BigMoeOnEdge commit
// message adding cache-aware substitution (cached experts get a bonus of L x
// (max - min of the token's scores), the k winners are picked again from the
// adjusted scores, and k experts still run).
//
// The arithmetic follows the routing numeric contract of include/moe.h
// operation by operation: no contraction (this header must be compiled under
// `#pragma clang fp contract(off)`), explicit fma, correctly rounded division,
// fixed summation tree.  Lane l holds experts l, l+64, ... (E <= 1024).
#pragma once
#include <math.h>

#include "../../include/moe.h"
#include "moe_dev.h"

namespace moe {

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

// exp_contract without a branch, so that independent calls interleave: the same
// arithmetic for x >= -86 (the clamp does not touch those), 0 below.  For
// finite x only (a NaN gives a finite value here).
__device__ __forceinline__ float exp_contract_nb(float x)
{
    const float xc = fmaxf(x, -87.0f);
    const float n = __builtin_rintf(xc * 1.44269502f);
    float r = __builtin_fmaf(-n, __uint_as_float(0x3f317218u), xc);
    r = __builtin_fmaf(-n, __uint_as_float(0xb102e308u), r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float y = p * __uint_as_float((uint32_t)((int)n + 127) << 23);
    return x < -86.0f ? 0.0f : y;
}

// Max / min over the wave, every lane gets the result: DPP moves within rows of
// 16 (quad xor 1, quad xor 2, half-row mirror, row mirror), then the gfx950 row
// swaps for lane i ^ 16 and i ^ 32 (each swap returns the lane's own value and
// its partner's, in some order).  No LDS traffic.
__device__ __forceinline__ float wave_max_f(float v)
{
    v = fmaxf(v, dpp_move<0xB1>(v));
    v = fmaxf(v, dpp_move<0x4E>(v));
    v = fmaxf(v, dpp_move<0x141>(v));
    v = fmaxf(v, dpp_move<0x140>(v));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_min_f(float v)
{
    v = fminf(v, dpp_move<0xB1>(v));
    v = fminf(v, dpp_move<0x4E>(v));
    v = fminf(v, dpp_move<0x141>(v));
    v = fminf(v, dpp_move<0x140>(v));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The fixed halving tree of the routing contract over one partial per lane:
// for off = 32, 16, ..., 1 lane l adds lane l + off; the result is lane 0's.
// Only lanes below off need a correct partner at each level: the row swaps
// bring lane l + 32 (l + 16) to lane l, DPP row shift left by n brings lane
// l + n within a row of 16.  Float addition is commutative, so operand order
// inside one add does not change the rounded sum.
__device__ __forceinline__ float tree_sum_lane0(float S)
{
    S = xor32_add(S);
    S = xor16_add(S);
    S = S + dpp_move<0x108>(S);
    S = S + dpp_move<0x104>(S);
    S = S + dpp_move<0x102>(S);
    S = S + dpp_move<0x101>(S);
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(S)));
}

// k-th largest (k = 1..64) of one value per lane: a bitonic network over the 64
// lanes sorts descending (lane 0 = largest), then lane k-1 is read.  Partner of
// lane l at distance s is lane l ^ s: quad DPP for s = 1, 2; two row shifts
// and a select for s = 4; row rotate by 8 for s = 8; the row swaps for 16, 32.
__device__ __forceinline__ float p4_partner(float v, int lane)
{
    const float up = dpp_move<0x114>(v);  // lane l - 4 (row shift right)
    const float dn = dpp_move<0x104>(v);  // lane l + 4 (row shift left)
    return (lane & 4) ? up : dn;
}

__device__ __forceinline__ float wave_kth_largest(float v, int k, int lane)
{
#define MOE_CX(PV, S, SIZE)                                                           \
    {                                                                                 \
        const float pv_ = (PV);                                                       \
        const float mx_ = fmaxf(v, pv_), mn_ = fminf(v, pv_);                         \
        const bool lo_ = (lane & (S)) == 0, dsc_ = (lane & (SIZE)) == 0;              \
        v = (lo_ == dsc_) ? mx_ : mn_;                                                \
    }
// both moves run with the full wave (a DPP source lane must be active), then select
#define MOE_P4(V) p4_partner(V, lane)
#define MOE_SW16(SIZE)                                                                \
    {                                                                                 \
        auto r_ = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false); \
        const float a_ = __uint_as_float(r_[0]), b_ = __uint_as_float(r_[1]);        \
        const bool lo_ = (lane & 16) == 0, dsc_ = (lane & (SIZE)) == 0;               \
        v = (lo_ == dsc_) ? fmaxf(a_, b_) : fminf(a_, b_);                            \
    }
#define MOE_SW32()                                                                    \
    {                                                                                 \
        auto r_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false); \
        const float a_ = __uint_as_float(r_[0]), b_ = __uint_as_float(r_[1]);        \
        v = (lane & 32) == 0 ? fmaxf(a_, b_) : fminf(a_, b_);                         \
    }
    MOE_CX(dpp_move<0xB1>(v), 1, 2)
    MOE_CX(dpp_move<0x4E>(v), 2, 4)
    MOE_CX(dpp_move<0xB1>(v), 1, 4)
    MOE_CX(MOE_P4(v), 4, 8)
    MOE_CX(dpp_move<0x4E>(v), 2, 8)
    MOE_CX(dpp_move<0xB1>(v), 1, 8)
    MOE_CX(dpp_move<0x128>(v), 8, 16)
    MOE_CX(MOE_P4(v), 4, 16)
    MOE_CX(dpp_move<0x4E>(v), 2, 16)
    MOE_CX(dpp_move<0xB1>(v), 1, 16)
    MOE_SW16(32)
    MOE_CX(dpp_move<0x128>(v), 8, 32)
    MOE_CX(MOE_P4(v), 4, 32)
    MOE_CX(dpp_move<0x4E>(v), 2, 32)
    MOE_CX(dpp_move<0xB1>(v), 1, 32)
    MOE_SW32()
    MOE_SW16(64)
    MOE_CX(dpp_move<0x128>(v), 8, 64)
    MOE_CX(MOE_P4(v), 4, 64)
    MOE_CX(dpp_move<0x4E>(v), 2, 64)
    MOE_CX(dpp_move<0xB1>(v), 1, 64)
#undef MOE_CX
#undef MOE_P4
#undef MOE_SW16
#undef MOE_SW32
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k - 1));
}

// DPP lane moves within rows of 16 (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// (key, id) precedes (ok, oi) in the selection order: larger key, then smaller id.
// Bitwise, not short-circuit: both operands are always evaluated, so the loads
// that feed them are never moved under a branch.
__device__ __forceinline__ bool precedes(float k, int i, float ok, int oi)
{
    return (k > ok) | ((k == ok) & (i < oi));
}

// Wave-wide first element in (key desc, id asc) order over one (key, id) per lane:
// DPP within rows of 16, then the four row winners through readlane.  Uniform.
__device__ __forceinline__ void wave_first(float& k, int& i)
{
#define MOE_STEP(CTRL)                                                                   \
    {                                                                                    \
        const float ok = dpp_f<CTRL>(k);                                                 \
        const int oi = dpp_i<CTRL>(i);                                                   \
        const bool b = precedes(ok, oi, k, i);                                           \
        k = b ? ok : k;                                                                  \
        i = b ? oi : i;                                                                  \
    }
    MOE_STEP(0xB1)
    MOE_STEP(0x4E)
    MOE_STEP(0x141)
    MOE_STEP(0x140)
#undef MOE_STEP
    float bk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k), 16 * r));
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (precedes(rk, ri, bk, bi)) {
            bk = rk;
            bi = ri;
        }
    }
    k = bk;
    i = bi;
}

// Route one token (called by all 64 lanes of a wave with the same arguments);
// MJ values per lane (E <= 64*MJ).  Writes ids[0..k) and w[0..k) from lanes
// 0..k-1.  Returns false if a logit is not finite (then ids = 0..k-1, w = 0).
//
// Top-k: each lane sorts its MJ (key, id, p) entries into selection order with a
// bitonic network, then k rounds pick the wave-wide first of the lane heads and
// the winning lane drops its head.  The order is total (key desc, id asc), so
// the result equals repeated argmax over all E experts.
// Per-wave LDS scratch of route_token: candidates and the chosen k.
struct alignas(16) RouteScratch {
    uint64_t ck[64];  // candidate order keys (order_key)
    float cp[64];     // candidate probabilities
    int sel_id[32];
    float sel_p[32];
};

// Candidate order key: selection keys are finite and >= 0, so their bit patterns
// order like their values; the low word ~id puts the smaller id first among
// equal keys.  A larger order key precedes a smaller one.
__device__ __forceinline__ uint64_t order_key(float key, int id)
{
    return ((uint64_t)__float_as_uint(key) << 32) | (uint32_t)~id;
}

// Rank the `total` (<= 64) candidates held in sc->ck/cp (one per lane) in the
// selection order (key desc, id asc), keep the first k, and write ids/w from
// lanes 0..k-1: w_r = p_r / (sum of the chosen p in rank order, left to right).
// One wave; the candidates must already be visible to it.
__device__ __forceinline__ void rank_select(RouteScratch* sc, int total, int k, int lane, int32_t* ids, float* w)
{
    const uint64_t mk = lane < total ? sc->ck[lane] : 0ull;
    const float mp = lane < total ? sc->cp[lane] : 0.0f;
    if (lane < 32) sc->sel_p[lane] = 0.0f;
    // rank = candidates ahead of this one (64-bit compares, two per LDS read)
    int rank = 0;
    for (int q = 0; q < total; q += 4) {
        const ulonglong2 a = *(const ulonglong2*)&sc->ck[q];
        const ulonglong2 b = *(const ulonglong2*)&sc->ck[q + 2];
        rank += (int)(a.x > mk);
        rank += (int)((q + 1 < total) & (a.y > mk));
        rank += (int)((q + 2 < total) & (b.x > mk));
        rank += (int)((q + 3 < total) & (b.y > mk));
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (lane < total && rank < k) {
        sc->sel_id[rank] = (int)~(uint32_t)mk;
        sc->sel_p[rank] = mp;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // renormalise: the chosen probabilities summed left to right (entries past k
    // are +0, which leaves a positive sum unchanged)
    float s = 0.0f;
    for (int r = 0; r < k; r += 8) {
        const float4 a = *(const float4*)&sc->sel_p[r];
        const float4 b = *(const float4*)&sc->sel_p[r + 4];
        s = s + a.x;
        s = s + a.y;
        s = s + a.z;
        s = s + a.w;
        s = s + b.x;
        s = s + b.y;
        s = s + b.z;
        s = s + b.w;
    }
    if (lane < k) {
        ids[lane] = sc->sel_id[lane];
        w[lane] = __fdiv_rn(sc->sel_p[lane], s);
    }
}

template <int MJ>
__device__ __attribute__((noinline)) bool route_token_t(const float* __restrict__ lr, int E, int k, int mode,
                                              float L, const int32_t* __restrict__ table, int lane,
                                              int32_t* ids, float* w, RouteScratch* sc)
{
    float v[MJ];
    bool bad = false;
    float m = -INFINITY;
    // every load is issued before any is used (no branch around a load)
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
        const int i = lane + 64 * j;
        v[j] = lr[i < E ? i : E - 1];
    }
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
        const int i = lane + 64 * j;
        if (i < E) {
            bad |= !isfinite(v[j]);
            m = fmaxf(m, v[j]);
        } else {
            v[j] = -INFINITY;
        }
    }
    if (__any(bad)) {
        if (lane < k) {
            ids[lane] = lane;
            w[lane] = 0.0f;
        }
        return false;
    }
    m = wave_max_f(m);

    // e_i, lane partial sums in ascending order, then the fixed halving tree
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
        const int i = lane + 64 * j;
        v[j] = (i < E) ? exp_contract(v[j] - m) : 0.0f;
        S = S + v[j];
    }
    const float Z = tree_sum_lane0(S);

    // probabilities and selection keys (invalid entries: key -inf, never chosen)
    float key[MJ];
    int id[MJ];
    float pmax = -INFINITY, pmin = INFINITY;
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
        const int i = lane + 64 * j;
        if (i < E) {
            v[j] = __fdiv_rn(v[j], Z);
            pmax = fmaxf(pmax, v[j]);
            pmin = fminf(pmin, v[j]);
        }
        key[j] = (i < E) ? v[j] : -INFINITY;
        id[j] = i;
    }
    if (mode == MOE_ROUTE_SUBST) {
        int res[MJ];
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            const int i = lane + 64 * j;
            res[j] = table[i < E ? i : E - 1];
        }
        pmax = wave_max_f(pmax);
        pmin = wave_min_f(pmin);
        const float range = pmax - pmin;
        const float c = L * range;
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            const int i = lane + 64 * j;
            if (i < E && res[j] >= 0) key[j] = v[j] + c;
        }
    }

    // ---- fast path: bound the k-th element by the k-th largest lane head ----
    // The k lane heads that lead the selection order are k distinct elements, so
    // the k-th chosen element is at least the k-th largest head key tau: every
    // element with key < tau is out.  Candidates = valid elements with key >= tau
    // (a superset of the answer); each candidate's rank among candidates is its
    // global rank.  Falls back to k rounds when there are more than 64.
    {
        float hk = -INFINITY;
        int hid = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < MJ; ++j)
            if (precedes(key[j], id[j], hk, hid)) {
                hk = key[j];
                hid = id[j];
            }
        const float tau = wave_kth_largest(hk, k, lane);
        unsigned long long cm[MJ];
        int total = 0;
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            cm[j] = __ballot(key[j] >= tau);  // invalid entries have key -inf
            total += __popcll(cm[j]);
        }
        if (total <= 64) {
            int base = 0;
#pragma unroll
            for (int j = 0; j < MJ; ++j) {
                if ((cm[j] >> lane) & 1ull) {
                    const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(cm[j] >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)cm[j], 0u));
                    sc->ck[pos] = order_key(key[j], id[j]);
                    sc->cp[pos] = v[j];
                }
                base += __popcll(cm[j]);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            rank_select(sc, total, k, lane, ids, w);
            return true;
        }
    }

    // ---- fallback: per-lane bitonic sort into selection order (position 0 = first) ----
#pragma unroll
    for (int size = 2; size <= MJ; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
            for (int a = 0; a < MJ; ++a) {
                const int b = a ^ stride;
                if (b > a) {
                    // ascending selection order in runs whose (a & size) == 0
                    const bool up = (a & size) == 0;
                    const bool bfirst = precedes(key[b], id[b], key[a], id[a]);
                    if (bfirst == up) {
                        const float tk = key[a], tp = v[a];
                        const int ti = id[a];
                        key[a] = key[b];
                        id[a] = id[b];
                        v[a] = v[b];
                        key[b] = tk;
                        id[b] = ti;
                        v[b] = tp;
                    }
                }
            }
        }
    }

    // k rounds over the lane heads
    int my_id = 0;
    float my_p = 0.0f;
    for (int r = 0; r < k; ++r) {
        float bk = key[0];
        int bi = id[0];
        wave_first(bk, bi);
        const int wl = bi & 63;
        const float bp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[0]), wl));
        if (lane == r) {
            my_id = bi;
            my_p = bp;
        }
        if (lane == wl) {
#pragma unroll
            for (int j = 0; j + 1 < MJ; ++j) {
                key[j] = key[j + 1];
                id[j] = id[j + 1];
                v[j] = v[j + 1];
            }
            key[MJ - 1] = -INFINITY;
            id[MJ - 1] = 0x7fffffff;
        }
    }
    // renormalise over the chosen k, summed left to right
    float s = 0.0f;
    for (int r = 0; r < k; ++r) s = s + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_p), r));
    if (lane < k) {
        ids[lane] = my_id;
        w[lane] = __fdiv_rn(my_p, s);
    }
    return true;
}

// E <= 512 only (callers that hold many registers across the call).
__device__ __forceinline__ bool route_token_512(const float* __restrict__ lr, int E, int k, int mode,
                                                float L, const int32_t* __restrict__ table, int lane,
                                                int32_t* ids, float* w, RouteScratch* sc)
{
    if (E <= 128) return route_token_t<2>(lr, E, k, mode, L, table, lane, ids, w, sc);
    if (E <= 256) return route_token_t<4>(lr, E, k, mode, L, table, lane, ids, w, sc);
    return route_token_t<8>(lr, E, k, mode, L, table, lane, ids, w, sc);
}

// LDS scratch of route_token_wg for W waves.
template <int W>
struct alignas(16) RouteWgScratch {
    float top[64 + 4];  // per-wave top keys (wave w: [w*r, w*r + r)), padded for vector reads
    float red[3][W];    // per-wave max of the logits, max and min of p
    int bad[W];
    float tau;
    int count;          // candidates placed so far
    float v[64 * W];    // e_i by expert
};

// Route one token with all W waves of a workgroup (64 <= E <= min(512, 64*W)): lane l of
// wave w holds expert 64w + l.  Every thread of the workgroup calls it with the
// same arguments (it contains workgroup barriers); ids/w are written by wave 0.
// The arithmetic is the single-wave routine's, step for step: exact max; the
// same exp; lane partials S_l = sum over j ascending of e_{l+64j}, then the same
// halving tree; correctly rounded p; the same keys and selection order.  Only the
// candidate threshold is found differently: each of the Wf = E/64 full waves
// lists its r largest keys, r = ceil(k/Wf); these are Wf*r >= k keys of distinct
// experts, so their k-th largest, tau, is at most the k-th largest key overall
// and every chosen expert has key >= tau.  Candidates (key >= tau) are ranked
// by (key desc, id asc), which does not depend on the order they were stored in.
template <int W>
__device__ bool route_token_wg(const float* __restrict__ lr, int E, int k, int mode, float L,
                               const int32_t* __restrict__ table, int32_t* ids, float* w,
                               RouteScratch* sc0, RouteWgScratch<W>* ws)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = wave * 64 + lane;
    const bool valid = e < E;
    const float l = valid ? lr[e] : -INFINITY;
    const bool bad = valid && !isfinite(l);
    const float mw = wave_max_f(l);
    const bool anybad = __any(bad);
    if (lane == 0) {
        ws->red[0][wave] = mw;
        ws->bad[wave] = anybad ? 1 : 0;
    }
    __syncthreads();
    float m = -INFINITY;
    int nb = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        m = fmaxf(m, ws->red[0][i]);
        nb |= ws->bad[i];
    }
    if (nb) {
        if (wave == 0 && lane < k) {
            ids[lane] = lane;
            w[lane] = 0.0f;
        }
        return false;
    }
    const float v = valid ? exp_contract(l - m) : 0.0f;
    ws->v[e] = v;
    __syncthreads();
    const int nj = (E + 63) >> 6;
    float S = 0.0f;
    for (int j = 0; j < nj; ++j) S = S + ws->v[lane + 64 * j];
    const float Z = tree_sum_lane0(S);
    const float p = valid ? __fdiv_rn(v, Z) : 0.0f;
    float key = valid ? p : -INFINITY;
    if (mode == MOE_ROUTE_SUBST) {
        const float pmx = wave_max_f(valid ? p : -INFINITY);
        const float pmn = wave_min_f(valid ? p : INFINITY);
        if (lane == 0) {
            ws->red[1][wave] = pmx;
            ws->red[2][wave] = pmn;
        }
        __syncthreads();
        float pmax = -INFINITY, pmin = INFINITY;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            pmax = fmaxf(pmax, ws->red[1][i]);
            pmin = fminf(pmin, ws->red[2][i]);
        }
        const float range = pmax - pmin;
        const float c = L * range;
        if (valid && table[e] >= 0) key = p + c;
    }
    // each full wave lists its r largest keys (r rounds: wave max, drop one lane holding it)
    const int wf = E >> 6;
    const int r = (k + wf - 1) / wf;
    const int nt = wf * r;  // <= k + wf - 1 <= 39
    if (wave < wf) {
        float x = key;
        for (int i = 0; i < r; ++i) {
            const float mx = wave_max_f(x);
            if (lane == 0) ws->top[wave * r + i] = mx;
            const unsigned long long at = __ballot(x == mx);
            if (lane == __ffsll((long long)at) - 1) x = -INFINITY;
        }
    }
    __syncthreads();
    // tau = k-th largest of the listed keys (equal keys ranked by list position)
    if (wave == 0) {
        const float tv = lane < nt ? ws->top[lane] : -INFINITY;
        int rank = 0;
        for (int q = 0; q < nt; q += 4) {
            const float4 t4 = *(const float4*)&ws->top[q];
            rank += (int)((t4.x > tv) | ((t4.x == tv) & (q < lane)));
            rank += (int)((q + 1 < nt) & ((t4.y > tv) | ((t4.y == tv) & (q + 1 < lane))));
            rank += (int)((q + 2 < nt) & ((t4.z > tv) | ((t4.z == tv) & (q + 2 < lane))));
            rank += (int)((q + 3 < nt) & ((t4.w > tv) | ((t4.w == tv) & (q + 3 < lane))));
        }
        if (lane < nt && rank == k - 1) ws->tau = tv;
        if (lane == 0) ws->count = 0;
    }
    __syncthreads();
    const float tau = ws->tau;
    const bool cand = valid && key >= tau;
    const unsigned long long cm = __ballot(cand);
    int base = 0;
    if (cm) {
        if (lane == 0) base = atomicAdd(&ws->count, __popcll(cm));
        base = __builtin_amdgcn_readfirstlane(base);
        const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
        if (cand && pos < 64) {
            sc0->ck[pos] = order_key(key, e);
            sc0->cp[pos] = p;
        }
    }
    __syncthreads();
    const int total = ws->count;
    if (wave == 0) {
        if (total > 64) return route_token_512(lr, E, k, mode, L, table, lane, ids, w, sc0);
        rank_select(sc0, total, k, lane, ids, w);
    }
    return true;
}

// ---------------------------------------------------------------------------
// Plain-mode workgroup routing by logit order (64 <= E <= 512, k <= 15).
//
// p_i is a function of logit_i alone once m and Z are fixed, and that function
// rises with the logit except within rounding: if l_a < l_b - 2^-10 and
// l_b - m >= -64, the contract's arithmetic gives p_a < p_b.  (The rounded
// l - m is within 2^-18 of the exact difference for |l - m| < 128; exp_c is
// within a few ulp of e^x; e^(-2^-10 + 2^-17) < 1 - 2^-11, far more than those
// errors, and dividing both by the same Z keeps a gap of 2^-11 relative, far
// more than one ulp of a normal p.)  So when every logit outside a set of k
// experts is at least 2^-9 below every logit inside it, and those are at least
// m - 64, the set holds exactly the k experts of largest p, whatever the ties
// elsewhere; their order is then taken from their exact p (ties: smaller id
// first).  Otherwise (near-ties at the boundary, far underflow) the token is
// routed by the single-wave routine.  Either way the result is the contract's.
//
// The set is found on 32-bit keys: the logit's bits mapped to an unsigned
// integer that orders like the value, its low 9 bits replaced by 511 - id, so
// keys are distinct and a key bounds its logit to a bucket of 512 neighbouring
// floats.  Waves 0..nl-1 (nl = ceil(E/64)) each sort their 64 keys (bitonic,
// lane moves and min/max) and list their 16 largest; wave zw computes m and Z
// meanwhile.  After one barrier wave zw merges the lists into the 16 largest
// keys overall, c_0 > c_1 > ...; the chosen set is c_0..c_(k-1), every other
// logit is at most the top of c_k's bucket, every chosen one at least the
// bottom of c_(k-1)'s, and the test above is made on those two bounds.
// ---------------------------------------------------------------------------
struct alignas(16) RouteSelScratch {
    uint32_t list[2][8][16];  // per token parity: per wave its 16 largest keys, descending
    int bad[2][8];            // per token parity: wave saw a non-finite logit
};

__device__ __forceinline__ uint32_t logit_order_bits(float l)
{
    const uint32_t u = __float_as_uint(l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// inverse of logit_order_bits
__device__ __forceinline__ float order_bits_logit(uint32_t v)
{
    return __uint_as_float((v & 0x80000000u) ? (v & 0x7fffffffu) : ~v);
}
__device__ __forceinline__ uint32_t logit_key32(float l, int id)
{
    return (logit_order_bits(l) & ~0x1ffu) | (uint32_t)(0x1ff - id);
}
constexpr uint32_t kPadKey32 = 0u;  // below every logit's key

// (every lane reads a lane of its own row for the moves used with it, except the
// row shifts of xor4_u32, whose out-of-row lanes are not selected)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
// lane i ^ 4 within a row: row shift right by 4 (lane i - 4) or left by 4 (lane i + 4)
__device__ __forceinline__ uint32_t xor4_u32(uint32_t v, int lane)
{
    const uint32_t up = dpp_u32<0x114>(v), dn = dpp_u32<0x104>(v);
    return (lane & 4) ? up : dn;
}
// lane i ^ 16 resp. i ^ 32: each swap returns this lane's value and its partner's
// in some order, so the partner's is their xor with this lane's
__device__ __forceinline__ uint32_t swap16_u32(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return r[0] ^ r[1] ^ v;
}
__device__ __forceinline__ uint32_t swap32_u32(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] ^ r[1] ^ v;
}

// One compare-exchange of a sorting network: the larger of this lane's key and
// its partner's when keep_max, else the smaller.
__device__ __forceinline__ uint32_t cx_u32(uint32_t own, uint32_t partner, bool keep_max)
{
    const uint32_t mx = own > partner ? own : partner, mn = own < partner ? own : partner;
    return keep_max ? mx : mn;
}

// A row of 16 lanes holding a bitonic sequence -> sorted descending.
__device__ __forceinline__ uint32_t row_clean_u32(uint32_t K, int lane)
{
    K = cx_u32(K, dpp_u32<0x128>(K), (lane & 8) == 0);  // row rotate by 8 = lane i ^ 8
    K = cx_u32(K, xor4_u32(K, lane), (lane & 4) == 0);
    K = cx_u32(K, dpp_u32<0x4E>(K), (lane & 2) == 0);
    K = cx_u32(K, dpp_u32<0xB1>(K), (lane & 1) == 0);
    return K;
}

// Every row of 16 lanes sorted descending: blocks of 2, 4, 8, 16 in turn, each
// merged from its two sorted halves by comparing lane i with its mirror in the
// block (the halves become bitonic) and cleaning the halves.
__device__ __forceinline__ uint32_t row_sort_u32(uint32_t K, int lane)
{
    K = cx_u32(K, dpp_u32<0xB1>(K), (lane & 1) == 0);   // blocks of 2
    K = cx_u32(K, dpp_u32<0x1B>(K), (lane & 2) == 0);   // blocks of 4: quad mirror
    K = cx_u32(K, dpp_u32<0xB1>(K), (lane & 1) == 0);
    K = cx_u32(K, dpp_u32<0x141>(K), (lane & 4) == 0);  // blocks of 8: half-row mirror
    K = cx_u32(K, dpp_u32<0x4E>(K), (lane & 2) == 0);
    K = cx_u32(K, dpp_u32<0xB1>(K), (lane & 1) == 0);
    K = cx_u32(K, dpp_u32<0x140>(K), (lane & 8) == 0);  // the row: row mirror
    K = cx_u32(K, xor4_u32(K, lane), (lane & 4) == 0);
    K = cx_u32(K, dpp_u32<0x4E>(K), (lane & 2) == 0);
    K = cx_u32(K, dpp_u32<0xB1>(K), (lane & 1) == 0);
    return K;
}

// Rows holding descending runs A (this row) and B (`other`, the partner row's
// run brought to this row): the 16 largest of both, descending.  max(A_i,
// B_(15-i)) is those 16 as a bitonic sequence.
__device__ __forceinline__ uint32_t row_merge_u32(uint32_t K, uint32_t other, int lane)
{
    const uint32_t b = dpp_u32<0x140>(other);
    return row_clean_u32(K > b ? K : b, lane);
}

// The wave of route_token_sel that computes m and Z and writes the result, and
// the list (experts 64 L .. 64 L + 63) each wave sorts, -1 for none.  With a
// spare wave the result wave is nl - 1 and list nl - 1 moves to wave nl: waves
// go to the four SIMDs round-robin, so the result wave shares its SIMD with one
// list wave instead of two (W = 10, nl = 8: SIMD 3 holds waves 3 and 7).
template <int W>
__device__ __forceinline__ int route_sel_wave(int E)
{
    const int nl = (E + 63) >> 6;
    return nl < W ? nl - 1 : 0;
}
template <int W>
__device__ __forceinline__ int route_sel_list(int wave, int E)
{
    const int nl = (E + 63) >> 6;
    if (nl >= W) return wave < nl ? wave : -1;
    return wave < nl - 1 ? wave : (wave == nl ? nl - 1 : -1);
}

// Before the barrier: the list waves list their 16 largest keys (own = this
// thread's logit, expert 64 * route_sel_list + lane); wave zw computes m and Z
// from v[j] = logit of expert lane + 64j (entries past E ignored).  No barrier
// inside.
// Z of the routing contract from v[j] = logit of expert lane + 64j (entries at
// or past E ignored) and the largest logit m.  (A non-finite logit makes the
// token's result be discarded, so the branch-free exp may see only finite values
// that matter; -inf gives 0.)
__device__ __forceinline__ float route_sel_z(const float (&v)[8], int E, float m)
{
    const int lane = threadIdx.x & 63;
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = lane + 64 * j < E ? exp_contract_nb(v[j] - m) : 0.0f;
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) S = S + e[j];
    return tree_sum_lane0(S);
}

template <int W>
__device__ __forceinline__ void route_sel_lists(float own, const float (&v_in)[8], int E, RouteSelScratch* rs,
                                                int par, float& m, float& Z)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = route_sel_list<W>(wave, E);
    if (li >= 0) {
        const int e = li * 64 + lane;
        const bool valid = e < E;
        const float l = valid ? own : 0.0f;
        const bool bad = __any(valid && !isfinite(l));
        uint32_t K = valid ? logit_key32(l, e) : kPadKey32;
        K = row_sort_u32(K, lane);
        K = row_merge_u32(K, swap16_u32(K), lane);  // rows 0 and 2: 16 largest of rows 0-1, 2-3
        K = row_merge_u32(K, swap32_u32(K), lane);  // row 0: 16 largest of the wave
        if (lane < 16) rs->list[par][li][lane] = K;
        if (lane == 0) rs->bad[par][li] = bad ? 1 : 0;
    }
    m = -INFINITY;
    Z = 0.0f;
    if (wave == route_sel_wave<W>(E)) {
        // m and Z exactly as the single-wave routine: lane l holds experts l + 64j
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = lane + 64 * j < E ? v_in[j] : -INFINITY;
        m = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
        m = wave_max_f(m);
        Z = route_sel_z(v, E, m);
    }
}

// After the barrier that follows route_sel_lists (lists and logits lr in LDS),
// in two steps.
//
// route_sel_choose: every thread returns false if a logit is not finite (wave
// zw then writes ids 0..k-1 with weight 0 to ids / w), else true.  Wave zw merges
// the lists; if the gap test holds, K holds the 16 largest keys in lanes 0..15
// (the chosen set: lanes 0..k-1) and *by_key = false; otherwise the token is
// routed by key now (ids / w written) and *by_key = true.  The chosen set is
// final after this step; only its order and weights come from route_sel_weights.
template <int W>
__device__ __forceinline__ bool route_sel_choose(const float* __restrict__ lr, int E, int k, float m, int32_t* ids,
                                                 float* w, RouteScratch* sc, RouteSelScratch* rs, int par,
                                                 uint32_t& K, bool& by_key)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nl = (E + 63) >> 6;
    const int zw = route_sel_wave<W>(E);
    by_key = true;
    K = kPadKey32;
    int nb = 0;
    for (int i = 0; i < nl; ++i) nb |= rs->bad[par][i];
    if (nb) {
        if (wave == zw && lane < k) {
            ids[lane] = lane;
            w[lane] = 0.0f;
        }
        return false;
    }
    if (wave != zw) return true;

    // merge the lists: lists 0-3 in rows 0-3, lists 4-7 under them
    const int r = lane >> 4;
    const uint32_t A = r < nl ? rs->list[par][r][lane & 15] : kPadKey32;
    const uint32_t Bv = r + 4 < nl ? rs->list[par][r + 4][lane & 15] : kPadKey32;
    K = row_merge_u32(A, Bv, lane);
    K = row_merge_u32(K, swap16_u32(K), lane);
    K = row_merge_u32(K, swap32_u32(K), lane);  // row 0: the 16 largest keys, descending

    const uint32_t c_last = (uint32_t)__builtin_amdgcn_readlane((int)K, k - 1);
    const uint32_t c_next = (uint32_t)__builtin_amdgcn_readlane((int)K, k);
    const float lo_in = order_bits_logit(c_last & ~0x1ffu);                         // every chosen logit >=
    const float hi_out = c_next == kPadKey32 ? -INFINITY : order_bits_logit(c_next | 0x1ffu);  // every other <=
    if (!(lo_in - m >= -64.0f && lo_in - hi_out >= 0x1p-9f)) {
        route_token_512(lr, E, k, MOE_ROUTE_PLAIN, 0.0f, nullptr, lane, ids, w, sc);
        return true;
    }
    by_key = false;
    return true;
}

// The expert of a chosen key (lanes 0..k-1 of wave zw after route_sel_choose).
__device__ __forceinline__ int key32_id(uint32_t K) { return 0x1ff - (int)(K & 0x1ffu); }

// Wave zw, by_key false: exact p of the chosen k, ordered by (p desc, id asc),
// weights p / (sum in that order, left to right); writes ids / w and returns
// this lane's expert in that order (lanes 0..k-1).
__device__ __forceinline__ int route_sel_weights(const float* __restrict__ lr, int k, float m, float Z, uint32_t K,
                                                 int32_t* ids, float* w)
{
    const int lane = threadIdx.x & 63;
    const int id = key32_id(K);
    const float lx = lane < k ? lr[id] : 0.0f;  // exact logit of a chosen expert
    const float p = lane < k ? __fdiv_rn(exp_contract_nb(lx - m), Z) : 0.0f;
    uint64_t P = lane < k ? (((uint64_t)__float_as_uint(p) << 32) | (uint32_t)~id) : 0ull;
    const uint64_t next = ((uint64_t)dpp_u32<0x101>((uint32_t)(P >> 32)) << 32) | dpp_u32<0x101>((uint32_t)P);
    if (__ballot(lane + 1 < k && !(P > next))) {
        // rare (p rounds equal or out of logit order): sort the 16 lanes of row 0
        // by (p, ~id) with the 64-bit keys, two words per step
#pragma unroll
        for (int st = 0; st < 16; ++st) {
            // odd-even transposition sort, 16 rounds over 16 lanes (row shifts by 1)
            const uint32_t dh = (st & 1) == (lane & 1) ? dpp_u32<0x101>((uint32_t)(P >> 32)) : dpp_u32<0x111>((uint32_t)(P >> 32));
            const uint32_t dl = (st & 1) == (lane & 1) ? dpp_u32<0x101>((uint32_t)P) : dpp_u32<0x111>((uint32_t)P);
            const uint64_t Q = ((uint64_t)dh << 32) | dl;
            const bool lower = (st & 1) == (lane & 1);  // this lane is the left one of its pair
            const bool edge = lower ? (lane & 15) == 15 : (lane & 15) == 0;
            if (!edge) P = lower ? (P > Q ? P : Q) : (P < Q ? P : Q);
        }
    }
    const float ps = __uint_as_float((uint32_t)(P >> 32));
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q)  // lanes past k hold p = +0, which leaves the sum unchanged
        s = s + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ps), q));
    const int out_id = (int)~(uint32_t)P;
    if (lane < k) {
        ids[lane] = out_id;
        w[lane] = __fdiv_rn(ps, s);
    }
    return out_id;
}

// Both steps at once: returns as route_sel_choose; wave zw writes ids / w.
template <int W>
__device__ __forceinline__ bool route_sel_finish(const float* __restrict__ lr, int E, int k, float m, float Z,
                                                 int32_t* ids, float* w, RouteScratch* sc, RouteSelScratch* rs,
                                                 int par)
{
    uint32_t K;
    bool by_key;
    const bool ok = route_sel_choose<W>(lr, E, k, m, ids, w, sc, rs, par, K, by_key);
    if (ok && (threadIdx.x >> 6) == route_sel_wave<W>(E) && !by_key) route_sel_weights(lr, k, m, Z, K, ids, w);
    return ok;
}

// One token by logit order with all W waves (logits lr in LDS); contains one barrier.
template <int W>
__device__ __forceinline__ bool route_token_sel(const float* __restrict__ lr, int E, int k, int32_t* ids, float* w,
                                                RouteScratch* sc, RouteSelScratch* rs, int par)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int i = lane + 64 * j;
        v[j] = lr[i < E ? i : E - 1];
    }
    const int li = route_sel_list<W>(wave, E);
    const int e = (li < 0 ? 0 : li) * 64 + lane;
    const float own = lr[e < E ? e : E - 1];
    float m, Z;
    route_sel_lists<W>(own, v, E, rs, par, m, Z);
    __syncthreads();
    return route_sel_finish<W>(lr, E, k, m, Z, ids, w, sc, rs, par);
}

__device__ __forceinline__ bool route_token(const float* __restrict__ lr, int E, int k, int mode,
                                            float L, const int32_t* __restrict__ table, int lane,
                                            int32_t* ids, float* w, RouteScratch* sc)
{
    if (E <= 128) return route_token_t<2>(lr, E, k, mode, L, table, lane, ids, w, sc);
    if (E <= 256) return route_token_t<4>(lr, E, k, mode, L, table, lane, ids, w, sc);
    if (E <= 512) return route_token_t<8>(lr, E, k, mode, L, table, lane, ids, w, sc);
    return route_token_t<16>(lr, E, k, mode, L, table, lane, ids, w, sc);
}

}  // namespace moe
