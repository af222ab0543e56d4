// route_dev.h — one wavefront routes one token: softmax over E router logits,
// top-k, renormalised weights, optional cache-aware substitution.
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", Motivation
// (each token uses k of E experts; only the top-k are read); BigMoeOnEdge commit
// message adding cache-aware substitution (every cached expert's score is
// raised by L times the token's score range, then top-k is taken again; the
// same number of experts runs).
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

__device__ __forceinline__ float wave_max_f(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_min_f(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
    return v;
}

// DPP lane moves within rows of 16 (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// (key, id) precedes (ok, oi) in the selection order: larger key, then smaller id.
__device__ __forceinline__ bool precedes(float k, int i, float ok, int oi)
{
    return k > ok || (k == ok && i < oi);
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
struct RouteScratch {
    float ck[64];
    int ci[64];
    float cp[64];
    int sel_id[32];
    float sel_p[32];
};

template <int MJ>
__device__ __forceinline__ bool route_token_t(const float* __restrict__ lr, int E, int k, int mode,
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
    for (int off = 32; off > 0; off >>= 1) S = S + __shfl_down(S, off, 64);
    const float Z = __shfl(S, 0, 64);

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
        const uint32_t hu = hk >= 0.0f ? __float_as_uint(hk) : 0u;  // keys are >= 0
        uint32_t prefix = 0;
        int need = k;
        for (int bit = 30; bit >= 0; --bit) {
            const uint32_t msk = 0xFFFFFFFFu << bit;
            const uint32_t want = prefix | (1u << bit);
            const int cnt = __popcll(__ballot((hu & msk) == want));
            if (cnt >= need) prefix = want;
            else need -= cnt;
        }
        const float tau = __uint_as_float(prefix);
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
                    sc->ck[pos] = key[j];
                    sc->ci[pos] = id[j];
                    sc->cp[pos] = v[j];
                }
                base += __popcll(cm[j]);
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            float mk = -INFINITY, mp = 0.0f;
            int mi = 0x7fffffff;
            if (lane < total) {
                mk = sc->ck[lane];
                mi = sc->ci[lane];
                mp = sc->cp[lane];
            }
            int rank = 0;
            for (int q = 0; q < total; ++q) {
                const float qk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mk), q));
                const int qi = __builtin_amdgcn_readlane(mi, q);
                rank += precedes(qk, qi, mk, mi) ? 1 : 0;
            }
            if (lane < total && rank < k) {
                sc->sel_id[rank] = mi;
                sc->sel_p[rank] = mp;
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            float s = 0.0f;
            for (int r = 0; r < k; ++r) s = s + sc->sel_p[r];
            if (lane < k) {
                ids[lane] = sc->sel_id[lane];
                w[lane] = __fdiv_rn(sc->sel_p[lane], s);
            }
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
