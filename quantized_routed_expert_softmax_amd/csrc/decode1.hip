// decode1.hip — the routed-expert layer for ONE token in one launch on gfx950,
// laid out for the shortest critical path: route -> request every weight row ->
// gate/up + SwiGLU -> h exchange -> down -> weighted combine.
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", Motivation
// (each token reads only its k routed experts) and How the prototype works
// (gated, concatenated, untransposed experts without bias, each layer mapping
// expert ids to slots; a fully resident model runs without host round trips);
// "POC: Experts offload", commit messages (queued GPU work must not idle
// between a layer's steps).
//
// A decode layer moves ~14 MB (10 experts of 1.38 MB at 3 bits): ~2 us of HBM
// time against ~1 us per dependent memory round trip, so the kernel is shaped
// by its dependency chain, not by arithmetic.  One workgroup of W waves per
// compute unit:
//   1. one round of loads shared through LDS: the router logits and the slot
//      table (list wave j takes experts 64 j .. 64 j + 63 and sorts its 16
//      largest logit keys), x, and the workgroup's call-tag counter;
//   2. every wave merges the eight lists itself and checks that the top k by
//      logit is the contract's top k (a gap of at least 2^-9 between the k-th
//      and (k+1)-th logit, the k-th within 64 of the largest); then hit h is
//      routing position h and its slot comes from the table, with no further
//      barrier.  Otherwise (near-ties, non-finite logits, or given ids) wave 0
//      runs the contract's own routine and builds the hit list in id order
//      while the others wait;
//   3. each wave then requests ALL its weight rows: its phase-1 item(s) (rows
//      n, n+16 of gate and of up of one expert) and its phase-2 rows (the
//      workgroup's output rows of down for its own expert(s)), so the layer's
//      bytes are in flight from the first microsecond of streaming;
//   4. phase 1: SwiGLU pairs published as 64-bit (h pair, call tag) words;
//   5. one wave then computes the routing weights (they need Z over all logits;
//      nothing before the final combine uses them, and computing them before
//      its phase-1 item would delay words that every consumer waits for);
//   6. phase 2: a wave polls only its own expert's h words (first one word that
//      a workgroup's last item slot writes, with pauses, then all of them),
//      stages them in its own LDS, computes its rows
//      of down and weights them; partial sums meet in LDS and become the bf16
//      output rows, summed over the hits in ascending expert id (fixed order,
//      the same whichever routing order the hits were numbered in).
// Measured on MI355X (in-kernel timestamps, median over workgroups, from the
// first workgroup's start): routing done 1.9 us, rows requested 2.3 us, phase 1
// done 3.9-5.3 us (the third wave on a SIMD finishes last: 10 items on 4 SIMDs,
// ~0.6 us of VALU work each), h complete 7.2 us, end 8.4 us; plus ~1.4 us from
// the previous kernel's end to this one's start.  (Taken before the poll read a
// last-slot word first, which moved the end about 0.4 us earlier.)
// All workgroups are co-resident (one per compute unit, occupancy checked on the
// host), so every polled word is eventually written; the poll is bounded and
// reports MOE_ERRW_TIMEOUT instead of hanging.
//
// Call tags, the h words and the expert -> word layout follow the reserved
// workspace region shared with decode.hip (counters at kGenBase; all counters
// equal between calls; tag = counter + 1, never 0).
#pragma clang fp contract(off)

#include "../../include/moe.h"
#include "moe_dev.h"
#include "decode_dev.h"
#include "moe_internal.h"
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kD1MaxK = 16;   // routed experts per token on this path
// Per variant: MI phase-1 items per wave, MH phase-2 experts per wave and ML
// phase-2 row loads per expert and wave at most (registers are sized for them).

struct D1Params {
    const float* logits;    // route in-kernel when not null
    const int32_t* ids_in;  // else the routing comes from here
    const float* w_in;
    int32_t* ids_out;  // routing result (workgroup 0, may be null)
    float* w_out;
    int E, k, I;
    const uint16_t* x;
    const int32_t* table;
    const uint8_t* pool;
    int64_t n_slots, slot_bytes, off_gu_codes, off_gu_sb, off_d_codes, off_d_sb;
    uint16_t* out;
    uint32_t* gen;
    uint64_t* xw;
    uint32_t* err;
    int rows_per_wg;  // output rows per workgroup (a multiple of 64 / LPRD)
    int ipw;          // phase-1 items per workgroup: ceil(k * I/2 / grid)
    unsigned spin_limit;
};

__device__ __forceinline__ void d1_flag(uint32_t* err, uint32_t bit)
{
    if (err) atomicOr(err, bit);
}

// Maximum of an unsigned value over the wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    v = max(v, swap16_u32(v));
    return max(v, swap32_u32(v));
}

// value of lane (i & 63), register i >> 6, of eight per-lane registers (i wave-uniform)
__device__ __forceinline__ uint32_t pick8(const uint32_t (&r)[8], int i)
{
    uint32_t v = r[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
        if ((i >> 6) == j) v = r[j];
    return (uint32_t)__builtin_amdgcn_readlane((int)v, i & 63);
}

// value of lane (i & 63), register i >> 6, for a per-lane index i
__device__ __forceinline__ uint32_t gather8(const uint32_t (&r)[8], int i)
{
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t g = (uint32_t)__builtin_amdgcn_ds_bpermute((i & 63) << 2, (int)r[j]);
        v = (i >> 6) == j ? g : v;
    }
    return v;
}

// Sort eight keys descending (a 19-comparator network).
__device__ __forceinline__ void sort8_desc(uint32_t (&k)[8])
{
#define MOE_CE(a, b)                                          \
    {                                                         \
        const uint32_t hi_ = max(k[a], k[b]), lo_ = min(k[a], k[b]); \
        k[a] = hi_;                                           \
        k[b] = lo_;                                           \
    }
    MOE_CE(0, 2) MOE_CE(1, 3) MOE_CE(4, 6) MOE_CE(5, 7)
    MOE_CE(0, 4) MOE_CE(1, 5) MOE_CE(2, 6) MOE_CE(3, 7)
    MOE_CE(0, 1) MOE_CE(2, 3) MOE_CE(4, 5) MOE_CE(6, 7)
    MOE_CE(2, 4) MOE_CE(3, 5)
    MOE_CE(1, 4) MOE_CE(3, 6)
    MOE_CE(1, 2) MOE_CE(3, 4) MOE_CE(5, 6)
#undef MOE_CE
}

// P16 pairs of 32 bf16 values held as 16 consecutive words (value 2m, 2m+1 in
// word m): pair i = (value i, value i + 16).
__device__ __forceinline__ void p16_from_words(const uint32_t (&w)[16], uint32_t (&pr)[16])
{
#pragma unroll
    for (int i = 0; i < 16; ++i)
        pr[i] = __builtin_amdgcn_perm(w[8 + (i >> 1)], w[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
}

// One lane's unit of one row against P16 activations xp with unit sum xs:
// s * sum x (off + c) + (z - off s) * sum x, or the plain dot for width 16.
template <int B>
__device__ __forceinline__ float unit_dot(const uint32_t (&w)[B], uint32_t sb, const uint32_t (&xp)[16], float xs)
{
    uint32_t cp[16];
    unit_pairs<B>(w, cp);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = dot2(cp[i], xp[i], acc);
    if constexpr (Code<B>::affine) {
        constexpr float off = Code<B>::offset;
        const float s = half_bits_to_f32(sb & 0xFFFFu);
        const float z = __builtin_fmaf(-off, s, half_bits_to_f32(sb >> 16));
        return __builtin_fmaf(s, acc, z * xs);
    } else {
        return acc;
    }
}

template <int B>
struct Unit {
    uint32_t w[B];
    uint32_t sb;
};

template <int B>
__device__ __forceinline__ void load_unit1(Unit<B>& u, const uint8_t* __restrict__ base, uint32_t codes, uint32_t sb)
{
    load_unit<B>(u.w, (const uint32_t*)(base + codes));
    if constexpr (Code<B>::affine) u.sb = *(const uint32_t*)(base + sb);
    else u.sb = 0u;
}

template <int BG, int BD, int LPRD, int UD, int W, int MI, int MH, int ML>
__global__ __launch_bounds__(64 * W) void decode1_kernel(D1Params P)
{
    static_assert(W >= 8, "eight list waves route 512 logits");
    constexpr int RPL = 64 / LPRD;          // down rows per wave load
    constexpr int H = 2048;
    __shared__ uint32_t s_x[H / 2];         // x as bf16 pairs, in order
    __shared__ float s_logit[512];
    __shared__ int32_t s_table[512];
    __shared__ uint32_t s_list[8][16];      // per list wave: its 16 largest keys, descending
    __shared__ int s_bad[8];
    __shared__ uint32_t s_h[W][512];        // h of the wave's current expert (P16, layout swz)
    __shared__ float s_hs[W][32];           // its unit sums
    __shared__ float s_y[MH][W][64];        // down rows of each wave's experts
    __shared__ float s_hw[kD1MaxK];         // weight of each hit
    __shared__ int32_t s_hslot[kD1MaxK];    // slot of each hit, -1 not resident (slow path)
    __shared__ int32_t s_ord[kD1MaxK];      // hits by ascending expert id
    __shared__ int s_nhit;
    __shared__ float s_sel[kD1MaxK];        // routing: p by position
    __shared__ RouteScratch s_rsc[1];       // routing fallback (wave 0)
    __shared__ int32_t s_fid[1][32];
    __shared__ float s_fw[1][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform
    const int G = gridDim.x;
    const int E = P.E, k = P.k, I = P.I;
    const bool wg0 = blockIdx.x == 0;
    const int nl = (E + 63) >> 6;  // list waves

    // ---- 1. one round of loads, shared through LDS ----
    const uint32_t gen0 = __hip_atomic_load(&P.gen[kGenBase + blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    {
        const int e = wave * 64 + lane;
        const bool on = wave < nl && e < E;
        const int32_t tb = wave < nl ? P.table[e < E ? e : E - 1] : 0;
        const float l = (P.logits && wave < nl) ? P.logits[e < E ? e : E - 1] : 0.0f;
        uint4 xv = {0u, 0u, 0u, 0u};
        const int t = (int)threadIdx.x;
        if (t < H / 8) xv = ((const uint4*)P.x)[t];
        if (on) s_table[e] = tb;
        if (t < H / 8) *(uint4*)&s_x[4 * t] = xv;
        if (P.logits && wave < nl) {
            // the wave's 16 largest keys by logit (keys order like logits; the low
            // 9 bits carry 511 - id, so keys are distinct)
            if (on) s_logit[e] = l;
            const bool bad = __any(on && !isfinite(l));
            uint32_t K = on ? logit_key32(l, e) : kPadKey32;
            K = row_sort_u32(K, lane);
            K = row_merge_u32(K, swap16_u32(K), lane);
            K = row_merge_u32(K, swap32_u32(K), lane);
            if (lane < 16) s_list[wave][lane] = K;
            if (lane == 0) s_bad[wave] = bad ? 1 : 0;
        }
    }
    __syncthreads();
    uint32_t tag = gen0 + 1u;
    if (tag == 0u) tag = 1u;

    // ---- 2. routing ----
    // Every wave merges the eight lists and takes the gap test itself (same
    // inputs, same result in every wave), so on the usual path no wave waits for
    // another before requesting its rows.  Lanes < k: the expert of pair `lane`
    // (idv), its weight when given or from the fallback (wv, wave 0), its hit
    // index (hidx) and whether it is the first pair of its expert (first).
    int32_t idv = 0;
    float wv = 0.0f;
    bool fast = false, nonfinite = false, first = false;
    int hidx = 0;
    if (P.logits) {
        int nb = 0;
        for (int i = 0; i < nl; ++i) nb |= s_bad[i];
        if (nb) {
            nonfinite = true;
        } else {
            const int r = lane >> 4;
            const uint32_t A = r < nl ? s_list[r][lane & 15] : kPadKey32;
            const uint32_t Bv = r + 4 < nl ? s_list[r + 4][lane & 15] : kPadKey32;
            uint32_t K = row_merge_u32(A, Bv, lane);
            K = row_merge_u32(K, swap16_u32(K), lane);
            K = row_merge_u32(K, swap32_u32(K), lane);  // lanes 0-15: the 16 largest keys
            const uint32_t c0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)K);
            const uint32_t c_last = (uint32_t)__builtin_amdgcn_readlane((int)K, k - 1);
            const uint32_t c_next = (uint32_t)__builtin_amdgcn_readlane((int)K, k);
            const float m_hi = order_bits_logit(c0 | 0x1ffu);        // >= the largest logit
            const float lo_in = order_bits_logit(c_last & ~0x1ffu);  // <= every chosen logit
            const float hi_out = c_next == kPadKey32 ? -INFINITY : order_bits_logit(c_next | 0x1ffu);
            fast = lo_in - m_hi >= -64.0f && lo_in - hi_out >= 0x1p-9f;
            idv = key32_id(K);
        }
    }
    // slots: on the fast path lane h of every wave holds hit h's slot (hit h =
    // routing position h: the k ids are distinct and in range), else s_hslot
    int32_t hsl = -1;
    int n_hit = k;
    if (fast) {
        if (lane < k) {
            const int32_t sl = s_table[idv];
            const bool res = sl >= 0 && sl < P.n_slots;
            if (!res && wg0 && wave == 0) d1_flag(P.err, sl < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
            hsl = res ? sl : -1;
        }
        first = lane < k;
        hidx = lane;  // s_ord puts the hits in id order after phase 1
    } else {
        // wave 0 routes with the contract's own routine (near-ties at the
        // boundary, the k-th logit far below the largest, or a non-finite logit)
        // or takes the given routing, and builds the hit list; the others wait
        if (wave == 0) {
            if (P.logits) {
                if (nonfinite) {
                    idv = lane;  // ids 0..k-1 with weight 0 (the token's result is discarded)
                } else {
                    route_token_512(s_logit, E, k, MOE_ROUTE_PLAIN, 0.0f, nullptr, lane, s_fid[0], s_fw[0],
                                    &s_rsc[0]);
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    idv = lane < k ? s_fid[0][lane] : 0;
                    wv = lane < k ? s_fw[0][lane] : 0.0f;
                }
            } else if (lane < k) {
                idv = P.ids_in[lane];
                wv = P.w_in[lane];
            }
            // hit list: distinct ids ascending (pairs with an id outside [0, E)
            // dropped); hit index = distinct ids below this one
            const bool valid = lane < k && idv >= 0 && idv < E;
            if (lane < k && !valid && wg0) d1_flag(P.err, MOE_ERRW_BAD_ID);
            int dup = 0;
#pragma unroll 1
            for (int q = 0; q < k; ++q) {
                const int o = __builtin_amdgcn_readlane(idv, q);
                dup += (o == idv && q < lane) ? 1 : 0;
            }
            first = valid && dup == 0;
            const unsigned long long fm = __ballot(first);
#pragma unroll 1
            for (int q = 0; q < k; ++q) {
                const int o = __builtin_amdgcn_readlane(idv, q);
                hidx += (((fm >> q) & 1ull) && o < idv) ? 1 : 0;
            }
            if (first) {
                const int32_t sl = s_table[idv];
                const bool res = sl >= 0 && sl < P.n_slots;
                if (!res && wg0) d1_flag(P.err, sl < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
                s_hslot[hidx] = res ? sl : -1;
            }
            if (lane == 0) s_nhit = __popcll(fm);
            if (lane < k) s_ord[lane] = lane;  // hits already ascending
        }
        __syncthreads();
        n_hit = s_nhit;
    }

    // ---- 3. every weight row this wave needs, requested now ----
    // phase-1 items: (hit, pair p) over n_hit * I/2 items, P.ipw per workgroup
    // (sized for k hits; with repeated ids the last workgroups idle); wave w
    // takes the workgroup's items w, w + W
    const int half_i = I >> 1;
    const int n_items = n_hit * half_i;
    const int ipw = P.ipw;
    Unit<BG> gu[MI][4];
    int it_hit[MI], it_p[MI], it_slot[MI];
    const uint32_t g_row_b = (uint32_t)(H * BG / 8), g_sb_b = (uint32_t)(H / 16);
#pragma unroll
    for (int q = 0; q < MI; ++q) {
        const int li = wave + W * q;
        const int it = blockIdx.x * ipw + li;
        const bool on = li < ipw && it < n_items;
        const int h = on ? udiv(it, half_i) : 0;
        it_hit[q] = on ? h : -1;
        it_p[q] = on ? it - h * half_i : 0;
        it_slot[q] = !on ? -1 : fast ? __builtin_amdgcn_readlane(hsl, h) : s_hslot[h];
        if (it_slot[q] >= 0) {
            const uint8_t* base = P.pool + (size_t)it_slot[q] * (size_t)P.slot_bytes;
            const uint32_t n0 = (uint32_t)pair_row(2 * it_p[q]);
            const uint32_t rows[4] = {n0, n0 + 16u, (uint32_t)I + n0, (uint32_t)I + n0 + 16u};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                load_unit1<BG>(gu[q][r], base,
                               (uint32_t)P.off_gu_codes + rows[r] * g_row_b + (uint32_t)lane * (uint32_t)(4 * BG),
                               (uint32_t)P.off_gu_sb + rows[r] * g_sb_b + (uint32_t)(lane >> 1) * 4u);
        }
    }
    // phase 2: this workgroup's output rows of down, for hits wave, wave + W
    const int row0 = blockIdx.x * P.rows_per_wg;
    const int n_ld = P.rows_per_wg / RPL;  // row loads per hit
    const int seg = lane & (LPRD - 1), rl = lane / LPRD;
    const uint32_t d_row_b = (uint32_t)(I * BD / 8), d_sb_b = (uint32_t)(I / 16);
    RowLoad<BD, UD> dr[MH][ML];
    int hs_slot[MH];
    // bf16 experts (a layer of ~63 MB, bound by bandwidth rather than by round
    // trips): a wave requests its down rows only once its gate/up rows are in, so
    // the bytes phase 1 waits for are not shared with bytes only phase 2 needs
    constexpr bool late_down = (BG == 16);
#define MOE_D1_REQUEST_DOWN                                                                   \
    for (int q = 0; q < MH; ++q) {                                                            \
        const int h = wave + W * q;                                                           \
        hs_slot[q] = h >= n_hit ? -1 : fast ? __builtin_amdgcn_readlane(hsl, h) : s_hslot[h]; \
        if (hs_slot[q] >= 0) {                                                                \
            const uint8_t* base = P.pool + (size_t)hs_slot[q] * (size_t)P.slot_bytes;         \
            _Pragma("unroll") for (int ld = 0; ld < ML; ++ld) {                               \
                const int row = row0 + ld * RPL + rl;                                         \
                if (ld < n_ld && row < H)                                                     \
                    load_row<BD, UD>(dr[q][ld], base, (uint32_t)P.off_d_codes + (uint32_t)row * d_row_b, \
                                     (uint32_t)P.off_d_sb + (uint32_t)row * d_sb_b, seg, LPRD);  \
            }                                                                                 \
        }                                                                                     \
    }
    if constexpr (late_down) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's gate/up rows are in
#pragma unroll
    MOE_D1_REQUEST_DOWN
#undef MOE_D1_REQUEST_DOWN

    // ---- 4. phase 1: gate/up + SwiGLU -> tagged h pair words ----
    const uint64_t tag_hi = (uint64_t)tag << 32;
    if (it_hit[0] >= 0) {
        uint32_t xw16[16], xp[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 v = *(const uint4*)&s_x[16 * lane + 4 * c];
            xw16[4 * c] = v.x;
            xw16[4 * c + 1] = v.y;
            xw16[4 * c + 2] = v.z;
            xw16[4 * c + 3] = v.w;
        }
        p16_from_words(xw16, xp);
        float xsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) xsum = dot2(xp[i], MOE_ONES_PAIR, xsum);
#pragma unroll
        for (int q = 0; q < MI; ++q) {
            if (it_hit[q] < 0) continue;
            uint64_t word = tag_hi;  // not resident: zeros, so readers are not kept waiting
            if (it_slot[q] >= 0) {
                const float g0 = unit_dot<BG>(gu[q][0].w, gu[q][0].sb, xp, xsum);
                const float g1 = unit_dot<BG>(gu[q][1].w, gu[q][1].sb, xp, xsum);
                const float u0 = unit_dot<BG>(gu[q][2].w, gu[q][2].sb, xp, xsum);
                const float u1 = unit_dot<BG>(gu[q][3].w, gu[q][3].sb, xp, xsum);
                // lanes 0-15: g0, 16-31: g1, 32-47: u0, 48-63: u1; the i^32 swap
                // brings u next to g
                const float sm = wave_sum4(g0, g1, u0, u1, lane);
                const auto ru = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm), __float_as_uint(sm), false, false);
                const uint32_t hh = f32_to_bf16(silu_mul(sm, __uint_as_float(ru[1])));
                const uint32_t h0 = (uint32_t)__builtin_amdgcn_readlane((int)hh, 0);
                const uint32_t h1 = (uint32_t)__builtin_amdgcn_readlane((int)hh, 16);
                word = tag_hi | h0 | (h1 << 16);
            }
            if (lane == 0)
                __hip_atomic_store(&P.xw[(size_t)it_hit[q] * half_i + it_p[q]], word, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- 5. routing weights, after the wave's phase-1 items (nothing before the
    // final combine needs them; computed earlier they would hold up phase 1,
    // which every expert's consumers wait for).  On the fast path every wave has
    // the routing, and wave 2 takes it: its SIMD runs two waves, not three; the
    // slow path's routing lives in wave 0 ----
    if (wave == (fast ? 2 : 0)) {
        if (P.logits && fast) {
            // m and Z of the contract over every logit, p of the chosen, ordered by
            // (p desc, id asc), weights = p / (their sum in that order)
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = lane + 64 * j < E ? s_logit[lane + 64 * j] : -INFINITY;
            float m = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
            m = wave_max_f(m);
            const float Z = route_sel_z(v, E, m);
            const float lx = lane < k ? s_logit[idv] : 0.0f;
            const float p = lane < k ? __fdiv_rn(exp_contract_nb(lx - m), Z) : 0.0f;
            int pos = 0;
#pragma unroll 1
            for (int q = 0; q < k; ++q) {
                const float po = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), q));
                const int io = __builtin_amdgcn_readlane(idv, q);
                pos += (po > p || (po == p && io < idv)) ? 1 : 0;
            }
            if (lane < k) s_sel[pos] = p;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            float ssum = 0.0f;
            for (int q = 0; q < k; ++q) ssum = ssum + s_sel[q];
            wv = lane < k ? __fdiv_rn(p, ssum) : 0.0f;
            if (wg0 && lane < k && P.ids_out) {
                P.ids_out[pos] = idv;
                P.w_out[pos] = wv;
            }
        } else if (P.logits) {
            if (nonfinite && wg0 && lane == 0) d1_flag(P.err, MOE_ERRW_NONFINITE);
            if (wg0 && lane < k && P.ids_out) {  // fallback or non-finite: already in contract order
                P.ids_out[lane] = idv;
                P.w_out[lane] = wv;
            }
        }
        if (fast) {
            // one pair per hit; hits in id order for the combine
            if (lane < k) s_hw[lane] = wv;
            int rank = 0;
#pragma unroll 1
            for (int q = 0; q < k; ++q) rank += __builtin_amdgcn_readlane(idv, q) < idv ? 1 : 0;
            if (lane < k) s_ord[rank] = lane;
        } else if (first) {
            // weight of each hit: the weights of its pairs, in pair order
            float ws = 0.0f;
            for (int q = 0; q < k; ++q) {
                const int o = __builtin_amdgcn_readlane(idv, q);
                const float wo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), q));
                if (o == idv) ws = ws + wo;
            }
            s_hw[hidx] = ws;
        }
    }

    // ---- 6. phase 2: own experts' h, down rows ----
    const int Ud = I >> 5;
#pragma unroll
    for (int q = 0; q < MH; ++q) {
        const int h = wave + W * q;
        if (h >= n_hit) continue;
        if (hs_slot[q] < 0) {  // not resident (flagged): contributes zeros
#pragma unroll
            for (int ld = 0; ld < ML; ++ld)
                if (ld < n_ld && seg == 0) s_y[q][wave][ld * RPL + rl] = 0.0f;
            continue;
        }
        // poll the expert's I/2 words.  While its producers are still at work, one
        // word is read, with a pause between reads (every wave of the grid polls at
        // once, and full-width polls compete with the weight streams); once it is
        // fresh, lane l takes words l, l + 64, ...  The word read first is one that
        // a workgroup's last item slot writes (item ipw - 1 of its workgroup: the
        // third wave on its SIMD, which finishes phase 1 last), so when it is fresh
        // the others mostly are too (-0.4 us per layer against the middle word).
        const uint64_t* src = P.xw + (size_t)h * half_i;
        {
            unsigned spins = 0;
            const int pw = min((ipw - 1 - (h * half_i) % ipw) % ipw, half_i - 1);
            while ((uint32_t)(__hip_atomic_load(src + pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) !=
                   tag) {
                if (++spins > P.spin_limit) break;  // the full poll below reports the timeout
                __builtin_amdgcn_s_sleep(2);
            }
        }
        for (int w0 = 0; w0 < half_i; w0 += 256) {
            uint64_t hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int wi = w0 + lane + 64 * r;
                hv[r] = wi < half_i ? __hip_atomic_load(src + wi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tag_hi;
            }
            unsigned spins = 0;
            for (;;) {
                bool ready = true;
#pragma unroll
                for (int r = 0; r < 4; ++r) ready = ready && (uint32_t)(hv[r] >> 32) == tag;
                if (__all(ready)) break;
                if (++spins > P.spin_limit) {
                    d1_flag(P.err, MOE_ERRW_TIMEOUT);
                    break;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int wi = w0 + lane + 64 * r;
                    if (wi < half_i && (uint32_t)(hv[r] >> 32) != tag)
                        hv[r] = __hip_atomic_load(src + wi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int wi = w0 + lane + 64 * r;
                if (wi < half_i) s_h[wave][swz(wi >> 4, wi & 15)] = (uint32_t)hv[r];
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        if (lane < Ud) s_hs[wave][lane] = unit_sum(s_h[wave], lane);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int ld = 0; ld < ML; ++ld) {
            if (ld >= n_ld) continue;
            float y = row_dot_raw<BD, UD>(dr[q][ld], s_h[wave], s_hs[wave], seg, LPRD);
            y = seg_sum_w<LPRD>(y);
            if (seg == 0) s_y[q][wave][ld * RPL + rl] = y;
        }
    }
    __syncthreads();
    // the next call's counters: b, b + G, ... (every wave has read counter b)
    for (int j = blockIdx.x + G * (int)threadIdx.x; j < kMaxGrid; j += G * 64 * W)
        __hip_atomic_store(&P.gen[kGenBase + j], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // out[row] = sum over hits (ascending expert id) of weight * y, in fp32
    if ((int)threadIdx.x < P.rows_per_wg) {
        const int row = row0 + (int)threadIdx.x;
        if (row < H) {
            float o = 0.0f;
            for (int r = 0; r < n_hit; ++r) {
                const int h = s_ord[r];
                const int q = h / W, w = h - q * W;
                o = __builtin_fmaf(s_hw[h], s_y[q][w][threadIdx.x], o);
            }
            P.out[row] = f32_to_bf16(o);
        }
    }
}

struct D1Variant {
    int bg, bd, lprd, ud, w, mi, mh, ml;
    hipError_t (*launch)(const D1Params&, int, hipStream_t);
    int (*occ)();
};

template <int BG, int BD, int LPRD, int UD, int W, int MI, int MH, int ML>
hipError_t d1_launch(const D1Params& P, int G, hipStream_t s)
{
    hipLaunchKernelGGL((decode1_kernel<BG, BD, LPRD, UD, W, MI, MH, ML>), dim3(G), dim3(64 * W), 0, s, P);
    return hipGetLastError();
}

template <int BG, int BD, int LPRD, int UD, int W, int MI, int MH, int ML>
int d1_occ()
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode1_kernel<BG, BD, LPRD, UD, W, MI, MH, ML>, 64 * W,
                                                     0) != hipSuccess)
        return 0;
    return nb;
}

#define MOE_D1(BG, BD, LPRD, UD, W, MI, MH, ML)                                    \
    {BG, BD, LPRD, UD, W, MI, MH, ML, d1_launch<BG, BD, LPRD, UD, W, MI, MH, ML>, \
     d1_occ<BG, BD, LPRD, UD, W, MI, MH, ML>}
const D1Variant kD1Variants[] = {
    MOE_D1(3, 3, 16, 1, 10, 2, 2, 4),  // hidden 2048, intermediate 512, 3-bit
    MOE_D1(4, 4, 16, 1, 10, 2, 2, 4),
    MOE_D1(8, 8, 16, 1, 10, 2, 2, 4),
    MOE_D1(4, 4, 8, 3, 8, 2, 2, 4),    // hidden 2048, intermediate 768, 4-bit
    MOE_D1(4, 6, 8, 3, 8, 2, 2, 4),    // ... with 6-bit down
    MOE_D1(16, 16, 16, 1, 10, 1, 1, 2),  // bf16 experts, intermediate 512: one item, expert and two down loads per wave
};
#undef MOE_D1

int d1_cus()
{
    static thread_local int cached_dev = -1, cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev != cached_dev) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 0;
        cus = p.multiProcessorCount;
        cached_dev = dev;
    }
    return cus;
}

// Lanes per down row and units per lane for I / 32 units.
void d1_lanes(int units, int* lprd, int* ud)
{
    int l = units & -units;
    if (l > 64) l = 64;
    *lprd = l;
    *ud = units / l;
}

const D1Variant* d1_find(const ClassView& c)
{
    int lprd, ud;
    d1_lanes(c.I / 32, &lprd, &ud);
    for (const D1Variant& v : kD1Variants)
        if (v.bg == c.bits_gu && v.bd == c.bits_d && v.lprd == lprd && v.ud == ud) return &v;
    return nullptr;
}

// Grid and rows: one workgroup per compute unit (at most H / rows-per-load),
// rows per workgroup a multiple of the rows one load covers.
bool d1_grid(const ClassView& c, const D1Variant* v, int* G, int* rows_per_wg)
{
    const int cus = d1_cus();
    if (cus <= 0) return false;
    const int rpl = 64 / v->lprd;
    const int n_rg = c.H / rpl;
    int g = n_rg < cus ? n_rg : cus;
    if (g > kMaxGrid) g = kMaxGrid;
    const int rows = ((n_rg + g - 1) / g) * rpl;
    if (rows / rpl > v->ml || rows > 64) return false;
    *G = g;
    *rows_per_wg = rows;
    return true;
}

}  // namespace

bool decode1_supported(int T, int k, int E, int mode, bool routes, const ClassView& c)
{
    if (T != 1 || mode != MOE_ROUTE_PLAIN) return false;
    if (E < 1 || E > 512 || k < 1 || k > kD1MaxK || k > E) return false;
    if (routes && k > kD1MaxK - 1) return false;  // the (k+1)-th of the 16 merged keys is needed
    if (c.H != 2048 || c.I < 64 || c.I > 1024 || c.I % 64) return false;
    if (c.slot_bytes >= ((int64_t)1 << 31)) return false;
    const D1Variant* v = d1_find(c);
    if (!v) return false;
    int G, rows;
    if (!d1_grid(c, v, &G, &rows)) return false;
    // phase-1 items and phase-2 experts per wave within the kernel's limits
    const int64_t items = (int64_t)k * (c.I / 2);
    if ((items + G - 1) / G > (int64_t)v->mi * v->w) return false;
    if ((k + v->w - 1) / v->w > v->mh) return false;
    if ((int64_t)k * (c.I / 2) > MOE_WS_XWORDS) return false;
    return v->occ() >= 1;
}

hipError_t launch_decode1(const float* logits, const int32_t* ids_in, const float* w_in, int32_t* ids_out,
                          float* w_out, int E, int k, const uint16_t* x, const int32_t* table,
                          const uint8_t* pool, const ClassView& c, uint16_t* out, void* reserved,
                          uint32_t* err, hipStream_t s)
{
    const D1Variant* v = d1_find(c);
    if (!v) return hipErrorInvalidValue;
    int G, rows;
    if (!d1_grid(c, v, &G, &rows)) return hipErrorInvalidConfiguration;
    D1Params P;
    P.logits = logits;
    P.ids_in = ids_in;
    P.w_in = w_in;
    P.ids_out = ids_out;
    P.w_out = w_out;
    P.E = E;
    P.k = k;
    P.I = c.I;
    P.x = x;
    P.table = table;
    P.pool = pool;
    P.n_slots = c.n_slots;
    P.slot_bytes = c.slot_bytes;
    P.off_gu_codes = c.off_gu_codes;
    P.off_gu_sb = c.off_gu_sb;
    P.off_d_codes = c.off_d_codes;
    P.off_d_sb = c.off_d_sb;
    P.out = out;
    P.gen = (uint32_t*)reserved;
    P.xw = (uint64_t*)((uint8_t*)reserved + MOE_WS_GEN_BYTES);
    P.err = err;
    P.rows_per_wg = rows;
    P.ipw = (int)(((int64_t)k * (c.I / 2) + G - 1) / G);
    P.spin_limit = 1u << 20;
    return v->launch(P, G, s);
}

}  // namespace moe
