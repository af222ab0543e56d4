// decode.hip — the whole routed-expert layer for decode-sized batches in ONE
// persistent launch on gfx950: (route) -> sort by expert -> slot resolve ->
// gate/up dequant-GEMV + SwiGLU -> h exchange -> down dequant-GEMV -> weighted
// combine.
//
// Sources: "POC: Experts offload", PR description and commit messages (quantized
// experts through a gather quantized matmul on the device cache; the GPU should
// not idle between a layer's sub-steps); "RFC: stream MoE experts from disk in
// from_pretrained", How the prototype works (gated, concatenated, untransposed
// experts, no bias; each layer maps expert ids to slots; a fully resident model
// runs its layers without host round trips); BigMoeOnEdge commit message
// (cache-aware substitution, optional).
//
// Why one kernel: a decode layer moves ~14 MB (10 experts of 1.38 MB at 3 bits),
// about 2 us of HBM time, while every extra launch and every dependent global
// load costs ~1-5 us.  So each workgroup
//   1. stages router logits, the token rows and the slot table, routes (one wave
//      per token, identical arithmetic to the router kernel) and sorts the
//      <= 64 (token, j) pairs by expert in LDS -- redundantly in every
//      workgroup, which costs a few hundred cycles and saves a launch and a
//      global round trip;
//   2. looks up the hit experts' slots, then issues the loads of ALL its weight
//      rows at once (one vector load per pack unit): the gate/up rows of phase 1
//      and the down rows of phase 2 (the down weights do not depend on h, so
//      they stream in while gate/up computes);
//   3. phase 1: a wave owns gate rows n, n+16 (one P16 pair) and the matching
//      up rows of one hit expert (or, for short rows, several pairs side by
//      side); codes become bf16 pairs (128 + c) and bf16 dot2 sums them against
//      the P16 paired activations; per unit s*acc + (z - 128 s)*sum(x), with
//      sum(x) per unit computed once; h = silu(g)*u in bf16;
//   4. h exchange without a grid barrier: the wave publishes each h pair word
//      as one 64-bit relaxed atomic store of (pair, call tag) into the reserved
//      workspace region; readers poll each word until it carries this call's
//      tag.  A word holds its own proof of freshness, so no fence, flag or
//      central counter sits between the last producer and the consumers;
//   5. phase 2: h of all pairs is in LDS; wave w of a workgroup takes hits w,
//      w+8, ... for the workgroup's output rows and accumulates w_j*y per token;
//      the waves' partial sums are added in wave order, so the result is
//      bit-reproducible.
// All workgroups are co-resident (grid <= compute units, occupancy checked on
// the host), so every polled word is eventually written; the poll is bounded
// and reports MOE_ERRW_TIMEOUT instead of hanging.
//
// Call tags: each workgroup slot b < kMaxGrid has a counter in the reserved
// region.  All counters are equal between calls; workgroup b reads counter b,
// uses tag = counter + 1 (never 0, the value of a cleared region) and stores the
// tag into counters b, b+G, b+2G, ... of the next call right away (no other
// workgroup of this call reads them).  A word written by an earlier call carries
// an older tag, so it is never taken for this call's value.
#pragma clang fp contract(off)

#include "../../include/moe.h"
#include "moe_dev.h"
#include "moe_internal.h"
#include "decode_dev.h"
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kMaxPairs = 64;
constexpr int kMaxE = 1024;

struct DecodeParams {
    const float* logits;  // routing in-kernel when not null
    int mode;
    float L;
    const int32_t* ids_in;  // otherwise the routing comes from here
    const float* w_in;
    int32_t* ids_out;  // routing result (may be null; written by workgroup 0)
    float* w_out;
    int T, E, k, H, I;
    const uint16_t* x;
    const int32_t* table;
    const uint8_t* pool;
    int64_t n_slots, slot_bytes, off_gu_codes, off_gu_sb, off_d_codes, off_d_sb;
    uint16_t* out;
    uint32_t* gen;     // call-tag counters (reserved workspace region)
    uint64_t* xw;      // tagged h pair words (reserved workspace region)
    uint32_t* err;
    int lpr_gu, lpr_d;
    int rows_per_wg;   // phase-2 output rows per workgroup (multiple of 64/lpr_d)
    int xs1_dw, h2_dw, xs2_dw, part_dw;  // dword offsets in dynamic LDS (see lds_layout)
    int nw_q, nw_r;    // (grid waves) / (phase-1 items per hit) and remainder
    unsigned spin_limit;
};

__device__ __forceinline__ void flag(uint32_t* err, uint32_t bit)
{
    if (err) atomicOr(err, bit);
}

template <int B, int UPL>
__device__ __forceinline__ void unpack_row(const RowLoad<B, UPL>& r, uint32_t (&cp)[UPL][16],
                                           float (&s)[UPL], float (&z)[UPL])
{
    constexpr float off = Code<B>::offset;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
        unit_pairs<B>(r.w[j], cp[j]);
        s[j] = half_bits_to_f32(r.sb[j] & 0xFFFFu);
        z[j] = __builtin_fmaf(-off, s[j], half_bits_to_f32(r.sb[j] >> 16));
    }
}

template <int BG, int BD, int UG, int UD, int W>
__global__ __launch_bounds__(64 * W) void decode_layer_kernel(DecodeParams P)
{
    constexpr int kWaves = W;  // waves per workgroup
    constexpr int kThreads = 64 * W;
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // x, logits, x unit sums, h, h unit sums, partials
    __shared__ int32_t s_table[kMaxE];
    __shared__ int32_t s_ids[kMaxPairs];
    __shared__ float s_w[kMaxPairs];
    __shared__ alignas(16) int32_t s_e[kMaxPairs];
    __shared__ int32_t s_sorted[kMaxPairs];
    __shared__ int32_t s_hit[kMaxPairs];
    __shared__ int32_t s_base[kMaxPairs + 1];
    __shared__ int32_t s_slot[kMaxPairs];  // slot of each hit (-1: not resident, skipped)
    __shared__ int s_hstate[kMaxPairs];    // h of a hit in LDS: 0 not yet, 1 being staged, 2 ready
    __shared__ int32_t s_cnt[2];  // n_hit, n_valid
    __shared__ unsigned s_gen;
    __shared__ RouteScratch s_rsc[kWaves];
    __shared__ RouteWgScratch<kWaves> s_rwg;
    __shared__ RouteSelScratch s_rsel;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x;
    const int T = P.T, k = P.k, H = P.H, I = P.I, E = P.E;
    const int n = T * k;
    const bool wg0 = blockIdx.x == 0;

    // ---- one round of loads: call tag, x, slot table, routing input ----
    // x goes to LDS as P16 pairs, unit-contiguous (layout swz)
    const int Ug = H / 32;
    uint32_t* s_act = s_dyn;
    float* s_logit = (float*)(s_dyn + T * H / 2);
    float* s_xs1 = (float*)(s_dyn + P.xs1_dw);  // [t][unit] sums of x
    uint32_t* s_h2 = s_dyn + P.h2_dw;           // h of every valid pair (P16, layout swz)
    float* s_xs2 = (float*)(s_dyn + P.xs2_dw);  // [pos][unit] sums of h
    if (tid == 0) s_gen = __hip_atomic_load(&P.gen[kGenBase + blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // one routed token in plain mode: routed by logit order, its lists and m, Z
    // computed from registers before the staging barrier
    const bool fast1 = P.logits && T == 1 && P.mode == MOE_ROUTE_PLAIN && E >= 64 && k <= 15 &&
                       E <= 64 * (kWaves < 8 ? kWaves : 8);
    float r_m = 0.0f, r_Z = 0.0f;  // routing: max logit and Z
    uint32_t r_K = 0;                // routing: the chosen keys (wave zw)
    bool r_late = false;             // routing: weights and pair order still to come (wave zw)
    {
        // all loads of this round are issued before any LDS store
        constexpr int R = 4;
        const int nx = T * H / 2;
        for (int q0 = tid; q0 < nx; q0 += kThreads * R) {
            uint32_t lo[R], hi[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                const int qq = q < nx ? q : nx - 1;
                const int t = T == 1 ? 0 : qq / (H / 2);
                const int rr = qq - t * (H / 2);
                const uint16_t* src = P.x + (size_t)t * H + 32 * (rr >> 4) + (rr & 15);
                lo[r] = src[0];
                hi[r] = src[16];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                if (q < nx) {
                    const int t = T == 1 ? 0 : q / (H / 2);
                    const int rr = q - t * (H / 2);
                    s_act[t * (H / 2) + swz(rr >> 4, rr & 15)] = lo[r] | (hi[r] << 16);
                }
            }
        }
        constexpr int RT = (kMaxE + kThreads - 1) / kThreads;
        int32_t tb[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int i = tid + kThreads * r;
            tb[r] = P.table[i < E ? i : E - 1];
        }
        float own = 0.0f, zv[8];
        const int own_e = (fast1 ? max(route_sel_list<kWaves>(wave, E), 0) : 0) * 64 + lane;  // own expert
        if (fast1) {
            own = P.logits[own_e < E ? own_e : E - 1];
            if (wave == route_sel_wave<kWaves>(E)) {
#pragma unroll
                for (int j = 0; j < 8; ++j) zv[j] = P.logits[lane + 64 * j < E ? lane + 64 * j : E - 1];
            }
        }
        float lgv[R];
        const int nl = (P.logits && !fast1) ? T * E : 0;
        for (int q0 = tid; q0 < nl; q0 += kThreads * R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                lgv[r] = P.logits[q < nl ? q : nl - 1];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                if (q < nl) s_logit[q] = lgv[r];
            }
        }
        if (!P.logits && tid < n) {
            s_ids[tid] = P.ids_in[tid];
            s_w[tid] = P.w_in[tid];
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int i = tid + kThreads * r;
            if (i < E) s_table[i] = tb[r];
        }
        if (fast1) {
            if (route_sel_list<kWaves>(wave, E) >= 0 && own_e < E) s_logit[own_e] = own;
            route_sel_lists<kWaves>(own, zv, E, &s_rsel, 0, r_m, r_Z);
        }
    }
    __syncthreads();
    unsigned tag = s_gen + 1u;
    if (tag == 0u) tag = 1u;
    // the next call's counters: b, b+G, ... (read by no other workgroup of this call)
    for (int j = blockIdx.x + G * tid; j < kMaxGrid; j += G * kThreads)
        __hip_atomic_store(&P.gen[kGenBase + j], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // per-unit sums of x (read by phase 1, after the sort's barrier)
    for (int q = tid; q < T * Ug; q += kThreads) {
        const int t = T == 1 ? 0 : q / Ug, u = q - t * Ug;
        s_xs1[q] = unit_sum(s_act + t * (H / 2), u);
    }

    if (tid < kMaxPairs) s_hstate[tid] = 0;  // read in phase 2, after the barriers below

    // ---- routing from LDS (one wave per token), identical to the router kernel ----
    // (few tokens: all waves route each token together; more: one wave per token)
    bool presorted = false;  // one routed token: the routing wave also sorts its pairs
    if (P.logits) {
        if (T <= 3 && E >= 64) {
            // plain mode: by logit order (one barrier); else by selection key
            const bool by_logit = P.mode == MOE_ROUTE_PLAIN && k <= 15 && E <= 64 * (kWaves < 8 ? kWaves : 8);
            // (one token without a loop: the loop's hoisted set-up costs more than the routing)
            if (fast1) {
                // the chosen set now; with routing by logit order its weights and pair
                // order come after the phase-1 loads are issued (they need the set only)
                bool by_key;
                const bool ok = route_sel_choose<kWaves>(s_logit, E, k, r_m, s_ids, s_w, &s_rsc[0], &s_rsel, 0, r_K,
                                                         by_key);
                if (!ok && wg0 && tid == 0) flag(P.err, MOE_ERRW_NONFINITE);
                if (wave == route_sel_wave<kWaves>(E)) {
                    // the k experts of one token are distinct: hit index = rank of the
                    // expert (one pair per hit); pair j is known now only if routed by key
                    r_late = ok && !by_key;
                    const int e = lane < k ? (r_late ? key32_id(r_K) : s_ids[lane]) : 0x7fffffff;
                    int rank = 0;
#pragma unroll
                    for (int q = 0; q < 16; ++q) rank += __builtin_amdgcn_readlane(e, q) < e ? 1 : 0;
                    if (lane < k) {
                        if (!r_late) s_sorted[rank] = lane;
                        s_hit[rank] = e;
                        s_base[rank] = rank;
                        int32_t slot = s_table[e];
                        if (slot < 0 || slot >= P.n_slots) {
                            if (wg0) flag(P.err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
                            slot = -1;
                        }
                        s_slot[rank] = slot;
                    }
                    if (lane == 0) {
                        s_cnt[0] = k;
                        s_cnt[1] = k;
                        s_base[k] = k;
                    }
                }
                presorted = true;
            } else {
                for (int t = 0; t < T; ++t) {
                    const bool ok =
                        by_logit ? route_token_sel<kWaves>(s_logit + t * E, E, k, s_ids + t * k, s_w + t * k,
                                                           &s_rsc[0], &s_rsel, t & 1)
                                 : route_token_wg<kWaves>(s_logit + t * E, E, k, P.mode, P.L, s_table, s_ids + t * k,
                                                          s_w + t * k, &s_rsc[0], &s_rwg);
                    if (!ok && wg0 && tid == 0) flag(P.err, MOE_ERRW_NONFINITE);
                }
            }
        } else {
            for (int t = wave; t < T; t += kWaves) {
                const bool ok = route_token_512(s_logit + t * E, E, k, P.mode, P.L, s_table, lane,
                                                s_ids + t * k, s_w + t * k, &s_rsc[wave]);
                if (!ok && wg0 && lane == 0) flag(P.err, MOE_ERRW_NONFINITE);
            }
        }
        __syncthreads();
        if (!fast1 && wg0 && P.ids_out && tid < n) {
            P.ids_out[tid] = s_ids[tid];
            P.w_out[tid] = s_w[tid];
        }
    }

    // ---- sort the pairs by expert (stable by pair id), hit list, slots ----
    // Lane l holds pair l's expert e; lt = pairs with a smaller expert (bit mask),
    // dup = earlier pairs with the same expert.  Sorted position = |lt| + dup;
    // hit index = first occurrences among lt.  Experts are read back from LDS
    // four at a time (broadcast reads); pairs past n hold the sentinel.
    if (!presorted && wave == 0) {
        int e = 0x7fffffff;  // invalid pairs sort after every expert and are dropped
        if (lane < n) {
            e = s_ids[lane];
            if (e < 0 || e >= E) {
                if (wg0) flag(P.err, MOE_ERRW_BAD_ID);
                e = 0x7fffffff;
            }
        }
        s_e[lane] = e;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        const bool valid = e != 0x7fffffff;
        uint64_t lt = 0;
        int dup = 0;
        for (int q = 0; q < n; q += 4) {
            const int4 eq = *(const int4*)&s_e[q];
            lt |= (uint64_t)(eq.x < e) << q;
            lt |= (uint64_t)(eq.y < e) << (q + 1);
            lt |= (uint64_t)(eq.z < e) << (q + 2);
            lt |= (uint64_t)(eq.w < e) << (q + 3);
            dup += (eq.x == e && q < lane) ? 1 : 0;
            dup += (eq.y == e && q + 1 < lane) ? 1 : 0;
            dup += (eq.z == e && q + 2 < lane) ? 1 : 0;
            dup += (eq.w == e && q + 3 < lane) ? 1 : 0;
        }
        const bool first = valid && dup == 0;
        const int pos = __popcll(lt) + dup;  // stable: equal experts keep pair order
        const unsigned long long fm = __ballot(first);
        const unsigned long long vm = __ballot(valid);
        if (valid) s_sorted[pos] = lane;
        if (first) {
            const int hidx = __popcll(fm & lt);
            s_hit[hidx] = e;
            s_base[hidx] = pos;
            int32_t slot = s_table[e];
            if (slot < 0 || slot >= P.n_slots) {
                if (wg0) flag(P.err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
                slot = -1;
            }
            s_slot[hidx] = slot;
        }
        const int nh = __popcll(fm);
        if (lane == 0) {
            s_cnt[0] = nh;
            s_cnt[1] = __popcll(vm);
            s_base[nh] = __popcll(vm);
        }
    }
    if (!presorted) __syncthreads();  // (presorted: the routing's barrier ordered the sort)
    const int n_hit = s_cnt[0];

    // ---- weight loads: phase 1 rows now, the phase-2 rows once phase 1 is done
    //      (they do not depend on h, so they stream in during the h exchange) ----
    // A hit's rows are visited in P16 pair order (index j -> row pair_row(j)).  A
    // phase-1 item is RW = max(rpp, 2) consecutive indices -- whole pairs -- so the
    // wave that computes it publishes its h words itself.  Wave gw takes items
    // gw, gw + NW, ...; (hit, item in hit) advance by (nw_q, nw_r) per step.
    const int lpr = P.lpr_gu, rpp = udiv(64, lpr);
    const int seg = lane & (lpr - 1), rloc = udiv(lane, lpr);
    const int RW = rpp > 1 ? rpp : 2;  // pair-order indices per item
    const int nsub = rpp > 1 ? 1 : 2;  // rows per lane per item
    const int n_ipr = udiv(I, RW);     // items per hit
    const int n_items = n_hit * n_ipr;
    const int gw = blockIdx.x * kWaves + wave, NW = G * kWaves;
    const size_t g_row_dw = (size_t)H * BG / 32;
    constexpr int D1 = (64 / (4 * UG * (BG + 1))) < 1 ? 1 : ((64 / (4 * UG * (BG + 1))) > 2 ? 2 : (64 / (4 * UG * (BG + 1))));
    RowLoad<BG, UG> gr[D1][2], ur[D1][2];
    int ih[D1], iii[D1], islot[D1];
    const uint32_t g_row_b = (uint32_t)(g_row_dw * 4), g_sb_b = (uint32_t)(H / 16);  // bytes per row
    int h_next = udiv(gw, n_ipr), ii_next = gw - h_next * n_ipr;  // item at it0
    auto issue_p1 = [&](int it0) {
        int h = h_next, ii = ii_next;
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            ih[d] = h;
            iii[d] = ii;
            h += P.nw_q;
            ii += P.nw_r;
            if (ii >= n_ipr) {
                ii -= n_ipr;
                ++h;
            }
        }
        h_next = h;
        ii_next = ii;
#pragma unroll
        for (int d = 0; d < D1; ++d)
            islot[d] = __builtin_amdgcn_readfirstlane(s_slot[ih[d] < kMaxPairs ? ih[d] : kMaxPairs - 1]);
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            if (it0 + d * NW < n_items && islot[d] >= 0) {
                const uint8_t* base = P.pool + (size_t)islot[d] * (size_t)P.slot_bytes;
                const uint32_t oc = (uint32_t)P.off_gu_codes, os = (uint32_t)P.off_gu_sb;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    if (sb < nsub) {
                        const uint32_t nr = (uint32_t)pair_row(iii[d] * RW + sb * rpp + rloc);
                        load_row<BG, UG>(gr[d][sb], base, oc + nr * g_row_b, os + nr * g_sb_b, seg, lpr);
                        load_row<BG, UG>(ur[d][sb], base, oc + (nr + I) * g_row_b, os + (nr + I) * g_sb_b, seg, lpr);
                    }
                }
            }
        }
    };
    issue_p1(gw);
    if (fast1) {
        // weights and pair order of the routed token (routing by logit order)
        if (r_late) {
            const int e = route_sel_weights(s_logit, k, r_m, r_Z, r_K, s_ids, s_w);  // expert of pair `lane`
            int rank = 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int o = __builtin_amdgcn_readlane(e, q);
                rank += (q < k && o < e) ? 1 : 0;
            }
            if (lane < k) s_sorted[rank] = lane;
        }
    }

    const int lpr_d = P.lpr_d, rpp_d = udiv(64, lpr_d);
    const int seg_d = lane & (lpr_d - 1), rloc_d = udiv(lane, lpr_d);
    const int Ud = I / 32;
    const int row0 = blockIdx.x * P.rows_per_wg;
    const int n_rg = udiv(P.rows_per_wg, rpp_d);  // row groups of this workgroup
    const uint32_t d_row_b = (uint32_t)(I * BD / 8), d_sb_b = (uint32_t)(I / 16);  // bytes per row
    constexpr int D2 = (64 / (UD * (BD + 1))) < 1 ? 1 : ((64 / (UD * (BD + 1))) > 4 ? 4 : (64 / (UD * (BD + 1))));
    // phase-2 items of the workgroup: (row group, hit), i = rg * n_hit + hit; wave w
    // takes i = w, w + kWaves, ... (balanced to within one item per wave)
    const int n_all2 = n_rg * n_hit;
    const int n_items2 = n_all2 > wave ? (n_all2 - wave + kWaves - 1) / kWaves : 0;
    RowLoad<BD, UD> pre[D2];
    int hh2[D2], rr2[D2];
    int h2_next = wave, rg2_next = 0;  // (wave / n_hit, wave % n_hit) without a division
    while (h2_next >= n_hit && n_hit > 0) {
        h2_next -= n_hit;
        ++rg2_next;
    }
    auto issue_p2 = [&](RowLoad<BD, UD>* dst, int d0) {
        int h = h2_next, rg = rg2_next;
#pragma unroll
        for (int d = 0; d < D2; ++d) {
            hh2[d] = h;
            rr2[d] = rg;
            h += kWaves;
            while (h >= n_hit && n_hit > 0) {
                h -= n_hit;
                ++rg;
            }
        }
        h2_next = h;
        rg2_next = rg;
        int sl[D2];
#pragma unroll
        for (int d = 0; d < D2; ++d)
            sl[d] = __builtin_amdgcn_readfirstlane(s_slot[hh2[d] < kMaxPairs ? hh2[d] : kMaxPairs - 1]);
#pragma unroll
        for (int d = 0; d < D2; ++d) {
            const int nrow = row0 + rr2[d] * rpp_d + rloc_d;
            if (d0 + d < n_items2 && sl[d] >= 0 && nrow < H) {
                const uint8_t* base = P.pool + (size_t)sl[d] * (size_t)P.slot_bytes;
                load_row<BD, UD>(dst[d], base, (uint32_t)P.off_d_codes + (uint32_t)nrow * d_row_b,
                                 (uint32_t)P.off_d_sb + (uint32_t)nrow * d_sb_b, seg_d, lpr_d);
            }
        }
    };

    // ---- phase 1: gate/up + SwiGLU -> tagged h pair words ----
    // Publisher of an item's pair words: lane 0 (rpp = 1: the lane holds both rows
    // of the pair), else the first lane of each even row (its odd partner row
    // sits lpr lanes up).  A hit that is not resident publishes zeros, so the
    // readers of its words are not kept waiting.
    const uint64_t tag_hi = (uint64_t)tag << 32;
    const bool pub_lane = nsub == 2 ? lane == 0 : (seg == 0 && (rloc & 1) == 0);
    for (int it0 = gw; it0 < n_items;) {
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            const int it = it0 + d * NW;
            if (it >= n_items) continue;
            const int h = ih[d];
            const int pidx = nsub == 2 ? iii[d] : ((iii[d] * RW + rloc) >> 1);
            const int pb = s_base[h], pe = s_base[h + 1];
            if (islot[d] < 0) {  // uniform per wave
                if (pub_lane)
                    for (int pos = pb; pos < pe; ++pos)
                        __hip_atomic_store(&P.xw[(size_t)pos * (I / 2) + pidx], tag_hi, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                continue;
            }
            for (int pos = pb; pos < pe; ++pos) {
                const int t = T == 1 ? 0 : s_sorted[pos] / k;
                const uint32_t* act = s_act + t * (H / 2);
                const float* xs = s_xs1 + t * Ug;
                uint32_t hb[2] = {0u, 0u};
                if (nsub == 2) {
                    // both rows of the pair on all 64 lanes: one transposed reduction of
                    // (g0, g1, u0, u1); lanes 0-15 then hold g0 and, after the i^32 swap,
                    // u0; lanes 16-31 hold g1 and u1
                    const float g0 = row_dot_raw<BG, UG>(gr[d][0], act, xs, seg, lpr);
                    const float g1 = row_dot_raw<BG, UG>(gr[d][1], act, xs, seg, lpr);
                    const float u0 = row_dot_raw<BG, UG>(ur[d][0], act, xs, seg, lpr);
                    const float u1 = row_dot_raw<BG, UG>(ur[d][1], act, xs, seg, lpr);
                    const float sm = wave_sum4(g0, g1, u0, u1, lane);
                    const auto ru = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm), __float_as_uint(sm), false, false);
                    const uint32_t h = f32_to_bf16(silu_mul(sm, __uint_as_float(ru[1])));
                    hb[0] = __builtin_amdgcn_readlane(h, 0);
                    hb[1] = __builtin_amdgcn_readlane(h, 16);
                } else {
                    float g = row_dot_raw<BG, UG>(gr[d][0], act, xs, seg, lpr);
                    float u = row_dot_raw<BG, UG>(ur[d][0], act, xs, seg, lpr);
                    g = seg_sum(g, lpr);
                    u = seg_sum(u, lpr);
                    hb[0] = f32_to_bf16(silu_mul(g, u));
                    hb[1] = (uint32_t)__shfl_xor((int)hb[0], lpr, 64);
                }
                if (pub_lane)
                    __hip_atomic_store(&P.xw[(size_t)pos * (I / 2) + pidx], tag_hi | hb[0] | (hb[1] << 16),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        it0 += NW * D1;
        if (it0 < n_items) issue_p1(it0);
    }


    // ---- h of each hit, staged when a wave first needs it: the wave that claims
    //      a hit polls the tagged words of its pairs (P16, unit-contiguous layout
    //      swz) until they carry this call's tag, adds their unit sums, and marks
    //      the hit ready; a wave that needs a hit claimed by another waits for that
    //      mark in LDS.  A wave so waits only for the experts of its own items, not
    //      for the slowest expert of the layer. ----
    issue_p2(pre, 0);  // the phase-2 weights stream in while h is exchanged
    // one token: phase 1 used only what the routing barrier published (hit list,
    // slots, staged x), so the weights and pair order the routing wave wrote after
    // its phase-1 loads are ordered here, before phase 2 reads them; phase 1 did
    // not wait for them
    if (fast1) {
        __syncthreads();
        if (wg0 && P.ids_out && tid < n) {
            P.ids_out[tid] = s_ids[tid];
            P.w_out[tid] = s_w[tid];
        }
    }
    float* s_part = (float*)(s_dyn + P.part_dw);  // [wave][row][t]
    float* part = s_part + wave * P.rows_per_wg * T;
    for (int q = lane; q < P.rows_per_wg * T; q += 64) part[q] = 0.0f;  // this wave's rows only
    auto ensure_hit = [&](int hh) {
        if (__hip_atomic_load(&s_hstate[hh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 2) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            return;
        }
        int claim = 0;
        if (lane == 0) claim = atomicCAS(&s_hstate[hh], 0, 1) == 0 ? 1 : 0;
        claim = __builtin_amdgcn_readfirstlane(claim);
        if (claim) {
            // pair by pair, word rr = w0 + lane + 64 r of the pair's I / 2 (no division)
            constexpr int R = 4;
            const int pb = s_base[hh], pe = s_base[hh + 1];
            for (int pos = pb; pos < pe; ++pos) {
                for (int w0 = 0; w0 < I / 2; w0 += 64 * R) {
                    const uint64_t* src = P.xw + (size_t)pos * (I / 2) + w0 + lane;
                    const int nv = I / 2 - w0 - lane;  // word r of this lane exists iff 64 r < nv
                    uint64_t hv[R];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        hv[r] = 64 * r < nv ? __hip_atomic_load(src + 64 * r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                            : tag_hi;
                    unsigned spins = 0;
                    for (;;) {
                        bool ready = true;
#pragma unroll
                        for (int r = 0; r < R; ++r) ready = ready && (uint32_t)(hv[r] >> 32) == tag;
                        if (ready) break;
                        if (++spins > P.spin_limit) {
                            flag(P.err, MOE_ERRW_TIMEOUT);
                            break;
                        }
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            if ((uint32_t)(hv[r] >> 32) != tag)
                                hv[r] = __hip_atomic_load(src + 64 * r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    uint32_t* dst = s_h2 + pos * (I / 2);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const int rr = w0 + lane + 64 * r;
                        if (64 * r < nv) dst[swz(rr >> 4, rr & 15)] = (uint32_t)hv[r];
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            for (int pos = pb; pos < pe; ++pos)
                for (int u = lane; u < Ud; u += 64) s_xs2[pos * Ud + u] = unit_sum(s_h2 + pos * (I / 2), u);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            if (lane == 0) __hip_atomic_store(&s_hstate[hh], 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
            unsigned spins = 0;
            while (__hip_atomic_load(&s_hstate[hh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 2) {
                if (++spins > P.spin_limit) {
                    flag(P.err, MOE_ERRW_TIMEOUT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
    };

    // ---- phase 2: down + weighted combine ----
    for (int d0 = 0; d0 < n_items2; d0 += D2) {
        if (d0 > 0) issue_p2(pre, d0);
        RowLoad<BD, UD>* cur = pre;
#pragma unroll
        for (int d = 0; d < D2; ++d) {
            const int it = d0 + d;
            const int rg = rr2[d], h = hh2[d];
            if (it >= n_items2) continue;
            const int lrow = rg * rpp_d + rloc_d;
            const int nrow = row0 + lrow;
            if (s_slot[h] < 0) continue;
            // the first pair's id and weight are read before waiting for h
            const int pb = s_base[h], pend = s_base[h + 1];
            const int pair0 = s_sorted[pb];
            const float w0 = s_w[pair0];
            ensure_hit(h);
            for (int pos = pb; pos < pend; ++pos) {
                const int pair = pos == pb ? pair0 : s_sorted[pos];
                const float wp = pos == pb ? w0 : s_w[pair];
                float y = row_dot_raw<BD, UD>(cur[d], s_h2 + pos * (I / 2), s_xs2 + pos * Ud, seg_d, lpr_d);
                y = seg_sum(y, lpr_d);
                if (seg_d == 0 && nrow < H) {
                    const int t = T == 1 ? 0 : pair / k;
                    // this wave's own partials: LDS add without a return value, applied
                    // in the wave's program order
                    atomicAdd(&part[lrow * T + t], wp * y);
                }
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < P.rows_per_wg * T; q += kThreads) {
        const int lrow = T == 1 ? q : q / T, t = q - lrow * T;
        const int nrow = row0 + lrow;
        if (nrow >= H) continue;
        float acc = s_part[q];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) acc += s_part[w * P.rows_per_wg * T + q];
        P.out[(size_t)t * H + nrow] = f32_to_bf16(acc);
    }
}

template <int BG, int BD, int UG, int UD, int W>
hipError_t launch_t(const DecodeParams& P, int G, size_t lds, hipStream_t s)
{
    hipLaunchKernelGGL((decode_layer_kernel<BG, BD, UG, UD, W>), dim3(G), dim3(64 * W), lds, s, P);
    return hipGetLastError();
}

template <int BG, int BD, int UG, int UD, int W>
int occupancy_t(size_t lds)
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_layer_kernel<BG, BD, UG, UD, W>, 64 * W, lds) != hipSuccess)
        return 0;
    return nb;
}

bool lanes_of(int units, int* lpr, int* upl)
{
    int l = units & -units;
    if (l > 64) l = 64;
    *lpr = l;
    *upl = units / l;
    return true;
}

using LaunchFn = hipError_t (*)(const DecodeParams&, int, size_t, hipStream_t);
using OccFn = int (*)(size_t);

struct Variant {
    int bg, bd, ug, ud, w;  // bits gate/up, bits down, units per lane, waves per workgroup
    LaunchFn launch;
    OccFn occ;
};

// Waves per workgroup: 10 where the kernel fits 3 waves per SIMD without
// spilling (one phase-1 item per wave at the decode shape), else 8.
#define MOE_V(BG, BD, UG, UD, W) {BG, BD, UG, UD, W, launch_t<BG, BD, UG, UD, W>, occupancy_t<BG, BD, UG, UD, W>}
const Variant kVariants[] = {
    MOE_V(3, 3, 1, 1, 10), MOE_V(4, 4, 1, 1, 10), MOE_V(6, 6, 1, 1, 8), MOE_V(8, 8, 1, 1, 10),
    MOE_V(4, 6, 1, 1, 10), MOE_V(3, 3, 1, 3, 8), MOE_V(4, 4, 1, 3, 8), MOE_V(4, 6, 1, 3, 8),
    MOE_V(8, 8, 2, 1, 8), MOE_V(4, 4, 2, 1, 8), MOE_V(3, 3, 2, 1, 8), MOE_V(6, 6, 1, 3, 8),
    MOE_V(16, 16, 1, 1, 8),
};
#undef MOE_V

const Variant* find_variant(int bg, int bd, int ug, int ud)
{
    for (const Variant& v : kVariants)
        if (v.bg == bg && v.bd == bd && v.ug == ug && v.ud == ud) return &v;
    return nullptr;
}

struct DevInfo {
    int cus = 0;
    size_t lds_per_block = 0;
};

DevInfo dev_info()
{
    static thread_local int cached_dev = -1;
    static thread_local DevInfo info;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DevInfo{};
    if (dev != cached_dev) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return DevInfo{};
        info.cus = p.multiProcessorCount;
        info.lds_per_block = p.sharedMemPerBlock;
        cached_dev = dev;
    }
    return info;
}

// Dynamic LDS layout (dwords): x (T*H/2), logits (T*E), x unit sums (T*H/32),
// staged h (n*I/2), h unit sums (n*I/32), then the phase-2 partials.
struct LdsLayout {
    int xs1, h2, xs2, part;
    size_t bytes;
};

LdsLayout lds_layout(int T, int k, int E, int H, int I, int rows_per_wg, int W)
{
    LdsLayout L;
    const int n = T * k;
    auto up4 = [](int v) { return (v + 3) & ~3; };  // 16-byte aligned regions
    L.xs1 = up4(T * H / 2 + T * E);
    L.h2 = up4(L.xs1 + T * (H / 32));
    L.xs2 = up4(L.h2 + n * (I / 2));
    L.part = up4(L.xs2 + n * (I / 32));
    L.bytes = (size_t)4 * L.part + sizeof(float) * (size_t)W * rows_per_wg * T;
    return L;
}

}  // namespace

bool decode_fused_supported(int T, int k, int E, const ClassView& c)
{
    const int n = T * k;
    if (n > kMaxPairs || T < 1 || E > kMaxE) return false;
    int lg, ug, ld, ud;
    lanes_of(c.H / 32, &lg, &ug);
    lanes_of(c.I / 32, &ld, &ud);
    const Variant* v = find_variant(c.bits_gu, c.bits_d, ug, ud);
    if (!v) return false;
    const DevInfo di = dev_info();
    if (di.cus <= 0) return false;
    const int rpp_d = 64 / ld;
    const int n_rg = c.H / rpp_d;
    const int rows = ((n_rg + di.cus - 1) / di.cus) * rpp_d;
    if ((size_t)n * (c.I / 2) > (size_t)MOE_WS_XWORDS) return false;  // tagged h words
    if (c.slot_bytes >= ((int64_t)1 << 31)) return false;                // 32-bit offsets in a slot
    const size_t static_lds = sizeof(int32_t) * (kMaxE + 8 * kMaxPairs) + sizeof(RouteScratch) * v->w +
                              sizeof(RouteWgScratch<10>) + sizeof(RouteSelScratch) + 64;
    return lds_layout(T, k, E, c.H, c.I, rows, v->w).bytes + static_lds <= di.lds_per_block;
}

hipError_t launch_decode_fused(const float* logits, int mode, float L, const int32_t* ids_in,
                               const float* w_in, int32_t* ids_out, float* w_out, int T, int E,
                               int k, const uint16_t* x, const int32_t* table, const uint8_t* pool,
                               const ClassView& c, uint16_t* out, void* reserved, uint32_t* err,
                               hipStream_t s)
{
    int lg, ug, ld, ud;
    lanes_of(c.H / 32, &lg, &ug);
    lanes_of(c.I / 32, &ld, &ud);
    const Variant* v = find_variant(c.bits_gu, c.bits_d, ug, ud);
    if (!v) return hipErrorInvalidValue;
    const DevInfo di = dev_info();
    if (di.cus <= 0) return hipErrorInvalidDevice;
    const int rpp_d = 64 / ld;
    const int n_rg = c.H / rpp_d;
    // one workgroup per compute unit: every workgroup is resident, so every
    // polled h word is eventually written; fewer if there are fewer row groups
    int G = n_rg < di.cus ? n_rg : di.cus;
    if (G > kMaxGrid) G = kMaxGrid;
    const int rows = ((n_rg + G - 1) / G) * rpp_d;
    const LdsLayout LL = lds_layout(T, k, E, c.H, c.I, rows, v->w);
    const size_t lds = LL.bytes;
    if (v->occ(lds) < 1) return hipErrorInvalidConfiguration;
    DecodeParams P;
    P.logits = logits;
    P.mode = mode;
    P.L = L;
    P.ids_in = ids_in;
    P.w_in = w_in;
    P.ids_out = ids_out;
    P.w_out = w_out;
    P.T = T;
    P.E = E;
    P.k = k;
    P.H = c.H;
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
    P.lpr_gu = lg;
    P.lpr_d = ld;
    P.rows_per_wg = rows;
    P.xs1_dw = LL.xs1;
    P.h2_dw = LL.h2;
    P.xs2_dw = LL.xs2;
    P.part_dw = LL.part;
    const int rpp = 64 / lg;
    const int n_ipr = c.I / (rpp > 1 ? rpp : 2);
    P.nw_q = G * v->w / n_ipr;
    P.nw_r = G * v->w % n_ipr;
    P.spin_limit = 1u << 20;
    return v->launch(P, G, lds, s);
}

}  // namespace moe
