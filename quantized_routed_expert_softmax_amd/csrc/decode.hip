// decode.hip — the whole routed-expert layer for decode-sized batches in ONE
// persistent launch on gfx950: (route) -> sort by expert -> slot resolve ->
// gate/up dequant-GEMV + SwiGLU -> grid barrier -> down dequant-GEMV ->
// weighted combine.
//
// Sources: "POC: Experts offload", PR description and commit messages (quantized
// experts through a gather quantized matmul on the device cache; the GPU should
// not idle between a layer's sub-steps); "RFC: stream MoE experts from disk in
// from_pretrained", How the prototype works (gated, concatenated, untransposed
// experts, no bias; per-layer expert -> slot table; when every expert is
// resident, layers never synchronise with the host); BigMoeOnEdge commit message
// (cache-aware substitution, optional).
//
// Why one kernel: a decode layer moves ~14 MB (10 experts of 1.38 MB at 3 bits),
// about 2 us of HBM time, while every extra launch and every dependent global
// load costs ~1-5 us.  So each workgroup
//   1. stages router logits, the token rows and nothing else, routes (one wave
//      per token, identical arithmetic to the router kernel) and sorts the
//      <= 64 (token, j) pairs by expert in LDS -- redundantly in every
//      workgroup, which costs a few hundred cycles and saves a launch and a
//      global round trip;
//   2. looks up the hit experts' slots, then issues the loads of ALL its weight
//      rows at once: the gate/up rows of phase 1 and the down rows of phase 2
//      (the down weights do not depend on h, so they stream in while gate/up
//      computes);
//   3. phase 1: a wave owns gate row n and up row I+n of one hit expert; codes
//      become bf16 pairs (128 + c) and bf16 dot2 sums them against the P16
//      paired activations; per unit s*acc + (z - 128 s)*sum(x); h = silu(g)*u
//      goes to the workspace in bf16;
//   4. grid barrier (one atomic counter + generation word, bounded spin that
//      reports MOE_ERRW_TIMEOUT instead of hanging);
//   5. phase 2: h of all pairs is staged in LDS; wave w of a workgroup takes
//      hits w, w+4, ... for the workgroup's output rows and accumulates w_j*y per
//      token; the four waves' partial sums are added in wave order, so the
//      result is bit-reproducible.
// All workgroups are co-resident (grid <= compute units, occupancy checked on
// the host), so the barrier always completes.
#pragma clang fp contract(off)

#include "../../include/moe.h"
#include "moe_dev.h"
#include "moe_internal.h"
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kMaxPairs = 64;
constexpr int kMaxE = 1024;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxGrid = 1024;  // arrival flags in the workspace barrier region

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
    uint16_t* hbuf;
    uint32_t* bar;
    uint32_t* err;
    int lpr_gu, lpr_d;
    int rows_per_wg;  // phase-2 output rows per workgroup (multiple of 64/lpr_d)
    int act_dw;       // dwords of the activation region of dynamic LDS
    unsigned spin_limit;
};

__device__ __forceinline__ void flag(uint32_t* err, uint32_t bit)
{
    if (err) atomicOr(err, bit);
}

template <int B, int UPL>
struct RowLoad {
    uint32_t w[UPL][B];
    uint32_t sb[UPL];
};

template <int B, int UPL>
__device__ __forceinline__ void load_row(RowLoad<B, UPL>& r, const uint32_t* __restrict__ codes_row,
                                         const uint32_t* __restrict__ sb_row, int seg, int lpr)
{
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
        const int u = seg + lpr * j;
#pragma unroll
        for (int b = 0; b < B; ++b) r.w[j][b] = codes_row[u * B + b];
        r.sb[j] = sb_row[u >> 1];
    }
}

// Dot of one row's lane share (UPL units) with activations read from LDS in the
// transposed P16 layout act[j][u] (16 dwords per unit, U units per row).
template <int B, int UPL>
__device__ __forceinline__ float row_dot(const uint32_t (&cp)[UPL][16], const float (&s)[UPL],
                                         const float (&z)[UPL], const uint32_t* __restrict__ act,
                                         int U, int seg, int lpr)
{
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
        const int u = seg + lpr * j;
        float X = 0.0f, a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t xv = act[i * U + u];
            X = dot2(xv, MOE_ONES_PAIR, X);
            a = dot2(cp[j][i], xv, a);
        }
        y = __builtin_fmaf(s[j], a, __builtin_fmaf(z[j], X, y));
    }
    return y;
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

template <int BG, int BD, int UG, int UD>
__global__ __launch_bounds__(kThreads) void decode_layer_kernel(DecodeParams P)
{
    extern __shared__ uint32_t s_dyn[];  // activations (x then h), logits, then partials
    __shared__ int32_t s_table[kMaxE];
    __shared__ int32_t s_ids[kMaxPairs];
    __shared__ float s_w[kMaxPairs];
    __shared__ int32_t s_sorted[kMaxPairs];
    __shared__ int32_t s_hit[kMaxPairs];
    __shared__ int32_t s_base[kMaxPairs + 1];
    __shared__ int32_t s_slot[kMaxPairs];
    __shared__ const uint8_t* s_rowb[kMaxPairs];  // slot row of each hit (null: skip)
    __shared__ int32_t s_cnt[2];  // n_hit, n_valid
    __shared__ unsigned s_gen;
    __shared__ RouteScratch s_rsc[kWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x;
    const int T = P.T, k = P.k, H = P.H, I = P.I, E = P.E;
    const int n = T * k;
    const bool wg0 = blockIdx.x == 0;

    // ---- one round of loads: barrier generation, x, slot table, routing input ----
    // x goes to LDS as P16 pairs, transposed: dword (t, i, u) at t*H/2 + i*U + u
    const int Ug = H / 32;
    uint32_t* s_act = s_dyn;
    float* s_logit = (float*)(s_dyn + T * H / 2);
    if (tid == 0) s_gen = __hip_atomic_load(&P.bar[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
                const int t = qq / (H / 2);
                const int rr = qq - t * (H / 2);
                const uint16_t* src = P.x + (size_t)t * H + 32 * (rr >> 4) + (rr & 15);
                lo[r] = src[0];
                hi[r] = src[16];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                if (q < nx) {
                    const int t = q / (H / 2);
                    const int rr = q - t * (H / 2);
                    s_act[t * (H / 2) + (rr & 15) * Ug + (rr >> 4)] = lo[r] | (hi[r] << 16);
                }
            }
        }
        int32_t tb[kMaxE / kThreads];
#pragma unroll
        for (int r = 0; r < kMaxE / kThreads; ++r) {
            const int i = tid + kThreads * r;
            tb[r] = P.table[i < E ? i : E - 1];
        }
        float lgv[R];
        const int nl = P.logits ? T * E : 0;
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
        for (int r = 0; r < kMaxE / kThreads; ++r) {
            const int i = tid + kThreads * r;
            if (i < E) s_table[i] = tb[r];
        }
    }
    __syncthreads();

    // ---- routing from LDS (one wave per token), identical to the router kernel ----
    if (P.logits) {
        for (int t = wave; t < T; t += kWaves) {
            const bool ok = route_token(s_logit + t * E, E, k, P.mode, P.L, s_table, lane,
                                        s_ids + t * k, s_w + t * k, &s_rsc[wave]);
            if (!ok && wg0 && lane == 0) flag(P.err, MOE_ERRW_NONFINITE);
        }
        __syncthreads();
        if (wg0 && P.ids_out && tid < n) {
            P.ids_out[tid] = s_ids[tid];
            P.w_out[tid] = s_w[tid];
        }
    }

    // ---- sort the pairs by expert (stable by pair id), hit list, slots ----
    if (wave == 0) {
        int e = 0x7fffffff;  // invalid pairs sort after every expert and are dropped
        if (lane < n) {
            e = s_ids[lane];
            if (e < 0 || e >= E) {
                if (wg0) flag(P.err, MOE_ERRW_BAD_ID);
                e = 0x7fffffff;
            }
        }
        const bool valid = e != 0x7fffffff;
        int pos = 0, dup = 0;
        for (int q0 = 0; q0 < n; q0 += 8) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int q = q0 + r;
                if (q < n) {
                    const int eq = __builtin_amdgcn_readlane(e, q);
                    pos += (eq < e) ? 1 : 0;
                    dup += (eq == e && q < lane) ? 1 : 0;
                }
            }
        }
        const bool first = valid && dup == 0;
        pos += dup;  // stable: equal experts keep pair order
        const unsigned long long fm = __ballot(first);
        const unsigned long long vm = __ballot(valid);
        // hit index = distinct valid experts below e (first occurrences with a smaller expert)
        int hidx = 0;
        for (int q0 = 0; q0 < n; q0 += 8) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int q = q0 + r;
                if (q < n) {
                    const int eq = __builtin_amdgcn_readlane(e, q);
                    hidx += ((fm >> q) & 1ull) && eq < e ? 1 : 0;
                }
            }
        }
        if (valid) s_sorted[pos] = lane;
        if (first) {
            s_hit[hidx] = e;
            s_base[hidx] = pos;
            int32_t slot = s_table[e];
            if (slot < 0 || slot >= P.n_slots) {
                if (wg0) flag(P.err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
                slot = -1;
            }
            s_slot[hidx] = slot;
            s_rowb[hidx] = slot >= 0 ? P.pool + (size_t)slot * (size_t)P.slot_bytes : nullptr;
        }
        const int nh = __popcll(fm);
        if (lane == 0) {
            s_cnt[0] = nh;
            s_cnt[1] = __popcll(vm);
            s_base[nh] = __popcll(vm);
        }
    }
    __syncthreads();
    const int n_hit = s_cnt[0];

    // ---- weight loads: phase 1 rows first, then the phase-2 rows (they do not
    //      depend on h, so they stream in while phase 1 computes) ----
    const int lpr = P.lpr_gu, rpp = 64 / lpr;
    const int seg = lane & (lpr - 1), rloc = lane / lpr;
    const int n_rg1 = (I + rpp - 1) / rpp;
    const int n_items = n_hit * n_rg1;
    const int gw = blockIdx.x * kWaves + wave, NW = G * kWaves;
    const size_t g_row_dw = (size_t)H * BG / 32;
    constexpr int D1 = (64 / (2 * UG * (BG + 1))) < 1 ? 1 : ((64 / (2 * UG * (BG + 1))) > 8 ? 8 : (64 / (2 * UG * (BG + 1))));
    RowLoad<BG, UG> gr[D1], ur[D1];
    auto issue_p1 = [&](int it0) {
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            const int it = it0 + d * NW;
            if (it < n_items) {
                const int h = it / n_rg1, rg = it - h * n_rg1;
                const int nr = rg * rpp + rloc;
                const uint8_t* rowb = s_rowb[h];
                if (rowb && nr < I) {
                    const uint32_t* cb = (const uint32_t*)(rowb + P.off_gu_codes);
                    const uint32_t* sbb = (const uint32_t*)(rowb + P.off_gu_sb);
                    load_row<BG, UG>(gr[d], cb + (size_t)nr * g_row_dw, sbb + (size_t)nr * (H / 64), seg, lpr);
                    load_row<BG, UG>(ur[d], cb + (size_t)(I + nr) * g_row_dw,
                                     sbb + (size_t)(I + nr) * (H / 64), seg, lpr);
                }
            }
        }
    };
    issue_p1(gw);

    const int lpr_d = P.lpr_d, rpp_d = 64 / lpr_d;
    const int seg_d = lane & (lpr_d - 1), rloc_d = lane / lpr_d;
    const int Ud = I / 32;
    const int row0 = blockIdx.x * P.rows_per_wg;
    const int n_rg = P.rows_per_wg / rpp_d;   // row groups of this workgroup
    const size_t d_row_dw = (size_t)I * BD / 32;
    constexpr int D2 = (64 / (UD * (BD + 1))) < 1 ? 1 : ((64 / (UD * (BD + 1))) > 8 ? 8 : (64 / (UD * (BD + 1))));
    // items of this wave: (row group rg, hit h = wave + kWaves*q), rg-major
    const int hits_w = n_hit > wave ? (n_hit - wave + kWaves - 1) / kWaves : 0;
    const int n_items2 = n_rg * hits_w;
    RowLoad<BD, UD> pre[D2];
    auto issue_p2 = [&](RowLoad<BD, UD>* dst, int d0) {
#pragma unroll
        for (int d = 0; d < D2; ++d) {
            const int it = d0 + d;
            if (it < n_items2) {
                const int rg = it / hits_w, h = wave + kWaves * (it - rg * hits_w);
                const int nrow = row0 + rg * rpp_d + rloc_d;
                const uint8_t* rowb = s_rowb[h];
                if (rowb && nrow < H)
                    load_row<BD, UD>(dst[d], (const uint32_t*)(rowb + P.off_d_codes) + (size_t)nrow * d_row_dw,
                                     (const uint32_t*)(rowb + P.off_d_sb) + (size_t)nrow * (I / 64), seg_d, lpr_d);
            }
        }
    };
    issue_p2(pre, 0);

    // ---- phase 1: gate/up + SwiGLU ----
    for (int it0 = gw; it0 < n_items;) {
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            const int it = it0 + d * NW;
            if (it >= n_items) continue;
            const int h = it / n_rg1, rg = it - h * n_rg1;
            const int nr = rg * rpp + rloc;
            if (!s_rowb[h]) continue;  // uniform per wave
            uint32_t gp[UG][16], up[UG][16];
            float gs[UG], gz[UG], us[UG], uz[UG];
            unpack_row<BG, UG>(gr[d], gp, gs, gz);
            unpack_row<BG, UG>(ur[d], up, us, uz);
            const int pend = s_base[h + 1];
            for (int pos = s_base[h]; pos < pend; ++pos) {
                const int t = s_sorted[pos] / k;
                const uint32_t* act = s_act + t * (H / 2);
                float g = row_dot<BG, UG>(gp, gs, gz, act, Ug, seg, lpr);
                float u = row_dot<BG, UG>(up, us, uz, act, Ug, seg, lpr);
                g = seg_sum(g, lpr);
                u = seg_sum(u, lpr);
                if (seg == 0 && nr < I) {
                    const int hp = (nr & ~31) | p16_pos(nr & 31);
                    P.hbuf[(size_t)pos * I + hp] = f32_to_bf16(silu_mul(g, u));
                }
            }
        }
        it0 += NW * D1;
        if (it0 < n_items) issue_p1(it0);
    }

    // ---- grid barrier: per-workgroup arrival flags, one poller, one release word ----
    // Workspace words: bar[0] = generation, bar[64 + b] = arrival flag of
    // workgroup b.  No read-modify-write: every word has one writer.
    __syncthreads();
    {
        const unsigned target = s_gen + 1u;
        uint32_t* flags = P.bar + 64;
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // h is visible device-wide
            __hip_atomic_store(&flags[blockIdx.x], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (wg0) {
            if (wave == 0) {
                unsigned spins = 0;
                for (;;) {
                    bool mine = true;
                    for (int j = lane; j < G; j += 64)
                        mine = mine && __hip_atomic_load(&flags[j], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT) == target;
                    if (__all(mine)) break;
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > P.spin_limit) {
                        if (lane == 0) flag(P.err, MOE_ERRW_TIMEOUT);
                        break;
                    }
                }
                if (lane == 0) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    __hip_atomic_store(&P.bar[0], target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        } else if (tid == 0) {
            unsigned spins = 0;
            while (__hip_atomic_load(&P.bar[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > P.spin_limit) {
                    flag(P.err, MOE_ERRW_TIMEOUT);
                    break;
                }
            }
        }
        __syncthreads();
        if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
    }

    // ---- stage h of every valid pair (transposed P16: (pos, i, u) at pos*I/2 + i*Ud + u) ----
    const int n_valid = s_cnt[1];
    {
        constexpr int R = 8;
        const int nh = n_valid * (I / 2);
        const uint32_t* hsrc = (const uint32_t*)P.hbuf;
        for (int q0 = tid; q0 < nh; q0 += kThreads * R) {
            uint32_t hv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                hv[r] = hsrc[q < nh ? q : nh - 1];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = q0 + kThreads * r;
                if (q < nh) {
                    const int pos = q / (I / 2);
                    const int rr = q - pos * (I / 2);
                    s_act[pos * (I / 2) + (rr & 15) * Ud + (rr >> 4)] = hv[r];
                }
            }
        }
    }
    float* s_part = (float*)(s_dyn + P.act_dw);  // [wave][row][t]
    for (int q = tid; q < kWaves * P.rows_per_wg * T; q += kThreads) s_part[q] = 0.0f;
    __syncthreads();

    // ---- phase 2: down + weighted combine ----
    float* part = s_part + wave * P.rows_per_wg * T;
    for (int d0 = 0; d0 < n_items2; d0 += D2) {
        if (d0 > 0) issue_p2(pre, d0);
        RowLoad<BD, UD>* cur = pre;
#pragma unroll
        for (int d = 0; d < D2; ++d) {
            const int it = d0 + d;
            if (it >= n_items2) break;
            const int rg = it / hits_w, h = wave + kWaves * (it - rg * hits_w);
            const int lrow = rg * rpp_d + rloc_d;
            const int nrow = row0 + lrow;
            if (!s_rowb[h]) continue;
            uint32_t cp[UD][16];
            float s[UD], z[UD];
            unpack_row<BD, UD>(cur[d], cp, s, z);
            const int pend = s_base[h + 1];
            for (int pos = s_base[h]; pos < pend; ++pos) {
                const int pair = s_sorted[pos];
                float y = row_dot<BD, UD>(cp, s, z, s_act + pos * (I / 2), Ud, seg_d, lpr_d);
                y = seg_sum(y, lpr_d);
                if (seg_d == 0 && nrow < H) {
                    const int t = pair / k;
                    part[lrow * T + t] += s_w[pair] * y;
                }
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < P.rows_per_wg * T; q += kThreads) {
        const int lrow = q / T, t = q - lrow * T;
        const int nrow = row0 + lrow;
        if (nrow >= H) continue;
        float acc = s_part[q];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) acc += s_part[w * P.rows_per_wg * T + q];
        P.out[(size_t)t * H + nrow] = f32_to_bf16(acc);
    }
}

template <int BG, int BD, int UG, int UD>
hipError_t launch_t(const DecodeParams& P, int G, size_t lds, hipStream_t s)
{
    hipLaunchKernelGGL((decode_layer_kernel<BG, BD, UG, UD>), dim3(G), dim3(kThreads), lds, s, P);
    return hipGetLastError();
}

template <int BG, int BD, int UG, int UD>
int occupancy_t(size_t lds)
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_layer_kernel<BG, BD, UG, UD>, kThreads, lds) != hipSuccess)
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
    int bg, bd, ug, ud;
    LaunchFn launch;
    OccFn occ;
};

#define MOE_V(BG, BD, UG, UD) {BG, BD, UG, UD, launch_t<BG, BD, UG, UD>, occupancy_t<BG, BD, UG, UD>}
const Variant kVariants[] = {
    MOE_V(3, 3, 1, 1), MOE_V(4, 4, 1, 1), MOE_V(6, 6, 1, 1), MOE_V(8, 8, 1, 1),
    MOE_V(4, 6, 1, 1), MOE_V(3, 3, 1, 3), MOE_V(4, 4, 1, 3), MOE_V(4, 6, 1, 3),
    MOE_V(8, 8, 2, 1), MOE_V(4, 4, 2, 1), MOE_V(3, 3, 2, 1), MOE_V(6, 6, 1, 3),
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

int act_dwords(int T, int k, int E, int H, int I)
{
    const int a = T * H / 2 + T * E, b = T * k * I / 2;  // phase 1: x + logits; phase 2: h
    return a > b ? a : b;
}

size_t dyn_lds(int T, int k, int E, int H, int I, int rows_per_wg)
{
    return (size_t)4 * act_dwords(T, k, E, H, I) + sizeof(float) * (size_t)kWaves * rows_per_wg * T;
}

}  // namespace

bool decode_fused_supported(int T, int k, int E, const ClassView& c)
{
    const int n = T * k;
    if (n > kMaxPairs || T < 1 || E > kMaxE) return false;
    int lg, ug, ld, ud;
    lanes_of(c.H / 32, &lg, &ug);
    lanes_of(c.I / 32, &ld, &ud);
    if (!find_variant(c.bits_gu, c.bits_d, ug, ud)) return false;
    const DevInfo di = dev_info();
    if (di.cus <= 0) return false;
    const int rpp_d = 64 / ld;
    const int n_rg = c.H / rpp_d;
    const int rows = ((n_rg + di.cus - 1) / di.cus) * rpp_d;
    const size_t static_lds = sizeof(int32_t) * (kMaxE + 7 * kMaxPairs) + sizeof(void*) * kMaxPairs +
                              sizeof(RouteScratch) * kWaves + 64;
    return dyn_lds(T, k, E, c.H, c.I, rows) + static_lds <= di.lds_per_block;
}

hipError_t launch_decode_fused(const float* logits, int mode, float L, const int32_t* ids_in,
                               const float* w_in, int32_t* ids_out, float* w_out, int T, int E,
                               int k, const uint16_t* x, const int32_t* table, const uint8_t* pool,
                               const ClassView& c, uint16_t* out, uint16_t* hbuf, uint32_t* bar,
                               uint32_t* err, hipStream_t s)
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
    // one workgroup per compute unit: every workgroup is resident, so the grid
    // barrier completes; fewer if there are fewer row groups than units
    int G = n_rg < di.cus ? n_rg : di.cus;
    if (G > kMaxGrid) G = kMaxGrid;
    const int rows = ((n_rg + G - 1) / G) * rpp_d;
    const size_t lds = dyn_lds(T, k, E, c.H, c.I, rows);
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
    P.hbuf = hbuf;
    P.bar = bar;
    P.err = err;
    P.lpr_gu = lg;
    P.lpr_d = ld;
    P.rows_per_wg = rows;
    P.act_dw = act_dwords(T, k, E, c.H, c.I);
    P.spin_limit = 1u << 20;
    return v->launch(P, G, lds, s);
}

}  // namespace moe
