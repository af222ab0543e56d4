// gemv.hip — decode path of the routed-expert layer on gfx950: dequantizing
// GEMV over the slot pool for few tokens per expert.
//
// Sources: "POC: Experts offload", PR description (quantized experts run through
// a gather quantized matmul on the device cache); "RFC: stream MoE experts from
// disk in from_pretrained", How the prototype works (gated, concatenated,
// untransposed experts without bias; each layer maps expert ids to slots).
//
// Decode reads each routed expert's bytes once and does ~2 flop per weight, so
// it is bound by HBM bandwidth.  Design:
//  * lanes read whole pack units of a row (B dwords per lane, consecutive lanes
//    on consecutive units: coalesced), and the fp16 scale/bias dword of the unit's
//    group;
//  * codes become bf16 pairs (128 + c) in registers with two shifts/masks per
//    pair (see moe_dev.h), and bf16 dot2 instructions accumulate them against
//    the P16-paired activations; the affine map is applied once per unit:
//    s * acc + (z - 128 s) * sum(x);
//  * a row's partial sums are reduced across its lanes with a fixed butterfly;
//  * gate/up: a wave owns a gate row and the matching up row, so SwiGLU happens
//    in registers; h goes out as bf16 in the P16 layout the down pass reads;
//  * down: a workgroup owns a block of output rows for all tokens, walks the hit
//    experts in ascending id (prefetching D experts' rows at a time) and adds
//    w * y per token in that fixed order: no atomics, bit-reproducible.
#include "../../include/moe.h"
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void x_unit_pairs(const uint32_t* __restrict__ xr, int u, uint32_t (&xp)[16])
{
    // xr: a token's bf16 row as dwords; unit u covers inputs 32u..32u+31.
    uint32_t d[16];
    const uint4* q = (const uint4*)(xr + 16 * u);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint4 t = q[v];
        d[4 * v + 0] = t.x;
        d[4 * v + 1] = t.y;
        d[4 * v + 2] = t.z;
        d[4 * v + 3] = t.w;
    }
    // pair i = (x_i, x_{i+16}); x_i is half (i & 1) of dword i/2
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t lo = d[i >> 1], hi = d[8 + (i >> 1)];
        xp[i] = (i & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                        : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
}

template <int B, int UPL>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(
    const uint16_t* __restrict__ x, int H, int I, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ pass_table,
    const int32_t* __restrict__ table, const uint8_t* __restrict__ pool, int64_t n_slots,
    int64_t slot_bytes, int64_t off_codes, int64_t off_sb, uint16_t* __restrict__ hbuf,
    uint32_t* __restrict__ err, int LPR)
{
    const int hit = blockIdx.y;
    if (hit >= pass_table[0]) return;
    const int e = pass_table[2 + hit];
    const int32_t slot = table[e];
    if (slot < 0 || slot >= n_slots) {
        if (threadIdx.x == 0 && err) atomicOr(err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
        return;
    }
    const int base = offsets[e], cnt = offsets[e + 1] - base;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int RPP = 64 / LPR;
    const int n = (blockIdx.x * 4 + wave) * RPP + lane / LPR;  // gate row; up row is I + n
    const int seg = lane & (LPR - 1);
    if (n >= I) return;  // whole lane segments leave together

    const uint8_t* rowb = pool + (size_t)slot * (size_t)slot_bytes;
    const size_t row_dw = (size_t)H * B / 32;
    const uint32_t* gc = (const uint32_t*)(rowb + off_codes) + (size_t)n * row_dw;
    const uint32_t* uc = (const uint32_t*)(rowb + off_codes) + (size_t)(I + n) * row_dw;
    const uint32_t* gsb = (const uint32_t*)(rowb + off_sb) + (size_t)n * (H / 64);
    const uint32_t* usb = (const uint32_t*)(rowb + off_sb) + (size_t)(I + n) * (H / 64);
    constexpr float off = Code<B>::offset;

    uint32_t gp[UPL][16], up[UPL][16];
    float gs[UPL], gz[UPL], us[UPL], uz[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
        const int u = seg + LPR * j;
        uint32_t gw[B], uw[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            gw[b] = gc[u * B + b];
            uw[b] = uc[u * B + b];
        }
        unit_pairs<B>(gw, gp[j]);
        unit_pairs<B>(uw, up[j]);
        if constexpr (Code<B>::affine) {
            const uint32_t g2 = gsb[u >> 1], u2 = usb[u >> 1];
            gs[j] = half_bits_to_f32(g2 & 0xFFFFu);
            gz[j] = __builtin_fmaf(-off, gs[j], half_bits_to_f32(g2 >> 16));
            us[j] = half_bits_to_f32(u2 & 0xFFFFu);
            uz[j] = __builtin_fmaf(-off, us[j], half_bits_to_f32(u2 >> 16));
        }
    }

    for (int p = 0; p < cnt; ++p) {
        const int pair = sorted_pairs[base + p];
        const int t = pair / k;
        const uint32_t* xr = (const uint32_t*)(x + (size_t)t * H);
        float g = 0.0f, uu = 0.0f;
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            uint32_t xpair[16];
            x_unit_pairs(xr, seg + LPR * j, xpair);
            float X = 0.0f, ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (Code<B>::affine) X = dot2(xpair[i], MOE_ONES_PAIR, X);
                ag = dot2(gp[j][i], xpair[i], ag);
                au = dot2(up[j][i], xpair[i], au);
            }
            if constexpr (Code<B>::affine) {
                g += gs[j] * ag + gz[j] * X;
                uu += us[j] * au + uz[j] * X;
            } else {
                g += ag;
                uu += au;
            }
        }
        g = seg_sum(g, LPR);
        uu = seg_sum(uu, LPR);
        if (seg == 0) {
            const int pos = (n & ~31) | p16_pos(n & 31);
            hbuf[(size_t)(base + p) * I + pos] = f32_to_bf16(silu_mul(g, uu));
        }
    }
}

template <int B, int UPL, int D>
__global__ __launch_bounds__(64) void gemv_down_kernel(
    int T, int H, int I, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ pass_table,
    const float* __restrict__ topk_w, const int32_t* __restrict__ table,
    const uint8_t* __restrict__ pool, int64_t n_slots, int64_t slot_bytes, int64_t off_codes,
    int64_t off_sb, const uint16_t* __restrict__ hbuf, uint16_t* __restrict__ out,
    uint32_t* __restrict__ err, int LPR)
{
    extern __shared__ float s_acc[];  // [T][RPP]
    const int lane = threadIdx.x;
    const int RPP = 64 / LPR;
    const int rloc = lane / LPR, seg = lane & (LPR - 1);
    const int n = blockIdx.x * RPP + rloc;  // output row
    for (int i = lane; i < T * RPP; i += 64) s_acc[i] = 0.0f;
    __syncthreads();

    const size_t row_dw = (size_t)I * B / 32;
    constexpr float off = Code<B>::offset;
    const int n_hit = pass_table[0];
    for (int h0 = 0; h0 < n_hit; h0 += D) {
        uint32_t cw[D][UPL][B];
        uint32_t sb[D][UPL];
        int ebase[D], ecnt[D];
        bool ok[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            ok[d] = false;
            ebase[d] = 0;
            ecnt[d] = 0;
            if (h0 + d < n_hit) {
                const int e = pass_table[2 + h0 + d];
                const int32_t slot = table[e];
                if (slot < 0 || slot >= n_slots) {
                    if (lane == 0 && err)
                        atomicOr(err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
                } else {
                    ok[d] = true;
                    ebase[d] = offsets[e];
                    ecnt[d] = offsets[e + 1] - ebase[d];
                    const uint8_t* rowb = pool + (size_t)slot * (size_t)slot_bytes;
                    const uint32_t* c = (const uint32_t*)(rowb + off_codes) + (size_t)n * row_dw;
                    const uint32_t* s2 = (const uint32_t*)(rowb + off_sb) + (size_t)n * (I / 64);
#pragma unroll
                    for (int j = 0; j < UPL; ++j) {
                        const int u = seg + LPR * j;
#pragma unroll
                        for (int b = 0; b < B; ++b) cw[d][j][b] = c[u * B + b];
                        if constexpr (Code<B>::affine) sb[d][j] = s2[u >> 1];
                    }
                }
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (!ok[d]) continue;
            uint32_t cp[UPL][16];
            float s[UPL], z[UPL];
#pragma unroll
            for (int j = 0; j < UPL; ++j) {
                unit_pairs<B>(cw[d][j], cp[j]);
                if constexpr (Code<B>::affine) {
                    s[j] = half_bits_to_f32(sb[d][j] & 0xFFFFu);
                    z[j] = __builtin_fmaf(-off, s[j], half_bits_to_f32(sb[d][j] >> 16));
                }
            }
            for (int p = 0; p < ecnt[d]; ++p) {
                const int pos = ebase[d] + p;
                const int pair = sorted_pairs[pos];
                const uint32_t* hr = (const uint32_t*)(hbuf + (size_t)pos * I);
                float y = 0.0f;
#pragma unroll
                for (int j = 0; j < UPL; ++j) {
                    const uint4* q = (const uint4*)(hr + 16 * (seg + LPR * j));
                    uint32_t hp[16];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint4 t4 = q[v];
                        hp[4 * v + 0] = t4.x;
                        hp[4 * v + 1] = t4.y;
                        hp[4 * v + 2] = t4.z;
                        hp[4 * v + 3] = t4.w;
                    }
                    float X = 0.0f, a = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        if constexpr (Code<B>::affine) X = dot2(hp[i], MOE_ONES_PAIR, X);
                        a = dot2(cp[j][i], hp[i], a);
                    }
                    if constexpr (Code<B>::affine) y += s[j] * a + z[j] * X;
                    else y += a;
                }
                y = seg_sum(y, LPR);
                if (seg == 0) {
                    const int t = pair / k;
                    s_acc[t * RPP + rloc] += topk_w[pair] * y;
                }
            }
        }
    }
    __syncthreads();
    for (int i = lane; i < T * RPP; i += 64) {
        const int t = i / RPP, r = i - t * RPP;
        out[(size_t)t * H + (size_t)blockIdx.x * RPP + r] = f32_to_bf16(s_acc[i]);
    }
}

// lanes per row (power of two <= 64 dividing the row's unit count) and units per lane
bool lanes_for(int units, int* lpr, int* upl)
{
    int l = units & -units;
    if (l > 64) l = 64;
    const int u = units / l;
    if (u < 1 || u > 4) return false;
    *lpr = l;
    *upl = u;
    return true;
}

template <int B>
hipError_t gateup_b(int upl, dim3 grid, hipStream_t s, const uint16_t* x, int H, int I, int k,
                    const SortView& sv, const int32_t* table, const uint8_t* pool,
                    const ClassView& c, uint16_t* hbuf, uint32_t* err, int lpr)
{
#define MOE_GU(U)                                                                              \
    hipLaunchKernelGGL((gemv_gateup_kernel<B, U>), grid, dim3(256), 0, s, x, H, I, k, sv.offsets, \
                       sv.sorted_pairs, sv.pass_table, table, pool, c.n_slots, c.slot_bytes,     \
                       c.off_gu_codes, c.off_gu_sb, hbuf, err, lpr)
    switch (upl) {
    case 1: MOE_GU(1); break;
    case 2: MOE_GU(2); break;
    case 3: MOE_GU(3); break;
    case 4: MOE_GU(4); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_GU
    return hipGetLastError();
}

template <int B>
hipError_t down_b(int upl, dim3 grid, size_t lds, hipStream_t s, int T, int H, int I, int k,
                  const SortView& sv, const float* w, const int32_t* table, const uint8_t* pool,
                  const ClassView& c, const uint16_t* hbuf, uint16_t* out, uint32_t* err, int lpr)
{
#define MOE_DN(U, D)                                                                             \
    hipLaunchKernelGGL((gemv_down_kernel<B, U, D>), grid, dim3(64), lds, s, T, H, I, k,           \
                       sv.offsets, sv.sorted_pairs, sv.pass_table, w, table, pool, c.n_slots,      \
                       c.slot_bytes, c.off_d_codes, c.off_d_sb, hbuf, out, err, lpr)
    // experts prefetched per step (bf16 rows hold 16 words per unit, so fewer)
    constexpr bool W16 = B == 16;
    switch (upl) {
    case 1: MOE_DN(1, W16 ? 5 : 8); break;
    case 2: MOE_DN(2, W16 ? 2 : 4); break;
    case 3: MOE_DN(3, W16 ? 1 : 2); break;
    case 4: MOE_DN(4, W16 ? 1 : 2); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_DN
    return hipGetLastError();
}

}  // namespace

constexpr int kGemvMaxT = 64;

bool gemv_supported(int T, int k, const ClassView& c)
{
    int l, u;
    (void)k;
    return T <= kGemvMaxT && lanes_for(c.H / 32, &l, &u) && lanes_for(c.I / 32, &l, &u);
}

hipError_t launch_gemv_gateup(const uint16_t* x, int T, int k, int E, const SortView& sv,
                              const int32_t* table, const uint8_t* pool, const ClassView& c,
                              uint16_t* hbuf, uint32_t* err, hipStream_t s)
{
    int lpr, upl;
    if (!lanes_for(c.H / 32, &lpr, &upl)) return hipErrorInvalidValue;
    const int rpp = 64 / lpr;
    const int max_hit = (int64_t)T * k < E ? T * k : E;
    dim3 grid((c.I + 4 * rpp - 1) / (4 * rpp), max_hit);
    switch (c.bits_gu) {
    case 3: return gateup_b<3>(upl, grid, s, x, c.H, c.I, k, sv, table, pool, c, hbuf, err, lpr);
    case 4: return gateup_b<4>(upl, grid, s, x, c.H, c.I, k, sv, table, pool, c, hbuf, err, lpr);
    case 6: return gateup_b<6>(upl, grid, s, x, c.H, c.I, k, sv, table, pool, c, hbuf, err, lpr);
    case 8: return gateup_b<8>(upl, grid, s, x, c.H, c.I, k, sv, table, pool, c, hbuf, err, lpr);
    case 16: return gateup_b<16>(upl, grid, s, x, c.H, c.I, k, sv, table, pool, c, hbuf, err, lpr);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_down(int T, int k, int E, const SortView& sv, const float* topk_w,
                            const int32_t* table, const uint8_t* pool, const ClassView& c,
                            const uint16_t* hbuf, uint16_t* out, uint32_t* err, hipStream_t s)
{
    (void)E;
    int lpr, upl;
    if (!lanes_for(c.I / 32, &lpr, &upl)) return hipErrorInvalidValue;
    const int rpp = 64 / lpr;
    dim3 grid(c.H / rpp);
    const size_t lds = (size_t)T * rpp * sizeof(float);
    switch (c.bits_d) {
    case 3: return down_b<3>(upl, grid, lds, s, T, c.H, c.I, k, sv, topk_w, table, pool, c, hbuf, out, err, lpr);
    case 4: return down_b<4>(upl, grid, lds, s, T, c.H, c.I, k, sv, topk_w, table, pool, c, hbuf, out, err, lpr);
    case 6: return down_b<6>(upl, grid, lds, s, T, c.H, c.I, k, sv, topk_w, table, pool, c, hbuf, out, err, lpr);
    case 8: return down_b<8>(upl, grid, lds, s, T, c.H, c.I, k, sv, topk_w, table, pool, c, hbuf, out, err, lpr);
    case 16: return down_b<16>(upl, grid, lds, s, T, c.H, c.I, k, sv, topk_w, table, pool, c, hbuf, out, err, lpr);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
