// mfma.hip — prefill path of the routed-expert layer on gfx950: a grouped
// dequantizing GEMM on bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", How the
// prototype works, Prefill (a long prompt touches almost all experts, which are
// then processed by a sorted, gathered quantized matmul, 64 experts per batch)
// and Quantized experts (group-wise affine format); "POC: Experts offload",
// commit messages (the sorted prefill's batches of 64 experts).
//
// Work split: a workgroup owns (hit expert, 64 output columns); each of its 4
// waves owns 16 columns and loops over the expert's rows (its sorted pairs) in
// M-tiles of 16, MT M-tiles per sweep of K.  The K sweep is a software pipeline
// of 128-input stages: coalesced 16-byte loads of the stage's raw codes,
// scale/bias and activation rows go to registers two stages ahead, are written
// to an LDS double buffer one stage ahead, and the matrix cores consume the
// current stage from LDS.  Workgroup barriers fence LDS only, so the global
// loads of later stages stay in flight across them.  Lane (column n, lane group
// g) turns the dwords of its unit in LDS into 4 bf16 pairs (128 + c, the P16
// pairing); the activations were laid out in the same P16 order, so one 16-byte
// LDS read per lane is the A operand.
//
// The affine map is applied per group of 64 inputs after the matrix core has
// summed codes against activations:
//     sum_{i in g} x_i (s c_i + z) = s * [sum x (128 + c)] + (z - 128 s) * [sum x]
// Both brackets are MFMA results (the second against a B operand of ones), so
// the codes never need a scale multiply or a float conversion.
//
// gate/up: SwiGLU in registers (a wave holds gate column n and up column I + n
// in identical accumulator layouts), h written as bf16 in P16 order.
// down: y per (pair, output) in bf16 to a workspace; a combine kernel adds the
// k contributions of each token in j order (deterministic).
//
// Widths 3, 4, 6 and 8 run mfma_lds_kernel instead: the same arithmetic with
// each stage loaded straight into LDS (no staging registers), and down with 128
// output columns per workgroup.  Width 16 runs mfma_grouped_kernel, staging 64
// inputs at a time (its rows are four times wider than 3-bit rows).
#include <utility>

#include "../../include/moe.h"
#include "moe_dev.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// Calls f(std::integral_constant<int, i>) for i = 0..N-1 (indices known at compile time).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ f32x4_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// The 4 P16 pairs (codes 4g+r and 4g+r+16, r = 0..3) of lane group g in the
// unit starting at dword pointer `unit`.
template <int B>
__device__ __forceinline__ u32x4_t lane_pairs(const uint32_t* __restrict__ unit, int g)
{
    u32x4_t r;
    if constexpr (B == 16) {  // bf16 weights: values 4g+r at half r&1 of word 2g + r/2, +16 at word 8 + ...
        const uint32_t l0 = unit[2 * g], l1 = unit[2 * g + 1];
        const uint32_t h0 = unit[8 + 2 * g], h1 = unit[9 + 2 * g];
        r.x = __builtin_amdgcn_perm(h0, l0, 0x05040100u);
        r.y = __builtin_amdgcn_perm(h0, l0, 0x07060302u);
        r.z = __builtin_amdgcn_perm(h1, l1, 0x05040100u);
        r.w = __builtin_amdgcn_perm(h1, l1, 0x07060302u);
    } else if constexpr (B == 8) {
        const uint32_t lo = unit[g], hi = unit[4 + g];
        const float a0 = ubyte_f32<0>(lo), b0 = ubyte_f32<0>(hi);
        const float a1 = ubyte_f32<1>(lo), b1 = ubyte_f32<1>(hi);
        const float a2 = ubyte_f32<2>(lo), b2 = ubyte_f32<2>(hi);
        const float a3 = ubyte_f32<3>(lo), b3 = ubyte_f32<3>(hi);
        r.x = __builtin_amdgcn_perm(__float_as_uint(b0), __float_as_uint(a0), 0x07060302u);
        r.y = __builtin_amdgcn_perm(__float_as_uint(b1), __float_as_uint(a1), 0x07060302u);
        r.z = __builtin_amdgcn_perm(__float_as_uint(b2), __float_as_uint(a2), 0x07060302u);
        r.w = __builtin_amdgcn_perm(__float_as_uint(b3), __float_as_uint(a3), 0x07060302u);
    } else {
        const int ol = 4 * g * B;              // first low code bit
        const int oh = ol + 16 * B - 16;       // window whose bit 16 is the first high code bit
        const int dl = ol >> 5, sl = ol & 31;
        const int dh = oh >> 5, sh = oh & 31;
        constexpr int S = Code<B>::per_t;  // 5 (B=3), 4 (B=4), 2 (B=6)
        constexpr uint32_t M2 = Code<B>::mask2;
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 4; q += S) {
            // 32-bit funnel shifts of two adjacent words (the shift stays below 32:
            // sl, sh < 32 and q * B + sl < 32 whenever q > 0 is reached)
            const int ql = sl + q * B, qh = sh + q * B;
            const uint32_t wl = __builtin_amdgcn_alignbit(unit[dl + 1 + (ql >> 5)], unit[dl + (ql >> 5)], ql & 31);
            const uint32_t wh = __builtin_amdgcn_alignbit(unit[dh + 1 + (qh >> 5)], unit[dh + (qh >> 5)], qh & 31);
            const uint32_t t = __builtin_amdgcn_perm(wh, wl, 0x07060100u);  // low half of wl, high half of wh
#pragma unroll
            for (int m = 0; m < S; ++m)
                if (q + m < 4) p[q + m] = bits_or_magic<M2>(t >> (B * m));
        }
        r.x = p[0];
        r.y = p[1];
        r.z = p[2];
        r.w = p[3];
    }
    return r;
}

constexpr int kKC = 128;          // K per pipeline stage
constexpr int kUPC = kKC / 32;    // pack units per stage
constexpr int kGPC = kKC / 64;    // groups per stage

// K per pipeline stage of the register-staged kernel: 128 inputs, 64 for width 16
// (its code rows are four times wider: 128 inputs would take 87 KB of LDS per
// gate/up workgroup, one workgroup per CU).
template <int B>
constexpr int stage_k() { return B == 16 ? 64 : kKC; }

// Dwords of padding after each staged code row.  The 16 lanes of a lane group
// read one column of 16 consecutive rows, and the lane group that shares their
// LDS cycle reads the same column or a neighbouring one (width 16: 64-bit reads,
// columns two apart).  A row stride of 2 (mod 4) dwords puts the 16 rows on
// distinct even banks (mod 32) and a column one dword over on the odd ones, so
// no read conflicts; the unpadded widths put rows r and r + 8 (or more) on one
// bank.  Rows stay 8-byte aligned.
template <int B>
constexpr int code_pad() { return 2; }

// One pipeline stage in LDS: raw codes and scale/bias of the workgroup's NB*64
// weight rows for stage_k<B>() inputs, and as many activations of up to MT*16
// rows (rows padded by 8 bf16: conflict-free reads).
template <int B, int NB, int MT>
struct Stage {
    uint32_t codes[NB * 64][stage_k<B>() / 32 * B + code_pad<B>()];
    uint32_t sb[NB * 64][stage_k<B>() / 64];
    uint16_t a[MT * 16][stage_k<B>() + 8];
};

// Workgroup barrier that orders LDS only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The 4 P16 pairs of lane group g from the dwords of one unit held in LDS
// (same bit arithmetic as lane_pairs, reading LDS instead of global memory).
template <int B>
__device__ __forceinline__ u32x4_t lds_pairs(const uint32_t* __restrict__ unit, int g)
{
    if constexpr (B == 8) {
        return lane_pairs<8>(unit, g);
    } else {
        return lane_pairs<B>(unit, g);
    }
}

// Grouped dequantizing GEMM for one hit expert and 64 output columns per
// workgroup (16 per wave), pipelined through registers and LDS in stages of KC
// inputs (see the top of this file).
//   GU = true : gate/up.  Weight rows: gate n0..n0+63 and up I+n0..; A = P16 x
//               rows of the expert's pairs (via sorted_pairs); epilogue SwiGLU
//               -> h (bf16, P16) at the pair's sorted position.
//   GU = false: down.  Weight rows n0..n0+63 of the down matrix; A = h rows;
//               epilogue y (bf16) at [pair id][n].
// 32-row sweeps of narrow codes (and of width 16, with its 64-input stages) fit
// 168 VGPRs: three waves per SIMD.
template <int B, bool GU, int MT, int CBW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((B <= 4 || B == 16) && MT == 2 ? 3 : 1)))
void mfma_grouped_kernel(
    const uint16_t* __restrict__ act, int H, int I, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ pass_table, int E,
    int pass_lo, int pass_hi, const int32_t* __restrict__ table, const uint8_t* __restrict__ pool,
    int64_t n_slots, int64_t slot_bytes, int64_t off_codes, int64_t off_sb,
    uint16_t* __restrict__ hbuf, uint16_t* __restrict__ ybuf, uint32_t* __restrict__ err)
{
    constexpr int NB = GU ? 2 : 1;
    constexpr int KC = stage_k<B>(), UPC = KC / 32, GPC = KC / 64;
    __shared__ Stage<B, NB, MT> st[2];
    // XCD-aware tile order: workgroup L runs on XCD L % 8, so the workgroups of
    // one expert are given the same L % 8 -- they share one L2 and fetch the
    // expert's activation rows from memory once, not once per workgroup.  A
    // workgroup takes CBW consecutive column blocks of 64.
    const int ncb = (GU ? I : H) / 64;          // column blocks per expert
    const int nwg = (ncb + CBW - 1) / CBW;      // workgroups per expert
    const int L = blockIdx.x, r8 = L >> 3;
    const int cb0 = (r8 % nwg) * CBW;
    const int ncb_wg = min(CBW, ncb - cb0);     // column blocks of this workgroup
    // the hit experts of passes [pass_lo, pass_hi): a contiguous run of the hit list
    const int hit = pass_table[2 + E + pass_lo] + (r8 / nwg) * 8 + (L & 7);
    if (hit >= pass_table[2 + E + pass_hi]) return;
    const int e = pass_table[2 + hit];
    const int32_t slot = table[e];
    if (slot < 0 || slot >= n_slots) {
        if (threadIdx.x == 0 && err) atomicOr(err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
        return;
    }
    const int base = offsets[e], cnt = offsets[e + 1] - base;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int K = GU ? H : I;            // reduction length
    const int NC = K / KC;              // full K stages per column block
    const bool tail = (K % KC) != 0;    // a last half stage of 64 inputs
    const int n_kc = NC + (tail ? 1 : 0);
    const int n_stages = ncb_wg * n_kc;  // stage s: column block cb0 + s / n_kc, K chunk s % n_kc

    const uint8_t* rowb = pool + (size_t)slot * (size_t)slot_bytes;
    const size_t row_dw = (size_t)K * B / 32;
    const uint32_t* codes = (const uint32_t*)(rowb + off_codes);
    const uint32_t* sbg = (const uint32_t*)(rowb + off_sb);
    constexpr float off = Code<B>::offset;
    const u32x4_t ones = {MOE_ONES_PAIR, MOE_ONES_PAIR, MOE_ONES_PAIR, MOE_ONES_PAIR};
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

    // weight row (in the whole matrix) of local row r of the column block at n0
#define wrow(R) (GU ? ((R) < 64 ? n0_ + (R) : I + n0_ + ((R) - 64)) : n0_ + (R))

    // staging assignment: B pieces (16 B), sb dwords, A pieces (16 B)
    constexpr int PPR = KC * B / 128;                    // 16-byte pieces per row per stage
    constexpr int BPIECES = NB * 64 * PPR;               // per stage
    constexpr int BPT = (BPIECES + 255) / 256;
    constexpr int SBN = NB * 64 * GPC;                  // sb dwords per stage
    constexpr int APT = MT * 16 * (KC / 8) / 256;       // A pieces per thread

    for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
        const int rows = min(16 * MT, cnt - m0);
        const int nmt = (rows + 15) >> 4;
        // activation row pointers of this thread's A pieces (fixed for the sweep)
        // rows past the expert's last pair re-read its last row (results discarded)
        const uint16_t* arow[APT];
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int q = tid + 256 * i;
            int m = q / (KC / 8);
            m = m < rows ? m : rows - 1;
            if (GU) arow[i] = act + (size_t)(sorted_pairs[base + m0 + m] / k) * H;
            else arow[i] = act + (size_t)(base + m0 + m) * I;
        }
        // two register sets (stages in flight); every staging load is unconditional
        // (indices clamped to valid data), so the staging registers are never spilled
        u32x4_t rb0[BPT], ra0[APT], rb1[BPT], ra1[APT];
        uint32_t rs0, rs1;
#define MOE_LOAD_STAGE(C, RB, RS, RA)                                                           \
    {                                                                                           \
        const int cbl_ = (C) / n_kc;                                                            \
        const int n0_ = (cb0 + cbl_) * 64;                                                      \
        const int kin_ = ((C) - cbl_ * n_kc) * KC;                                             \
        const int units_ = (kin_ + KC <= K) ? UPC : (K - kin_) / 32;                          \
        static_for<BPT>([&](auto I_) {                                                          \
            constexpr int i = decltype(I_)::value;                                              \
            int q = tid + 256 * i;                                                              \
            q = q < BPIECES ? q : BPIECES - 1;                                                  \
            const int r = q / PPR;                                                              \
            int p = q - r * PPR;                                                                \
            p = p * 4 < units_ * B ? p : 0;                                                     \
            RB[i] = *(const u32x4_t*)(codes + (size_t)wrow(r) * row_dw + (size_t)(kin_ / 32) * B + p * 4); \
        });                                                                                     \
        if constexpr (Code<B>::affine) {                                                        \
            const int qs = tid < SBN ? tid : SBN - 1;                                           \
            const int r = qs / GPC;                                                            \
            int gg = qs - r * GPC;                                                             \
            gg = gg * 64 < units_ * 32 ? gg : 0;                                                \
            RS = sbg[(size_t)wrow(r) * (K / 64) + kin_ / 64 + gg];                              \
        }                                                                                       \
        static_for<APT>([&](auto I_) {                                                          \
            constexpr int i = decltype(I_)::value;                                              \
            int p = (tid + 256 * i) % (KC / 8);                                                \
            p = p * 8 < units_ * 32 ? p : 0;                                                    \
            RA[i] = *(const u32x4_t*)(arow[i] + kin_ + p * 8);                                  \
        });                                                                                     \
    }
#define MOE_STORE_STAGE(BUF, RB, RS, RA)                                                        \
    {                                                                                           \
        Stage<B, NB, MT>& S_ = st[(BUF)];                                                       \
        static_for<BPT>([&](auto I_) {                                                          \
            constexpr int i = decltype(I_)::value;                                              \
            const int q = tid + 256 * i;                                                        \
            if (q < BPIECES) {                                                                  \
                const int r = q / PPR, p = q - r * PPR;                                         \
                *(u32x2_t*)(&S_.codes[r][p * 4]) = u32x2_t{RB[i].x, RB[i].y};                   \
                *(u32x2_t*)(&S_.codes[r][p * 4 + 2]) = u32x2_t{RB[i].z, RB[i].w};               \
            }                                                                                   \
        });                                                                                     \
        if (Code<B>::affine && tid < SBN) S_.sb[tid / GPC][tid % GPC] = RS;                   \
        static_for<APT>([&](auto I_) {                                                          \
            constexpr int i = decltype(I_)::value;                                              \
            const int q = tid + 256 * i;                                                        \
            *(u32x4_t*)(&S_.a[q / (KC / 8)][(q % (KC / 8)) * 8]) = RA[i];                    \
        });                                                                                     \
    }
#define MOE_COMPUTE_STAGE(BUF, C)                                                               \
    {                                                                                           \
        const Stage<B, NB, MT>& S = st[(BUF)];                                                  \
        const int cbl = (C) / n_kc;                                                             \
        const int kin = ((C) - cbl * n_kc) * KC;                                               \
        const int groups = (kin + KC <= K) ? GPC : (K - kin) / 64;                            \
        for (int G2 = 0; G2 < groups; ++G2) compute_group(S, G2);                               \
        if (kin + KC >= K) {                                                                   \
            epilogue((cb0 + cbl) * 64 + wave * 16 + c16);                                       \
            _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                   \
                _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = zero;           \
        }                                                                                       \
    }

        f32x4_t acc[NB][MT];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = zero;
        // results of this lane's column n for the sweep's rows
        auto epilogue = [&](int n) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < nmt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = m0 + mt * 16 + 4 * g + i;
                        if (r < cnt) {
                            if constexpr (GU) {
                                const int pos = (n & ~31) | p16_pos(n & 31);
                                hbuf[(size_t)(base + r) * I + pos] = f32_to_bf16(silu_mul(acc[0][mt][i], acc[1][mt][i]));
                            } else {
                                ybuf[(size_t)sorted_pairs[base + r] * H + n] = f32_to_bf16(acc[0][mt][i]);
                            }
                        }
                    }
                }
            }
        };

        // one group of 64 inputs of the stage in LDS: B operands, then the matrix cores
        auto compute_group = [&](const Stage<B, NB, MT>& S, int G2) __attribute__((always_inline)) {
            u32x4_t bw[NB][2];
            float sc[NB], zc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int r = nb * 64 + wave * 16 + c16;
                bw[nb][0] = lds_pairs<B>(&S.codes[r][(2 * G2) * B], g);
                bw[nb][1] = lds_pairs<B>(&S.codes[r][(2 * G2 + 1) * B], g);
                if constexpr (Code<B>::affine) {
                    const uint32_t s2 = S.sb[r][G2];
                    sc[nb] = half_bits_to_f32(s2 & 0xFFFFu);
                    zc[nb] = __builtin_fmaf(-off, sc[nb], half_bits_to_f32(s2 >> 16));
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < nmt) {
                    const u32x4_t a0 = *(const u32x4_t*)(&S.a[mt * 16 + c16][(2 * G2) * 32 + 8 * g]);
                    const u32x4_t a1 = *(const u32x4_t*)(&S.a[mt * 16 + c16][(2 * G2 + 1) * 32 + 8 * g]);
                    if constexpr (Code<B>::affine) {
                        f32x4_t tx = mfma(a0, ones, zero);
                        tx = mfma(a1, ones, tx);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            f32x4_t t = mfma(a0, bw[nb][0], zero);
                            t = mfma(a1, bw[nb][1], t);
#pragma unroll
                            for (int q_ = 0; q_ < 4; ++q_)
                                acc[nb][mt][q_] = __builtin_fmaf(sc[nb], t[q_], __builtin_fmaf(zc[nb], tx[q_], acc[nb][mt][q_]));
                        }
                    } else {  // bf16 weights: the matrix cores accumulate in place
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            acc[nb][mt] = mfma(a0, bw[nb][0], acc[nb][mt]);
                            acc[nb][mt] = mfma(a1, bw[nb][1], acc[nb][mt]);
                        }
                    }
                }
            }
        };

        // prologue: stages 0 and 1 in flight, stage 0 into LDS
        MOE_LOAD_STAGE(0, rb0, rs0, ra0)
        if (n_stages > 1) MOE_LOAD_STAGE(1, rb1, rs1, ra1)
        MOE_STORE_STAGE(0, rb0, rs0, ra0)
        lds_barrier();
        for (int c = 0; c < n_stages; c += 2) {
            // even stage c: registers 0 take stage c+2, LDS 1 takes stage c+1
            if (c + 2 < n_stages) MOE_LOAD_STAGE(c + 2, rb0, rs0, ra0)
            MOE_COMPUTE_STAGE(0, c)
            if (c + 1 < n_stages) MOE_STORE_STAGE(1, rb1, rs1, ra1)
            lds_barrier();
            if (c + 1 >= n_stages) break;
            // odd stage c+1: registers 1 take stage c+3, LDS 0 takes stage c+2
            if (c + 3 < n_stages) MOE_LOAD_STAGE(c + 3, rb1, rs1, ra1)
            MOE_COMPUTE_STAGE(1, c + 1)
            if (c + 2 < n_stages) MOE_STORE_STAGE(0, rb0, rs0, ra0)
            lds_barrier();
        }
#undef MOE_LOAD_STAGE
#undef MOE_STORE_STAGE
#undef MOE_COMPUTE_STAGE

    }
#undef wrow
}

// Widths 3, 4, 6, 8: the same grouped GEMM with the stages moved from global memory
// straight into LDS (global_load_lds_dwordx4 / _dword: lane i of a load writes
// 16 or 4 bytes at the wave's LDS base + 16 i or 4 i).  No staging registers
// and no VALU copies into LDS: gate/up spends the registers saved on both
// groups of a stage in flight at once.  Down takes two blocks of 64 columns per
// workgroup (128 weight rows, like gate and up), so each wave carries two
// independent chains and one staging of the h rows serves both.  Two LDS
// buffers: stage c + 1 lands while stage c is consumed.  Layouts in a buffer:
//   codes  row r at 16-byte slots [S r, S r + B): the row's B pieces (S = B, or
//          B + 1 for even B, see row_slots)
//   sb     row r at dwords 2 r, 2 r + 1
//   a      row m at dwords [64 m, 64 m + 64); its 16-byte chunk c sits in slot
//          c ^ (m & 15), so the 16 rows read by one lane group spread over the banks
constexpr int kKC3 = 128;               // inputs per stage of the LDS-loading kernel
constexpr int kGPC3 = kKC3 / 64;         // groups per stage
constexpr int kCPR3 = kKC3 / 8;          // 16-byte activation chunks per row and stage
static_assert(kKC3 % 128 == 0, "whole 16-byte code pieces per row");
// 16-byte code pieces per row and stage, and the LDS slots a staged row takes:
// one more (never loaded) for widths whose piece count is even, so that the 16
// rows a lane group reads start on 16 distinct banks (a row stride of 3, 5, 7
// or 9 pieces; 4, 6 or 8 would put several rows on one bank)
template <int B>
constexpr int ppr() { return kKC3 * B / 128; }
template <int B>
constexpr int row_slots() { return ppr<B>() % 2 ? ppr<B>() : ppr<B>() + 1; }
template <int B, int NB, int MT>
struct DmaStage {
    uint32_t codes[NB * 64 * 4 * row_slots<B>()];
    uint32_t sb[NB * 64 * kGPC3];
    uint32_t a[MT * 16 * (kKC3 / 2)];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_wave_base, 4, 0, 0);
}

template <int B, bool GU, int MT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT <= 2 ? (GU ? 3 : 4) : 1)))
void mfma_lds_kernel(
    const uint16_t* __restrict__ act, int H, int I, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ pass_table, int E,
    int pass_lo, int pass_hi, const int32_t* __restrict__ table, const uint8_t* __restrict__ pool,
    int64_t n_slots, int64_t slot_bytes, int64_t off_codes, int64_t off_sb,
    uint16_t* __restrict__ hbuf, uint16_t* __restrict__ ybuf, uint32_t* __restrict__ err)
{
    constexpr int NB = 2;  // gate and up / two blocks of 64 down columns
    constexpr int ROWS = NB * 64;
    __shared__ DmaStage<B, NB, MT> st[2];
    constexpr int PPR = ppr<B>(), RS = row_slots<B>();
    // tile order as in mfma_grouped_kernel (one column block per workgroup)
    const int ncb = GU ? I / 64 : (H / 64 + 1) / 2;
    const int L = blockIdx.x, r8 = L >> 3;
    const int cb0 = r8 % ncb;
    const int hit = pass_table[2 + E + pass_lo] + (r8 / ncb) * 8 + (L & 7);
    if (hit >= pass_table[2 + E + pass_hi]) return;
    const int e = pass_table[2 + hit];
    const int32_t slot = table[e];
    if (slot < 0 || slot >= n_slots) {
        if (threadIdx.x == 0 && err) atomicOr(err, slot < 0 ? MOE_ERRW_NOT_RESIDENT : MOE_ERRW_BAD_SLOT);
        return;
    }
    const int base = offsets[e], cnt = offsets[e + 1] - base;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int K = GU ? H : I;
    const int NC = K / kKC3;
    const bool tail = (K % kKC3) != 0;
    const int n_stages = NC + (tail ? 1 : 0);
    const int n0 = cb0 * (GU ? 64 : 128);

    const uint8_t* rowb = pool + (size_t)slot * (size_t)slot_bytes;
    const size_t row_dw = (size_t)K * B / 32;
    const uint32_t* codes = (const uint32_t*)(rowb + off_codes);
    const uint32_t* sbg = (const uint32_t*)(rowb + off_sb);
    constexpr float off = Code<B>::offset;
    const u32x4_t ones = {MOE_ONES_PAIR, MOE_ONES_PAIR, MOE_ONES_PAIR, MOE_ONES_PAIR};
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    auto wrow = [&](int r) { return GU ? (r < 64 ? n0 + r : I + n0 + (r - 64)) : min(n0 + r, H - 1); };

    // loads of one stage: code slots q = 256 i + tid (row q / RS, piece q % RS;
    // the padding slot is not loaded), sb dwords q = 256 i + tid (row q / kGPC3,
    // group q % kGPC3), activation pieces q = 256 i + tid
    constexpr int BPIECES = ROWS * RS;                   // 16-byte code slots per stage
    constexpr int BPT = (BPIECES + 255) / 256;
    constexpr int SBN = ROWS * kGPC3;                    // sb dwords per stage
    constexpr int SBT = (SBN + 255) / 256;
    constexpr int APT = MT * 16 * kCPR3 / 256;          // 16-byte activation pieces per thread
    static_assert(BPIECES % 64 == 0 && SBN % 64 == 0, "whole waves per load");
    const uint32_t* bsrc[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int q = min(256 * i + tid, BPIECES - 1);
        const int r = q / RS;
        bsrc[i] = codes + (size_t)wrow(r) * row_dw + min(q - r * RS, PPR - 1) * 4;
    }
    const uint32_t* ssrc[SBT];
#pragma unroll
    for (int i = 0; i < SBT; ++i) {
        const int q = min(256 * i + tid, SBN - 1);
        ssrc[i] = sbg + (size_t)wrow(q / kGPC3) * (K / 64) + q % kGPC3;
    }
    const uint16_t* arow_[APT];  // activation row of each A piece, set per sweep
    // stage kin: piece p of a code row is clamped to 0 past the tail's units (the
    // copy lands in LDS but is never read), likewise the sb group and A chunk
    auto issue = [&](int c, int buf) {
        const int kin = c * kKC3;
        const int units = (kin + kKC3 <= K) ? kKC3 / 32 : (K - kin) / 32;
        DmaStage<B, NB, MT>& S = st[buf];
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (256 * i + wave * 64 < BPIECES) {  // wave-uniform
                const int q = 256 * i + tid;
                const int p = q % RS;
                const uint32_t* src = bsrc[i] + (size_t)(kin / 32) * B;
                if (p < PPR) dma16(p * 4 < units * B ? src : src - p * 4, &S.codes[(256 * i + wave * 64) * 4]);
            }
        }
#pragma unroll
        for (int i = 0; i < SBT; ++i) {
            if (256 * i + wave * 64 < SBN) {  // wave-uniform
                const int gg = (256 * i + tid) % kGPC3;
                dma4(ssrc[i] + kin / 64 - (gg * 64 < units * 32 ? 0 : gg), &S.sb[256 * i + wave * 64]);
            }
        }
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int q = 256 * i + tid;
            const int m = q / kCPR3;
            int ch = (q % kCPR3) ^ (m & 15);    // global chunk held by this slot
            ch = ch * 8 < units * 32 ? ch : 0;
            dma16(arow_[i] + kin + ch * 8, &S.a[(256 * i + wave * 64) * 4]);
        }
    };

    for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
        const int rows = min(16 * MT, cnt - m0);
        const int nmt = (rows + 15) >> 4;
        // rows past the expert's last pair re-read its last row (results discarded)
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int m = min((256 * i + tid) / kCPR3, rows - 1);
            if (GU) arow_[i] = act + (size_t)(sorted_pairs[base + m0 + m] / k) * H;
            else arow_[i] = act + (size_t)(base + m0 + m) * I;
        }
        // the row indices have landed before any stage load is issued (the compiler
        // does not count LDS-DMA loads, so its own wait for them would be a vmcnt(0)
        // behind stage 0's code loads)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        f32x4_t acc[NB][MT];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = zero;

        // one group of 64 inputs of the stage in LDS: B operands, then the matrix cores
        auto compute_group = [&](const DmaStage<B, NB, MT>& S, int G2) __attribute__((always_inline)) {
            u32x4_t bw[NB][2];
            float sc[NB], zc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int r = nb * 64 + wave * 16 + c16;
                bw[nb][0] = lds_pairs<B>(&S.codes[r * 4 * RS + (2 * G2) * B], g);
                bw[nb][1] = lds_pairs<B>(&S.codes[r * 4 * RS + (2 * G2 + 1) * B], g);
                const uint32_t s2 = S.sb[r * kGPC3 + G2];
                sc[nb] = half_bits_to_f32(s2 & 0xFFFFu);
                zc[nb] = __builtin_fmaf(-off, sc[nb], half_bits_to_f32(s2 >> 16));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt < nmt) {
                    const int m = mt * 16 + c16;  // m & 15 == c16
                    const u32x4_t a0 = *(const u32x4_t*)(&S.a[m * (kKC3 / 2) + (((8 * G2 + g) ^ c16) * 4)]);
                    const u32x4_t a1 = *(const u32x4_t*)(&S.a[m * (kKC3 / 2) + (((8 * G2 + 4 + g) ^ c16) * 4)]);
                    f32x4_t tx = mfma(a0, ones, zero);
                    tx = mfma(a1, ones, tx);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        f32x4_t t = mfma(a0, bw[nb][0], zero);
                        t = mfma(a1, bw[nb][1], t);
#pragma unroll
                        for (int q_ = 0; q_ < 4; ++q_)
                            acc[nb][mt][q_] = __builtin_fmaf(sc[nb], t[q_], __builtin_fmaf(zc[nb], tx[q_], acc[nb][mt][q_]));
                    }
                }
            }
        };
        auto compute_stage = [&](const DmaStage<B, NB, MT>& S, int c) __attribute__((always_inline)) {
            const int kin = c * kKC3;
            const int groups = (kin + kKC3 <= K) ? kGPC3 : (K - kin) / 64;
            if (GU && groups == kGPC3) {  // gate/up: the stage's groups in one block for the scheduler
#pragma unroll
                for (int G2 = 0; G2 < kGPC3; ++G2) compute_group(S, G2);
            } else {
                for (int G2 = 0; G2 < groups; ++G2) compute_group(S, G2);
            }
        };

        // stage c + 1 lands in the other buffer while stage c is consumed; each
        // wave waits for its own loads, the barrier for everyone's (and for the
        // reads of the buffer the next loads overwrite)
        issue(0, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        lds_barrier();
        for (int c = 0; c < n_stages; c += 2) {
            if (c + 1 < n_stages) issue(c + 1, 1);
            compute_stage(st[0], c);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            lds_barrier();
            if (c + 1 >= n_stages) break;
            if (c + 2 < n_stages) issue(c + 2, 0);
            compute_stage(st[1], c + 1);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            lds_barrier();
        }

        // results of this lane's column n for the sweep's rows
        const int n = n0 + wave * 16 + c16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (mt < nmt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = m0 + mt * 16 + 4 * g + i;
                    if (r < cnt) {
                        if constexpr (GU) {
                            const int pos = (n & ~31) | p16_pos(n & 31);
                            hbuf[(size_t)(base + r) * I + pos] = f32_to_bf16(silu_mul(acc[0][mt][i], acc[1][mt][i]));
                        } else {
                            const size_t yr = (size_t)sorted_pairs[base + r] * H;
                            ybuf[yr + n] = f32_to_bf16(acc[0][mt][i]);
                            if (n + 64 < H) ybuf[yr + n + 64] = f32_to_bf16(acc[1][mt][i]);
                        }
                    }
                }
            }
        }
    }
}

// out[t, n] = bf16( sum_j w[t, j] * y[t*k + j, n] ), j ascending, in fp32 (y is
// stored in bf16, like h: the weighted sum of the k expert outputs is the only
// place they meet).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ ybuf,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, uint16_t* __restrict__ out)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4 outputs per thread
    const int64_t per_t = H / 4;
    if (q >= (int64_t)T * per_t) return;
    const int t = (int)(q / per_t);
    const int n4 = (int)(q - (int64_t)t * per_t) * 4;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const uint2 y = *(const uint2*)(ybuf + ((size_t)t * k + j) * H + n4);
        a0 += wj * bf16lo(y.x);
        a1 += wj * bf16hi(y.x);
        a2 += wj * bf16lo(y.y);
        a3 += wj * bf16hi(y.y);
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
    o.y = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
    *(uint2*)(out + (size_t)t * H + n4) = o;
}

}  // namespace

// Most hit experts passes [pass_lo, pass_hi) can hold: kPassExperts each, and no
// more than the distinct experts the T*k pairs can reach.
static int pass_hits_max(int T, int k, int E, int pass_lo, int pass_hi)
{
    int64_t m = (int64_t)T * k;
    if (m > E) m = E;
    const int64_t p = (int64_t)kPassExperts * (pass_hi - pass_lo);
    return (int)(m < p ? m : p);
}

// M-tiles per sweep: 1 (16 rows) when experts average at most two rows (small
// batches: half the activation loads and matrix work of 32-row sweeps, and room
// for a fourth workgroup per CU), 2 (32 rows) when they average few, else 4.
// Width 16's register-staged kernel has no 1-tile variant and takes 2.
static int pick_mt(int T, int k, int E)
{
    const int64_t pairs = (int64_t)T * k;
    const int64_t hits = pairs < E ? pairs : E;
    return pairs > 40 * hits ? 4 : pairs <= 2 * hits ? 1 : 2;
}

hipError_t launch_mfma_gateup(const uint16_t* xp, int T, int k, int E, const SortView& sv,
                              int pass_lo, int pass_hi, const int32_t* table, const uint8_t* pool,
                              const ClassView& c, uint16_t* hbuf, uint32_t* err, hipStream_t s)
{
    const int max_hit = pass_hits_max(T, k, E, pass_lo, pass_hi);
    constexpr int CBW = 1;  // column blocks per workgroup
    dim3 grid((unsigned)(((c.I / 64 + CBW - 1) / CBW) * ((max_hit + 7) / 8) * 8));  // see the kernel's tile order
    const int mt = pick_mt(T, k, E);
#define MOE_MG(BB, MM)                                                                             \
    hipLaunchKernelGGL((mfma_grouped_kernel<BB, true, MM, CBW>), grid, dim3(256), 0, s, xp, c.H, c.I, k, \
                       sv.offsets, sv.sorted_pairs, sv.pass_table, E, pass_lo, pass_hi, table, pool, c.n_slots,         \
                       c.slot_bytes, c.off_gu_codes, c.off_gu_sb, hbuf, nullptr, err)
#define MOE_MG2(BB) { if (mt == 4) MOE_MG(BB, 4); else MOE_MG(BB, 2); }
#define MOE_MG3(BB, MM)                                                                            \
    hipLaunchKernelGGL((mfma_lds_kernel<BB, true, MM>), dim3((unsigned)((c.I / 64) * ((max_hit + 7) / 8) * 8)), \
                       dim3(256), 0, s, xp, c.H, c.I, k, sv.offsets, sv.sorted_pairs, sv.pass_table, \
                       E, pass_lo, pass_hi, table, pool, c.n_slots, c.slot_bytes, c.off_gu_codes, c.off_gu_sb, hbuf,    \
                       nullptr, err)
    switch (c.bits_gu) {
    case 3: if (mt == 4) MOE_MG3(3, 4); else if (mt == 1) MOE_MG3(3, 1); else MOE_MG3(3, 2); break;
    case 4: if (mt == 4) MOE_MG3(4, 4); else if (mt == 1) MOE_MG3(4, 1); else MOE_MG3(4, 2); break;
    case 6: if (mt == 4) MOE_MG3(6, 4); else if (mt == 1) MOE_MG3(6, 1); else MOE_MG3(6, 2); break;
    case 8: if (mt == 4) MOE_MG3(8, 4); else if (mt == 1) MOE_MG3(8, 1); else MOE_MG3(8, 2); break;
    case 16: MOE_MG2(16); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_MG
#undef MOE_MG2
#undef MOE_MG3
    return hipGetLastError();
}

hipError_t launch_mfma_down(int T, int k, int E, const SortView& sv, int pass_lo, int pass_hi,
                            const int32_t* table, const uint8_t* pool, const ClassView& c,
                            const uint16_t* hbuf, uint16_t* ybuf, uint32_t* err, hipStream_t s)
{
    const int max_hit = pass_hits_max(T, k, E, pass_lo, pass_hi);
    constexpr int CBW = 1;  // column blocks per workgroup
    dim3 grid((unsigned)(((c.H / 64 + CBW - 1) / CBW) * ((max_hit + 7) / 8) * 8));  // see the kernel's tile order
    const int mt = pick_mt(T, k, E);
#define MOE_MD(BB, MM)                                                                             \
    hipLaunchKernelGGL((mfma_grouped_kernel<BB, false, MM, CBW>), grid, dim3(256), 0, s, hbuf, c.H, c.I, \
                       k, sv.offsets, sv.sorted_pairs, sv.pass_table, E, pass_lo, pass_hi, table, pool, c.n_slots,      \
                       c.slot_bytes, c.off_d_codes, c.off_d_sb, nullptr, ybuf, err)
#define MOE_MD2(BB) { if (mt == 4) MOE_MD(BB, 4); else MOE_MD(BB, 2); }
#define MOE_MD3(BB, MM)                                                                            \
    hipLaunchKernelGGL((mfma_lds_kernel<BB, false, MM>), dim3((unsigned)(((c.H / 64 + 1) / 2) * ((max_hit + 7) / 8) * 8)), \
                       dim3(256), 0, s, hbuf, c.H, c.I, k, sv.offsets, sv.sorted_pairs, sv.pass_table, \
                       E, pass_lo, pass_hi, table, pool, c.n_slots, c.slot_bytes, c.off_d_codes, c.off_d_sb, nullptr,  \
                       ybuf, err)
    switch (c.bits_d) {
    case 3: if (mt == 4) MOE_MD3(3, 4); else if (mt == 1) MOE_MD3(3, 1); else MOE_MD3(3, 2); break;
    case 4: if (mt == 4) MOE_MD3(4, 4); else if (mt == 1) MOE_MD3(4, 1); else MOE_MD3(4, 2); break;
    case 6: if (mt == 4) MOE_MD3(6, 4); else if (mt == 1) MOE_MD3(6, 1); else MOE_MD3(6, 2); break;
    case 8: if (mt == 4) MOE_MD3(8, 4); else if (mt == 1) MOE_MD3(8, 1); else MOE_MD3(8, 2); break;
    case 16: MOE_MD2(16); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_MD
#undef MOE_MD2
#undef MOE_MD3
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* ybuf, const float* topk_w, int T, int k, int H,
                          uint16_t* out, hipStream_t s)
{
    const int64_t n = (int64_t)T * (H / 4);
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ybuf, topk_w, T, k,
                       H, out);
    return hipGetLastError();
}

}  // namespace moe
