// moe_internal.h — launchers shared between the C-ABI layer and the kernel
// translation units.  Host code only; every launcher enqueues on `s` and
// returns hipGetLastError() of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Experts per pass of the sorted prefill: a long prompt's hit experts run in
// passes of at most this many ("RFC: stream MoE experts from disk in
// from_pretrained", How the prototype works, Prefill bullet).
constexpr int kPassExperts = 64;

// Reserved workspace region of the one-launch decode kernels: call-tag counter of
// workgroup slot b at dword kGenBase + b (b < kMaxGrid), then the tagged h words.
constexpr int kMaxGrid = 1024;
constexpr int kGenBase = 64;

// Record `msg` as this thread's moe_last_error() text; returns `code`.
int set_error(int code, const char* msg);

struct ClassView {
    int H, I, bits_gu, bits_d;
    int64_t n_slots, slot_bytes;
    int64_t off_gu_codes, off_gu_sb, off_d_codes, off_d_sb;
};

// Sorted-by-expert view of the routed pairs (all device pointers).
struct SortView {
    const int32_t* offsets;       // [E+1]
    const int32_t* sorted_pairs;  // [n]
    const int32_t* pass_table;    // [2 + E + n_pass_max + 1]
};

hipError_t launch_route(const float* logits, int T, int E, int k, int mode, float L,
                        const int32_t* table, int32_t* ids, float* w, uint32_t* err, hipStream_t s);

// Router logits of n_mats consecutive layers: logits [n_mats][T][E] fp32 from
// x bf16 [T][H] and w bf16 [n_mats][E][H].
hipError_t launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* w, int n_mats, int E,
                                float* logits, hipStream_t s);

size_t sort_ws_bytes(int T, int k, int E);
// x_perm (may be null): also write x [T, H] in the P16 layout of the MFMA path
// to xp, by extra workgroups of the sort's first launch (independent work, one
// launch fewer than a separate permute)
hipError_t launch_sort(const int32_t* ids, int T, int k, int E, int P, int32_t* offsets,
                       int32_t* sorted_pairs, int32_t* pass_table, void* ws, uint32_t* err,
                       hipStream_t s, const uint16_t* x_perm = nullptr, int H = 0, uint16_t* xp = nullptr);

// Decode path: dequant-GEMV gate/up + SwiGLU, then down + weighted combine.
hipError_t launch_gemv_gateup(const uint16_t* x, int T, int k, int E, const SortView& sv,
                              const int32_t* table, const uint8_t* pool, const ClassView& c,
                              uint16_t* hbuf, uint32_t* err, hipStream_t s);
hipError_t launch_gemv_down(int T, int k, int E, const SortView& sv, const float* topk_w,
                            const int32_t* table, const uint8_t* pool, const ClassView& c,
                            const uint16_t* hbuf, uint16_t* out, uint32_t* err, hipStream_t s);
bool gemv_supported(int T, int k, const ClassView& c);

// Decode path fused into one persistent launch (routing optional: logits != null).
// `reserved` points at the workspace's reserved prefix (MOE_WS_RESERVED_BYTES,
// zero before the first call): call-tag counters, then the tagged h words.
bool decode_fused_supported(int T, int k, int E, const ClassView& c);
hipError_t launch_decode_fused(const float* logits, int mode, float L, const int32_t* ids_in,
                               const float* w_in, int32_t* ids_out, float* w_out, int T, int E,
                               int k, const uint16_t* x, const int32_t* table, const uint8_t* pool,
                               const ClassView& c, uint16_t* out, void* reserved, uint32_t* err,
                               hipStream_t s);

// Decode path for one token: a leaner one-launch kernel (every wave routes in
// registers, all weight rows are requested at once, each wave stages only its
// own experts' h).  Plain routing only (logits != null) or given ids / weights.
bool decode1_supported(int T, int k, int E, int mode, bool routes, const ClassView& c);
hipError_t launch_decode1(const float* logits, const int32_t* ids_in, const float* w_in, int32_t* ids_out,
                          float* w_out, int E, int k, const uint16_t* x, const int32_t* table,
                          const uint8_t* pool, const ClassView& c, uint16_t* out, void* reserved,
                          uint32_t* err, hipStream_t s);

// Prefill path: P16-permuted x (written by launch_sort's launch), MFMA gate/up +
// SwiGLU, MFMA down (y in bf16), combine (fp32 sum in j order).
// Both run the hit experts of passes [pass_lo, pass_hi) of the pass table only
// (0 and ceil(E / kPassExperts) for every hit expert).
hipError_t launch_mfma_gateup(const uint16_t* xp, int T, int k, int E, const SortView& sv,
                              int pass_lo, int pass_hi, const int32_t* table, const uint8_t* pool,
                              const ClassView& c, uint16_t* hbuf, uint32_t* err, hipStream_t s);
hipError_t launch_mfma_down(int T, int k, int E, const SortView& sv, int pass_lo, int pass_hi,
                            const int32_t* table, const uint8_t* pool, const ClassView& c,
                            const uint16_t* hbuf, uint16_t* ybuf, uint32_t* err, hipStream_t s);
hipError_t launch_combine(const uint16_t* ybuf, const float* topk_w, int T, int k, int H,
                          uint16_t* out, hipStream_t s);
// one-time conversion: fp32 / bf16 (bf16_in) weights of n experts -> n slot rows
hipError_t launch_convert(const void* w_gu, const void* w_d, int bf16_in, int64_t n, const ClassView& c,
                          void* rows, hipStream_t s);

}  // namespace moe
