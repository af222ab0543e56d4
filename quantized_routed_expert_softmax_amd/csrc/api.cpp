// api.cpp — the C-ABI of include/moe.h: argument checks, workspace carving and
// kernel launches.  No entry point allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// code widths: 3, 4, 6, 8 (group-wise affine), 16 (unquantized bf16 weights)
bool bits_ok(int b) { return b == 3 || b == 4 || b == 6 || b == 8 || b == 16; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

using moe::kPassExperts;

int check_desc(const moe_size_class_desc* d)
{
    if (!d) return fail(MOE_E_INVALID, "size class descriptor is NULL");
    moe_size_class_desc ref;
    if (moe_size_class_init(&ref, d->H, d->I, d->bits_gu, d->bits_d, d->group, d->align, d->n_slots) != MOE_OK)
        return MOE_E_INVALID;
    if (ref.off_gu_codes != d->off_gu_codes || ref.off_gu_sb != d->off_gu_sb ||
        ref.off_d_codes != d->off_d_codes || ref.off_d_sb != d->off_d_sb ||
        ref.slot_bytes != d->slot_bytes)
        return fail(MOE_E_INVALID, "size class descriptor offsets do not match its shape");
    return MOE_OK;
}

moe::ClassView view_of(const moe_size_class_desc* d)
{
    moe::ClassView c;
    c.H = d->H;
    c.I = d->I;
    c.bits_gu = d->bits_gu;
    c.bits_d = d->bits_d;
    c.n_slots = d->n_slots;
    c.slot_bytes = d->slot_bytes;
    c.off_gu_codes = d->off_gu_codes;
    c.off_gu_sb = d->off_gu_sb;
    c.off_d_codes = d->off_d_codes;
    c.off_d_sb = d->off_d_sb;
    return c;
}

// Forward workspace.  The first MOE_WS_RESERVED_BYTES hold the fused decode
// kernel's h exchange (call-tag counters + tagged h words): zero before the
// first call on a workspace, kept consistent by every call, overlapped by
// nothing else.
struct FwdLayout {
    size_t reserved, offsets, sorted, pass, sort_ws, hbuf, xp, ybuf, total;
};

FwdLayout fwd_layout(int T, int k, int E, const moe_size_class_desc* d)
{
    FwdLayout L;
    const size_t n = (size_t)T * k;
    size_t o = 0;
    L.reserved = o;
    o += MOE_WS_RESERVED_BYTES;
    L.offsets = o;
    o = align_up(o + sizeof(int32_t) * (E + 1), 256);
    L.sorted = o;
    o = align_up(o + sizeof(int32_t) * n, 256);
    L.pass = o;
    o = align_up(o + sizeof(int32_t) * (size_t)moe_pass_table_size(E, kPassExperts), 256);
    L.sort_ws = o;
    o = align_up(o + moe::sort_ws_bytes(T, k, E), 256);
    L.hbuf = o;
    o = align_up(o + sizeof(uint16_t) * n * (size_t)d->I, 256);
    L.xp = o;
    o = align_up(o + sizeof(uint16_t) * (size_t)T * d->H, 256);
    L.ybuf = o;
    o = align_up(o + sizeof(uint16_t) * n * (size_t)d->H, 256);  // y in bf16
    L.total = o;
    return L;
}

int n_pass_max(int E) { return (E + kPassExperts - 1) / kPassExperts; }

// gate/up + SwiGLU and down of the hit experts of passes [p0, p1): h and y of
// their pairs in the workspace (sort and permuted x already there).
int run_passes(int T, int k, int E, int p0, int p1, const int32_t* slot_table, const uint8_t* pool,
               const moe::ClassView& c, const FwdLayout& L, char* w, uint32_t* err_word,
               hipStream_t stream)
{
    const moe::SortView sv{(const int32_t*)(w + L.offsets), (const int32_t*)(w + L.sorted),
                           (const int32_t*)(w + L.pass)};
    uint16_t* hbuf = (uint16_t*)(w + L.hbuf);
    hipError_t e = moe::launch_mfma_gateup((const uint16_t*)(w + L.xp), T, k, E, sv, p0, p1, slot_table,
                                           pool, c, hbuf, err_word, stream);
    if (e != hipSuccess) return hip_fail(e, "mfma gate/up launch");
    e = moe::launch_mfma_down(T, k, E, sv, p0, p1, slot_table, pool, c, hbuf, (uint16_t*)(w + L.ybuf),
                              err_word, stream);
    if (e != hipSuccess) return hip_fail(e, "mfma down launch");
    return MOE_OK;
}

// Shared checks of the forward-shaped calls: T, E, k ranges and the workspace.
int check_fwd(int T, int k, int E, const moe_size_class_desc* d, const void* ws, size_t ws_bytes,
              FwdLayout* L)
{
    if (int rc = check_desc(d)) return rc;
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if ((int64_t)T * k > (int64_t)1 << 26) return fail(MOE_E_INVALID, "T*k too large");
    *L = fwd_layout(T, k, E, d);
    if (T == 0) return MOE_OK;
    if (!ws || !aligned(ws, 256)) return fail(MOE_E_INVALID, "ws must be a 256-byte aligned buffer");
    if (ws_bytes < L->total)
        return fail(MOE_E_WORKSPACE, "forward workspace %zu bytes < %zu", ws_bytes, L->total);
    return MOE_OK;
}

}  // namespace

// ---- the library-owned scratch of moe_layer_forward_static ------------------
// One array per GPU the library runs on, held until the process ends.  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress once per device and is kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_dwords_kernel(uint32_t* __restrict__ p, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Device address of the current device's scratch; the first call on a device
// looks it up and clears its reserved prefix (the fused decode kernel's call-tag
// counters and tagged h words) with a fill kernel on `stream`.
int static_scratch(hipStream_t stream, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_E_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || (uintptr_t)ptr % 256) return fail(MOE_E_HIP, "scratch has no 256-byte aligned device address");
        const size_t n = MOE_WS_RESERVED_BYTES / 4;
        hipLaunchKernelGGL(zero_dwords_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (uint32_t*)ptr, n);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

int moe::set_error(int code, const char* msg)
{
    g_last_error = msg;
    return code;
}

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_size_class_init(moe_size_class_desc* d, int H, int I, int bits_gu, int bits_d, int group,
                        int align, int64_t n_slots)
{
    if (!d) return fail(MOE_E_INVALID, "descriptor is NULL");
    if (group != 64) return fail(MOE_E_INVALID, "group must be 64 (got %d)", group);
    if (align != 256) return fail(MOE_E_INVALID, "align must be 256 (got %d)", align);
    if (H <= 0 || I <= 0 || H % 64 || I % 64)
        return fail(MOE_E_INVALID, "H and I must be positive multiples of 64 (H=%d I=%d)", H, I);
    if (!bits_ok(bits_gu) || !bits_ok(bits_d))
        return fail(MOE_E_INVALID, "bits must be 3, 4, 6, 8 or 16 (gate_up %d, down %d)", bits_gu, bits_d);
    if (n_slots < 0) return fail(MOE_E_INVALID, "n_slots < 0");
    const int64_t gu_codes = (int64_t)2 * I * H * bits_gu / 8;
    const int64_t gu_sb = bits_gu == 16 ? 0 : (int64_t)2 * I * (H / 64) * 4;
    const int64_t d_codes = (int64_t)H * I * bits_d / 8;
    const int64_t d_sb = bits_d == 16 ? 0 : (int64_t)H * (I / 64) * 4;
    d->H = H;
    d->I = I;
    d->bits_gu = bits_gu;
    d->bits_d = bits_d;
    d->group = group;
    d->align = align;
    d->n_slots = n_slots;
    d->off_gu_codes = 0;
    d->off_gu_sb = (int64_t)align_up((size_t)gu_codes, align);
    d->off_d_codes = (int64_t)align_up((size_t)(d->off_gu_sb + gu_sb), align);
    d->off_d_sb = (int64_t)align_up((size_t)(d->off_d_codes + d_codes), align);
    d->slot_bytes = (int64_t)align_up((size_t)(d->off_d_sb + d_sb), align);
    return MOE_OK;
}

int moe_route_topk(const float* logits, int T, int E, int k, int mode, float L,
                   const int32_t* slot_table, int32_t* topk_ids, float* topk_w, uint32_t* err_word,
                   hipStream_t stream)
{
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if (mode != MOE_ROUTE_PLAIN && mode != MOE_ROUTE_SUBST)
        return fail(MOE_E_INVALID, "unknown routing mode %d", mode);
    if (mode == MOE_ROUTE_SUBST) {
        if (!slot_table) return fail(MOE_E_INVALID, "substitution needs the slot table");
        if (!(L >= 0.0f) || !std::isfinite(L)) return fail(MOE_E_INVALID, "L must be finite and >= 0");
    }
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return fail(MOE_E_INVALID, "NULL buffer");
    hipError_t e = moe::launch_route(logits, T, E, k, mode, L, slot_table, topk_ids, topk_w,
                                     err_word, stream);
    if (e != hipSuccess) return hip_fail(e, "route_topk launch");
    return MOE_OK;
}

int moe_router_logits(const void* x, int T, int H, const void* w, int n_mats, int E, float* logits,
                      hipStream_t stream)
{
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (H < 8 || H % 8) return fail(MOE_E_INVALID, "H must be a positive multiple of 8 (got %d)", H);
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (n_mats < 1 || n_mats > 8) return fail(MOE_E_INVALID, "n_mats must be in [1, 8] (got %d)", n_mats);
    if (T == 0) return MOE_OK;
    if (!x || !w || !logits) return fail(MOE_E_INVALID, "NULL buffer");
    if (!aligned(x, 16) || !aligned(w, 16)) return fail(MOE_E_INVALID, "x and w need 16-byte alignment");
    hipError_t e = moe::launch_router_logits((const uint16_t*)x, T, H, (const uint16_t*)w, n_mats, E,
                                             logits, stream);
    if (e != hipSuccess) return hip_fail(e, "router logits launch");
    return MOE_OK;
}

int moe_pass_table_size(int E, int pass_experts)
{
    if (E < 1 || pass_experts < 1) return 0;
    return 2 + E + (E + pass_experts - 1) / pass_experts + 1;
}

size_t moe_sort_workspace_size(int T, int k, int E)
{
    if (T < 0 || k < 1 || E < 1) return 0;
    return moe::sort_ws_bytes(T, k, E);
}

int moe_sort_by_expert(const int32_t* topk_ids, int T, int k, int E, int pass_experts,
                       int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pass_table,
                       void* ws, size_t ws_bytes, uint32_t* err_word, hipStream_t stream)
{
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if (pass_experts < 1) return fail(MOE_E_INVALID, "pass_experts must be >= 1");
    if ((int64_t)T * k > (int64_t)1 << 26) return fail(MOE_E_INVALID, "T*k too large");
    if (T == 0) return MOE_OK;
    if (!topk_ids || !expert_offsets || !sorted_pairs || !pass_table)
        return fail(MOE_E_INVALID, "NULL buffer");
    const size_t need = moe::sort_ws_bytes(T, k, E);
    if (ws_bytes < need || (need && !ws))
        return fail(MOE_E_WORKSPACE, "sort workspace %zu bytes < %zu", ws_bytes, need);
    hipError_t e = moe::launch_sort(topk_ids, T, k, E, pass_experts, expert_offsets, sorted_pairs,
                                    pass_table, ws, err_word, stream);
    if (e != hipSuccess) return hip_fail(e, "sort launch");
    return MOE_OK;
}

size_t moe_forward_workspace_size(int T, int k, int E, const moe_size_class_desc* d)
{
    if (T < 0 || k < 1 || E < 1 || !d || d->H <= 0 || d->I <= 0) return 0;
    return fwd_layout(T, k, E, d).total;
}

int moe_experts_forward_ex(const void* x, int T, const int32_t* topk_ids, const float* topk_w,
                           int k, int E, const int32_t* slot_table, const void* slot_pool,
                           const moe_size_class_desc* d, void* out, void* ws, size_t ws_bytes,
                           uint32_t* err_word, int path, hipStream_t stream)
{
    if (int rc = check_desc(d)) return rc;
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if (path != MOE_PATH_AUTO && path != MOE_PATH_GEMV && path != MOE_PATH_MFMA && path != MOE_PATH_GEMV3)
        return fail(MOE_E_INVALID, "unknown path %d", path);
    if ((int64_t)T * k > (int64_t)1 << 26) return fail(MOE_E_INVALID, "T*k too large");
    if (T == 0) return MOE_OK;
    if (!x || !topk_ids || !topk_w || !slot_table || !slot_pool || !out)
        return fail(MOE_E_INVALID, "NULL buffer");
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(slot_pool, 256) || !aligned(ws, 256))
        return fail(MOE_E_INVALID, "x/out need 16-byte, slot_pool/ws 256-byte alignment");
    const FwdLayout L = fwd_layout(T, k, E, d);
    if (ws_bytes < L.total) return fail(MOE_E_WORKSPACE, "forward workspace %zu bytes < %zu", ws_bytes, L.total);

    const moe::ClassView c = view_of(d);
    const bool gemv_ok = moe::gemv_supported(T, k, c);
    if ((path == MOE_PATH_GEMV || path == MOE_PATH_GEMV3) && !gemv_ok)
        return fail(MOE_E_UNSUPPORTED, "GEMV path supports T <= 64 and H/32, I/32 with an odd part <= 4");
    if (path == MOE_PATH_AUTO) {
        // the one-launch decode kernel when it takes the shape; otherwise the
        // three-launch GEMV only for a handful of pairs (measured: 8 pairs of the
        // mixed layer 28 us GEMV vs 38 us MFMA, 16 pairs 48 vs 43, 64 pairs 155
        // vs 72), the MFMA path above that
        if (gemv_ok && (moe::decode1_supported(T, k, E, MOE_ROUTE_PLAIN, false, c) || moe::decode_fused_supported(T, k, E, c)))
            path = MOE_PATH_GEMV;
        else path = (gemv_ok && (int64_t)T * k <= 8) ? MOE_PATH_GEMV : MOE_PATH_MFMA;
    }

    char* w = (char*)ws;
    int32_t* offsets = (int32_t*)(w + L.offsets);
    int32_t* sorted = (int32_t*)(w + L.sorted);
    int32_t* pass = (int32_t*)(w + L.pass);
    uint16_t* hbuf = (uint16_t*)(w + L.hbuf);
    const uint8_t* pool = (const uint8_t*)slot_pool;
    hipError_t e;
    if (path == MOE_PATH_GEMV && moe::decode1_supported(T, k, E, MOE_ROUTE_PLAIN, false, c)) {
        e = moe::launch_decode1(nullptr, topk_ids, topk_w, nullptr, nullptr, E, k, (const uint16_t*)x, slot_table,
                                pool, c, (uint16_t*)out, w + L.reserved, err_word, stream);
        if (e != hipSuccess) return hip_fail(e, "one-token decode launch");
        return MOE_OK;
    }
    if (path == MOE_PATH_GEMV && moe::decode_fused_supported(T, k, E, c)) {
        e = moe::launch_decode_fused(nullptr, MOE_ROUTE_PLAIN, 0.0f, topk_ids, topk_w, nullptr,
                                     nullptr, T, E, k, (const uint16_t*)x, slot_table, pool, c,
                                     (uint16_t*)out, w + L.reserved, err_word, stream);
        if (e != hipSuccess) return hip_fail(e, "fused decode launch");
        return MOE_OK;
    }
    const bool mfma = !(path == MOE_PATH_GEMV || path == MOE_PATH_GEMV3);
    e = moe::launch_sort(topk_ids, T, k, E, kPassExperts, offsets, sorted, pass, w + L.sort_ws, err_word,
                         stream, mfma ? (const uint16_t*)x : nullptr, c.H, (uint16_t*)(w + L.xp));
    if (e != hipSuccess) return hip_fail(e, "sort launch");
    moe::SortView sv{offsets, sorted, pass};
    if (path == MOE_PATH_GEMV || path == MOE_PATH_GEMV3) {
        e = moe::launch_gemv_gateup((const uint16_t*)x, T, k, E, sv, slot_table, pool, c, hbuf,
                                    err_word, stream);
        if (e != hipSuccess) return hip_fail(e, "gemv gate/up launch");
        e = moe::launch_gemv_down(T, k, E, sv, topk_w, slot_table, pool, c, hbuf, (uint16_t*)out,
                                  err_word, stream);
        if (e != hipSuccess) return hip_fail(e, "gemv down launch");
        return MOE_OK;
    }
    // MFMA: every pass in one launch pair (the whole hit list is resident; x
    // was permuted by the sort's launch)
    if (int rc = run_passes(T, k, E, 0, n_pass_max(E), slot_table, pool, c, L, w, err_word, stream))
        return rc;
    e = moe::launch_combine((const uint16_t*)(w + L.ybuf), topk_w, T, k, c.H, (uint16_t*)out, stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return MOE_OK;
}

int moe_layer_forward(const float* logits, int T, int E, int k, int mode, float L, const void* x,
                      const int32_t* slot_table, const void* slot_pool, const moe_size_class_desc* d,
                      int32_t* topk_ids, float* topk_w, void* out, void* ws, size_t ws_bytes,
                      uint32_t* err_word, hipStream_t stream)
{
    if (int rc = check_desc(d)) return rc;
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if (mode != MOE_ROUTE_PLAIN && mode != MOE_ROUTE_SUBST)
        return fail(MOE_E_INVALID, "unknown routing mode %d", mode);
    if (mode == MOE_ROUTE_SUBST && (!(L >= 0.0f) || !std::isfinite(L)))
        return fail(MOE_E_INVALID, "L must be finite and >= 0");
    if ((int64_t)T * k > (int64_t)1 << 26) return fail(MOE_E_INVALID, "T*k too large");
    if (T == 0) return MOE_OK;
    if (!logits || !x || !slot_table || !slot_pool || !out || !topk_ids || !topk_w)
        return fail(MOE_E_INVALID, "NULL buffer");
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(slot_pool, 256) || !aligned(ws, 256))
        return fail(MOE_E_INVALID, "x/out need 16-byte, slot_pool/ws 256-byte alignment");
    const FwdLayout Lw = fwd_layout(T, k, E, d);
    if (ws_bytes < Lw.total) return fail(MOE_E_WORKSPACE, "forward workspace %zu bytes < %zu", ws_bytes, Lw.total);
    const moe::ClassView c = view_of(d);
    if (moe::decode1_supported(T, k, E, mode, true, c)) {
        hipError_t e = moe::launch_decode1(logits, nullptr, nullptr, topk_ids, topk_w, E, k, (const uint16_t*)x,
                                           slot_table, (const uint8_t*)slot_pool, c, (uint16_t*)out,
                                           (char*)ws + Lw.reserved, err_word, stream);
        if (e != hipSuccess) return hip_fail(e, "one-token decode launch");
        return MOE_OK;
    }
    // in-kernel routing covers E <= 512; larger E routes with the router kernel first
    if (E <= 512 && moe::decode_fused_supported(T, k, E, c)) {
        char* w = (char*)ws;
        hipError_t e = moe::launch_decode_fused(logits, mode, L, nullptr, nullptr, topk_ids, topk_w, T, E,
                                                k, (const uint16_t*)x, slot_table, (const uint8_t*)slot_pool,
                                                c, (uint16_t*)out, w + Lw.reserved, err_word, stream);
        if (e != hipSuccess) return hip_fail(e, "fused decode launch");
        return MOE_OK;
    }
    if (int rc = moe_route_topk(logits, T, E, k, mode, L, slot_table, topk_ids, topk_w, err_word, stream))
        return rc;
    return moe_experts_forward_ex(x, T, topk_ids, topk_w, k, E, slot_table, slot_pool, d, out, ws,
                                  ws_bytes, err_word, MOE_PATH_AUTO, stream);
}

int moe_layer_forward_static(const float* logits, int T, int E, int k, int mode, float L, const void* x,
                             const int32_t* slot_table, const void* slot_pool,
                             const moe_size_class_desc* d, int32_t* topk_ids, float* topk_w, void* out,
                             uint32_t* err_word, hipStream_t stream)
{
    if (int rc = check_desc(d)) return rc;
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if ((int64_t)T * k > (int64_t)1 << 26) return fail(MOE_E_INVALID, "T*k too large");
    const size_t need = fwd_layout(T, k, E, d).total;
    if (need > (size_t)MOE_STATIC_SCRATCH_BYTES)
        return fail(MOE_E_WORKSPACE, "this layer needs %zu bytes of scratch, more than the library's %zu",
                    need, (size_t)MOE_STATIC_SCRATCH_BYTES);
    if (T == 0) return MOE_OK;
    void* ws = nullptr;
    if (int rc = static_scratch(stream, &ws)) return rc;
    return moe_layer_forward(logits, T, E, k, mode, L, x, slot_table, slot_pool, d, topk_ids, topk_w, out,
                             ws, (size_t)MOE_STATIC_SCRATCH_BYTES, err_word, stream);
}

int moe_experts_forward(const void* x, int T, const int32_t* topk_ids, const float* topk_w, int k,
                        int E, const int32_t* slot_table, const void* slot_pool,
                        const moe_size_class_desc* d, void* out, void* ws, size_t ws_bytes,
                        uint32_t* err_word, hipStream_t stream)
{
    return moe_experts_forward_ex(x, T, topk_ids, topk_w, k, E, slot_table, slot_pool, d, out, ws,
                                  ws_bytes, err_word, MOE_PATH_AUTO, stream);
}

int moe_pass_table_host(const int32_t* topk_ids, int T, int k, int E, int pass_experts,
                        int32_t* pass_table)
{
    if (T < 0) return fail(MOE_E_INVALID, "T < 0");
    if (E < 1 || E > 1024) return fail(MOE_E_INVALID, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E || k > 32) return fail(MOE_E_INVALID, "k must be in [1, min(E, 32)] (got %d)", k);
    if (pass_experts < 1) return fail(MOE_E_INVALID, "pass_experts must be >= 1");
    if (!pass_table || (T > 0 && !topk_ids)) return fail(MOE_E_INVALID, "NULL buffer");
    std::vector<char> hit((size_t)E, 0);
    for (int64_t p = 0; p < (int64_t)T * k; ++p) {
        const int32_t e = topk_ids[p];
        if (e < 0 || e >= E) return fail(MOE_E_INVALID, "expert id %d of pair %lld outside [0, %d)", e, (long long)p, E);
        hit[(size_t)e] = 1;
    }
    int n_hit = 0;
    for (int e = 0; e < E; ++e) {
        pass_table[2 + e] = -1;
        if (hit[(size_t)e]) pass_table[2 + n_hit++] = e;
    }
    const int n_max = (E + pass_experts - 1) / pass_experts;
    pass_table[0] = n_hit;
    pass_table[1] = (n_hit + pass_experts - 1) / pass_experts;
    for (int q = 0; q <= n_max; ++q) {
        const int64_t start = (int64_t)q * pass_experts;
        pass_table[2 + E + q] = start < n_hit ? (int32_t)start : n_hit;
    }
    return MOE_OK;
}

int moe_prefill_sort(const void* x, int T, const int32_t* topk_ids, int k, int E,
                     const moe_size_class_desc* d, void* ws, size_t ws_bytes, uint32_t* err_word,
                     hipStream_t stream)
{
    FwdLayout L;
    if (int rc = check_fwd(T, k, E, d, ws, ws_bytes, &L)) return rc;
    if (T == 0) return MOE_OK;
    if (!x || !topk_ids) return fail(MOE_E_INVALID, "NULL buffer");
    if (!aligned(x, 16)) return fail(MOE_E_INVALID, "x needs 16-byte alignment");
    char* w = (char*)ws;
    hipError_t e = moe::launch_sort(topk_ids, T, k, E, kPassExperts, (int32_t*)(w + L.offsets),
                                    (int32_t*)(w + L.sorted), (int32_t*)(w + L.pass), w + L.sort_ws,
                                    err_word, stream, (const uint16_t*)x, d->H, (uint16_t*)(w + L.xp));
    if (e != hipSuccess) return hip_fail(e, "sort launch");
    return MOE_OK;
}

int moe_prefill_pass(int T, int k, int E, int pass_begin, int pass_end, const int32_t* slot_table,
                     const void* slot_pool, const moe_size_class_desc* d, void* ws, size_t ws_bytes,
                     uint32_t* err_word, hipStream_t stream)
{
    FwdLayout L;
    if (int rc = check_fwd(T, k, E, d, ws, ws_bytes, &L)) return rc;
    const int nmax = n_pass_max(E);
    if (pass_begin < 0 || pass_end > nmax || pass_begin > pass_end)
        return fail(MOE_E_INVALID, "pass range [%d, %d) outside [0, %d]", pass_begin, pass_end, nmax);
    if (T == 0 || pass_begin == pass_end) return MOE_OK;
    if (!slot_table || !slot_pool) return fail(MOE_E_INVALID, "NULL buffer");
    if (!aligned(slot_pool, 256)) return fail(MOE_E_INVALID, "slot_pool needs 256-byte alignment");
    return run_passes(T, k, E, pass_begin, pass_end, slot_table, (const uint8_t*)slot_pool, view_of(d),
                      L, (char*)ws, err_word, stream);
}

int moe_prefill_combine(int T, int k, int E, const float* topk_w, const moe_size_class_desc* d,
                        void* out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    FwdLayout L;
    if (int rc = check_fwd(T, k, E, d, ws, ws_bytes, &L)) return rc;
    if (T == 0) return MOE_OK;
    if (!topk_w || !out) return fail(MOE_E_INVALID, "NULL buffer");
    if (!aligned(out, 16)) return fail(MOE_E_INVALID, "out needs 16-byte alignment");
    hipError_t e = moe::launch_combine((const uint16_t*)((char*)ws + L.ybuf), topk_w, T, k, d->H,
                                       (uint16_t*)out, stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return MOE_OK;
}

int moe_quantize_experts(const void* w_gu, const void* w_d, int dtype, int n_experts,
                         const moe_size_class_desc* d, void* rows, hipStream_t stream)
{
    if (int rc = check_desc(d)) return rc;
    if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return fail(MOE_E_INVALID, "unknown weight dtype %d", dtype);
    if (n_experts < 0) return fail(MOE_E_INVALID, "n_experts %d < 0", n_experts);
    if (n_experts == 0) return MOE_OK;
    if (!w_gu || !w_d || !rows) return fail(MOE_E_INVALID, "NULL buffer");
    if (((uintptr_t)rows & 255) != 0) return fail(MOE_E_INVALID, "rows must be 256-byte aligned");
    const size_t el = dtype == MOE_DTYPE_F32 ? 4 : 2;
    if (((uintptr_t)w_gu | (uintptr_t)w_d) & (el - 1)) return fail(MOE_E_INVALID, "weights not aligned to their element");
    hipError_t e = moe::launch_convert(w_gu, w_d, dtype == MOE_DTYPE_BF16, n_experts, view_of(d), rows, stream);
    if (e != hipSuccess) return hip_fail(e, "convert launch");
    return MOE_OK;
}

int moe_cache_install(void* slot_pool, const moe_size_class_desc* d, int64_t slot, const void* src,
                      int src_kind, hipStream_t copy_stream, hipEvent_t done)
{
    if (int rc = check_desc(d)) return rc;
    if (!slot_pool || !src) return fail(MOE_E_INVALID, "NULL buffer");
    if (slot < 0 || slot >= d->n_slots)
        return fail(MOE_E_INVALID, "slot %lld outside [0, %lld)", (long long)slot, (long long)d->n_slots);
    hipMemcpyKind kind;
    if (src_kind == MOE_SRC_HOST) kind = hipMemcpyHostToDevice;
    else if (src_kind == MOE_SRC_DEVICE) kind = hipMemcpyDeviceToDevice;
    else return fail(MOE_E_INVALID, "unknown source kind %d", src_kind);
    char* dst = (char*)slot_pool + (size_t)slot * (size_t)d->slot_bytes;
    hipError_t e = hipMemcpyAsync(dst, src, (size_t)d->slot_bytes, kind, copy_stream);
    if (e != hipSuccess) return hip_fail(e, "install copy");
    if (done) {
        e = hipEventRecord(done, copy_stream);
        if (e != hipSuccess) return hip_fail(e, "install event");
    }
    return MOE_OK;
}

}  // extern "C"
