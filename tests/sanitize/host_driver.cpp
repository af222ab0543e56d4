// Drives the library's host code (size-class cache, expert store, miss
// pipeline with its I/O threads and event rings) on the host-only HIP stand-in,
// for runs under the address / undefined-behaviour and thread sanitizers.
// "Device" pools and tables are host memory; copies run on stream worker
// threads.  Every layer step checks, on the compute stream after the waits that
// moe_pipeline_prepare enqueued, that each routed expert's slot holds exactly
// that expert's store row: a missing wait shows up as a wrong row here and as a
// data race under the thread sanitizer.
//
// Exit status 0 when every check passed; prints one summary line.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <random>
#include <string>
#include <vector>

#include <unistd.h>

#include "../../include/moe.h"
#include "hip_stub_ext.h"

namespace moe {
// The library's error text lives in its C-ABI translation unit, which is not
// part of this build; keep the last message here.
thread_local std::string g_last;
int set_error(int code, const char* msg)
{
    g_last = msg ? msg : "";
    return code;
}
}  // namespace moe

// Entry points the pipeline's prefill path calls; not exercised here.
extern "C" {
int moe_pass_table_size(int E, int pass_experts) { return 2 + E + (E + pass_experts - 1) / pass_experts + 1; }
int moe_pass_table_host(const int32_t*, int, int, int, int, int32_t*) { return MOE_E_UNSUPPORTED; }
int moe_prefill_sort(const void*, int, const int32_t*, int, int, const moe_size_class_desc*, void*, size_t,
                     uint32_t*, hipStream_t)
{
    return MOE_E_UNSUPPORTED;
}
int moe_prefill_pass(int, int, int, int, int, const int32_t*, const void*, const moe_size_class_desc*, void*,
                     size_t, uint32_t*, hipStream_t)
{
    return MOE_E_UNSUPPORTED;
}
int moe_prefill_combine(int, int, int, const float*, const moe_size_class_desc*, void*, void*, size_t, hipStream_t)
{
    return MOE_E_UNSUPPORTED;
}
const char* moe_last_error(void) { return moe::g_last.c_str(); }
}

namespace {

int g_fail = 0;
constexpr int kSteps = 40;  // layer sweeps per pipeline configuration

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);            \
            std::fprintf(stderr, "\n");                   \
            ++g_fail;                                     \
        }                                                 \
    } while (0)

// A size class of the given row size (the cache and pipeline only use the
// slot count and row size; the block offsets are filled consistently).
moe_size_class_desc make_class(int64_t slot_bytes, int64_t n_slots)
{
    moe_size_class_desc d;
    std::memset(&d, 0, sizeof d);
    d.H = 64;
    d.I = 64;
    d.bits_gu = 4;
    d.bits_d = 4;
    d.group = 64;
    d.align = 256;
    d.n_slots = n_slots;
    d.off_gu_codes = 0;
    d.off_gu_sb = slot_bytes / 4;
    d.off_d_codes = slot_bytes / 2;
    d.off_d_sb = 3 * slot_bytes / 4;
    d.slot_bytes = slot_bytes;
    return d;
}

uint8_t row_byte(int layer, int expert, int64_t i)
{
    uint64_t h = (uint64_t)layer * 0x9E3779B97F4A7C15ull ^ (uint64_t)expert * 0xC2B2AE3D27D4EB4Full ^
                 (uint64_t)i * 0x165667B19E3779F9ull;
    h ^= h >> 29;
    h *= 0xBF58476D1CE4E5B9ull;
    h ^= h >> 32;
    return (uint8_t)h;
}

// ---- cache: random acquire / fill / pin sequences against its own invariants ----
void cache_run(unsigned seed, int per_layer, int policy)
{
    const int L = 6, E = 40;
    moe_size_class_desc cls[2] = {make_class(512, 24), make_class(768, 20)};
    int32_t lc[L];
    for (int l = 0; l < L; ++l) lc[l] = l % 2;
    moe_cache* c = moe_cache_create_ex(cls, 2, lc, L, E, policy, per_layer);
    CHECK(c != nullptr, "cache create");
    if (!c) return;
    std::mt19937 rng(seed);
    std::vector<std::vector<int>> pinned(L);
    for (int it = 0; it < 4000; ++it) {
        const int l = (int)(rng() % L), e = (int)(rng() % E);
        const int op = (int)(rng() % 10);
        if (op < 6) {
            int64_t slot = -1;
            int nf = 0;
            const int rc = moe_cache_acquire(c, l, e, &slot, &nf);
            CHECK(rc == MOE_OK || rc == MOE_E_NO_SLOT || rc == MOE_E_BUSY, "acquire rc %d", rc);
            if (rc == MOE_OK && nf) {
                if (rng() % 8 == 0) moe_cache_abort_fill(c, l, e);
                else moe_cache_fill_done(c, l, e, nullptr);
            }
        } else if (op < 8) {
            int64_t slot = -1;
            if (moe_cache_lookup(c, l, e, &slot) == MOE_OK && slot >= 0 && pinned[l].size() < 3 &&
                moe_cache_pin(c, l, e) == MOE_OK)
                pinned[l].push_back(e);
        } else if (!pinned[l].empty()) {
            CHECK(moe_cache_unpin(c, l, pinned[l].back()) == MOE_OK, "unpin");
            pinned[l].pop_back();
        }
        if (it % 97 == 0) {
            moe_cache_poll(c);
            // every class's table entries point at distinct slots inside the class
            for (int k = 0; k < 2; ++k) {
                std::vector<int> owner((size_t)cls[k].n_slots, 0);
                for (int ll = 0; ll < L; ++ll) {
                    if (lc[ll] != k) continue;
                    std::vector<int32_t> t((size_t)E);
                    CHECK(moe_cache_table(c, ll, t.data()) == MOE_OK, "table");
                    for (int ee = 0; ee < E; ++ee) {
                        if (t[ee] < 0) continue;
                        CHECK(t[ee] < cls[k].n_slots, "slot range");
                        if (t[ee] < cls[k].n_slots) ++owner[(size_t)t[ee]];
                    }
                }
                for (int v : owner) CHECK(v <= 1, "slot shared by two entries");
            }
        }
    }
    for (int l = 0; l < L; ++l)
        for (int e : pinned[l]) moe_cache_unpin(c, l, e);
    int64_t h = 0, m = 0, ev = 0;
    moe_cache_stats(c, &h, &m, &ev);
    CHECK(h + m > 0, "stats");
    moe_cache_destroy(c);
}

// ---- store: memory- and file-backed rows read back from several threads ----
struct Layout {
    int L, E;
    std::vector<moe_size_class_desc> cls;
    std::vector<int32_t> lc;
};

std::vector<uint8_t> store_image(const Layout& s, moe_store* probe)
{
    std::vector<uint8_t> img((size_t)moe_store_bytes(probe));
    for (int l = 0; l < s.L; ++l)
        for (int e = 0; e < s.E; ++e) {
            const int64_t off = moe_store_row_offset(probe, l, e);
            const int64_t n = s.cls[(size_t)s.lc[(size_t)l]].slot_bytes;
            for (int64_t i = 0; i < n; ++i) img[(size_t)(off + i)] = row_byte(l, e, i);
        }
    return img;
}

// ---- pipeline: layer steps with checks on the compute stream ----
struct PipeCfg {
    int64_t host_tier_bytes;
    int preload, io_threads, staging, copies, per_layer, use_file, prefetch;
};

void pipeline_run(const PipeCfg& pc, unsigned seed)
{
    Layout s;
    s.L = 8;
    s.E = 48;
    const int k = 6;
    // class 0 holds six layers: with one LRU per layer each needs k slots
    s.cls = {make_class(1024, pc.per_layer ? 6 * k : 16), make_class(1536, 12)};
    s.lc.resize((size_t)s.L);
    for (int l = 0; l < s.L; ++l) s.lc[(size_t)l] = (l % 4 == 3) ? 1 : 0;

    // the store image: sized and laid out by the library's own offsets
    std::vector<uint8_t> tmp(1);
    moe_store* probe = moe_store_open_memory(tmp.data(), 1, s.cls.data(), 2, s.lc.data(), s.L, s.E);
    // a 1-byte region is too short: the library refuses it; size it properly
    if (probe) moe_store_close(probe);
    int64_t need = 0;
    for (int l = 0; l < s.L; ++l) need += (int64_t)s.E * s.cls[(size_t)s.lc[(size_t)l]].slot_bytes;
    std::vector<uint8_t> mem((size_t)need);
    probe = moe_store_open_memory(mem.data(), need, s.cls.data(), 2, s.lc.data(), s.L, s.E);
    CHECK(probe != nullptr, "store open memory");
    if (!probe) return;
    const std::vector<uint8_t> img = store_image(s, probe);
    moe_store_close(probe);
    std::memcpy(mem.data(), img.data(), img.size());

    moe_store* store = nullptr;
    std::string path;
    if (pc.use_file) {
        char name[] = "/tmp/moe_sanitize_storeXXXXXX";
        const int fd = mkstemp(name);
        CHECK(fd >= 0, "mkstemp");
        if (fd < 0) return;
        path = name;
        CHECK(write(fd, img.data(), img.size()) == (ssize_t)img.size(), "write store file");
        close(fd);
        store = moe_store_open_file(path.c_str(), s.cls.data(), 2, s.lc.data(), s.L, s.E);
    } else {
        store = moe_store_open_memory(mem.data(), need, s.cls.data(), 2, s.lc.data(), s.L, s.E);
    }
    CHECK(store != nullptr, "store open");
    if (!store) return;
    {
        std::vector<uint8_t> row((size_t)s.cls[1].slot_bytes);
        CHECK(moe_store_read(store, 3, 5, row.data()) == MOE_OK, "store read");
        for (int64_t i = 0; i < s.cls[1].slot_bytes; ++i)
            if (row[(size_t)i] != row_byte(3, 5, i)) {
                CHECK(false, "store row bytes");
                break;
            }
    }

    moe_cache* cache = moe_cache_create_ex(s.cls.data(), 2, s.lc.data(), s.L, s.E, MOE_EVICT_LRU, pc.per_layer);
    CHECK(cache != nullptr, "cache");
    // "device" pools: 256-byte aligned host memory, as the pipeline requires
    std::vector<std::unique_ptr<uint8_t, void (*)(void*)>> pools;
    void* pool_ptrs[2];
    for (int c = 0; c < 2; ++c) {
        const size_t n = (size_t)(s.cls[(size_t)c].n_slots * s.cls[(size_t)c].slot_bytes);
        pools.emplace_back((uint8_t*)std::aligned_alloc(256, (n + 255) / 256 * 256), std::free);
        std::memset(pools.back().get(), 0, n);
        pool_ptrs[c] = pools.back().get();
    }
    hipStream_t copies[4];
    for (int i = 0; i < pc.copies; ++i) copies[i] = stub_stream_create();
    hipStream_t compute = stub_stream_create();
    moe_pipeline_config cfg;
    std::memset(&cfg, 0, sizeof cfg);
    cfg.host_tier_bytes = pc.host_tier_bytes;
    cfg.host_preload = pc.preload;
    cfg.io_threads = pc.io_threads;
    cfg.staging_rows = pc.staging;
    moe_pipeline* p = moe_pipeline_create(cache, store, pool_ptrs, &cfg, copies, pc.copies);
    CHECK(p != nullptr, "pipeline create: %s", moe_last_error());
    if (!p) return;

    std::vector<std::vector<int32_t>> tables((size_t)s.L, std::vector<int32_t>((size_t)s.E, -2));
    std::atomic<int> bad_rows{0}, checked{0};
    std::mt19937 rng(seed);
    auto pick = [&](int n) {
        std::vector<int32_t> ids((size_t)n);
        for (int j = 0; j < n; ++j) {
            // skewed: low ids more often, and duplicates now and then
            const uint32_t r = rng();
            ids[(size_t)j] = (int32_t)((r % 3 == 0) ? (r >> 8) % 8 : (r >> 8) % (uint32_t)s.E);
        }
        return ids;
    };
    for (int step = 0; step < kSteps; ++step) {
        for (int l = 0; l < s.L; ++l) {
            const std::vector<int32_t> ids = pick(k);
            int32_t* tdev = tables[(size_t)l].data();
            const int rc = moe_pipeline_prepare(p, l, ids.data(), k, tdev, compute);
            CHECK(rc == MOE_OK, "prepare layer %d: %d %s", l, rc, moe_last_error());
            if (rc != MOE_OK) continue;
            const int cls = s.lc[(size_t)l];
            const int64_t rb = s.cls[(size_t)cls].slot_bytes;
            const uint8_t* pool = pools[(size_t)cls].get();
            stub_host_task(compute, [&, ids, l, tdev, rb, pool] {
                for (int32_t e : ids) {
                    const int32_t slot = tdev[e];
                    if (slot < 0) {
                        ++bad_rows;
                        continue;
                    }
                    const uint8_t* row = pool + (size_t)slot * (size_t)rb;
                    for (int64_t i = 0; i < rb; i += 61)
                        if (row[i] != row_byte(l, e, i)) {
                            ++bad_rows;
                            break;
                        }
                    ++checked;
                }
            });
            CHECK(moe_pipeline_release(p, l, compute) == MOE_OK, "release");
            if (pc.prefetch && l + 1 < s.L) {
                const std::vector<int32_t> guess = pick(k);
                CHECK(moe_pipeline_prefetch(p, l + 1, guess.data(), k) >= 0, "prefetch");
            }
        }
    }
    CHECK(moe_pipeline_drain(p) == MOE_OK, "drain");
    hipStreamSynchronize(compute);
    CHECK(bad_rows.load() == 0, "%d routed experts read a wrong or absent row", bad_rows.load());
    CHECK(checked.load() == kSteps * s.L * k, "checked %d", checked.load());
    for (int c = 0; c < 2; ++c) {
        moe_pipeline_stats st;
        CHECK(moe_pipeline_stats_get(p, c, &st) == MOE_OK, "stats");
        CHECK(st.requests > 0, "requests");
    }
    moe_pipeline_destroy(p);
    moe_cache_destroy(cache);
    moe_store_close(store);
    if (!path.empty()) unlink(path.c_str());
}

}  // namespace

int main()
{
    for (unsigned seed = 1; seed <= 3; ++seed)
        for (int per_layer = 0; per_layer < 2; ++per_layer)
            for (int policy = 0; policy < 2; ++policy) cache_run(seed, per_layer, policy);
    const PipeCfg cfgs[] = {
        {0, 0, 1, 1, 1, 0, 0, 0},            // no host tier, one reader, one staging row
        {0, 0, 4, 8, 3, 0, 1, 1},            // file store, four readers, three copy streams, guesses
        {64 << 10, 0, 2, 4, 2, 1, 0, 1},     // partial host tier, per-layer LRU
        {1 << 20, 1, 3, 6, 4, 0, 1, 0},      // host tier preloaded with every row
    };
    unsigned seed = 11;
    for (const PipeCfg& pc : cfgs) pipeline_run(pc, seed++);
    stub_shutdown();
    std::printf("host driver: %s (%d failures)\n", g_fail ? "FAILED" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
