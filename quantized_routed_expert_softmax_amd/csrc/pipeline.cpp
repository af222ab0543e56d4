// pipeline.cpp — the miss path of the bounded expert cache: an expert store
// (a file, or host memory standing in for one), an optional pinned-host level of
// expert rows, I/O threads that read missing experts into reused pinned staging
// buffers, installs on a copy stream, and the stream-ordered reservations
// that let installs overlap compute without a host synchronisation.
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", How the
// prototype works, Cache and Reads bullets (a missing expert is fetched by a
// worker thread as a single read into a pinned staging buffer that is reused,
// then moved to its slot by one asynchronous copy; experts that later layers are
// predicted to need are fetched ahead of time; a fully resident model never
// makes a layer wait on the host) and Host tier bullet (a pinned host copy of
// expert rows forms a level under the device cache and may be filled when
// the model loads); "POC: Experts offload", commit messages (one open file per
// shard serves all reads; each layer's slot numbers go to the device in a single
// small copy; a host row is not reused before the copy reading it has finished;
// a predicted read that has not landed yet is bypassed rather than awaited).
//
// Ordering without host waits.  Three event rings carry every dependency:
//   fill rings (one per copy   — recorded after each install copy.  The compute
//   stream)
//                                stream waits on it before the layer that reads the
//                                slot; the slot stays "in flight" in the cache until
//                                it completes; a host row or staging buffer is not
//                                reused before the copy that read it has run.
//   use ring (compute stream)  — recorded when a layer's forward has been enqueued
//                                (release).  An install into a slot first makes the
//                                copy stream wait on the use event of the slot's
//                                previous owner, so a slot is never overwritten
//                                while a queued forward may still read it.
//   table ring (compute)       — the pinned copy of a layer's expert -> slot table
//                                is reused only after its transfer has run.
// A ring entry may be re-recorded by a later operation, always on the same stream
// (each copy stream has its own fill ring, and every copy that reads a given host
// row or staging buffer runs on that buffer's stream); since each stream runs in
// order, waiting on (or querying) the later record is conservative, never wrong.  Every wait targets a record made before the waiting
// operation was enqueued, so the two streams cannot wait on each other in a cycle.
#include <hip/hip_runtime.h>

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <list>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

// --------------------------------------------------------------------------
// Expert store: one row per (layer, expert), layer-major; the row of (l, e)
// starts at base[l] + e * row_bytes[l], base[l] = sum over l' < l of E * row_bytes[l'].
// --------------------------------------------------------------------------
struct moe_store {
    int fd = -1;                    // file store: one descriptor shared by every reader
    const uint8_t* mem = nullptr;   // memory store: caller-owned bytes
    int E = 0;
    std::vector<int64_t> base, row_bytes;
    int64_t total = 0;
};

namespace {

int pfail(int code, const char* msg) { return moe::set_error(code, msg); }

moe_store* store_layout(const moe_size_class_desc* classes, int n_classes, const int32_t* layer_class,
                        int n_layers, int E)
{
    if (!classes || n_classes < 1 || !layer_class || n_layers < 1 || E < 1) {
        pfail(MOE_E_INVALID, "moe_store: bad arguments");
        return nullptr;
    }
    moe_store* s = new (std::nothrow) moe_store;
    if (!s) return nullptr;
    s->E = E;
    s->base.resize(n_layers);
    s->row_bytes.resize(n_layers);
    int64_t o = 0;
    for (int l = 0; l < n_layers; ++l) {
        const int c = layer_class[l];
        if (c < 0 || c >= n_classes || classes[c].slot_bytes <= 0) {
            delete s;
            pfail(MOE_E_INVALID, "moe_store: layer class out of range or empty row size");
            return nullptr;
        }
        s->base[l] = o;
        s->row_bytes[l] = classes[c].slot_bytes;
        o += (int64_t)E * classes[c].slot_bytes;
    }
    s->total = o;
    return s;
}

bool store_row_ok(const moe_store* s, int layer, int expert)
{
    return s && layer >= 0 && layer < (int)s->base.size() && expert >= 0 && expert < s->E;
}

// One contiguous read of a whole row.  0 on success, else an errno value.
int store_read(const moe_store* s, int layer, int expert, void* dst)
{
    const int64_t off = s->base[layer] + (int64_t)expert * s->row_bytes[layer];
    const int64_t n = s->row_bytes[layer];
    if (s->mem) {
        std::memcpy(dst, s->mem + off, (size_t)n);
        return 0;
    }
    int64_t done = 0;
    while (done < n) {
        const ssize_t r = pread(s->fd, (char*)dst + done, (size_t)(n - done), (off_t)(off + done));
        if (r < 0) {
            if (errno == EINTR) continue;
            return errno;
        }
        if (r == 0) return EIO;  // short file
        done += r;
    }
    return 0;
}

}  // namespace

extern "C" {

moe_store* moe_store_open_file(const char* path, const moe_size_class_desc* classes, int n_classes,
                               const int32_t* layer_class, int n_layers, int E)
{
    if (!path) {
        pfail(MOE_E_INVALID, "moe_store_open_file: NULL path");
        return nullptr;
    }
    moe_store* s = store_layout(classes, n_classes, layer_class, n_layers, E);
    if (!s) return nullptr;
    s->fd = open(path, O_RDONLY | O_CLOEXEC);
    if (s->fd < 0) {
        delete s;
        pfail(MOE_E_IO, "moe_store_open_file: cannot open the file");
        return nullptr;
    }
    struct stat st;
    if (fstat(s->fd, &st) != 0 || (int64_t)st.st_size < s->total) {
        close(s->fd);
        delete s;
        pfail(MOE_E_IO, "moe_store_open_file: file shorter than the rows it must hold");
        return nullptr;
    }
    return s;
}

moe_store* moe_store_open_memory(const void* mem, int64_t bytes, const moe_size_class_desc* classes,
                                 int n_classes, const int32_t* layer_class, int n_layers, int E)
{
    if (!mem) {
        pfail(MOE_E_INVALID, "moe_store_open_memory: NULL memory");
        return nullptr;
    }
    moe_store* s = store_layout(classes, n_classes, layer_class, n_layers, E);
    if (!s) return nullptr;
    if (bytes < s->total) {
        delete s;
        pfail(MOE_E_INVALID, "moe_store_open_memory: memory smaller than the rows it must hold");
        return nullptr;
    }
    s->mem = (const uint8_t*)mem;
    return s;
}

void moe_store_close(moe_store* s)
{
    if (!s) return;
    if (s->fd >= 0) close(s->fd);
    delete s;
}

int64_t moe_store_bytes(const moe_store* s) { return s ? s->total : -1; }

int64_t moe_store_row_offset(const moe_store* s, int layer, int expert)
{
    if (!store_row_ok(s, layer, expert)) {
        pfail(MOE_E_INVALID, "moe_store_row_offset: bad arguments");
        return -1;
    }
    return s->base[layer] + (int64_t)expert * s->row_bytes[layer];
}

int moe_store_read(const moe_store* s, int layer, int expert, void* dst)
{
    if (!store_row_ok(s, layer, expert) || !dst) return pfail(MOE_E_INVALID, "moe_store_read: bad arguments");
    if (store_read(s, layer, expert, dst) != 0) return pfail(MOE_E_IO, "moe_store_read: read failed");
    return MOE_OK;
}

}  // extern "C"

// --------------------------------------------------------------------------
// Pipeline
// --------------------------------------------------------------------------
namespace {

constexpr int kMaxCopyStreams = 4;
constexpr int kFillRing = 1024;  // per copy stream
constexpr int kUseRing = 256;
constexpr int kTableRing = 64;

struct HostRow {
    int32_t layer = -1, expert = -1;
    int readers = 0;       // installs that read the row and have not yet enqueued their copy
    bool loading = false;  // a store read into the row is running
    int ev = -1;           // fill-ring entry of the last copy that read the row
    std::list<int64_t>::iterator it;
};

struct HostClass {
    uint8_t* mem = nullptr;  // pinned, rows * row_bytes
    int64_t rows = 0, row_bytes = 0;
    std::vector<HostRow> row;
    std::list<int64_t> lru;  // front = most recently used
};

struct Staging {
    uint8_t* mem = nullptr;  // pinned, max row bytes
    bool busy = false;
    int ev = -1;
};

struct SlotState {
    int use_ev = -1;       // use-ring entry of the last release that covered the slot
    int fill_ev = -1;      // fill-ring entry of the slot's last install
    uint64_t fill_seq = 0; // order in which that install's copy was enqueued
    bool pending = false;  // install accepted, copy not yet enqueued
    bool failed = false;   // the store read of the last install failed
};

// A host-tier install of a prepare whose copy is enqueued after the prepare's
// acquisitions, merged with its neighbours (see flush_deferred).
struct Deferred {
    int layer, expert;
    int64_t row, slot;
    int use_ev;
};

enum JobKind { kInstall, kPreload };

struct Job {
    JobKind kind;
    int layer, expert, cls;
    int64_t slot;   // kInstall
    int use_ev;     // kInstall: use event of the slot's previous owner
    bool guess;     // kInstall started by moe_pipeline_prefetch
    int64_t row;    // kPreload: host row to fill
};

struct Held {
    std::vector<int> experts;
    std::vector<int64_t> slots;
    bool active = false;
};

bool event_done(hipEvent_t e) { return hipEventQuery(e) == hipSuccess; }

}  // namespace

struct moe_pipeline {
    moe_cache* cache = nullptr;
    moe_store* store = nullptr;
    int device = 0;
    int n_classes = 0, n_layers = 0, E = 0;
    std::vector<moe_size_class_desc> desc;
    std::vector<int> layer_class;
    std::vector<uint8_t*> pools;
    std::vector<hipStream_t> copies;
    hipStream_t compute = nullptr;  // the one compute stream prepare/release run on
    bool compute_set = false;

    std::vector<HostClass> host;
    std::vector<int64_t> host_of;  // [layer * E + expert] -> host row, -1 absent
    std::vector<Staging> staging;
    std::vector<std::vector<SlotState>> slot;  // [class][slot]
    std::vector<Held> held;                    // [layer]
    std::vector<moe_pipeline_stats> stats;     // [class]

    hipEvent_t fill_ring[kMaxCopyStreams * kFillRing] = {};  // entry q * kFillRing + j on stream q
    hipEvent_t use_ring[kUseRing] = {};
    hipEvent_t table_ring[kTableRing] = {};
    bool table_used[kTableRing] = {};
    int32_t* table_host = nullptr;  // pinned [kTableRing][E]
    int64_t fill_next[kMaxCopyStreams] = {};
    int64_t use_next = 0, table_next = 0;
    uint64_t fill_count = 0;            // installs enqueued so far (fill_seq source)
    uint64_t use_gen[kUseRing] = {};    // records made of each use-ring entry
    int last_wait[kMaxCopyStreams] = {-1, -1, -1, -1};  // use-ring entry a copy stream last waited for ...
    uint64_t last_wait_gen[kMaxCopyStreams] = {};  // ... and which record of it

    mutable std::mutex mu;  // everything above that threads share
    std::mutex copy_mu[kMaxCopyStreams];  // per copy stream: enqueue + fill-ring record
    std::condition_variable cv_jobs, cv_done;
    std::deque<Job> jobs;
    int active_jobs = 0;
    bool stop = false;
    std::vector<std::thread> threads;
    int io_error = 0;  // first thread-side HIP error (sticky)

    // --- helpers (callers hold `mu` where noted) ---
    int cls_of(int layer) const { return layer_class[layer]; }
    uint8_t* slot_ptr(int cls, int64_t s) const
    {
        return pools[cls] + (size_t)s * (size_t)desc[cls].slot_bytes;
    }
    uint8_t* host_ptr(int cls, int64_t r) const
    {
        return host[cls].mem + (size_t)r * (size_t)host[cls].row_bytes;
    }

    // Copy stream of a source buffer: fixed per host row / staging buffer, so every
    // copy that reads one buffer runs on one stream.
    int row_queue(int64_t r) const { return (int)(r % (int64_t)copies.size()); }

    // Enqueue one install copy on copy stream q; returns the fill-ring entry, or
    // -1 on a HIP error.
    int enqueue_copy(int q, int cls, int64_t s, const uint8_t* src, int use_ev)
    {
        std::lock_guard<std::mutex> g(copy_mu[q]);
        const hipStream_t st = copies[(size_t)q];
        // a stream that already waits for this record of the use event (installs
        // of one layer or pass share their victims' release) need not wait again
        if (use_ev >= 0) {
            const uint64_t gen = __atomic_load_n(&use_gen[use_ev], __ATOMIC_ACQUIRE);
            if (last_wait[q] != use_ev || last_wait_gen[q] != gen) {
                if (hipStreamWaitEvent(st, use_ring[use_ev], 0) != hipSuccess) return -1;
                last_wait[q] = use_ev;
                last_wait_gen[q] = gen;
            }
        }
        if (hipMemcpyAsync(slot_ptr(cls, s), src, (size_t)desc[cls].slot_bytes, hipMemcpyHostToDevice,
                           st) != hipSuccess)
            return -1;
        const int i = q * kFillRing + (int)(fill_next[q]++ % kFillRing);
        if (hipEventRecord(fill_ring[i], st) != hipSuccess) return -1;
        return i;
    }

    // One copy of n consecutive host rows into n consecutive slots on copy stream
    // q, after the stream waited for the use events of every victim slot; one
    // fill-ring entry for all of them, or -1 on a HIP error.
    int enqueue_run(int q, int cls, int64_t s0, int64_t n, const uint8_t* src, const std::vector<int>& use_evs)
    {
        std::lock_guard<std::mutex> g(copy_mu[q]);
        const hipStream_t st = copies[(size_t)q];
        for (int use_ev : use_evs) {
            if (use_ev < 0) continue;
            const uint64_t gen = __atomic_load_n(&use_gen[use_ev], __ATOMIC_ACQUIRE);
            if (last_wait[q] != use_ev || last_wait_gen[q] != gen) {
                if (hipStreamWaitEvent(st, use_ring[use_ev], 0) != hipSuccess) return -1;
                last_wait[q] = use_ev;
                last_wait_gen[q] = gen;
            }
        }
        if (hipMemcpyAsync(slot_ptr(cls, s0), src, (size_t)n * (size_t)desc[cls].slot_bytes,
                           hipMemcpyHostToDevice, st) != hipSuccess)
            return -1;
        const int i = q * kFillRing + (int)(fill_next[q]++ % kFillRing);
        if (hipEventRecord(fill_ring[i], st) != hipSuccess) return -1;
        return i;
    }

    // Enqueue a prepare's deferred host-tier installs: sorted by host row, each
    // run of consecutive rows going to consecutive slots becomes one copy (a
    // prefill pass of consecutive experts whose rows sit in order in the host
    // tier is one or a few large copies instead of 64 of 1.38 MB, each of which
    // pays the copy engine's per-copy cost).  Caller holds mu (released while
    // enqueueing); the rows keep a reader and the slots stay pending until done.
    void flush_deferred(std::unique_lock<std::mutex>& lk, int cls, std::vector<Deferred>& d)
    {
        if (d.empty()) return;
        std::sort(d.begin(), d.end(), [](const Deferred& a, const Deferred& b) { return a.row < b.row; });
        struct Run {
            size_t first, n;
            int ev;
        };
        std::vector<Run> runs;
        for (size_t i = 0; i < d.size(); ++i) {
            if (!runs.empty()) {
                const Deferred& prev = d[i - 1];
                if (d[i].row == prev.row + 1 && d[i].slot == prev.slot + 1) {
                    runs.back().n++;
                    continue;
                }
            }
            runs.push_back(Run{i, 1, -1});
        }
        lk.unlock();
        for (Run& run : runs) {
            const Deferred& f = d[run.first];
            std::vector<int> use_evs;
            for (size_t i = run.first; i < run.first + run.n; ++i)
                if (std::find(use_evs.begin(), use_evs.end(), d[i].use_ev) == use_evs.end()) use_evs.push_back(d[i].use_ev);
            run.ev = enqueue_run(row_queue(f.row), cls, f.slot, (int64_t)run.n, host_ptr(cls, f.row), use_evs);
        }
        lk.lock();
        for (const Run& run : runs)
            for (size_t i = run.first; i < run.first + run.n; ++i) {
                HostRow& row = host[cls].row[(size_t)d[i].row];
                row.readers--;
                if (run.ev >= 0) row.ev = run.ev;
                else if (!io_error) io_error = MOE_E_HIP;
                moe_pipeline_stats& st = stats[cls];
                st.host_hits++;
                if (run.ev >= 0) st.bytes_copied += desc[cls].slot_bytes;
                finish_install(d[i].layer, d[i].expert, cls, d[i].slot, run.ev);
            }
        d.clear();
        cv_done.notify_all();
    }

    void sync_copies()
    {
        for (hipStream_t st : copies) hipStreamSynchronize(st);
    }

    // A host row that may be overwritten: least recently used, nobody reading or
    // loading it, and its last copy has run.  Caller holds mu.  -1 if none.
    int64_t host_victim(int cls)
    {
        HostClass& h = host[cls];
        for (auto it = h.lru.rbegin(); it != h.lru.rend(); ++it) {
            HostRow& r = h.row[(size_t)*it];
            if (r.readers > 0 || r.loading) continue;
            if (r.ev >= 0 && !event_done(fill_ring[r.ev])) continue;
            return *it;
        }
        return -1;
    }

    void host_map(int cls, int64_t r, int layer, int expert)
    {
        HostRow& row = host[cls].row[(size_t)r];
        if (row.layer >= 0) host_of[(size_t)row.layer * E + row.expert] = -1;
        row.layer = layer;
        row.expert = expert;
        host_of[(size_t)layer * E + expert] = r;
    }

    void host_unmap(int cls, int64_t r)
    {
        HostRow& row = host[cls].row[(size_t)r];
        if (row.layer >= 0) host_of[(size_t)row.layer * E + row.expert] = -1;
        row.layer = row.expert = -1;
        host[cls].lru.splice(host[cls].lru.end(), host[cls].lru, row.it);
    }

    void host_touch(int cls, int64_t r)
    {
        HostClass& h = host[cls];
        h.lru.splice(h.lru.begin(), h.lru, h.row[(size_t)r].it);
    }

    // Mark the install of `s` finished (copy enqueued or failed) and tell the cache.
    // Caller holds mu.
    void finish_install(int layer, int expert, int cls, int64_t s, int ev)
    {
        SlotState& ss = slot[cls][(size_t)s];
        ss.pending = false;
        ss.failed = ev < 0;
        ss.fill_ev = ev;
        ss.fill_seq = ++fill_count;
        if (ev >= 0) {
            moe_cache_fill_done(cache, layer, expert, fill_ring[ev]);
        } else {
            // a guess nobody waits for is dropped here; a pinned entry is dropped by
            // the prepare that pinned it
            moe_cache_abort_fill(cache, layer, expert);
        }
    }

    // Try the host tier for an install.  Caller holds mu; returns true when the
    // row is present (the copy is then enqueued here, with mu released meanwhile,
    // or, given `defer`, recorded there for flush_deferred).
    bool install_from_host(std::unique_lock<std::mutex>& lk, int layer, int expert, int cls, int64_t s,
                           int use_ev, std::vector<Deferred>* defer = nullptr)
    {
        if (host.empty() || host[cls].rows == 0) return false;
        const int64_t r = host_of[(size_t)layer * E + expert];
        if (r < 0 || host[cls].row[(size_t)r].loading) return false;
        host[cls].row[(size_t)r].readers++;
        host_touch(cls, r);
        if (defer) {
            defer->push_back(Deferred{layer, expert, r, s, use_ev});
            return true;
        }
        lk.unlock();
        const int ev = enqueue_copy(row_queue(r), cls, s, host_ptr(cls, r), use_ev);
        lk.lock();
        HostRow& row = host[cls].row[(size_t)r];
        row.readers--;
        if (ev >= 0) row.ev = ev;
        else if (!io_error) io_error = MOE_E_HIP;
        moe_pipeline_stats& st = stats[cls];
        st.host_hits++;
        if (ev >= 0) st.bytes_copied += desc[cls].slot_bytes;
        finish_install(layer, expert, cls, s, ev);
        cv_done.notify_all();
        return true;
    }

    void run_install(const Job& j)
    {
        std::unique_lock<std::mutex> lk(mu);
        // rows being loaded for the same expert by a preload: wait for them
        for (;;) {
            const int64_t r = host.empty() ? -1 : host_of[(size_t)j.layer * E + j.expert];
            if (r < 0 || !host[j.cls].row[(size_t)r].loading) break;
            cv_done.wait(lk);
        }
        if (install_from_host(lk, j.layer, j.expert, j.cls, j.slot, j.use_ev)) return;
        // read from the store into a host row (kept for later misses) or a staging buffer
        int64_t r = -1;
        int sidx = -1;
        if (!host.empty() && host[j.cls].rows > 0) r = host_victim(j.cls);
        if (r >= 0) {
            host_map(j.cls, r, j.layer, j.expert);
            HostRow& row = host[j.cls].row[(size_t)r];
            row.loading = true;
            row.readers++;
            host_touch(j.cls, r);
        } else {
            for (;;) {
                int wait_on = -1;
                for (size_t i = 0; i < staging.size(); ++i) {
                    Staging& b = staging[i];
                    if (b.busy) continue;
                    if (b.ev >= 0 && !event_done(fill_ring[b.ev])) {
                        if (wait_on < 0) wait_on = (int)i;
                        continue;
                    }
                    sidx = (int)i;
                    break;
                }
                if (sidx >= 0) break;
                if (wait_on >= 0) {  // wait for that buffer's copy outside the lock
                    const hipEvent_t e = fill_ring[staging[(size_t)wait_on].ev];
                    lk.unlock();
                    hipEventSynchronize(e);
                    lk.lock();
                } else {
                    cv_done.wait(lk);
                }
            }
            staging[(size_t)sidx].busy = true;
        }
        uint8_t* buf = r >= 0 ? host_ptr(j.cls, r) : staging[(size_t)sidx].mem;
        lk.unlock();
        const bool read_ok = store_read(store, j.layer, j.expert, buf) == 0;
        const int q = r >= 0 ? row_queue(r) : sidx % (int)copies.size();
        const int ev = read_ok ? enqueue_copy(q, j.cls, j.slot, buf, j.use_ev) : -1;
        lk.lock();
        if (r >= 0) {
            HostRow& row = host[j.cls].row[(size_t)r];
            row.loading = false;
            row.readers--;
            if (ev >= 0) row.ev = ev;
            if (!read_ok) host_unmap(j.cls, r);
        } else {
            staging[(size_t)sidx].busy = false;
            if (ev >= 0) staging[(size_t)sidx].ev = ev;
        }
        if (read_ok && ev < 0 && !io_error) io_error = MOE_E_HIP;
        moe_pipeline_stats& st = stats[j.cls];
        st.store_reads++;
        if (read_ok) st.bytes_read += desc[j.cls].slot_bytes;
        if (ev >= 0) st.bytes_copied += desc[j.cls].slot_bytes;
        finish_install(j.layer, j.expert, j.cls, j.slot, ev);
        cv_done.notify_all();
    }

    void run_preload(const Job& j)
    {
        const bool ok = store_read(store, j.layer, j.expert, host_ptr(j.cls, j.row)) == 0;
        std::lock_guard<std::mutex> g(mu);
        HostRow& row = host[j.cls].row[(size_t)j.row];
        row.loading = false;
        if (ok) stats[j.cls].bytes_read += desc[j.cls].slot_bytes;
        else {
            host_unmap(j.cls, j.row);
            if (!io_error) io_error = MOE_E_IO;
        }
        cv_done.notify_all();
    }

    void worker()
    {
        hipSetDevice(device);
        for (;;) {
            Job j;
            {
                std::unique_lock<std::mutex> lk(mu);
                cv_jobs.wait(lk, [&] { return stop || !jobs.empty(); });
                if (jobs.empty()) return;  // stop requested and nothing left
                j = jobs.front();
                jobs.pop_front();
                active_jobs++;
            }
            if (j.kind == kInstall) run_install(j);
            else run_preload(j);
            {
                std::lock_guard<std::mutex> g(mu);
                active_jobs--;
            }
            cv_done.notify_all();
        }
    }

    // Accept a device miss of (layer, expert) into slot s.  Caller holds mu.
    void start_install(std::unique_lock<std::mutex>& lk, int layer, int expert, int64_t s, bool guess,
                       std::vector<Deferred>* defer = nullptr)
    {
        const int cls = cls_of(layer);
        SlotState& ss = slot[cls][(size_t)s];
        ss.pending = true;
        ss.failed = false;
        const int use_ev = ss.use_ev;
        if (install_from_host(lk, layer, expert, cls, s, use_ev, defer)) return;
        jobs.push_back(Job{kInstall, layer, expert, cls, s, use_ev, guess, -1});
        cv_jobs.notify_one();
    }

    // Every unpinned slot of class cls is being filled: wait for the oldest fill
    // still in flight (the copies queued behind it keep the copy engines busy),
    // or for a queued store read.  Caller holds mu (released while waiting).
    // False when nothing of the class is in flight.
    bool wait_oldest_fill(std::unique_lock<std::mutex>& lk, int cls)
    {
        int64_t best = -1;
        bool pending = false;
        for (size_t i = 0; i < slot[cls].size(); ++i) {
            const SlotState& ss = slot[cls][i];
            if (ss.pending) {
                pending = true;
                continue;
            }
            if (ss.fill_ev < 0 || event_done(fill_ring[ss.fill_ev])) continue;
            if (best < 0 || ss.fill_seq < slot[cls][(size_t)best].fill_seq) best = (int64_t)i;
        }
        if (best >= 0) {
            const hipEvent_t e = fill_ring[slot[cls][(size_t)best].fill_ev];
            lk.unlock();
            hipEventSynchronize(e);
            lk.lock();
            return true;
        }
        if (pending) {
            cv_done.wait(lk);
            return true;
        }
        return false;
    }

    void wait_idle(std::unique_lock<std::mutex>& lk)
    {
        cv_done.wait(lk, [&] { return jobs.empty() && active_jobs == 0; });
    }

    void unpin_all(int layer)
    {
        Held& h = held[(size_t)layer];
        for (int e : h.experts) moe_cache_unpin(cache, layer, e);
        h.experts.clear();
        h.slots.clear();
        h.active = false;
    }

    ~moe_pipeline()
    {
        {
            std::lock_guard<std::mutex> g(mu);
            stop = true;
        }
        cv_jobs.notify_all();
        for (auto& t : threads) t.join();
        sync_copies();
        for (auto& h : host)
            if (h.mem) hipHostFree(h.mem);
        for (auto& b : staging)
            if (b.mem) hipHostFree(b.mem);
        if (table_host) hipHostFree(table_host);
        for (auto& e : fill_ring)
            if (e) hipEventDestroy(e);
        for (auto& e : use_ring)
            if (e) hipEventDestroy(e);
        for (auto& e : table_ring)
            if (e) hipEventDestroy(e);
    }
};

namespace {

// prepare and release must all use one compute stream: the use and table rings
// are re-recorded on it, which is only conservative on a single in-order stream
bool same_compute(moe_pipeline* p, hipStream_t compute)
{
    if (!p->compute_set) {
        p->compute = compute;
        p->compute_set = true;
    }
    return p->compute == compute;
}

bool ids_ok(const moe_pipeline* p, int layer, const int32_t* ids, int n)
{
    if (!p || layer < 0 || layer >= p->n_layers || n < 0 || (n > 0 && !ids)) return false;
    for (int i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= p->E) return false;
    return true;
}

// Distinct ids in order of first appearance.
std::vector<int> distinct(const int32_t* ids, int n, int E)
{
    std::vector<char> seen((size_t)E, 0);
    std::vector<int> out;
    for (int i = 0; i < n; ++i)
        if (!seen[(size_t)ids[i]]) {
            seen[(size_t)ids[i]] = 1;
            out.push_back(ids[i]);
        }
    return out;
}

}  // namespace

extern "C" {

moe_pipeline* moe_pipeline_create(moe_cache* cache, moe_store* store, void* const* class_pools,
                                  const moe_pipeline_config* cfg, const hipStream_t* copy_streams,
                                  int n_copy_streams)
{
    if (!cache || !store || !class_pools || !cfg || !copy_streams) {
        pfail(MOE_E_INVALID, "moe_pipeline_create: NULL argument");
        return nullptr;
    }
    if (n_copy_streams < 1 || n_copy_streams > kMaxCopyStreams) {
        pfail(MOE_E_INVALID, "moe_pipeline_create: need 1 to 4 copy streams");
        return nullptr;
    }
    for (int q = 0; q < n_copy_streams; ++q)
        if (!copy_streams[q]) {
            pfail(MOE_E_INVALID, "moe_pipeline_create: NULL copy stream");
            return nullptr;
        }
    if (cfg->io_threads < 1 || cfg->io_threads > 64 || cfg->staging_rows < cfg->io_threads ||
        cfg->staging_rows > 1024 || cfg->host_tier_bytes < 0) {
        pfail(MOE_E_INVALID, "moe_pipeline_create: need 1 <= io_threads <= 64, "
                             "io_threads <= staging_rows <= 1024, host_tier_bytes >= 0");
        return nullptr;
    }
    int nc = 0, nl = 0, E = 0;
    moe_cache_shape(cache, &nc, &nl, &E);
    if (nl != (int)store->base.size() || E != store->E) {
        pfail(MOE_E_INVALID, "moe_pipeline_create: store and cache disagree on layers or experts");
        return nullptr;
    }
    moe_pipeline* p = new (std::nothrow) moe_pipeline;
    if (!p) {
        pfail(MOE_E_INVALID, "moe_pipeline_create: out of host memory");
        return nullptr;
    }
    auto bail = [&](int code, const char* msg) -> moe_pipeline* {
        delete p;
        pfail(code, msg);
        return nullptr;
    };
    p->cache = cache;
    p->store = store;
    p->copies.assign(copy_streams, copy_streams + n_copy_streams);
    p->n_classes = nc;
    p->n_layers = nl;
    p->E = E;
    if (hipGetDevice(&p->device) != hipSuccess) return bail(MOE_E_HIP, "moe_pipeline_create: no device");
    p->desc.resize(nc);
    p->pools.resize(nc);
    p->slot.resize(nc);
    p->stats.assign(nc, moe_pipeline_stats{});
    int64_t max_row = 0;
    for (int c = 0; c < nc; ++c) {
        moe_cache_class_desc(cache, c, &p->desc[c]);
        p->pools[c] = (uint8_t*)class_pools[c];
        if (!p->pools[c] && p->desc[c].n_slots > 0) return bail(MOE_E_INVALID, "moe_pipeline_create: NULL pool");
        if ((uintptr_t)p->pools[c] % 256) return bail(MOE_E_INVALID, "moe_pipeline_create: pools need 256-byte alignment");
        p->slot[c].resize((size_t)p->desc[c].n_slots);
        if (p->desc[c].slot_bytes > max_row) max_row = p->desc[c].slot_bytes;
    }
    p->layer_class.resize(nl);
    for (int l = 0; l < nl; ++l) {
        p->layer_class[l] = moe_cache_class_of(cache, l);
        if (store->row_bytes[l] != p->desc[p->layer_class[l]].slot_bytes)
            return bail(MOE_E_INVALID, "moe_pipeline_create: store row size differs from the layer's class");
    }
    p->held.resize(nl);

    for (auto* ring : {p->fill_ring, p->use_ring, p->table_ring}) {
        const int n = ring == p->fill_ring ? (int)p->copies.size() * kFillRing
                      : ring == p->use_ring ? kUseRing : kTableRing;
        for (int i = 0; i < n; ++i)
            if (hipEventCreateWithFlags(&ring[i], hipEventDisableTiming) != hipSuccess)
                return bail(MOE_E_HIP, "moe_pipeline_create: event creation failed");
    }
    if (hipHostMalloc((void**)&p->table_host, sizeof(int32_t) * (size_t)kTableRing * E, hipHostMallocDefault) != hipSuccess)
        return bail(MOE_E_HIP, "moe_pipeline_create: pinned table buffer");
    p->staging.resize((size_t)cfg->staging_rows);
    for (auto& b : p->staging)
        if (hipHostMalloc((void**)&b.mem, (size_t)max_row, hipHostMallocDefault) != hipSuccess)
            return bail(MOE_E_HIP, "moe_pipeline_create: pinned staging buffer");

    // host tier: the budget is split between classes in proportion to the bytes
    // of all their experts, so each layer gets an equal fraction
    if (cfg->host_tier_bytes > 0) {
        std::vector<double> weight(nc, 0.0);
        double sum = 0.0;
        for (int l = 0; l < nl; ++l) {
            const double w = (double)E * (double)p->desc[p->layer_class[l]].slot_bytes;
            weight[p->layer_class[l]] += w;
            sum += w;
        }
        p->host.resize(nc);
        p->host_of.assign((size_t)nl * E, -1);
        for (int c = 0; c < nc; ++c) {
            HostClass& h = p->host[c];
            h.row_bytes = p->desc[c].slot_bytes;
            const double share = sum > 0 ? (double)cfg->host_tier_bytes * weight[c] / sum : 0.0;
            int64_t rows = (int64_t)(share / (double)h.row_bytes);
            int64_t all = 0;  // never more rows than the class has experts
            for (int l = 0; l < nl; ++l) all += p->layer_class[l] == c ? E : 0;
            if (rows > all) rows = all;
            h.rows = rows;
            if (rows == 0) continue;
            if (hipHostMalloc((void**)&h.mem, (size_t)rows * (size_t)h.row_bytes, hipHostMallocDefault) != hipSuccess)
                return bail(MOE_E_HIP, "moe_pipeline_create: pinned host tier");
            h.row.resize((size_t)rows);
            for (int64_t r = 0; r < rows; ++r) {
                h.lru.push_back(r);
                h.row[(size_t)r].it = std::prev(h.lru.end());
            }
        }
    }
    for (int t = 0; t < cfg->io_threads; ++t) p->threads.emplace_back([p] { p->worker(); });

    if (cfg->host_preload && !p->host.empty()) {
        std::unique_lock<std::mutex> lk(p->mu);
        std::vector<int64_t> next(nc, 0);
        for (int l = 0; l < nl; ++l) {
            const int c = p->layer_class[l];
            for (int e = 0; e < E && next[c] < p->host[c].rows; ++e) {
                const int64_t r = next[c]++;
                p->host_map(c, r, l, e);
                p->host[c].row[(size_t)r].loading = true;
                p->host_touch(c, r);
                p->jobs.push_back(Job{kPreload, l, e, c, -1, -1, false, r});
            }
        }
        p->cv_jobs.notify_all();
        p->wait_idle(lk);
        if (p->io_error) {
            lk.unlock();
            return bail(MOE_E_IO, "moe_pipeline_create: a preload read failed");
        }
    }
    return p;
}

void moe_pipeline_destroy(moe_pipeline* p) { delete p; }

int moe_pipeline_prepare(moe_pipeline* p, int layer, const int32_t* ids, int n, int32_t* table_dev,
                         hipStream_t compute)
{
    if (!ids_ok(p, layer, ids, n) || !table_dev)
        return pfail(MOE_E_INVALID, "moe_pipeline_prepare: bad arguments");
    if (!same_compute(p, compute))
        return pfail(MOE_E_INVALID, "moe_pipeline_prepare: another compute stream than before");
    Held& h = p->held[(size_t)layer];
    if (h.active) return pfail(MOE_E_BUSY, "moe_pipeline_prepare: layer prepared and not yet released");
    const int cls = p->cls_of(layer);
    // experts are acquired last first: the class hands out victims in LRU order
    // and empty slots last-created first, so a run of ascending experts (a
    // prefill pass) lands in ascending slots, next to each other like their
    // host-tier rows, and its installs merge into few copies
    std::vector<int> want = distinct(ids, n, p->E);
    std::reverse(want.begin(), want.end());
    std::vector<int64_t> waits;
    std::vector<Deferred> deferred;
    std::unique_lock<std::mutex> lk(p->mu);
    if (p->io_error) return pfail(p->io_error, "moe_pipeline_prepare: an earlier install failed");
    h.active = true;
    for (int e : want) {
        int64_t s = -1;
        int needs_fill = 0;
        int rc = moe_cache_acquire(p->cache, layer, e, &s, &needs_fill);
        // installs still in flight (earlier passes' or guesses') may hold every
        // unpinned slot: wait for them one at a time, oldest first.  A fill can
        // complete between the cache's check and ours, so when nothing is left in
        // flight the cache is asked once more before the class counts as full.
        while (rc == MOE_E_NO_SLOT) {
            p->flush_deferred(lk, cls, deferred);  // what waits may be this prepare's own installs
            const bool waited = p->wait_oldest_fill(lk, cls);
            rc = moe_cache_acquire(p->cache, layer, e, &s, &needs_fill);
            if (!waited) break;
        }
        if (rc != MOE_OK && rc != MOE_E_BUSY) {
            p->flush_deferred(lk, cls, deferred);
            lk.unlock();
            p->unpin_all(layer);
            return pfail(rc, "moe_pipeline_prepare: no free slot in the layer's size class");
        }
        moe_cache_pin(p->cache, layer, e);
        h.experts.push_back(e);
        h.slots.push_back(s);
        moe_pipeline_stats& st = p->stats[cls];
        st.requests++;
        if (rc == MOE_E_BUSY) {
            st.inflight_hits++;
            waits.push_back(s);
        } else if (!needs_fill) {
            st.hits++;
        } else {
            p->start_install(lk, layer, e, s, false, &deferred);
            waits.push_back(s);
        }
    }
    p->flush_deferred(lk, cls, deferred);
    // every install this layer needs has its copy enqueued (or failed)
    p->cv_done.wait(lk, [&] {
        for (int64_t s : waits)
            if (p->slot[cls][(size_t)s].pending) return false;
        return true;
    });
    bool failed = false;
    std::vector<int> evs;
    for (int64_t s : waits) {
        const SlotState& ss = p->slot[cls][(size_t)s];
        if (ss.failed) failed = true;
        else if (ss.fill_ev >= 0) evs.push_back(ss.fill_ev);
    }
    if (failed) {
        std::vector<int> drop;
        for (size_t i = 0; i < h.experts.size(); ++i)
            if (p->slot[cls][(size_t)h.slots[i]].failed) drop.push_back(h.experts[i]);
        lk.unlock();
        p->unpin_all(layer);
        for (int e : drop) moe_cache_abort_fill(p->cache, layer, e);
        return pfail(MOE_E_IO, "moe_pipeline_prepare: reading an expert from the store failed");
    }
    const int t = (int)(p->table_next++ % kTableRing);
    lk.unlock();
    // one wait per distinct fill event: the slots of a coalesced run share one
    // (a wait costs several microseconds of host time; 64 of them per pass were
    // most of a pass's prepare)
    std::sort(evs.begin(), evs.end());
    evs.erase(std::unique(evs.begin(), evs.end()), evs.end());
    for (int ev : evs)
        if (hipStreamWaitEvent(compute, p->fill_ring[ev], 0) != hipSuccess)
            return pfail(MOE_E_HIP, "moe_pipeline_prepare: stream wait failed");
    // one small copy of the layer's expert -> slot table
    int32_t* tbl = p->table_host + (size_t)t * p->E;
    if (p->table_used[t] && hipEventSynchronize(p->table_ring[t]) != hipSuccess)
        return pfail(MOE_E_HIP, "moe_pipeline_prepare: table event");
    p->table_used[t] = true;
    moe_cache_table(p->cache, layer, tbl);
    if (hipMemcpyAsync(table_dev, tbl, sizeof(int32_t) * (size_t)p->E, hipMemcpyHostToDevice, compute) != hipSuccess ||
        hipEventRecord(p->table_ring[t], compute) != hipSuccess)
        return pfail(MOE_E_HIP, "moe_pipeline_prepare: table copy failed");
    return MOE_OK;
}

int moe_pipeline_release(moe_pipeline* p, int layer, hipStream_t compute)
{
    if (!p || layer < 0 || layer >= p->n_layers) return pfail(MOE_E_INVALID, "moe_pipeline_release: bad arguments");
    Held& h = p->held[(size_t)layer];
    if (!h.active) return pfail(MOE_E_INVALID, "moe_pipeline_release: layer not prepared");
    if (!same_compute(p, compute))
        return pfail(MOE_E_INVALID, "moe_pipeline_release: another compute stream than prepare's");
    const int u = (int)(p->use_next++ % kUseRing);
    if (hipEventRecord(p->use_ring[u], compute) != hipSuccess) {
        p->unpin_all(layer);
        return pfail(MOE_E_HIP, "moe_pipeline_release: event record failed");
    }
    // counted after the record: a copy stream that saw this count has waited for
    // this record or a later one
    __atomic_add_fetch(&p->use_gen[u], 1, __ATOMIC_RELEASE);
    {
        std::lock_guard<std::mutex> g(p->mu);
        const int cls = p->cls_of(layer);
        for (int64_t s : h.slots) p->slot[cls][(size_t)s].use_ev = u;
    }
    p->unpin_all(layer);
    return MOE_OK;
}

int moe_pipeline_prefetch(moe_pipeline* p, int layer, const int32_t* ids, int n)
{
    if (!ids_ok(p, layer, ids, n)) return pfail(MOE_E_INVALID, "moe_pipeline_prefetch: bad arguments");
    const int cls = p->cls_of(layer);
    const std::vector<int> want = distinct(ids, n, p->E);
    std::unique_lock<std::mutex> lk(p->mu);
    if (p->io_error) return pfail(p->io_error, "moe_pipeline_prefetch: an earlier install failed");
    int started = 0;
    for (int e : want) {
        int64_t s = -1;
        moe_cache_lookup(p->cache, layer, e, &s);
        moe_pipeline_stats& st = p->stats[cls];
        if (s >= 0) {  // resident or already on its way: a guess never waits
            st.prefetch_skipped++;
            continue;
        }
        int needs_fill = 0;
        const int rc = moe_cache_acquire(p->cache, layer, e, &s, &needs_fill);
        if (rc != MOE_OK || !needs_fill) {
            st.prefetch_skipped++;
            continue;
        }
        st.prefetches++;
        started++;
        p->start_install(lk, layer, e, s, true);
    }
    return started;
}

int moe_pipeline_drain(moe_pipeline* p)
{
    if (!p) return pfail(MOE_E_INVALID, "moe_pipeline_drain: NULL pipeline");
    {
        std::unique_lock<std::mutex> lk(p->mu);
        p->wait_idle(lk);
    }
    for (hipStream_t st : p->copies)
        if (hipStreamSynchronize(st) != hipSuccess) return pfail(MOE_E_HIP, "moe_pipeline_drain: copy stream");
    moe_cache_poll(p->cache);
    std::lock_guard<std::mutex> g(p->mu);
    if (p->io_error) return pfail(p->io_error, "moe_pipeline_drain: an install failed");
    return MOE_OK;
}

int moe_pipeline_prefill(moe_pipeline* p, int layer, const int32_t* ids_host, const void* x, int T,
                         const int32_t* topk_ids, const float* topk_w, int k, int32_t* table_dev,
                         void* out, void* ws, size_t ws_bytes, uint32_t* err_word, hipStream_t compute)
{
    if (!p || layer < 0 || layer >= p->n_layers)
        return pfail(MOE_E_INVALID, "moe_pipeline_prefill: bad arguments");
    if (T == 0) return 0;
    const int E = p->E;
    const int cls = p->cls_of(layer);
    const moe_size_class_desc* d = &p->desc[(size_t)cls];
    std::vector<int32_t> pt((size_t)moe_pass_table_size(E, moe::kPassExperts));
    if (pt.empty()) return pfail(MOE_E_INVALID, "moe_pipeline_prefill: bad E");
    if (int rc = moe_pass_table_host(ids_host, T, k, E, moe::kPassExperts, pt.data())) return rc;
    const int n_pass = pt[1];
    if (n_pass > 0 && d->n_slots < std::min<int64_t>(pt[0], moe::kPassExperts))
        return pfail(MOE_E_NO_SLOT, "moe_pipeline_prefill: the layer's class holds fewer slots than one pass");
    if (int rc = moe_prefill_sort(x, T, topk_ids, k, E, d, ws, ws_bytes, err_word, compute)) return rc;
    const int32_t* starts = pt.data() + 2 + E;
    for (int q = 0; q < n_pass; ++q) {
        // the pass's hit experts resident (their installs overlap the kernels of
        // the passes already enqueued), its kernels, then the slots released
        const int32_t* hits = pt.data() + 2 + starts[q];
        if (int rc = moe_pipeline_prepare(p, layer, hits, starts[q + 1] - starts[q], table_dev, compute))
            return rc;
        const int rc = moe_prefill_pass(T, k, E, q, q + 1, table_dev, p->pools[(size_t)cls], d, ws, ws_bytes,
                                        err_word, compute);
        const int rr = moe_pipeline_release(p, layer, compute);
        if (rc) return rc;
        if (rr) return rr;
    }
    if (int rc = moe_prefill_combine(T, k, E, topk_w, d, out, ws, ws_bytes, compute)) return rc;
    return n_pass;
}

int moe_pipeline_stats_get(const moe_pipeline* p, int cls, moe_pipeline_stats* out)
{
    if (!p || !out || cls < 0 || cls >= p->n_classes)
        return pfail(MOE_E_INVALID, "moe_pipeline_stats_get: bad arguments");
    std::lock_guard<std::mutex> g(p->mu);
    *out = p->stats[(size_t)cls];
    return MOE_OK;
}

int64_t moe_pipeline_host_rows(const moe_pipeline* p, int cls)
{
    if (!p || cls < 0 || cls >= p->n_classes) return -1;
    return p->host.empty() ? 0 : p->host[(size_t)cls].rows;
}

}  // extern "C"
