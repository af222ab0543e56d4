// cache.cpp — host side of the bounded expert cache: size classes, one eviction
// order per class (or per layer), per-layer expert -> slot tables, reservation of
// slots whose fill is in flight.
//
// Sources: "RFC: stream MoE experts from disk in from_pretrained", How the
// prototype works, Cache (a fixed pool of expert slots allocated up front, LRU
// eviction, the host holds each layer's map from expert to slot) and Reads (a
// miss lands in its slot through a single asynchronous copy); "POC: Experts
// offload", host-tier commit message (a host row is not reused before the copy
// reading it has finished);
// "moe: expert slots in size classes", PR description and the ExpertCache
// constructor in its review (a class = the layers whose experts take equal bytes,
// with a separate slot pool and LRU; a class's slots are adjacent; unused slots
// are queued at the LRU's tail and handed out before any eviction; no class
// borrows another's budget; --per-layer gives every layer an LRU of its own and
// an equal fraction); the RFC's Cache bullet (LRU, optional LFU).
//
// A class's slots form one partition (shared LRU) or one partition per layer of
// the class (per-layer mode: slots split as evenly as possible, in layer order,
// contiguous).  Each partition keeps its slots in a recency list.  LRU evicts the
// least recently used candidate; LFU evicts the candidate with the fewest uses
// since it became resident, ties to the least recently used.  A candidate is
// neither pinned nor in flight; empty slots always go first.  Hits, touches and
// LRU victims are O(1) (list splice + table lookup); an LFU victim scans its
// partition.  One mutex guards everything: fills may be reported from I/O threads.
#include <hip/hip_runtime.h>

#include <cstring>
#include <list>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.h"

struct CacheSlot {
    int32_t layer = -1;
    int32_t expert = -1;
    int32_t pins = 0;
    int32_t part = 0;  // partition of the class that owns the slot
    int64_t uses = 0;  // acquires since the slot took its current expert
    bool inflight = false;
    hipEvent_t ev = nullptr;
    std::list<int64_t>::iterator it;
};

struct CachePart {
    std::list<int64_t> lru;  // front = most recently used, back = least
};

struct CacheClass {
    moe_size_class_desc desc;
    std::vector<CacheSlot> slots;
    std::vector<CachePart> parts;
    int64_t hits = 0, misses = 0, evictions = 0;
};

struct moe_cache {
    std::vector<CacheClass> classes;
    std::vector<int32_t> layer_class;
    std::vector<int32_t> layer_part;  // partition of the layer within its class
    int policy = MOE_EVICT_LRU;
    int per_layer = 0;
    int E = 0;
    std::vector<std::vector<int64_t>> table;  // [layer][expert] -> slot, -1 absent
    int64_t hits = 0, misses = 0, evictions = 0;
    mutable std::mutex mu;
};

namespace {

int cache_fail(int code, const char* msg) { return moe::set_error(code, msg); }

// A slot whose fill event has completed is no longer in flight.
void poll_slot(CacheSlot& s)
{
    if (s.inflight && s.ev) {
        if (hipEventQuery(s.ev) == hipSuccess) {
            s.inflight = false;
            s.ev = nullptr;
        }
    }
}

bool layer_ok(const moe_cache* c, int layer, int expert)
{
    return c && layer >= 0 && layer < (int)c->layer_class.size() && expert >= 0 && expert < c->E;
}

// The victim of a partition: an empty slot if any (they sit at the back), else the
// least recently used (LRU) or least used, then least recently used (LFU)
// candidate.  -1 when every slot is pinned or in flight.
int64_t pick_victim(moe_cache* c, CacheClass& k, CachePart& part)
{
    int64_t best = -1;
    int64_t best_uses = 0;
    for (auto it = part.lru.rbegin(); it != part.lru.rend(); ++it) {
        CacheSlot& cs = k.slots[(size_t)*it];
        poll_slot(cs);
        if (cs.pins > 0 || cs.inflight) continue;
        if (cs.layer < 0) return *it;  // empty
        if (c->policy == MOE_EVICT_LRU) return *it;
        if (best < 0 || cs.uses < best_uses) {  // strict: ties stay with the less recent
            best = *it;
            best_uses = cs.uses;
        }
    }
    return best;
}

}  // namespace

extern "C" {

moe_cache* moe_cache_create(const moe_size_class_desc* classes, int n_classes,
                            const int32_t* layer_class, int n_layers, int E)
{
    return moe_cache_create_ex(classes, n_classes, layer_class, n_layers, E, MOE_EVICT_LRU, 0);
}

moe_cache* moe_cache_create_ex(const moe_size_class_desc* classes, int n_classes,
                               const int32_t* layer_class, int n_layers, int E, int policy,
                               int per_layer)
{
    if (!classes || n_classes < 1 || !layer_class || n_layers < 1 || E < 1) {
        cache_fail(MOE_E_INVALID, "moe_cache_create: bad arguments");
        return nullptr;
    }
    if (policy != MOE_EVICT_LRU && policy != MOE_EVICT_LFU) {
        cache_fail(MOE_E_INVALID, "moe_cache_create: unknown eviction policy");
        return nullptr;
    }
    for (int l = 0; l < n_layers; ++l)
        if (layer_class[l] < 0 || layer_class[l] >= n_classes) {
            cache_fail(MOE_E_INVALID, "moe_cache_create: layer class out of range");
            return nullptr;
        }
    moe_cache* c = new (std::nothrow) moe_cache;
    if (!c) return nullptr;
    c->E = E;
    c->policy = policy;
    c->per_layer = per_layer ? 1 : 0;
    c->layer_class.assign(layer_class, layer_class + n_layers);
    c->layer_part.assign(n_layers, 0);
    c->table.assign(n_layers, std::vector<int64_t>(E, -1));
    c->classes.resize(n_classes);
    for (int ci = 0; ci < n_classes; ++ci) {
        CacheClass& k = c->classes[ci];
        k.desc = classes[ci];
        if (k.desc.n_slots < 0) {
            delete c;
            cache_fail(MOE_E_INVALID, "moe_cache_create: negative slot count");
            return nullptr;
        }
        int n_parts = 1;
        if (c->per_layer) {
            n_parts = 0;
            for (int l = 0; l < n_layers; ++l)
                if (layer_class[l] == ci) c->layer_part[l] = n_parts++;
            if (n_parts == 0) n_parts = 1;  // a class no layer uses
        }
        k.parts.resize((size_t)n_parts);
        k.slots.resize((size_t)k.desc.n_slots);
        // partition p owns a contiguous run of n/P (+1 for the first n % P) slots
        const int64_t base = k.desc.n_slots / n_parts, extra = k.desc.n_slots % n_parts;
        int64_t s = 0;
        for (int pi = 0; pi < n_parts; ++pi) {
            const int64_t cnt = base + (pi < extra ? 1 : 0);
            for (int64_t i = 0; i < cnt; ++i, ++s) {
                CachePart& part = k.parts[(size_t)pi];
                part.lru.push_back(s);  // unused slots queue at the tail, where victims come from
                k.slots[(size_t)s].it = std::prev(part.lru.end());
                k.slots[(size_t)s].part = pi;
            }
        }
    }
    return c;
}

void moe_cache_destroy(moe_cache* c) { delete c; }

int moe_cache_shape(const moe_cache* c, int* n_classes, int* n_layers, int* E)
{
    if (!c) return cache_fail(MOE_E_INVALID, "moe_cache_shape: NULL cache");
    if (n_classes) *n_classes = (int)c->classes.size();
    if (n_layers) *n_layers = (int)c->layer_class.size();
    if (E) *E = c->E;
    return MOE_OK;
}

int moe_cache_class_desc(const moe_cache* c, int cls, moe_size_class_desc* d)
{
    if (!c || !d || cls < 0 || cls >= (int)c->classes.size())
        return cache_fail(MOE_E_INVALID, "moe_cache_class_desc: bad arguments");
    *d = c->classes[cls].desc;
    return MOE_OK;
}

int moe_cache_class_of(const moe_cache* c, int layer)
{
    if (!c || layer < 0 || layer >= (int)c->layer_class.size()) return -1;
    return c->layer_class[layer];
}

int moe_cache_acquire(moe_cache* c, int layer, int expert, int64_t* slot, int* needs_fill)
{
    if (!layer_ok(c, layer, expert) || !slot || !needs_fill)
        return cache_fail(MOE_E_INVALID, "moe_cache_acquire: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    CacheClass& k = c->classes[c->layer_class[layer]];
    CachePart& part = k.parts[(size_t)c->layer_part[layer]];
    *needs_fill = 0;
    int64_t s = c->table[layer][expert];
    if (s >= 0) {
        CacheSlot& cs = k.slots[(size_t)s];
        poll_slot(cs);
        *slot = s;
        part.lru.splice(part.lru.begin(), part.lru, cs.it);
        ++cs.uses;
        if (cs.inflight) return MOE_E_BUSY;
        ++c->hits;
        ++k.hits;
        return MOE_OK;
    }
    const int64_t v = pick_victim(c, k, part);
    if (v >= 0) {
        CacheSlot& cs = k.slots[(size_t)v];
        if (cs.layer >= 0) {
            c->table[cs.layer][cs.expert] = -1;
            ++c->evictions;
            ++k.evictions;
        }
        cs.layer = layer;
        cs.expert = expert;
        cs.uses = 1;
        cs.inflight = true;
        cs.ev = nullptr;
        c->table[layer][expert] = v;
        part.lru.splice(part.lru.begin(), part.lru, cs.it);
        ++c->misses;
        ++k.misses;
        *slot = v;
        *needs_fill = 1;
        return MOE_OK;
    }
    *slot = -1;
    return cache_fail(MOE_E_NO_SLOT, "moe_cache_acquire: every slot of the class is pinned or in flight");
}

int moe_cache_fill_done(moe_cache* c, int layer, int expert, hipEvent_t ev)
{
    if (!layer_ok(c, layer, expert)) return cache_fail(MOE_E_INVALID, "moe_cache_fill_done: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    const int64_t s = c->table[layer][expert];
    if (s < 0) return cache_fail(MOE_E_NOT_RESIDENT, "moe_cache_fill_done: entry not resident");
    CacheSlot& cs = c->classes[c->layer_class[layer]].slots[(size_t)s];
    if (!cs.inflight) return cache_fail(MOE_E_INVALID, "moe_cache_fill_done: no fill in flight");
    if (ev) {
        cs.ev = ev;
        poll_slot(cs);
    } else {
        cs.inflight = false;
        cs.ev = nullptr;
    }
    return MOE_OK;
}

int moe_cache_abort_fill(moe_cache* c, int layer, int expert)
{
    if (!layer_ok(c, layer, expert)) return cache_fail(MOE_E_INVALID, "moe_cache_abort_fill: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    const int64_t s = c->table[layer][expert];
    if (s < 0) return cache_fail(MOE_E_NOT_RESIDENT, "moe_cache_abort_fill: entry not resident");
    CacheClass& k = c->classes[c->layer_class[layer]];
    CacheSlot& cs = k.slots[(size_t)s];
    if (!cs.inflight) return cache_fail(MOE_E_INVALID, "moe_cache_abort_fill: no fill in flight");
    if (cs.pins > 0) return cache_fail(MOE_E_BUSY, "moe_cache_abort_fill: entry is pinned");
    // the slot holds nothing usable: empty it and put it where empty slots sit
    c->table[layer][expert] = -1;
    cs.layer = -1;
    cs.expert = -1;
    cs.uses = 0;
    cs.inflight = false;
    cs.ev = nullptr;
    CachePart& part = k.parts[(size_t)cs.part];
    part.lru.splice(part.lru.end(), part.lru, cs.it);
    return MOE_OK;
}

int moe_cache_poll(moe_cache* c)
{
    if (!c) return cache_fail(MOE_E_INVALID, "moe_cache_poll: NULL cache");
    std::lock_guard<std::mutex> lock(c->mu);
    int still = 0;
    for (auto& k : c->classes)
        for (auto& cs : k.slots) {
            poll_slot(cs);
            still += cs.inflight ? 1 : 0;
        }
    return still;
}

int moe_cache_pin(moe_cache* c, int layer, int expert)
{
    if (!layer_ok(c, layer, expert)) return cache_fail(MOE_E_INVALID, "moe_cache_pin: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    const int64_t s = c->table[layer][expert];
    if (s < 0) return cache_fail(MOE_E_NOT_RESIDENT, "moe_cache_pin: entry not resident");
    ++c->classes[c->layer_class[layer]].slots[(size_t)s].pins;
    return MOE_OK;
}

int moe_cache_unpin(moe_cache* c, int layer, int expert)
{
    if (!layer_ok(c, layer, expert)) return cache_fail(MOE_E_INVALID, "moe_cache_unpin: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    const int64_t s = c->table[layer][expert];
    if (s < 0) return cache_fail(MOE_E_NOT_RESIDENT, "moe_cache_unpin: entry not resident");
    CacheSlot& cs = c->classes[c->layer_class[layer]].slots[(size_t)s];
    if (cs.pins <= 0) return cache_fail(MOE_E_INVALID, "moe_cache_unpin: not pinned");
    --cs.pins;
    return MOE_OK;
}

int moe_cache_table(const moe_cache* c, int layer, int32_t* table)
{
    if (!c || !table || layer < 0 || layer >= (int)c->layer_class.size())
        return cache_fail(MOE_E_INVALID, "moe_cache_table: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    for (int e = 0; e < c->E; ++e) table[e] = (int32_t)c->table[layer][e];
    return MOE_OK;
}

int moe_cache_lookup(const moe_cache* c, int layer, int expert, int64_t* slot)
{
    if (!layer_ok(c, layer, expert) || !slot) return cache_fail(MOE_E_INVALID, "moe_cache_lookup: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    *slot = c->table[layer][expert];
    return MOE_OK;
}

int moe_cache_stats(const moe_cache* c, int64_t* hits, int64_t* misses, int64_t* evictions)
{
    if (!c) return cache_fail(MOE_E_INVALID, "moe_cache_stats: NULL cache");
    std::lock_guard<std::mutex> lock(c->mu);
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (evictions) *evictions = c->evictions;
    return MOE_OK;
}

int moe_cache_class_stats(const moe_cache* c, int cls, int64_t* hits, int64_t* misses,
                          int64_t* evictions)
{
    if (!c || cls < 0 || cls >= (int)c->classes.size())
        return cache_fail(MOE_E_INVALID, "moe_cache_class_stats: bad arguments");
    std::lock_guard<std::mutex> lock(c->mu);
    const CacheClass& k = c->classes[cls];
    if (hits) *hits = k.hits;
    if (misses) *misses = k.misses;
    if (evictions) *evictions = k.evictions;
    return MOE_OK;
}

}  // extern "C"
