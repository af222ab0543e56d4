// Host-only implementation of the HIP runtime subset in stub/hip/hip_runtime_api.h
// (see there).  Streams are worker threads with ordered queues; events carry a
// record generation and a completed generation, so re-recorded events behave as
// in HIP (queries and waits refer to the latest record at the time of the call).
// All hand-offs go through std::mutex / std::condition_variable, which the
// thread sanitizer understands: a consumer that touches memory before the event
// that orders it has completed shows up as a data race.
#include <hip/hip_runtime_api.h>

#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "hip_stub_ext.h"

struct ihipEvent_t {
    std::mutex m;
    std::condition_variable cv;
    uint64_t recorded = 0;   // generation of the latest record
    uint64_t completed = 0;  // highest generation its stream has reached
};

struct ihipStream_t {
    std::mutex m;
    std::condition_variable cv;
    std::deque<std::function<void()>> q;
    bool stop = false;
    std::thread th;

    ihipStream_t()
    {
        th = std::thread([this] {
            for (;;) {
                std::function<void()> task;
                {
                    std::unique_lock<std::mutex> lk(m);
                    cv.wait(lk, [this] { return stop || !q.empty(); });
                    if (q.empty()) return;
                    task = std::move(q.front());
                    q.pop_front();
                }
                task();
            }
        });
    }
    void push(std::function<void()> f)
    {
        {
            std::lock_guard<std::mutex> lk(m);
            q.push_back(std::move(f));
        }
        cv.notify_one();
    }
    void join()
    {
        {
            std::lock_guard<std::mutex> lk(m);
            stop = true;
        }
        cv.notify_one();
        if (th.joinable()) th.join();
    }
};

namespace {

std::mutex g_mu;
std::vector<std::unique_ptr<ihipStream_t>> g_streams;  // [0] = the null stream
std::vector<std::unique_ptr<ihipEvent_t>> g_events;    // freed at shutdown (tasks may still name them)

ihipStream_t* resolve(hipStream_t s)
{
    if (s) return s;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_streams.empty()) g_streams.emplace_back(new ihipStream_t());
    return g_streams[0].get();
}

}  // namespace

hipStream_t stub_stream_create()
{
    resolve(nullptr);  // the null stream first, so it is [0]
    std::lock_guard<std::mutex> lk(g_mu);
    g_streams.emplace_back(new ihipStream_t());
    return g_streams.back().get();
}

void stub_host_task(hipStream_t s, std::function<void()> fn) { resolve(s)->push(std::move(fn)); }

void stub_shutdown()
{
    std::vector<std::unique_ptr<ihipStream_t>> streams;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        streams.swap(g_streams);
    }
    for (auto& s : streams) s->join();
    streams.clear();
    std::lock_guard<std::mutex> lk(g_mu);
    g_events.clear();
}

extern "C" {

hipError_t hipGetDevice(int* device)
{
    if (!device) return hipErrorInvalidValue;
    *device = 0;
    return hipSuccess;
}

hipError_t hipSetDevice(int device) { return device == 0 ? hipSuccess : hipErrorInvalidValue; }

hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned)
{
    if (!e) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lk(g_mu);
    g_events.emplace_back(new ihipEvent_t());
    *e = g_events.back().get();
    return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidValue; }

hipError_t hipEventRecord(hipEvent_t e, hipStream_t s)
{
    if (!e) return hipErrorInvalidValue;
    uint64_t g;
    {
        std::lock_guard<std::mutex> lk(e->m);
        g = ++e->recorded;
    }
    resolve(s)->push([e, g] {
        {
            std::lock_guard<std::mutex> lk(e->m);
            if (e->completed < g) e->completed = g;
        }
        e->cv.notify_all();
    });
    return hipSuccess;
}

hipError_t hipEventQuery(hipEvent_t e)
{
    if (!e) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lk(e->m);
    return e->completed >= e->recorded ? hipSuccess : hipErrorNotReady;
}

hipError_t hipEventSynchronize(hipEvent_t e)
{
    if (!e) return hipErrorInvalidValue;
    std::unique_lock<std::mutex> lk(e->m);
    const uint64_t g = e->recorded;
    e->cv.wait(lk, [e, g] { return e->completed >= g; });
    return hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned)
{
    if (!e) return hipErrorInvalidValue;
    uint64_t g;
    {
        std::lock_guard<std::mutex> lk(e->m);
        g = e->recorded;
    }
    resolve(s)->push([e, g] {
        std::unique_lock<std::mutex> lk(e->m);
        e->cv.wait(lk, [e, g] { return e->completed >= g; });
    });
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t s)
{
    std::mutex m;
    std::condition_variable cv;
    bool done = false;
    resolve(s)->push([&] {
        std::lock_guard<std::mutex> lk(m);  // notify under the lock: the waiter owns m and cv
        done = true;
        cv.notify_all();
    });
    std::unique_lock<std::mutex> lk(m);
    cv.wait(lk, [&] { return done; });
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t s)
{
    if ((!dst || !src) && n) return hipErrorInvalidValue;
    resolve(s)->push([dst, src, n] { std::memcpy(dst, src, n); });
    return hipSuccess;
}

hipError_t hipHostMalloc(void** p, size_t n, unsigned)
{
    if (!p) return hipErrorInvalidValue;
    *p = std::aligned_alloc(256, (n + 255) / 256 * 256);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipHostFree(void* p)
{
    std::free(p);
    return hipSuccess;
}

}  // extern "C"
