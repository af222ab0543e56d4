// Extra calls of the host-only HIP stand-in, for the sanitizer driver only.
#pragma once
#include <hip/hip_runtime_api.h>

#include <functional>

// A new stream (a worker thread running its queue in order).
hipStream_t stub_stream_create();
// Enqueue a host function on a stream: it runs after everything enqueued before
// it on that stream (copies, event waits) and before everything after it.
void stub_host_task(hipStream_t s, std::function<void()> fn);
// Drain and join every stream, then free streams and events.
void stub_shutdown();
