// Host-only stand-in for the HIP runtime API, for building the library's host
// code (size-class cache, expert store, miss pipeline) with the compiler's
// address, undefined-behaviour and thread sanitizers on a machine without a GPU.
// Only what that code calls is declared.  The implementation
// (tests/sanitize/hip_stub.cpp) keeps HIP's ordering semantics: every stream is
// a worker thread that runs its queue in order, copies are asynchronous, an
// event completes when the stream reaches the point where it was recorded, and
// hipStreamWaitEvent makes a stream wait for the event's latest record.
#pragma once
#include <stddef.h>
#include <stdint.h>

typedef enum hipError_t {
    hipSuccess = 0,
    hipErrorInvalidValue = 1,
    hipErrorOutOfMemory = 2,
    hipErrorInvalidConfiguration = 9,
    hipErrorNotReady = 600,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum hipMemcpyKind {
    hipMemcpyHostToHost = 0,
    hipMemcpyHostToDevice = 1,
    hipMemcpyDeviceToHost = 2,
    hipMemcpyDeviceToDevice = 3,
    hipMemcpyDefault = 4,
} hipMemcpyKind;

#define hipEventDefault 0x0
#define hipEventDisableTiming 0x2
#define hipHostMallocDefault 0x0

#ifdef __cplusplus
extern "C" {
#endif
hipError_t hipGetDevice(int* device);
hipError_t hipSetDevice(int device);
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned flags);
hipError_t hipEventDestroy(hipEvent_t e);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventQuery(hipEvent_t e);
hipError_t hipEventSynchronize(hipEvent_t e);
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned flags);
hipError_t hipStreamSynchronize(hipStream_t s);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t s);
hipError_t hipHostMalloc(void** p, size_t n, unsigned flags);
hipError_t hipHostFree(void* p);
#ifdef __cplusplus
}
#endif
