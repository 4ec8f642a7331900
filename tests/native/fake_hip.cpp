// Host-memory stand-in for the HIP runtime calls the library's host code
// makes (plan and device-table management, resharding), so that code can be
// built with AddressSanitizer and UndefinedBehaviorSanitizer and run on a
// machine without a GPU.  "Device" memory is malloc'd host memory (ASan sees
// every table the library uploads), copies are memcpy, streams and events
// do nothing.  Test infrastructure only: the library links the real runtime.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

extern "C" {

hipError_t hipGetDevice(int *device) {
    *device = 0;
    return hipSuccess;
}

hipError_t hipSetDevice(int) { return hipSuccess; }

hipError_t hipMalloc(void **ptr, size_t size) {
    *ptr = std::malloc(size != 0 ? size : 1);
    return *ptr != nullptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipFree(void *ptr) {
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t) {
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

hipError_t hipGetLastError(void) { return hipSuccess; }

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

const char *hipGetErrorString(hipError_t e) {
    switch (e) {
        case hipSuccess: return "no error";
        case hipErrorLaunchFailure: return "unspecified launch failure";
        case hipErrorOutOfMemory: return "out of memory";
        default: return "HIP error";
    }
}

}  // extern "C"
