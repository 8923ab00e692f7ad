// workspace.cpp -- device workspace for launches that leave partial sums in
// memory (stream-K runs of the direct-load tiles, split-K slices of the
// few-rows skinny kernel).
//
// Outside graph capture a call takes the workspace cached for its (device,
// stream): work on one stream runs in order, so every call on that stream can
// reuse one buffer.  A request larger than the cached buffer replaces it: the
// old buffer is returned with hipFreeAsync on the same stream (after the work
// already queued there) and the new one taken with hipMallocAsync.  Cached
// buffers are held until sgemm_workspace_release or the end of the process.
//
// Under graph capture the workspace is the graph's own: hipMallocAsync and
// hipFreeAsync on the capturing stream record allocation and free nodes, so
// replays of the graph never share memory with eager calls.
#include <map>
#include <mutex>
#include <utility>

#include "gemm_internal.hpp"

namespace sg {
namespace {

struct Cached {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex &cache_mutex() {
    static std::mutex m;
    return m;
}

std::map<std::pair<int, hipStream_t>, Cached> &cache() {
    static std::map<std::pair<int, hipStream_t>, Cached> c;
    return c;
}

}  // namespace

hipError_t workspace_acquire(size_t bytes, hipStream_t stream, Workspace &w) {
    w = Workspace{};
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        e = hipMallocAsync(&w.ptr, bytes, stream);
        w.owned = (e == hipSuccess);
        return e;
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(cache_mutex());
    Cached &c = cache()[{dev, stream}];
    if (c.bytes < bytes) {
        if (c.ptr) {
            e = hipFreeAsync(c.ptr, stream);
            c = Cached{};
            if (e != hipSuccess) return e;
        }
        e = hipMallocAsync(&c.ptr, bytes, stream);
        if (e != hipSuccess) {
            c = Cached{};
            return e;
        }
        c.bytes = bytes;
    }
    w.ptr = c.ptr;
    return hipSuccess;
}

hipError_t workspace_release(const Workspace &w, hipStream_t stream) {
    return w.owned ? hipFreeAsync(w.ptr, stream) : hipSuccess;
}

hipError_t workspace_release_all() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(cache_mutex());
    for (auto it = cache().begin(); it != cache().end();) {
        if (it->first.first == dev) {
            const hipError_t f = hipFreeAsync(it->second.ptr, nullptr);
            if (f != hipSuccess && e == hipSuccess) e = f;
            it = cache().erase(it);
        } else {
            ++it;
        }
    }
    const hipError_t f = hipStreamSynchronize(nullptr);
    return e != hipSuccess ? e : f;
}

}  // namespace sg
