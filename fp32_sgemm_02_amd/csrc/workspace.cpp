// workspace.cpp -- device memory for launches that leave partial sums in
// memory (stream-K runs of the direct-load tiles, K slices of the few-rows
// skinny kernel), and the static scratch array of the entry point that
// allocates nothing.
//
// Layout of every workspace: kWorkspaceCounters arrival counters (zero
// between launches: a launch that counts arrivals on them sets each one back
// to zero before it ends), then the partial sums.
//
// Outside graph capture a call takes the workspace cached for its (device,
// stream): work on one stream runs in order, so every call on that stream can
// reuse one buffer.  The per-thread default stream (hipStreamPerThread) is a
// different stream on every host thread behind one handle value, so its
// buffers are kept per thread.  A request larger than the cached buffer
// replaces it: the old buffer is returned with hipFreeAsync on the same
// stream (after the work already queued there), the new one taken with
// hipMallocAsync and its counters cleared by a fill kernel on the stream.
// Cached buffers are held until sgemm_workspace_release or the end of the
// process.  A stream whose handle is destroyed and whose value a new stream
// later receives would inherit its buffer: sgemm_workspace_release must be
// called before destroying a stream that ran stream-K or split launches.
//
// Under graph capture the workspace is the graph's own: hipMallocAsync and
// hipFreeAsync on the capturing stream record allocation and free nodes (the
// counters cleared by a recorded fill kernel), so replays of the graph never
// share memory with eager calls.
//
// A problem that brings its own scratch (Problem::scratch, set by the entry
// point that allocates nothing) takes it instead, with no allocation at all.
#include <map>
#include <mutex>
#include <thread>
#include <tuple>

#include "gemm_internal.hpp"

namespace sg {
namespace {

// The static scratch: counters, then 16 MiB for partial sums.  Zero at load
// (so its counters start at zero); each device holds its own copy until the
// process ends.
constexpr size_t kStaticScratchBytes = kWorkspaceCounterBytes + ((size_t)16 << 20);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;

__global__ void __launch_bounds__(256) zero_counters(unsigned *c, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) c[i] = 0u;
}

hipError_t clear_counters(void *base, hipStream_t stream) {
    hipLaunchKernelGGL(zero_counters, dim3((kWorkspaceCounters + 255) / 256), dim3(256), 0, stream,
                       static_cast<unsigned *>(base), kWorkspaceCounters);
    return hipGetLastError();
}

struct Cached {
    void *ptr = nullptr;   // the allocation: counters, then the sums
    size_t bytes = 0;      // bytes for the sums
};

using Key = std::tuple<int, hipStream_t, std::thread::id>;

std::mutex &cache_mutex() {
    static std::mutex m;
    return m;
}

std::map<Key, Cached> &cache() {
    static std::map<Key, Cached> c;
    return c;
}

void fill(Workspace &w, void *base, bool owned) {
    w.base = base;
    w.counters = static_cast<unsigned *>(base);
    w.ptr = static_cast<unsigned char *>(base) + kWorkspaceCounterBytes;
    w.owned = owned;
}

}  // namespace

hipError_t static_scratch(void **ptr, size_t *bytes) {
    static std::mutex m;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(m);
    if (!addr[dev]) {
        // the array's device address on this device (the name itself is a
        // host-side stand-in and must never reach a kernel)
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = q;
    }
    *ptr = addr[dev];
    *bytes = kStaticScratchBytes - kWorkspaceCounterBytes;
    return hipSuccess;
}

hipError_t workspace_acquire(size_t bytes, hipStream_t stream, const Problem &p, Workspace &w) {
    w = Workspace{};
    if (p.scratch) {
        // the caller's scratch (checked against the plan before any launch)
        if (bytes > p.scratch_bytes) return hipErrorOutOfMemory;
        fill(w, p.scratch, false);
        return hipSuccess;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
        void *base = nullptr;
        e = hipMallocAsync(&base, bytes + kWorkspaceCounterBytes, stream);
        if (e != hipSuccess) return e;
        fill(w, base, true);
        return clear_counters(base, stream);
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const std::thread::id tid =
        stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
    std::lock_guard<std::mutex> lock(cache_mutex());
    Cached &c = cache()[Key{dev, stream, tid}];
    if (c.bytes < bytes || !c.ptr) {
        if (c.ptr) {
            e = hipFreeAsync(c.ptr, stream);
            c = Cached{};
            if (e != hipSuccess) return e;
        }
        void *base = nullptr;
        e = hipMallocAsync(&base, bytes + kWorkspaceCounterBytes, stream);
        if (e != hipSuccess) return e;
        e = clear_counters(base, stream);
        if (e != hipSuccess) {
            (void)hipFreeAsync(base, stream);   // the launch error is the one reported
            return e;
        }
        c.ptr = base;
        c.bytes = bytes;
    }
    fill(w, c.ptr, false);
    return hipSuccess;
}

hipError_t workspace_release(const Workspace &w, hipStream_t stream) {
    return w.owned ? hipFreeAsync(w.base, stream) : hipSuccess;
}

hipError_t workspace_release_all() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(cache_mutex());
    for (auto it = cache().begin(); it != cache().end();) {
        if (std::get<0>(it->first) == dev) {
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
