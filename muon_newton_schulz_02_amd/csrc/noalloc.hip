// Device scratch of muon_adamw_step_noalloc, the step for callers that
// cannot allocate memory.
//
// `scratch` is a fixed array in the library's code object: every GPU the
// library runs on holds one copy of it, at its own address, until the
// process ends.  Host code never uses the array's name as a device address
// (on the host it names a stand-in, not device memory): the device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept; kernels receive it like any other workspace pointer.
//
// The step's descriptor tables reach the scratch through kernel arguments
// (k_copy_args): the runtime copies a launch's arguments when the launch is
// enqueued, so the host buffer they come from is free again at once and no
// pinned staging memory is needed.

#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "ma_internal.h"

namespace {

static __device__ __align__(256) char scratch[ma::kNoAllocScratchBytes];

// Bytes of table data one copy launch carries in its arguments (with the
// destination and length, within the 4 KB argument limit).
constexpr int kArgChunkBytes = 3072;

struct __attribute__((aligned(16))) ArgChunk {
    unsigned char b[kArgChunkBytes];
};

__global__ __launch_bounds__(256) void k_copy_args(char* __restrict__ dst, ArgChunk c, int n) {
    for (int i = threadIdx.x * 16; i < n; i += 256 * 16)
        *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(c.b + i);
}

std::mutex g_mu;
std::vector<std::pair<int, void*>> g_addr;   // (device, address of `scratch` on it)

}  // namespace

namespace ma {

int noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    std::lock_guard<std::mutex> lock(g_mu);
    for (const auto& a : g_addr) {
        if (a.first == dev) {
            *out = a.second;
            return (int)hipSuccess;
        }
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return (int)hipErrorInvalidSymbol;
    g_addr.emplace_back(dev, p);
    *out = p;
    return (int)hipSuccess;
}

int launch_copy_args(void* dst, const void* src, size_t bytes, void* stream) {
    const unsigned char* s = static_cast<const unsigned char*>(src);
    for (size_t off = 0; off < bytes; off += kArgChunkBytes) {
        const int n = (int)(bytes - off < (size_t)kArgChunkBytes ? bytes - off : kArgChunkBytes);
        ArgChunk c;
        for (int i = 0; i < n; ++i) c.b[i] = s[off + i];
        for (int i = n; i < kArgChunkBytes; ++i) c.b[i] = 0;
        hipLaunchKernelGGL(k_copy_args, dim3(1), dim3(256), 0, (hipStream_t)stream,
                           static_cast<char*>(dst) + off, c, (n + 15) & ~15);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return (int)hipSuccess;
}

}  // namespace ma
