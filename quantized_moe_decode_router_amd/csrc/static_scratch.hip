// static_scratch.hip -- the fixed device scratch of the allocation-free decode entry point
// (moe_stack_decode_static): a file-scope device array used as the decode workspace, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops).
//
// Host code never passes the array's name to a kernel or a copy: in host code that name is only a
// host-side stand-in. The device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device; every later use goes
// through that address. Each GPU holds its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.hpp"

namespace moe {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device (null until set up)
bool g_clear[kMaxDevices] = {};  // the first use on a device clears the array first

// Zero-fills n bytes (n a multiple of 16) at p, grid-stride.
__global__ void __launch_bounds__(256) fill_zero(uint4 *p, size_t n16) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

}  // namespace

hipError_t static_scratch(size_t need, bool reset, hipStream_t stream, void **out) {
    *out = nullptr;
    if (need > kStaticScratchBytes) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    bool clear = reset;
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_ptr[dev]) {
            void *p = nullptr;
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess) return err;
            g_ptr[dev] = p;
            g_clear[dev] = true;
        }
        ptr = g_ptr[dev];
        clear = clear || g_clear[dev];
        g_clear[dev] = false;
    }
    if (clear) {
        // a fill kernel rather than a memset node: the call may be captured into a graph
        const size_t n16 = kStaticScratchBytes / 16;
        hipLaunchKernelGGL(fill_zero, dim3(1024), dim3(256), 0, stream, static_cast<uint4 *>(ptr), n16);
        if ((err = hipGetLastError()) != hipSuccess) {
            std::lock_guard<std::mutex> lock(g_mu);
            g_clear[dev] = true;  // try again on the next call
            return err;
        }
    }
    *out = ptr;
    return hipSuccess;
}

}  // namespace moe
