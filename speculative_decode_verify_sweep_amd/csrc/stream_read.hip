// Streaming-read ceiling: a plain kernel that reads a buffer once with 16-byte
// loads and does nothing else with it.  Its bytes / time is the practical HBM
// read ceiling on the device it runs on, the figure the attention sweep's own
// KV bandwidth (one sweep's K and V bytes / time, the measure of "ChunkedSmallT
// re-streams full KV per query chunk", section Measurement) is set against.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_internal.h"

namespace {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per thread per step

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each step a workgroup reads kReadThreads * kReadUnroll consecutive 16-byte
// vectors (64 KiB of contiguous memory); steps stride over the grid.  The XOR
// of every word feeds a store that only runs for one value, so the loads
// cannot be removed.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* buf, int64_t n,
                                                                   uint32_t* sink) {
    const int64_t step = int64_t(gridDim.x) * kReadThreads * kReadUnroll;
    uint32_t acc = 0;
    for (int64_t base = int64_t(blockIdx.x) * kReadThreads * kReadUnroll + threadIdx.x; base < n;
         base += step) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = base + int64_t(u) * kReadThreads;
            v[u] = i < n ? buf[i] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int small_w_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream,
                                   void* ev_start, void* ev_end) {
    if (!buf || !sink || bytes == 0 || (bytes & 15u) || (reinterpret_cast<uintptr_t>(buf) & 15u))
        return SMALLW_EINVAL;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) {
        smallw::set_device_error("compute-unit query", int(e));
        return SMALLW_EDEVICE;
    }
    const int64_t n = int64_t(bytes / 16);
    const int64_t per_block = int64_t(kReadThreads) * kReadUnroll;
    int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > int64_t(cus) * 8) blocks = int64_t(cus) * 8;  // 8 workgroups per CU, then stride
    const u32x4* p = static_cast<const u32x4*>(buf);
    void* args[] = {&p, const_cast<int64_t*>(&n), &sink};
    e = hipExtLaunchKernel(reinterpret_cast<const void*>(stream_read_kernel), dim3(unsigned(blocks)),
                           dim3(kReadThreads), args, 0, static_cast<hipStream_t>(stream),
                           hipEvent_t(ev_start), hipEvent_t(ev_end), 0);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
        smallw::set_device_error("stream read launch", int(e));
        return SMALLW_EDEVICE;
    }
    return SMALLW_OK;
}
