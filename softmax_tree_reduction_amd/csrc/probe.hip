// Read-bandwidth probe: streams a buffer once with 16-byte nontemporal loads (the
// width and cache policy of the partial kernel's K and V loads, which go through
// buffer resources; these are plain global loads) and computes nothing from the
// data. Its rate is the device's practical read ceiling for that kind of access.
#include "device_common.h"
#include "kernels.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup w reads the w-th contiguous slice of the buffer.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* buf, int64_t n16, uint32_t* sink) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t begin = (int64_t)blockIdx.x * per;
    const int64_t end = begin + per < n16 ? begin + per : n16;
    uint32_t acc = 0;
    for (int64_t i = begin + threadIdx.x; i < end; i += (int64_t)kProbeThreads * kProbeUnroll) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kProbeThreads;
            v[u] = j < end ? ta::load_stream(buf + j) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x5a5a5a5au) *sink = acc;  // keeps the loads; the value itself is of no use
}

}  // namespace

namespace ta {

// Launch shape by size. Up to 8 slices of 32 KiB per CU (one pass of the loop per
// thread) the whole buffer is in flight in one round of workgroups: a 34 MB read
// then took 7.0 us per call, against 8.3 with one workgroup per CU, which waits for
// four rounds of loads. Larger buffers take one workgroup per CU, each streaming one
// contiguous slice: the fastest of the shapes measured on 512 MiB to 1 GiB (1 to 8
// workgroups per CU, 256 to 1024 threads).
hipError_t launch_stream_read(const void* buf, int64_t n16, uint32_t* sink, int cus, hipStream_t stream) {
    constexpr int64_t kSlice = (int64_t)kProbeThreads * kProbeUnroll;  // 16-byte items per pass
    const int64_t grid = n16 <= (int64_t)cus * 8 * kSlice ? (n16 + kSlice - 1) / kSlice : (cus < n16 ? cus : n16);
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace ta
