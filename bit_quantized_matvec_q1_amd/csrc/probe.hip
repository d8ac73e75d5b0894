// Streaming-read probe: the rate at which this GPU delivers a buffer far larger than its caches to the
// vector units through 16-byte non-temporal loads -- the access pattern of the decode kernels' weight
// stream, so its rate bounds theirs (tritium "Architecture", section 3: a streaming-read probe run in the
// same invocation is the roofline the kernels are reported against).
//
// Each wave reads 1 KiB contiguous per load instruction (64 lanes x 16 bytes); a thread keeps UNROLL
// loads in flight, its loads strided by the whole grid, so at any moment the grid reads one contiguous
// window of the buffer.  The loaded words are folded into a checksum that is stored only when it equals
// a fixed constant: the loads cannot be removed, and (on any realistic data) nothing is written.
#include "lowbit_internal.h"

#include <algorithm>

namespace lb {

namespace {

typedef unsigned pv4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const pv4u gpv4u;

constexpr int PT = 256;     // threads per workgroup
constexpr int UNROLL = 8;   // 16-byte loads in flight per thread
constexpr uint32_t MAGIC = 0x9E3779B9u;

__global__ __launch_bounds__(PT) void read_probe_kernel(const pv4u *__restrict__ p, int64_t n16,
                                                        uint32_t *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * PT;
    int64_t i = (int64_t)blockIdx.x * PT + threadIdx.x;
    uint32_t acc = 0;
    const gpv4u *g = (const gpv4u *)p;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        pv4u v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; u++)
            v[u] = __builtin_nontemporal_load(g + (i + u * stride));
#pragma unroll
        for (int u = 0; u < UNROLL; u++)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const pv4u v = __builtin_nontemporal_load(g + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == MAGIC)
        sink[blockIdx.x & 0xFFFF] = acc;
}

} // namespace

hipError_t launch_read_probe(const void *buf, int64_t nbytes, uint32_t *sink, hipStream_t s)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const int64_t n16 = nbytes / 16;
    // 8 workgroups (32 waves) per CU, fewer for a buffer too small to give every thread one load
    int64_t blocks = (int64_t)cus * 8;
    blocks = std::min<int64_t>(blocks, std::max<int64_t>(1, (n16 + PT - 1) / PT));
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(PT), 0, s,
                       static_cast<const pv4u *>(buf), n16, sink);
    return hipGetLastError();
}

} // namespace lb
