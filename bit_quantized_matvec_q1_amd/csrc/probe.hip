// Streaming-read probe: the rate at which this GPU delivers a buffer far larger than its caches to the
// vector units through 16-byte non-temporal loads -- the access pattern of the decode kernels' weight
// stream, so its rate bounds theirs (tritium "Architecture", section 3: a streaming-read probe run in the
// same invocation is the roofline the kernels are reported against).
//
// Each workgroup streams one contiguous 64 KiB chunk of the buffer (as a decode workgroup streams its row
// tile): per step its 256 threads issue UNROLL 16-byte loads each, every wave-wide load one contiguous
// KiB; the grid is one workgroup per chunk, dispatched as slots free up.  (Measured on MI355X: chunks of
// 64 KiB-1 MiB read at 7.0-7.2 TB/s, a grid-stride loop over the whole buffer at 6.0-6.5 TB/s, cached
// loads at 6.3-6.4 TB/s.)  The loaded words are folded into a checksum that is stored only when it
// equals a fixed constant: the loads cannot be removed, and (on any realistic data) nothing is written.
#include "lowbit_internal.h"

namespace lb {

namespace {

typedef unsigned pv4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const pv4u gpv4u;

constexpr int PT = 256;             // threads per workgroup
constexpr int UNROLL = 4;           // 16-byte loads in flight per thread
constexpr int64_t CHUNK = 4096;     // 16-byte units per workgroup (64 KiB)
constexpr uint32_t MAGIC = 0x9E3779B9u;

__global__ __launch_bounds__(PT) void read_probe_kernel(const pv4u *__restrict__ p, int64_t n16,
                                                        uint32_t *__restrict__ sink)
{
    const int64_t b0 = (int64_t)blockIdx.x * CHUNK, e = min(b0 + CHUNK, n16);
    const gpv4u *g = (const gpv4u *)p;
    uint32_t acc = 0;
    int64_t i = b0 + threadIdx.x;
    for (; i + (UNROLL - 1) * PT < e; i += UNROLL * PT) {
        pv4u v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; u++)
            v[u] = __builtin_nontemporal_load(g + (i + u * PT));
#pragma unroll
        for (int u = 0; u < UNROLL; u++)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < e; i += PT) {
        const pv4u v = __builtin_nontemporal_load(g + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == MAGIC)
        sink[blockIdx.x & 0xFFFF] = acc;
}

} // namespace

hipError_t launch_read_probe(const void *buf, int64_t nbytes, uint32_t *sink, hipStream_t s)
{
    const int64_t n16 = nbytes / 16, blocks = (n16 + CHUNK - 1) / CHUNK;
    if (blocks > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(PT), 0, s, static_cast<const pv4u *>(buf), n16,
                       sink);
    return hipGetLastError();
}

} // namespace lb
