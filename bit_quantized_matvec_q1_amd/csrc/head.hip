// Dense bf16 head matvec: y[n] = sum_k f32(W[n][k]) * x[k] (tritium "Architecture", section 3: the
// tied output head is the largest single stream of a decode step, stored as bf16).
//
// Purely bandwidth-bound: each weight byte is read once with 16-byte loads (8 bf16), widened to fp32
// exactly (bf16 is the top half of a binary32), and multiply-added against x held in VGPRs.  A row is
// spread over one wave (each lane owns S chunks of 8 columns, strided so every wave-wide load is
// contiguous) and closed with a cross-lane tree.
#include "lowbit_internal.h"

namespace lb {

template <int S>
__global__ __launch_bounds__(WG) void head_kernel(const uint16_t *__restrict__ W, int N, int K,
                                                  const float *__restrict__ x, float *__restrict__ y, int tile_rows)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nch = K / 8; // chunks of 8 columns per row
    float xr[S][8];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int ch = lane + 64 * i;
        if (ch < nch) {
            const float4 a = reinterpret_cast<const float4 *>(x)[2 * ch];
            const float4 b = reinterpret_cast<const float4 *>(x)[2 * ch + 1];
            xr[i][0] = a.x, xr[i][1] = a.y, xr[i][2] = a.z, xr[i][3] = a.w;
            xr[i][4] = b.x, xr[i][5] = b.y, xr[i][6] = b.z, xr[i][7] = b.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++)
                xr[i][j] = 0.0f;
        }
    }
    const int row0 = blockIdx.x * tile_rows;
    const int nrows = min(tile_rows, N - row0);
    constexpr int U = 2;
    for (int it = 0; it < nrows; it += U * (WG / 64)) {
        uint4 w[U][S];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int rl = it + u * (WG / 64) + wave;
#pragma unroll
            for (int i = 0; i < S; i++) {
                const int ch = lane + 64 * i;
                w[u][i] = make_uint4(0, 0, 0, 0);
                if (rl < nrows && ch < nch)
                    w[u][i] = reinterpret_cast<const uint4 *>(W + (int64_t)(row0 + rl) * K)[ch];
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int rl = it + u * (WG / 64) + wave;
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < S; i++) {
                const uint32_t v[4] = {w[u][i].x, w[u][i].y, w[u][i].z, w[u][i].w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    acc = fmaf(__uint_as_float(v[j] << 16), xr[i][2 * j], acc);
                    acc = fmaf(__uint_as_float(v[j] & 0xffff0000u), xr[i][2 * j + 1], acc);
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1)
                acc += __shfl_xor(acc, off, 64);
            if (rl < nrows && lane == 0)
                y[row0 + rl] = acc;
        }
    }
}

hipError_t launch_head(const uint16_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s)
{
    const int nch = (int)(K / 8);
    const int S = (nch + 63) / 64;
    const int tile = 64;
    const int grid = (int)((N + tile - 1) / tile);
    switch (S) {
#define LB_HEAD(n)                                                                                            \
    case n:                                                                                                   \
        hipLaunchKernelGGL(head_kernel<n>, dim3(grid), dim3(WG), 0, s, W, (int)N, (int)K, x, y, tile);        \
        break;
        LB_HEAD(1) LB_HEAD(2) LB_HEAD(3) LB_HEAD(4) LB_HEAD(5) LB_HEAD(6) LB_HEAD(7) LB_HEAD(8)
#undef LB_HEAD
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace lb
