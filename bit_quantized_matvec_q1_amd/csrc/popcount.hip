// Bit-serial popcount formulation of the planar ternary product (tritium "Architecture", section 4.3
// "About popcount": the formulation that maps onto an adder tree, kept as a third independent
// implementation for differential tests; section 5: implementations of the same arithmetic must agree).
//
// With the int8 activation written in two's complement as q = sum_p t_p * bit_p(q), t_p = 2^p for p < 7
// and t_7 = -128, and the planes of a beat {pos, neg}:
//     acc = sum_k (pos_k - neg_k) q_k = sum_p t_p * (popcount(pos & Q_p) - popcount(neg & Q_p)),
// where Q_p is the bit mask of plane p of the activations over the beat's 64 columns.  The activation
// planes are built once per workgroup in LDS; per beat and plane a lane spends two ANDs and two
// v_bcnt_u32_b32 (which accumulates) per 32 columns.  The output rule is the planar one,
// y = ((float)acc * s_x) * s_w, so the result is bit-identical to the select-accumulate kernel.
//
// Work split: a row over L = 16 lanes, S beats per lane (strided by L), one DPP tree per row.
#include "lowbit_internal.h"

namespace lb {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u gv4u;
typedef __attribute__((address_space(1))) const uint8_t gu8;

constexpr int L = 16;   // lanes per row
constexpr int PREC = 16; // staged dwords per beat: 8 planes x 2 halves of 32 columns

template <int S, bool EMIT>
__global__ __launch_bounds__(WG) void popcount_kernel(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                                      const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                      float *__restrict__ y, int32_t *__restrict__ sums, int tile_rows)
{
    extern __shared__ uint32_t planes[];
    constexpr int GROUPS = 64 / L;
    constexpr int STEP = GROUPS * (WG / 64);
    const int nbeat = K / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, li = lane % L;
    const int row0 = blockIdx.x * tile_rows;
    const int nrows = min(tile_rows, N - row0);

    // plane p of 32 columns: bit c is bit p of q[32 h + c]; one thread per (beat, half, plane)
    for (int it = threadIdx.x; it < nbeat * PREC; it += WG) {
        const int bt = it / PREC, h = (it % PREC) / 8, p = it % 8;
        const int8_t *qc = xq + 64 * bt + 32 * h;
        uint32_t m = 0;
        for (int c = 0; c < 32; c++)
            m |= (uint32_t)(((uint8_t)qc[c] >> p) & 1u) << c;
        planes[bt * PREC + h * 8 + p] = m;
    }
    __syncthreads();

    uint32_t qp[S][PREC];
    uint32_t bo[S];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int bt = li + i * L;
        bo[i] = (uint32_t)min(bt, nbeat - 1) * 16u; // a lane past the row's end re-reads its last beat
#pragma unroll
        for (int j = 0; j < PREC; j++)
            qp[i][j] = bt < nbeat ? planes[bt * PREC + j] : 0u; // ... against empty planes
    }
    const float sx = xs[0];
    const uint32_t rowbytes = (uint32_t)nbeat * 16u;
    for (int cur = 0; cur < nrows; cur += STEP) {
        const int rl = cur + wave * GROUPS + g;
        const uint32_t off = (uint32_t)(row0 + min(rl, nrows - 1)) * rowbytes;
        int cnt[8];
#pragma unroll
        for (int p = 0; p < 8; p++)
            cnt[p] = 0;
#pragma unroll
        for (int i = 0; i < S; i++) {
            const v4u b = *(gv4u *)((gu8 *)W + (off + bo[i])); // {pos lo, pos hi, neg lo, neg hi}
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int p = 0; p < 8; p++) {
                    const uint32_t pl = qp[i][h * 8 + p];
                    // popcount(pos & Q_p) - popcount(neg & Q_p), accumulated per plane
                    cnt[p] += __builtin_popcount(b[h] & pl) - __builtin_popcount(b[2 + h] & pl);
                }
        }
        int acc = 0;
#pragma unroll
        for (int p = 0; p < 7; p++)
            acc += cnt[p] << p;
        acc -= cnt[7] << 7; // the sign plane weighs -128
        acc = group_sum_i<L>(acc);
        if (rl < nrows && li == L - 1) {
            if (EMIT)
                sums[row0 + rl] = acc;
            const float ys = (float)acc * sx;
            if (!EMIT || y != nullptr)
                y[row0 + rl] = ys * w_scale;
        }
    }
}

} // namespace

hipError_t launch_popcount(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *xq, const float *xs,
                           float *y, int32_t *sums, hipStream_t s)
{
    const int nbeat = (int)(K / 64);
    const int S = (nbeat + L - 1) / L;
    const int rpi = (64 / L) * (WG / 64);
    const int tile = 8 * rpi;
    const int grid = (int)((N + tile - 1) / tile);
    const size_t lds = (size_t)nbeat * PREC * 4;
    const int n = (int)N, k = (int)K;
    switch (S) {
#define LB_POP(sv)                                                                                            \
    case sv:                                                                                                  \
        if (sums)                                                                                             \
            hipLaunchKernelGGL((popcount_kernel<sv, true>), dim3(grid), dim3(WG), lds, s, W, n, k, w_scale, xq, xs, \
                               y, sums, tile);                                                                \
        else                                                                                                  \
            hipLaunchKernelGGL((popcount_kernel<sv, false>), dim3(grid), dim3(WG), lds, s, W, n, k, w_scale, xq,  \
                               xs, y, sums, tile);                                                            \
        break;
        LB_POP(1) LB_POP(2) LB_POP(3) LB_POP(4) LB_POP(5) LB_POP(6) LB_POP(7) LB_POP(8)
#undef LB_POP
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace lb
