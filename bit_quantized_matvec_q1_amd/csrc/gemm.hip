// Prefill product Y[M][N] on the int8 matrix cores (v_mfma_i32_32x32x32_i8).
//
// Prefill multiplies the same weights by many activation rows, so it is a dense contraction (tritium
// "Architecture", section 3: prefill runs compute-bound; bankml technical report, section III.3: a
// tile loads each weight block once and applies it to several activation columns).
//
// Mapping to CDNA4:
//  * A workgroup owns a tile of TN = 128 weight rows x TM = 64 activation rows.  Per K-step of 128
//    weights it loads the packed codes of its 128 rows once and unpacks them into LDS as int8 weights in
//    natural column order (shift and mask, a 4x4 byte transpose with v_perm_b32, and a v_perm_b32
//    table lookup from code to weight byte: Q2_0 c -> c - 1, Q1_0 bit -> +/-1, planar (pos, neg) ->
//    pos - neg).
//  * Each of the 4 waves computes 32 weight rows x 64 activation rows: per q8_0 block (32 columns, the
//    MFMA's K depth) one A operand from LDS and two B operands (activation rows, read straight from the
//    L2-resident activation matrix), two MFMAs.  Each MFMA result is one exact int32 sum per (row, block).
//  * The accumulator input of every MFMA is a constant register tile holding 0x4B400000 (1.5 * 2^23), so
//    each result, read as fp32, is 1.5 * 2^23 + isum exactly; one FMA with the block's activation scale
//    and the precomputed -d_x * 1.5 * 2^23 gives round(d_x * isum) without a conversion.  The weight
//    block scale is then applied with one more FMA (bankml technical report, section III.3: one multiply-
//    add per q8_0 block, then one per weight block).
//  * Planar weights have no block scales: the MFMA accumulates int32 over the whole row and the two
//    per-row/per-tensor scales are applied once at the end.
#include "lowbit_internal.h"

namespace lb {

namespace {

constexpr int TN = 128; // weight rows per workgroup
constexpr int TM = 64;  // activation rows per workgroup
constexpr int KS = 128; // weights per K-step
constexpr int WROW = KS / 4 + 4; // LDS dwords per unpacked weight row (padded against bank conflicts)
constexpr uint32_t BIAS = 0x4B400000u; // 1.5 * 2^23 as fp32 bits
constexpr float BIASF = 12582912.0f;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel)
{
    return __builtin_amdgcn_perm(s0, s1, sel);
}

// out[t].byte[s] = e[s].byte[t]
__device__ __forceinline__ void transpose4(const uint32_t e0, const uint32_t e1, const uint32_t e2, const uint32_t e3,
                                           uint32_t *out)
{
    const uint32_t lo01 = perm(e1, e0, 0x05010400u), hi01 = perm(e1, e0, 0x07030602u);
    const uint32_t lo23 = perm(e3, e2, 0x05010400u), hi23 = perm(e3, e2, 0x07030602u);
    out[0] = perm(lo23, lo01, 0x05040100u);
    out[1] = perm(lo23, lo01, 0x07060302u);
    out[2] = perm(hi23, hi01, 0x05040100u);
    out[3] = perm(hi23, hi01, 0x07060302u);
}

// Q2_0: one code dword (16 weights, weight 4t + s at bits 8t + 2s) -> 4 dwords of int8 weights in order.
__device__ __forceinline__ void unpack_q2_dword(uint32_t v, uint32_t *out)
{
    const uint32_t lut = 0x020100FFu; // code 0, 1, 2, 3 -> weight -1, 0, +1, +2
    uint32_t e[4];
#pragma unroll
    for (int s = 0; s < 4; s++)
        e[s] = perm(0u, lut, (v >> (2 * s)) & 0x03030303u);
    transpose4(e[0], e[1], e[2], e[3], out);
}

// Q1_0 / planar: 32 sign bits (or plane bits) -> 8 dwords of int8 weights in order, via an 8-entry
// byte table indexed by the 0/1 (Q1_0) or pos | neg << 1 (planar) selector of each weight.
__device__ __forceinline__ void unpack_bits_dword(uint32_t sel_lo_bits, uint32_t sel_hi_bits, bool planar,
                                                  uint32_t *out)
{
    const uint32_t lut = planar ? 0x00FF0100u /* 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0 */
                                : 0x000001FFu /* 0 -> -1, 1 -> +1 */;
    uint32_t e[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
        uint32_t s = (sel_lo_bits >> r) & 0x01010101u;
        if (planar)
            s |= ((sel_hi_bits >> r) & 0x01010101u) << 1;
        e[r] = perm(0u, lut, s);
    }
    uint32_t t0[4], t1[4];
    transpose4(e[0], e[1], e[2], e[3], t0);
    transpose4(e[4], e[5], e[6], e[7], t1);
#pragma unroll
    for (int t = 0; t < 4; t++) {
        out[2 * t] = t0[t];
        out[2 * t + 1] = t1[t];
    }
}

template <int FMT, bool EMIT>
__global__ __launch_bounds__(WG) void gemm_kernel(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                                  const int8_t *__restrict__ X, const void *__restrict__ Xscale, int M,
                                                  float *__restrict__ Y, int32_t *__restrict__ sums)
{
    __shared__ __attribute__((aligned(16))) uint32_t w_lds[TN * WROW];
    __shared__ __attribute__((aligned(16))) float dw_lds[2 * TN];

    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
    const int ns = K / 64;        // 16-byte records per row (Q2_0, planar) / half that for Q1_0
    const int nrec = FMT == LB_Q1_0 ? K / 128 : ns;
    const int nab = K / QK8;      // activation blocks per row
    const uint16_t *wsc = reinterpret_cast<const uint16_t *>(W + (int64_t)N * nrec * 16);

    // this lane's activation rows (clamped: rows past M are computed and never stored)
    int mrow[2];
#pragma unroll
    for (int s = 0; s < 2; s++)
        mrow[s] = min(m0 + 32 * s + l32, M - 1);

    v16i cbias;
#pragma unroll
    for (int i = 0; i < 16; i++)
        cbias[i] = (int)BIAS;

    float acc[2][16];
    v16i iacc[2];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
            acc[s][i] = 0.0f;
            iacc[s][i] = 0;
        }

    for (int kk = 0; kk < K; kk += KS) {
        const int kab = min(KS, K - kk) / QK8; // activation blocks in this step (4, or 2 on a Q2_0 / planar tail)
        // --- unpack this step's weights into LDS ---
        __syncthreads();
        if (FMT == LB_Q1_0) {
            if (tid < TN) {
                const int row = min(n0 + tid, N - 1);
                const uint4 c = *reinterpret_cast<const uint4 *>(W + ((int64_t)row * nrec + kk / 128) * 16);
                const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
                uint32_t *dst = w_lds + tid * WROW;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    uint32_t o[8];
                    unpack_bits_dword(cw[k], 0u, false, o);
                    *reinterpret_cast<uint4 *>(dst + 8 * k) = make_uint4(o[0], o[1], o[2], o[3]);
                    *reinterpret_cast<uint4 *>(dst + 8 * k + 4) = make_uint4(o[4], o[5], o[6], o[7]);
                }
                dw_lds[tid] = half_bits_to_float(wsc[(int64_t)row * nrec + kk / 128]);
            }
        } else {
            const int r = tid >> 1, bb = tid & 1;
            if (2 * bb < kab) {
                const int row = min(n0 + r, N - 1);
                const uint4 c = *reinterpret_cast<const uint4 *>(W + ((int64_t)row * ns + kk / 64 + bb) * 16);
                uint32_t *dst = w_lds + r * WROW + 16 * bb;
                if (PLANAR) {
                    // beat = {pos lo, pos hi, neg lo, neg hi}
                    uint32_t o[8];
                    unpack_bits_dword(c.x, c.z, true, o);
                    *reinterpret_cast<uint4 *>(dst + 0) = make_uint4(o[0], o[1], o[2], o[3]);
                    *reinterpret_cast<uint4 *>(dst + 4) = make_uint4(o[4], o[5], o[6], o[7]);
                    unpack_bits_dword(c.y, c.w, true, o);
                    *reinterpret_cast<uint4 *>(dst + 8) = make_uint4(o[0], o[1], o[2], o[3]);
                    *reinterpret_cast<uint4 *>(dst + 12) = make_uint4(o[4], o[5], o[6], o[7]);
                } else {
                    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        uint32_t o[4];
                        unpack_q2_dword(cw[k], o);
                        *reinterpret_cast<uint4 *>(dst + 4 * k) = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                    dw_lds[bb * TN + r] = half_bits_to_float(wsc[(int64_t)row * ns + kk / 64 + bb]);
                }
            }
        }
        __syncthreads();

        // --- this wave's 32 weight rows x 64 activation rows ---
        float t[2][16];
        for (int j = 0; j < kab; j++) {
            const int kb = kk / QK8 + j; // activation block index along K
            const uint4 a4 = *reinterpret_cast<const uint4 *>(w_lds + (32 * wave + l32) * WROW + 8 * j + 4 * h);
            const v4i A = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
#pragma unroll
            for (int s = 0; s < 2; s++) {
                const uint4 b4 = *reinterpret_cast<const uint4 *>(X + (int64_t)mrow[s] * K + kk + 32 * j + 16 * h);
                const v4i B = {(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
                if (PLANAR) {
                    iacc[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, iacc[s], 0, 0, 0);
                } else {
                    const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, cbias, 0, 0, 0);
                    const float dx = half_bits_to_float(reinterpret_cast<const uint16_t *>(Xscale)[(int64_t)mrow[s] * nab + kb]);
                    const float c = -dx * BIASF; // exact: an 11-bit significand times 3 * 2^22
                    const int jw = FMT == LB_Q1_0 ? j : (j & 1); // position inside the weight block
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        const float v = fmaf(dx, __int_as_float(D[i]), c); // round(d_x * isum)
                        t[s][i] = jw == 0 ? v : t[s][i] + v;
                    }
                    if (EMIT) {
                        const int m = m0 + 32 * s + l32;
#pragma unroll
                        for (int i = 0; i < 16; i++) {
                            const int n = n0 + 32 * wave + 8 * (i >> 2) + 4 * h + (i & 3);
                            if (m < M && n < N)
                                sums[((int64_t)m * N + n) * nab + kb] = D[i] - (int)BIAS;
                        }
                    }
                    const bool block_end = FMT == LB_Q1_0 ? j == 3 : (j & 1) == 1;
                    if (block_end) {
                        const int b = FMT == LB_Q1_0 ? 0 : (j >> 1);
#pragma unroll
                        for (int g = 0; g < 4; g++) {
                            const float4 dw = *reinterpret_cast<const float4 *>(dw_lds + b * TN + 32 * wave + 8 * g + 4 * h);
                            const float dwv[4] = {dw.x, dw.y, dw.z, dw.w};
#pragma unroll
                            for (int q = 0; q < 4; q++)
                                acc[s][4 * g + q] = fmaf(dwv[q], t[s][4 * g + q], acc[s][4 * g + q]);
                        }
                    }
                }
            }
        }
    }

    // --- store: lane holds rows n = 32 wave + 8 (i / 4) + 4 h + i % 4 of activation row m = 32 s + l32 ---
    const float *sxp = reinterpret_cast<const float *>(Xscale);
#pragma unroll
    for (int s = 0; s < 2; s++) {
        const int m = m0 + 32 * s + l32;
        if (m >= M)
            continue;
        const float sx = PLANAR ? sxp[m] : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int n = n0 + 32 * wave + 8 * (i >> 2) + 4 * h + (i & 3);
            if (n >= N)
                continue;
            if (PLANAR) {
                if (EMIT)
                    sums[(int64_t)m * N + n] = iacc[s][i];
                if (!EMIT || Y != nullptr) {
                    const float ys = (float)iacc[s][i] * sx;
                    Y[(int64_t)m * N + n] = ys * w_scale;
                }
            } else if (!EMIT || Y != nullptr) {
                Y[(int64_t)m * N + n] = acc[s][i];
            }
        }
    }
}

template <int FMT, bool EMIT>
hipError_t launch_fmt(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *Xq, const void *Xscale,
                      int64_t M, float *Y, int32_t *sums, hipStream_t s)
{
    const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    hipLaunchKernelGGL((gemm_kernel<FMT, EMIT>), grid, dim3(WG), 0, s, W, (int)N, (int)K, w_scale, Xq, Xscale, (int)M,
                       Y, sums);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemm(int fmt, const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *Xq,
                       const void *Xscale, int64_t M, float *Y, int32_t *sums, hipStream_t s)
{
    const bool emit = sums != nullptr;
    switch (fmt) {
    case LB_Q1_0:
        return emit ? launch_fmt<LB_Q1_0, true>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s)
                    : launch_fmt<LB_Q1_0, false>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s);
    case LB_Q2_0_G64:
        return emit ? launch_fmt<LB_Q2_0_G64, true>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s)
                    : launch_fmt<LB_Q2_0_G64, false>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s);
    case LB_TERNARY_PLANAR:
        return emit ? launch_fmt<LB_TERNARY_PLANAR, true>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s)
                    : launch_fmt<LB_TERNARY_PLANAR, false>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s);
    }
    return hipErrorInvalidValue;
}

} // namespace lb
