// Prefill product Y[M][N] on the int8 matrix cores (v_mfma_i32_32x32x32_i8).
//
// Prefill multiplies the same weights by many activation rows, so it is a dense contraction (tritium
// "Architecture", section 3: prefill runs compute-bound; bankml technical report, section III.3: a
// tile loads each weight block once and applies it to several activation columns).
//
// Mapping to CDNA4:
//  * A workgroup owns a tile of TN = 128 weight rows x TM = 64 activation rows and walks K in steps of
//    128 columns.  Each step is software-pipelined: the packed weight codes, activation tile and
//    activation scales of the step three ahead are loaded into a register ring while the current step
//    computes; at the top of a step they are written to double-buffered LDS -- the weights unpacked to
//    int8 in natural column order (shift and mask, a 4x4 byte transpose with v_perm_b32, and a
//    v_perm_b32 lookup from code to weight byte: Q2_0 c -> c - 1, Q1_0 bit -> +/-1, planar (pos, neg) ->
//    pos - neg) -- and one barrier per step separates the writes from the reads.  Waves 0-7 load and
//    unpack the weights, waves 8-15 load the activations.
//  * A workgroup is 16 waves (1024 threads).  Wave w computes the 32 x 32 output tile w mod 8 (32 weight
//    rows x 32 activation rows) over one half of every step's columns: per q8_0 block (32 columns, the
//    MFMA's K depth) one A operand (weights) and one B operand (activations) from LDS, one MFMA.  The
//    halves split at weight-block boundaries (a Q2_0 block, half a Q1_0 block), and the second half's
//    partial sums join the first's through LDS at the end: four waves per SIMD, so one wave's rescale
//    arithmetic overlaps another's matrix-core, LDS and load latency.  Each MFMA result is one exact
//    int32 sum per (weight row, activation row, block).
//  * The accumulator input of every MFMA is a constant register tile holding 0x4B400000 (1.5 * 2^23), so
//    each result, read as fp32, is 1.5 * 2^23 + isum exactly; one FMA with the block's activation scale
//    and -d_x * 1.5 * 2^23 gives round(d_x * isum) without a conversion.  The weight block scale is then
//    applied with one more FMA (bankml technical report, section III.3: one multiply-add per q8_0 block,
//    then one per weight block).
//  * Planar weights have no block scales: the MFMA accumulates int32 over the whole row and the two
//    per-row / per-tensor scales are applied once at the end.
#include "lowbit_internal.h"

namespace lb {

namespace {

constexpr int GT = 1024;         // threads per workgroup (16 waves)
constexpr int GH = GT / 2;       // threads of each role (weights / activations) and of each K half
constexpr int TN = 128;          // weight rows per workgroup
constexpr int TM = 64;           // activation rows per workgroup
constexpr int KS = 128;          // columns per K-step
constexpr int WROW = KS / 4 + 4; // LDS dwords per unpacked weight row (padded against bank conflicts)
constexpr int XROW = KS / 4 + 4; // LDS dwords per activation row
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

// Q1_0: one device sign dword m of a record (the sign of weight 32r + 8m + k at bit 4k + r) -> for each
// activation block r, the 8 int8 weights 32r + 8m .. 32r + 8m + 7 as two dwords out[2r], out[2r + 1].
// A byte table maps each 0/1 selector to -1/+1; byte t of e[s] is then the weight of bit 8t + s, i.e.
// k = 2t + (s >> 2) of block r = s & 3, and one byte interleave per half puts k in order.
__device__ __forceinline__ void unpack_q1_dword(uint32_t v, uint32_t *out)
{
    const uint32_t lut = 0x000001FFu; // 0 -> -1, 1 -> +1
    uint32_t e[8];
#pragma unroll
    for (int s = 0; s < 8; s++)
        e[s] = perm(0u, lut, (v >> s) & 0x01010101u);
#pragma unroll
    for (int r = 0; r < 4; r++) {
        out[2 * r] = perm(e[r + 4], e[r], 0x05010400u);     // k = 0, 1, 2, 3
        out[2 * r + 1] = perm(e[r + 4], e[r], 0x07030602u); // k = 4, 5, 6, 7
    }
}

// Planar: 32 plane bits -> 8 dwords of int8 weights in order, via a byte table indexed by the
// pos | neg << 1 selector of each weight.
__device__ __forceinline__ void unpack_planar_dword(uint32_t pos_bits, uint32_t neg_bits, uint32_t *out)
{
    const uint32_t lut = 0x00FF0100u; // 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0
    uint32_t e[8];
#pragma unroll
    for (int r = 0; r < 8; r++)
        e[r] = perm(0u, lut, ((pos_bits >> r) & 0x01010101u) | (((neg_bits >> r) & 0x01010101u) << 1));
    uint32_t t0[4], t1[4];
    transpose4(e[0], e[1], e[2], e[3], t0);
    transpose4(e[4], e[5], e[6], e[7], t1);
#pragma unroll
    for (int t = 0; t < 4; t++) {
        out[2 * t] = t0[t];
        out[2 * t + 1] = t1[t];
    }
}

// What one thread carries from global memory into a K-step, by role.  Weight threads (tid < GH): a
// quarter of one weight row's codes for the step in a.x, a.y (Q2_0: 2 code dwords; Q1_0: 1 sign dword;
// planar: pos dword, neg dword) and the weight block scale (binary16) in a.z where the thread stores it.
// Activation threads: 16 activation bytes in a and, for the first TM of them, the row's four binary16
// activation scales in b.
struct StepRegs {
    uint4 a;
    uint2 b;
};

template <int FMT>
__device__ __forceinline__ void load_step(StepRegs &r, const uint8_t *__restrict__ W, const uint16_t *__restrict__ wsc,
                                          int N, int K, const int8_t *__restrict__ X, const uint16_t *__restrict__ xsc,
                                          int M, int n0, int m0, int kk, int tid)
{
    const int kab = min(KS, K - kk) / QK8; // activation blocks in this step
    if (tid >= GH) { // activation threads
        const int t = tid - GH;
        // activation tile: 64 rows x kab * 32 bytes; thread -> (row t / 8, 16-byte chunk t % 8)
        const int m = min(m0 + (t >> 3), M - 1), ch = t & 7;
        if (ch < 2 * kab)
            r.a = *reinterpret_cast<const uint4 *>(X + (int64_t)m * K + kk + 16 * ch);
        if (FMT != LB_TERNARY_PLANAR && t < TM) {
            const int mm = min(m0 + t, M - 1);
            const uint16_t *pp = xsc + (int64_t)mm * (K / QK8) + kk / QK8;
            const uint32_t h0 = pp[0], h1 = pp[1];
            const uint32_t h2 = kab > 2 ? pp[2] : 0u, h3 = kab > 2 ? pp[3] : 0u;
            r.b = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        }
        return;
    }
    const int row = min(n0 + (tid >> 2), N - 1), p = tid & 3;
    if (FMT == LB_Q1_0) {
        // one 128-weight record per row; thread p takes its device sign dword p
        const int64_t idx = (int64_t)row * (K / 128) + kk / 128;
        r.a.x = *reinterpret_cast<const uint32_t *>(W + idx * 16 + 4 * p);
        if (p == 0)
            r.a.z = wsc[idx];
    } else {
        // two 64-weight records per row (one on a half step); thread p takes half p & 1 of record p >> 1
        const int bb = p >> 1, hh = p & 1;
        if (2 * bb < kab) {
            const int64_t idx = (int64_t)row * (K / 64) + kk / 64 + bb;
            if (FMT == LB_TERNARY_PLANAR) {
                r.a.x = *reinterpret_cast<const uint32_t *>(W + idx * 16 + 4 * hh);     // pos
                r.a.y = *reinterpret_cast<const uint32_t *>(W + idx * 16 + 8 + 4 * hh); // neg
            } else {
                const uint2 c2 = *reinterpret_cast<const uint2 *>(W + idx * 16 + 8 * hh);
                r.a.x = c2.x;
                r.a.y = c2.y;
                if (hh == 0)
                    r.a.z = wsc[idx];
            }
        }
    }
}

struct __attribute__((aligned(16))) Lds {
    uint32_t w[2][TN * WROW];
    uint32_t x[2][TM * XROW];
    float dw[2][2 * TN]; // weight block scales: [block within step][row]
    float dx[2][4 * TM]; // activation scales: [block within step][row]
};

template <int FMT>
__device__ __forceinline__ void store_step(Lds &lds, int buf, const StepRegs &r, int K, int kk, int tid)
{
    const int kab = min(KS, K - kk) / QK8;
    if (tid >= GH) { // activation threads
        const int t = tid - GH;
        const int mr = t >> 3, ch = t & 7;
        if (ch < 2 * kab)
            *reinterpret_cast<uint4 *>(lds.x[buf] + mr * XROW + 4 * ch) = r.a;
        if (FMT != LB_TERNARY_PLANAR && t < TM) {
            lds.dx[buf][0 * TM + t] = half_bits_to_float((uint16_t)(r.b.x & 0xffffu));
            lds.dx[buf][1 * TM + t] = half_bits_to_float((uint16_t)(r.b.x >> 16));
            lds.dx[buf][2 * TM + t] = half_bits_to_float((uint16_t)(r.b.y & 0xffffu));
            lds.dx[buf][3 * TM + t] = half_bits_to_float((uint16_t)(r.b.y >> 16));
        }
        return;
    }
    const int rr = tid >> 2, p = tid & 3;
    uint32_t *wrow = lds.w[buf] + rr * WROW;
    if (FMT == LB_Q1_0) {
        // sign dword p of the record holds 8 weights of each of the step's 4 activation blocks
        uint32_t o[8];
        unpack_q1_dword(r.a.x, o);
#pragma unroll
        for (int j = 0; j < 4; j++)
            *reinterpret_cast<uint2 *>(wrow + 8 * j + 2 * p) = make_uint2(o[2 * j], o[2 * j + 1]);
        if (p == 0)
            lds.dw[buf][rr] = half_bits_to_float((uint16_t)r.a.z);
    } else {
        const int bb = p >> 1, hh = p & 1;
        if (2 * bb < kab) {
            uint32_t *dst = wrow + 16 * bb + 8 * hh;
            uint32_t o[8];
            if (FMT == LB_TERNARY_PLANAR) {
                unpack_planar_dword(r.a.x, r.a.y, o);
            } else {
                unpack_q2_dword(r.a.x, o);
                unpack_q2_dword(r.a.y, o + 4);
                if (hh == 0)
                    lds.dw[buf][bb * TN + rr] = half_bits_to_float((uint16_t)r.a.z);
            }
            *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<uint4 *>(dst + 4) = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

// One K-step of one wave: NJ activation blocks (compile-time, so the pairing of blocks into weight
// blocks and every register index are static).
// One wave's share of a K-step: the two q8_0 blocks jb, jb + 1 (half of the step's 128 columns), which
// lie in one weight block (a whole Q2_0 block, half a Q1_0 block).
template <int FMT, bool EMIT>
__device__ __forceinline__ void step_compute(const Lds &lds, int buf, int jb, int h, int l32, int wn, int wm, int m0,
                                             int n0, int M, int N, int nab, int kk, float (&acc)[16], v16i &iacc,
                                             const v16i &cbias, int32_t *__restrict__ sums)
{
    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    constexpr int JW = FMT == LB_Q1_0 ? 4 : 2; // activation blocks per weight block
    const uint32_t *wl = lds.w[buf] + (32 * wn + l32) * WROW + 4 * h;
    const uint32_t *xl = lds.x[buf] + (32 * wm + l32) * XROW + 4 * h;
    float t[16];
#pragma unroll
    for (int jj = 0; jj < 2; jj++) {
        const int j = jb + jj;
        const uint4 a4 = *reinterpret_cast<const uint4 *>(wl + 8 * j);
        const uint4 b4 = *reinterpret_cast<const uint4 *>(xl + 8 * j);
        const v4i A = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
        const v4i B = {(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
        if (PLANAR) {
            iacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, iacc, 0, 0, 0);
            continue;
        }
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, cbias, 0, 0, 0);
        const float dx = lds.dx[buf][j * TM + 32 * wm + l32];
        const float c = -dx * BIASF; // exact: an 11-bit significand times 3 * 2^22
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float v = fmaf(dx, __int_as_float(D[i]), c); // round(d_x * isum)
            t[i] = jj == 0 ? v : t[i] + v;
        }
        if (EMIT) {
            const int m = m0 + 32 * wm + l32, kb = kk / QK8 + j;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int n = n0 + 32 * wn + 8 * (i >> 2) + 4 * h + (i & 3);
                if (m < M && n < N)
                    sums[((int64_t)m * N + n) * nab + kb] = D[i] - (int)BIAS;
            }
        }
    }
    if (!PLANAR) {
        const int b = jb / JW;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const float4 dw = *reinterpret_cast<const float4 *>(lds.dw[buf] + b * TN + 32 * wn + 8 * g + 4 * h);
            const float dwv[4] = {dw.x, dw.y, dw.z, dw.w};
#pragma unroll
            for (int q = 0; q < 4; q++)
                acc[4 * g + q] = fmaf(dwv[q], t[4 * g + q], acc[4 * g + q]);
        }
    }
}

template <int FMT, bool EMIT>
__global__ __launch_bounds__(GT, 1) void gemm_kernel(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                                     const int8_t *__restrict__ X, const void *__restrict__ Xscale,
                                                     int M, float *__restrict__ Y, int32_t *__restrict__ sums)
{
    __shared__ Lds lds;

    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    // this wave's 32 x 32 tile inside the 128 x 64 workgroup tile, and its half of each step's columns
    const int ti = wave & 7, kh = wave >> 3;
    const int wn = ti & 3, wm = ti >> 2;
    const int n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
    const int nrec = FMT == LB_Q1_0 ? K / 128 : K / 64; // 16-byte records per weight row
    const int nab = K / QK8;                             // activation blocks per row
    const uint16_t *wsc = reinterpret_cast<const uint16_t *>(W + (int64_t)N * nrec * 16);
    const uint16_t *xsc = reinterpret_cast<const uint16_t *>(Xscale);

    v16i cbias;
#pragma unroll
    for (int i = 0; i < 16; i++)
        cbias[i] = (int)BIAS;
    float acc[16];
    v16i iacc;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        acc[i] = 0.0f;
        iacc[i] = 0;
    }

    // Each workgroup walks its K-steps starting at a different step (rotating with the weight tile), so
    // at any moment the workgroups read different column ranges of the activation rows: with row strides
    // that are large powers of two, all workgroups reading the same column range at once pile onto a few
    // cache channels.  Integer block sums do not depend on the order; only the fp32 accumulation order
    // of the weight blocks does.
    const int nsteps = (K + KS - 1) / KS;
    const int rot = blockIdx.x % nsteps;
    auto step_k = [&](int s) { return ((s + rot) % nsteps) * KS; };

    // register ring: the loads of step s + PF are issued while step s computes
    constexpr int PF = 3;
    StepRegs ring[PF];
#pragma unroll
    for (int p = 0; p < PF; p++)
        if (p < nsteps)
            load_step<FMT>(ring[p], W, wsc, N, K, X, xsc, M, n0, m0, step_k(p), tid);

    int buf = 0;
    for (int s = 0; s < nsteps; s++, buf ^= 1) {
        const int kk = step_k(s);
        const int kab = min(KS, K - kk) / QK8;
        store_step<FMT>(lds, buf, ring[0], K, kk, tid);
        __syncthreads();
#pragma unroll
        for (int p = 0; p + 1 < PF; p++)
            ring[p] = ring[p + 1];
        if (s + PF < nsteps)
            load_step<FMT>(ring[PF - 1], W, wsc, N, K, X, xsc, M, n0, m0, step_k(s + PF), tid);
        // a full step: each K half takes two blocks; a half step (the K tail of Q2_0 / planar): the first
        // half takes both (uniform per wave)
        if (kab == KS / QK8 || kh == 0)
            step_compute<FMT, EMIT>(lds, buf, kab == KS / QK8 ? 2 * kh : 0, h, l32, wn, wm, m0, n0, M, N, nab, kk, acc,
                                    iacc, cbias, sums);
    }

    // the second K half hands its partial sums to the first through LDS (the weight buffers are free now)
    __syncthreads();
    uint32_t *red = lds.w[0];
    if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 16; i++)
            red[(ti * 16 + i) * 64 + lane] = PLANAR ? (uint32_t)iacc[i] : __float_as_uint(acc[i]);
    }
    __syncthreads();
    if (kh == 1)
        return;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t o = red[(ti * 16 + i) * 64 + lane];
        if (PLANAR)
            iacc[i] += (int)o;
        else
            acc[i] += __uint_as_float(o);
    }

    // store: lane holds weight rows n = 32 wn + 8 (i / 4) + 4 h + i % 4 of activation row m = 32 wm + l32
    const int m = m0 + 32 * wm + l32;
    if (m >= M)
        return;
    const float sx = PLANAR ? reinterpret_cast<const float *>(Xscale)[m] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int n = n0 + 32 * wn + 8 * (i >> 2) + 4 * h + (i & 3);
        if (n >= N)
            continue;
        if (PLANAR) {
            if (EMIT)
                sums[(int64_t)m * N + n] = iacc[i];
            if (!EMIT || Y != nullptr) {
                const float ys = (float)iacc[i] * sx;
                Y[(int64_t)m * N + n] = ys * w_scale;
            }
        } else if (!EMIT || Y != nullptr) {
            Y[(int64_t)m * N + n] = acc[i];
        }
    }
}

template <int FMT, bool EMIT>
hipError_t launch_fmt(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *Xq, const void *Xscale,
                      int64_t M, float *Y, int32_t *sums, hipStream_t s)
{
    const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    hipLaunchKernelGGL((gemm_kernel<FMT, EMIT>), grid, dim3(GT), 0, s, W, (int)N, (int)K, w_scale, Xq, Xscale, (int)M,
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
