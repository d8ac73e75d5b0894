// Prefill product Y[M][N] on the int8 matrix cores (v_mfma_i32_32x32x32_i8).
//
// Prefill multiplies the same weights by many activation rows, so it is a dense contraction (tritium
// "Architecture", section 3: prefill runs compute-bound; bankml technical report, section III.3: a
// tile loads each weight block once and applies it to several activation columns).
//
// Mapping to CDNA4:
//  * A workgroup owns a tile of TN = 64 weight rows x TM = 128 activation rows and walks K in steps of
//    128 columns.  Each step is software-pipelined: the packed weight codes, activation tile and
//    activation scales of the step two ahead are loaded into a register ring while the current step
//    computes; at the top of a step they are written to double-buffered LDS -- the weights unpacked to
//    int8 in natural column order (shift and mask, a 4x4 byte transpose with v_perm_b32, and a
//    v_perm_b32 lookup from code to weight byte: Q2_0 c -> c - 1, Q1_0 bit -> +/-1, planar (pos, neg) ->
//    pos - neg; Q8_0 weights are int8 already and copied as they are) -- and one barrier per step
//    separates the writes from the reads.  Every thread loads and
//    unpacks an equal share of the weight tile and copies an equal share of the activation tile.
//  * A workgroup is 8 waves (512 threads), two per SIMD, and two workgroups fit a CU.  Wave w computes
//    the 32 x 32 output tile (weight rows 32 (w mod 2), activation rows 32 (w / 2)) over every step's
//    four q8_0 blocks (32 columns each, the MFMA's K depth): per block one A operand (weights) and one B
//    operand (activations) from LDS, one MFMA, one exact int32 sum per (weight row, activation row,
//    block).  The weight unpack is shared by the 128 activation rows of the tile and the activation copy
//    by its 64 weight rows, so per MFMA the per-step work stays small next to the rescale below.
//  * Q2_0 and Q8_0: the accumulator input of every MFMA is a constant register tile holding 0x4B400000
//    (1.5 * 2^23), so each result, read as fp32, is 1.5 * 2^23 + isum exactly; one FMA with the block's activation
//    scale and -d_x * 1.5 * 2^23 gives round(d_x * isum) without a conversion.  Q1_0: a zero accumulator,
//    each exact int32 result converted and multiply-added into the weight block's sum (fewer registers,
//    which keeps two workgroups per CU).  The weight block scale is then applied with one more FMA (bankml
//    technical report, section III.3: one multiply-add per q8_0 block, then one per weight block).
//  * Planar weights have no block scales: the MFMA accumulates int32 over the whole row and the two
//    per-row / per-tensor scales are applied once at the end.
#include "lowbit_internal.h"

#include <atomic>

namespace lb {

namespace {

constexpr int GT = 512;          // threads per workgroup (8 waves)
constexpr int TN = 64;           // weight rows per workgroup
constexpr int TM = 128;          // activation rows per workgroup
constexpr int KS = 128;          // columns per K-step
constexpr int WROW = KS / 4 + 4; // LDS dwords per unpacked weight row (padded against bank conflicts)
constexpr int XROW = KS / 4 + 4; // LDS dwords per activation row
constexpr uint32_t BIAS = 0x4B400000u; // 1.5 * 2^23 as fp32 bits
constexpr float BIASF = 12582912.0f;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

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

// What one thread carries from global memory into a K-step.  Every thread takes one share of the weight
// tile -- Q2_0: one code dword (16 weights); Q1_0: one sign dword, of which it builds two of the four
// activation blocks; planar: one (pos, neg) dword pair, of which it builds half -- in a.x (planar neg in
// a.y, the weight block scale's binary16 in a.z where the thread stores it), 32 activation bytes (one
// q8_0 block of one activation row) in b0, b1, and, for the first TM threads, the four binary16
// activation scales of one activation row in c.
struct StepRegs {
    uint4 a;
    v4u b0, b1; // native vectors: copied as registers, never through memory
    uint2 c;
    uint32_t ws; // Q8_0: the binary16 scale of the thread's weight block
};

// Global-address-space views: loads take a scalar base and a 32-bit per-lane offset (the ABI keeps the
// weight tensor and the activation matrix under 4 GiB), so no 64-bit address arithmetic per load.
typedef __attribute__((address_space(1))) const uint8_t gu8;
typedef __attribute__((address_space(1))) const v4u gv4u;
typedef __attribute__((address_space(1))) const uint32_t gu32;
typedef __attribute__((address_space(1))) const uint16_t gu16;

template <int FMT>
__device__ __forceinline__ void load_step(StepRegs &r, const uint8_t *__restrict__ W, const uint16_t *__restrict__ wsc,
                                          int N, int K, const int8_t *__restrict__ X, const uint16_t *__restrict__ xsc,
                                          int M, int n0, int m0, int kk, int tid)
{
    // Every load is unconditional, its index clamped into the tensor: on a half step (the K tail) the
    // shares past the row's end re-read its last block and are not stored.  The registers are filled
    // straight from memory, so nothing waits on them until the step is stored.
    const int kab = min(KS, K - kk) / QK8; // activation blocks in this step
    // activation tile: 128 rows x kab blocks of 32 bytes; thread -> (row tid / 4, block tid % 4)
    {
        const int m = min(m0 + (tid >> 2), M - 1), ch = min(tid & 3, kab - 1);
        const uint32_t xo = (uint32_t)m * (uint32_t)K + (uint32_t)(kk + 32 * ch);
        r.b0 = *(gv4u *)((gu8 *)X + xo);
        r.b1 = *(gv4u *)((gu8 *)X + (xo + 16u));
    }
    if (FMT != LB_TERNARY_PLANAR && tid < TM) { // one activation row's four block scales
        const int mm = min(m0 + (tid & (TM - 1)), M - 1);
        const uint32_t so = ((uint32_t)mm * (uint32_t)(K / QK8) + (uint32_t)(kk / QK8)) * 2u;
        r.c.x = *(gu32 *)((gu8 *)xsc + so);                            // blocks 0, 1 (4-byte aligned: K / 32
        r.c.y = *(gu32 *)((gu8 *)xsc + (so + (kab > 2 ? 4u : 0u)));    // and kk / 32 are even); 2, 3
    }
    const int row = min(n0 + (tid >> 3), N - 1), p = tid & 7;
    if (FMT == LB_Q1_0) {
        // one 128-weight record per row and step; thread p takes sign dword p / 2
        const uint32_t idx = (uint32_t)row * (uint32_t)(K / 128) + (uint32_t)(kk / 128);
        r.a.x = *(gu32 *)((gu8 *)W + (idx * 16u + 4u * (uint32_t)(p >> 1)));
        r.a.z = *(gu16 *)((gu8 *)wsc + idx * 2u);
    } else if (FMT == LB_Q8_0) {
        // four 32-byte records per row (K is a whole number of steps); thread p takes half p % 2 of
        // record p / 2, and its scale
        const uint32_t idx = (uint32_t)row * (uint32_t)(K / 32) + (uint32_t)(kk / 32 + (p >> 1));
        const v4u t = *(gv4u *)((gu8 *)W + (idx * 32u + 16u * (uint32_t)(p & 1)));
        r.a = make_uint4(t.x, t.y, t.z, t.w);
        r.ws = *(gu16 *)((gu8 *)wsc + idx * 2u);
    } else if (FMT == LB_Q2_0_G64) {
        // two 64-weight records per row (one on a half step); thread p takes dword p % 4 of record p / 4
        const int bb = min(p >> 2, kab / 2 - 1), d = p & 3;
        const uint32_t idx = (uint32_t)row * (uint32_t)(K / 64) + (uint32_t)(kk / 64 + bb);
        r.a.x = *(gu32 *)((gu8 *)W + (idx * 16u + 4u * (uint32_t)d));
        r.a.z = *(gu16 *)((gu8 *)wsc + idx * 2u);
    } else {
        // two 64-column beats per row; thread p takes the (pos, neg) dword pair (p / 2) % 2 of beat p / 4
        const int bb = min(p >> 2, kab / 2 - 1), hh = (p >> 1) & 1;
        const uint32_t idx = (uint32_t)row * (uint32_t)(K / 64) + (uint32_t)(kk / 64 + bb);
        r.a.x = *(gu32 *)((gu8 *)W + (idx * 16u + 4u * (uint32_t)hh));       // pos
        r.a.y = *(gu32 *)((gu8 *)W + (idx * 16u + 8u + 4u * (uint32_t)hh)); // neg
    }
}

struct __attribute__((aligned(16))) Lds {
    uint32_t w[2][TN * WROW];
    uint32_t x[2][TM * XROW];
    float dw[2][4 * TN]; // weight block scales: [block within step][row]
    float dx[2][4 * TM]; // activation scales: [block within step][row]
};

template <int FMT>
__device__ __forceinline__ void store_step(Lds &lds, int buf, const StepRegs &r, int K, int kk, int tid)
{
    const int kab = min(KS, K - kk) / QK8;
    {
        const int mr = tid >> 2, ch = tid & 3;
        if (ch < kab) {
            v4u *dst = reinterpret_cast<v4u *>(lds.x[buf] + mr * XROW + 8 * ch);
            dst[0] = r.b0;
            dst[1] = r.b1;
        }
    }
    if (FMT != LB_TERNARY_PLANAR && tid < TM) {
        // (on a half step the values of blocks 2 and 3 are not read)
        lds.dx[buf][0 * TM + tid] = half_bits_to_float((uint16_t)(r.c.x & 0xffffu));
        lds.dx[buf][1 * TM + tid] = half_bits_to_float((uint16_t)(r.c.x >> 16));
        lds.dx[buf][2 * TM + tid] = half_bits_to_float((uint16_t)(r.c.y & 0xffffu));
        lds.dx[buf][3 * TM + tid] = half_bits_to_float((uint16_t)(r.c.y >> 16));
    }
    const int rr = tid >> 3, p = tid & 7;
    uint32_t *wrow = lds.w[buf] + rr * WROW;
    if (FMT == LB_Q1_0) {
        // sign dword m holds 8 weights of each activation block; this thread builds blocks 2 hb, 2 hb + 1
        const int m = p >> 1, hb = p & 1;
        const uint32_t v = r.a.x, lut = 0x000001FFu; // 0 -> -1, 1 -> +1
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int j = 2 * hb + q;
            const uint32_t e0 = __builtin_amdgcn_perm(0u, lut, (v >> j) & 0x01010101u);       // k = 0, 2, 4, 6
            const uint32_t e1 = __builtin_amdgcn_perm(0u, lut, (v >> (j + 4)) & 0x01010101u); // k = 1, 3, 5, 7
            *reinterpret_cast<uint2 *>(wrow + 8 * j + 2 * m) =
                make_uint2(__builtin_amdgcn_perm(e1, e0, 0x05010400u), __builtin_amdgcn_perm(e1, e0, 0x07030602u));
        }
        if (p == 0)
            lds.dw[buf][rr] = half_bits_to_float((uint16_t)r.a.z);
    } else if (FMT == LB_Q8_0) {
        // the weights are int8 already: copied as they are
        const int j = p >> 1;
        *reinterpret_cast<uint4 *>(wrow + 8 * j + 4 * (p & 1)) = r.a;
        if ((p & 1) == 0)
            lds.dw[buf][j * TN + rr] = half_bits_to_float((uint16_t)r.ws);
    } else if (FMT == LB_Q2_0_G64) {
        const int bb = p >> 2, d = p & 3;
        if (2 * bb < kab) {
            uint32_t o[4];
            unpack_q2_dword(r.a.x, o);
            *reinterpret_cast<uint4 *>(wrow + 16 * bb + 4 * d) = make_uint4(o[0], o[1], o[2], o[3]);
            if (d == 0)
                lds.dw[buf][bb * TN + rr] = half_bits_to_float((uint16_t)r.a.z);
        }
    } else {
        const int bb = p >> 2, hh = (p >> 1) & 1, sub = p & 1;
        if (2 * bb < kab) {
            // bits 4 sub .. 4 sub + 3 of each byte: weights 8 t + 4 sub + s of the dword pair's 32
            const uint32_t lut = 0x00FF0100u; // (pos, neg): 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0
            uint32_t e[4];
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const int rb = 4 * sub + s;
                e[s] = __builtin_amdgcn_perm(0u, lut, ((r.a.x >> rb) & 0x01010101u) | (((r.a.y >> rb) & 0x01010101u) << 1));
            }
            uint32_t t[4];
            transpose4(e[0], e[1], e[2], e[3], t);
            uint32_t *dst = wrow + 16 * bb + 8 * hh;
#pragma unroll
            for (int q = 0; q < 4; q++)
                dst[2 * q + sub] = t[q];
        }
    }
}

// One wave's share of a K-step: its 32 x 32 output tile over the step's kab q8_0 blocks (4, or 2 on the
// half step that ends a Q2_0 / planar row of an odd number of weight blocks).
template <int FMT, bool EMIT>
__device__ __forceinline__ void step_compute(const Lds &lds, int buf, int kab, int h, int l32, int wn, int wm, int m0,
                                             int n0, int M, int N, int nab, int kk, float (&acc)[16], v16i &iacc,
                                             const v16i &cbias, int32_t *__restrict__ sums)
{
    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    // accumulator preset to the bias (else zero); exact while |isum| < 2^22 (Q8_0: at most 2^19)
    constexpr bool BIASED = FMT == LB_Q2_0_G64 || FMT == LB_Q8_0;
    constexpr int JW = FMT == LB_Q1_0 ? 4 : FMT == LB_Q8_0 ? 1 : 2; // activation blocks per weight block
    const uint32_t *wl = lds.w[buf] + (32 * wn + l32) * WROW + 4 * h;
    const uint32_t *xl = lds.x[buf] + (32 * wm + l32) * XROW + 4 * h;
    float t[16];
#pragma unroll
    for (int j = 0; j < KS / QK8; j++) {
        if (j >= kab) // uniform
            break;
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
        if (BIASED) {
            const float c = -dx * BIASF; // exact: an 11-bit significand times 3 * 2^22
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float v = fmaf(dx, __int_as_float(D[i]), c); // round(d_x * isum)
                t[i] = j % JW == 0 ? v : t[i] + v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) // (float)isum is exact: |isum| < 2^24
                t[i] = j % JW == 0 ? dx * (float)D[i] : fmaf(dx, (float)D[i], t[i]);
        }
        if (EMIT) {
            const int m = m0 + 32 * wm + l32, kb = kk / QK8 + j;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int n = n0 + 32 * wn + 8 * (i >> 2) + 4 * h + (i & 3);
                if (m < M && n < N)
                    sums[((int64_t)m * N + n) * nab + kb] = BIASED ? D[i] - (int)BIAS : D[i];
            }
        }
        if (j % JW == JW - 1) { // the weight block is complete
            const int b = j / JW;
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
}

// KSPLIT = 2 (grids of fewer than two workgroups per CU): a workgroup of 16 waves, whose two 8-wave halves
// walk alternate K-steps of the same output tile with their own LDS buffers and add their partial sums
// at the end, so a CU holds 16 waves where the tile count alone would give it 8.
template <int FMT, bool EMIT, int KSPLIT>
__global__ __launch_bounds__(GT * KSPLIT, 2 * KSPLIT) void gemm_kernel(const uint8_t *__restrict__ W, int N, int K,
                                                                       float w_scale, const int8_t *__restrict__ X,
                                                                       const void *__restrict__ Xscale, int M,
                                                                       float *__restrict__ Y, int32_t *__restrict__ sums,
                                                                       int ntn)
{
    __shared__ Lds lds[KSPLIT];

    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    // (uniform per wave: readfirstlane keeps the step bookkeeping in scalar registers)
    const int half = KSPLIT == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / GT);
    const int tid = (int)threadIdx.x % GT, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    // this wave's 32 x 32 output tile inside the 64 x 128 workgroup tile
    const int wn = wave & 1, wm = wave >> 1;
    const int bn = blockIdx.x % ntn, bm = blockIdx.x / ntn; // weight tiles vary fastest
    const int n0 = bn * TN, m0 = bm * TM;
    const int64_t rowcode = FMT == LB_Q1_0 ? K / 8 : FMT == LB_Q8_0 ? K : K / 4; // code bytes per weight row
    const int nab = K / QK8;                                                  // activation blocks per row
    const uint16_t *wsc = reinterpret_cast<const uint16_t *>(W + (int64_t)N * rowcode);
    const uint16_t *xsc = reinterpret_cast<const uint16_t *>(Xscale);

    // Q2_0: 16 registers of the bias, each made opaque to the compiler: a tile it knows to be uniform it
    // rebuilds before every MFMA (16 moves each) instead of keeping it live.  Q1_0: a zero accumulator
    // (its results are converted instead: the bias registers would push it past 128 VGPRs, and so to one
    // workgroup per CU)
    v16i cbias;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        int b = (int)BIAS;
        if (FMT == LB_Q2_0_G64 || FMT == LB_Q8_0)
            asm volatile("; opaque bias %0" : "+v"(b));
        else
            b = 0;
        cbias[i] = b;
    }
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
    // of the weight blocks does.  Half h of a split workgroup takes steps h, h + 2, ...
    const int nsteps = (K + KS - 1) / KS;
    const int nsh = (nsteps + KSPLIT - 1) / KSPLIT; // steps of the first half (the second may have one fewer)
    const int rot = bn % nsteps;
    auto step_k = [&](int j) { // K offset of this half's j-th step, clamped to the last step
        return ((min(j * KSPLIT + half, nsteps - 1) + rot) % nsteps) * KS;
    };

    // register ring: the loads of step j + PF are issued into the slot step j frees; the step loop is
    // unrolled by the ring length so every slot is a fixed set of registers and the compiler can wait
    // for exactly the oldest step's loads
    constexpr int PF = 2; // (3 measured slower: its registers cost the second workgroup per CU)
    StepRegs ring[PF];
#pragma unroll
    for (int p = 0; p < PF; p++)
        load_step<FMT>(ring[p], W, wsc, N, K, X, xsc, M, n0, m0, step_k(p), tid);

    for (int j0 = 0; j0 < nsh; j0 += PF)
#pragma unroll
    for (int q = 0; q < PF; q++) {
        const int j = j0 + q;
        if (j >= nsh) // uniform
            break;
        // the second half of a split workgroup may run one step short: it still meets every barrier
        const bool active = j * KSPLIT + half < nsteps; // uniform per half
        const int buf = j & 1;
        const int kk = step_k(j);
        const int kab = min(KS, K - kk) / QK8;
        if (active)
            store_step<FMT>(lds[half], buf, ring[q], K, kk, tid);
        __syncthreads();
        // unconditional (the last steps re-load the final step, unused): a load under a branch would make
        // the compiler wait for every outstanding load at the next store instead of only this slot's
        load_step<FMT>(ring[q], W, wsc, N, K, X, xsc, M, n0, m0, step_k(j + PF), tid);
        if (active)
            step_compute<FMT, EMIT>(lds[half], buf, kab, h, l32, wn, wm, m0, n0, M, N, nab, kk, acc, iacc, cbias,
                                    sums);
    }

    if (KSPLIT == 2) {
        // the second half hands its partial sums to the first through LDS: 8 waves x 16 x 64 dwords = 32 KiB
        // over the first half's buffers, free once every wave has passed this barrier
        static_assert(sizeof(Lds) >= 8 * 16 * 64 * 4, "reduction area");
        __syncthreads();
        uint32_t *red = reinterpret_cast<uint32_t *>(&lds[0]);
        if (half == 1) {
#pragma unroll
            for (int i = 0; i < 16; i++)
                red[(wave * 16 + i) * 64 + lane] = PLANAR ? (uint32_t)iacc[i] : __float_as_uint(acc[i]);
        }
        __syncthreads();
        if (half == 1)
            return;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t o = red[(wave * 16 + i) * 64 + lane];
            if (PLANAR)
                iacc[i] += (int)o;
            else
                acc[i] += __uint_as_float(o);
        }
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

// Compute units of the current device, cached per device.
static int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
            v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int FMT, bool EMIT>
hipError_t launch_fmt(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *Xq, const void *Xscale,
                      int64_t M, float *Y, int32_t *sums, hipStream_t s)
{
    const int64_t ntn = (N + TN - 1) / TN, ntm = (M + TM - 1) / TM;
    if (ntn * ntm > INT32_MAX)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(ntn * ntm));
    // fewer tiles than two workgroups per CU: split K inside 16-wave workgroups (the block-sum instances
    // need more than the 128 registers a 16-wave workgroup allows, and keep 8 waves)
    if constexpr (!EMIT) {
        if (ntn * ntm < 2 * (int64_t)device_cus()) {
            hipLaunchKernelGGL((gemm_kernel<FMT, EMIT, 2>), grid, dim3(2 * GT), 0, s, W, (int)N, (int)K, w_scale, Xq,
                               Xscale, (int)M, Y, sums, (int)ntn);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_kernel<FMT, EMIT, 1>), grid, dim3(GT), 0, s, W, (int)N, (int)K, w_scale, Xq, Xscale,
                       (int)M, Y, sums, (int)ntn);
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
    case LB_Q8_0:
        return emit ? launch_fmt<LB_Q8_0, true>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s)
                    : launch_fmt<LB_Q8_0, false>(W, N, K, w_scale, Xq, Xscale, M, Y, sums, s);
    case LB_TERNARY_B3:
        return hipErrorNotSupported; // decode only
    }
    return hipErrorInvalidValue;
}

} // namespace lb
