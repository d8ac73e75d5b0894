// Prefill product Y[M][N] on the int8 matrix cores (v_mfma_i32_32x32x32_i8).
//
// Prefill multiplies the same weights by many activation rows, so it is a dense contraction (tritium
// "Architecture", section 3: prefill runs compute-bound; bankml technical report, section III.3: a
// tile loads each weight block once and applies it to several activation columns).
//
// Mapping to CDNA4:
//  * A workgroup owns a tile of TN = 64 weight rows x TM = 128 activation rows and walks K in steps of
//    128 columns.  Each step is software-pipelined: while a step computes, the next step's packed weight
//    codes, weight scales and activation scales are loaded into registers and its activation tile
//    streams HBM -> LDS through the load unit; at the top of a step the registers are written to
//    double-buffered LDS -- the weights unpacked to int8 in natural column order (shift and mask, a 4x4
//    byte transpose with v_perm_b32, and a v_perm_b32 lookup from code to weight byte: Q2_0 c -> c - 1,
//    Q1_0 bit -> +/-1, planar (pos, neg) -> pos - neg; Q8_0 weights are int8 already and copied as they
//    are) -- and one barrier per step separates the writes from the reads.  Every thread loads and
//    unpacks an equal share of the weight tile and issues an equal share of the activation tile.
//  * A workgroup is 8 waves (512 threads), two per SIMD, and two workgroups fit a CU.  Wave w computes
//    the 32 x 32 output tile (weight rows 32 (w mod 2), activation rows 32 (w / 2)) over every step's
//    four q8_0 blocks (32 columns each, the MFMA's K depth): per block one A operand (weights) and one B
//    operand (activations) from LDS, one MFMA, one exact int32 sum per (weight row, activation row,
//    block).  The weight unpack is shared by the 128 activation rows of the tile and the activation copy
//    by its 64 weight rows, so per MFMA the per-step work stays small next to the rescale below.
//  * Q1_0, Q2_0 and Q8_0: the accumulator input of every MFMA is a constant register tile holding
//    0x4B400000 (1.5 * 2^23), so each result, read as fp32, is 1.5 * 2^23 + isum exactly; one FMA with the
//    block's activation scale and -d_x * 1.5 * 2^23 gives round(d_x * isum) without a conversion.  The
//    weight block scale is then applied with one more FMA (bankml technical report, section III.3: one
//    multiply-add per q8_0 block, then one per weight block).
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
constexpr int XCH = KS / 16;     // 16-byte chunks per activation tile row
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

// What one thread carries from global memory into a K-step's weight tile.  Every thread takes one share of
// it -- Q2_0: one code dword (16 weights); Q1_0: one sign dword, of which it builds two of the four
// activation blocks; planar: one (pos, neg) dword pair, of which it builds half; Q8_0: 16 weight bytes --
// in a (planar neg in a.y; the weight block scale's binary16 where the thread stores it in
// sc, sh), and, for the first TM threads, the four binary16 activation scales of one activation row in c.
struct StepRegs {
    uint4 a;
    uint2 c;
    uint32_t sc; // the aligned dword holding the thread's weight block scale (binary16) ...
    uint32_t sh; // ... at this bit offset (0 or 16)
};

// Global-address-space views: loads take a scalar base and a 32-bit per-lane offset (the ABI keeps the
// weight tensor and the activation matrix under 4 GiB), so no 64-bit address arithmetic per load.
typedef __attribute__((address_space(1))) const uint8_t gu8;
typedef __attribute__((address_space(1))) const v4u gv4u;
typedef __attribute__((address_space(1))) const uint32_t gu32;
typedef __attribute__((address_space(1))) const uint16_t gu16;
typedef unsigned v2u_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef __attribute__((address_space(1))) const v2u_a4 gv2u;
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Per-thread load offsets, fixed for the whole K walk: every load of a step is a per-step scalar base (the
// tensor's address plus the step's offset, kept in scalar registers) plus one of these 32-bit lane offsets,
// so a step's loads cost no vector arithmetic.  Rows past N or M are clamped to the last row (re-read,
// never stored).
struct LaneOffs {
    uint32_t w;     // the thread's share of the weight codes (Q8_0: of the weight bytes)
    uint32_t ws;    // its weight block scale
    uint32_t dx;    // Q8_0: the four activation scales of activation row tid mod TM (the other formats rebuild it)
    uint32_t x[2];  // its two activation-tile slots: row offset + 16 x chunk (x_slot)
};

// Bytes a step advances each base by: weight records (16 bytes per 64 Q2_0 / planar or 128 Q1_0 weights, 32
// per 32 Q8_0 weights), their binary16 scales, the activation scales (binary16 per 32) and the activation
// bytes themselves.
template <int FMT> __device__ __forceinline__ uint32_t step_wbytes(int kk)
{
    return FMT == LB_Q1_0 ? (uint32_t)(kk / 128) * 16u : FMT == LB_Q8_0 ? (uint32_t)kk : (uint32_t)(kk / 64) * 16u;
}
template <int FMT> __device__ __forceinline__ uint32_t step_sbytes(int kk)
{
    return FMT == LB_Q1_0 ? (uint32_t)(kk / 128) * 2u : FMT == LB_Q8_0 ? (uint32_t)(kk / 32) * 2u : (uint32_t)(kk / 64) * 2u;
}

template <int FMT>
__device__ __forceinline__ LaneOffs lane_offsets(int N, int K, int M, int n0, int m0, int tid)
{
    LaneOffs o;
    const int row = min(n0 + (tid >> 3), N - 1), p = tid & 7;
    if (FMT == LB_Q1_0) { // one 128-weight record per row and step; thread p takes sign dword p / 2
        o.w = (uint32_t)row * (uint32_t)(K / 128) * 16u + 4u * (uint32_t)(p >> 1);
        o.ws = (uint32_t)row * (uint32_t)(K / 128) * 2u;
    } else if (FMT == LB_Q8_0) { // four 32-byte records per row; thread p takes half p % 2 of record p / 2
        o.w = (uint32_t)row * (uint32_t)K + 32u * (uint32_t)(p >> 1) + 16u * (uint32_t)(p & 1);
        o.ws = ((uint32_t)row * (uint32_t)(K / 32) + (uint32_t)(p >> 1)) * 2u;
    } else if (FMT == LB_Q2_0_G64) { // two 64-weight records per row; thread p takes dword p % 4 of record p / 4
        o.w = ((uint32_t)row * (uint32_t)(K / 64) + (uint32_t)(p >> 2)) * 16u + 4u * (uint32_t)(p & 3);
        o.ws = ((uint32_t)row * (uint32_t)(K / 64) + (uint32_t)(p >> 2)) * 2u;
    } else { // two 64-column beats per row; thread p takes the (pos, neg) dword pair (p / 2) % 2 of beat p / 4
        o.w = ((uint32_t)row * (uint32_t)(K / 64) + (uint32_t)(p >> 2)) * 16u + 4u * (uint32_t)((p >> 1) & 1);
        o.ws = 0;
    }
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int slot = 128 * wave + 64 * u + lane, r = slot / XCH;
        o.x[u] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + 16u * (uint32_t)((slot % XCH) ^ ((r >> 1) & 7));
    }
    o.dx = (uint32_t)min(m0 + (tid & (TM - 1)), M - 1) * (uint32_t)(K / QK8) * 2u;
    return o;
}

// One step's weight codes / scales and activation scales into registers.  A full step (128 columns) reads
// exactly the step's blocks.  The half step that ends a Q2_0 / planar row of an odd number of 64-column
// blocks (only one step of the walk) takes a branch whose lanes of the missing second block re-read the
// first.  Every thread loads the activation scales of activation row tid mod TM (the first TM threads
// store them).
template <int FMT>
__device__ __forceinline__ void load_step(StepRegs &r, const LaneOffs &o, const uint8_t *__restrict__ W,
                                          const uint8_t *__restrict__ wsc, const uint8_t *__restrict__ xsc, int kk,
                                          bool half_step, int tid, int m0, int M, int K)
{
    uint32_t ow = o.w + step_wbytes<FMT>(kk), os = o.ws + step_sbytes<FMT>(kk);
    if (half_step) { // uniform
        const uint32_t second = (uint32_t)((tid >> 2) & 1); // the lane's record / beat index within the step
        ow -= 16u * second;
        os -= 2u * second;
    }
    if (FMT != LB_TERNARY_PLANAR && tid < TM) {
        // Q1_0 and Q2_0 rebuild the row offset at every step (an opaque copy of tid stops the compiler from
        // keeping it live across the loop, where it costs a register that their two result tiles need);
        // Q8_0 keeps it
        uint32_t odx = o.dx;
        if (FMT != LB_Q8_0) {
            int t = tid;
            asm volatile("; activation-scale row %0" : "+v"(t));
            odx = (uint32_t)min(m0 + t, M - 1) * (uint32_t)(K / QK8) * 2u;
        }
        odx += (uint32_t)(kk / QK8) * 2u;
        // one 8-byte load per activation row (4-byte aligned: K / 32 and kk / 32 are even); the half step has
        // two blocks only
        if (half_step) { // (blocks 2 and 3 are stored as zero)
            r.c.x = *(const gu32 *)((const gu8 *)xsc + odx);
        } else {
            const v2u_a4 t = *(const gv2u *)((const gu8 *)xsc + odx);
            r.c.x = t.x, r.c.y = t.y;
        }
    }
    if (FMT == LB_Q8_0) {
        const v4u t = *(const gv4u *)((const gu8 *)W + ow);
        r.a = make_uint4(t.x, t.y, t.z, t.w);
    } else if (FMT == LB_TERNARY_PLANAR) {
        r.a.x = *(const gu32 *)((const gu8 *)W + ow);        // pos
        r.a.y = *(const gu32 *)((const gu8 *)W + (ow + 8u)); // neg
    } else {
        r.a.x = *(const gu32 *)((const gu8 *)W + ow);
    }
    if (FMT != LB_TERNARY_PLANAR) {
        // the scale's aligned dword (a 2-byte load would be widened by an instruction of its own, which makes the
        // compiler wait for the load as soon as it is issued)
        r.sc = *(const gu32 *)((const gu8 *)wsc + (os & ~3u));
        r.sh = (os & 2u) * 8u;
    }
}

// The activation tile of a step (TM rows x KS bytes) goes HBM -> LDS through the load unit, without
// registers: one global_load_lds_dwordx4 writes lane i's 16 bytes at the wave's LDS base + 16 i, so each
// instruction fills 64 consecutive 16-byte slots and each thread issues two.  Chunk c (16 bytes) of tile
// row r sits in slot r * XCH + (c ^ ((r >> 1) & 7)), so the operand reads (16 lanes, one chunk of 16
// consecutive rows each) meet 16 different bank groups; the lane that fills a slot loads the chunk that
// belongs there.  On the half step the lanes of the chunks past K load nothing (each wave holds whole
// rows, so every wave still issues both instructions).
__device__ __forceinline__ int x_slot(int r, int c) { return r * XCH + (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ void issue_x(uint32_t *lds_tile, const int8_t *__restrict__ X, const LaneOffs &o, int kk,
                                       bool half_step, int wave, int lane)
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
        uint32_t *dst = lds_tile + 4 * (128 * wave + 64 * u); // the wave's 64 slots
        if (!half_step || ((64 * u + lane) % XCH ^ (((128 * wave + 64 * u + lane) / XCH >> 1) & 7)) < 4)
            __builtin_amdgcn_global_load_lds((gvoid *)((const gu8 *)X + (o.x[u] + (uint32_t)kk)), (lvoid *)dst, 16, 0, 0);
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt(int vm, int lgkm) { return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14); }
constexpr int wait_vmcnt(int n) { return waitcnt(n, 15); }
constexpr int WAIT_LGKM0 = waitcnt(63, 0);
static_assert(wait_vmcnt(0) == 0x0F70 && WAIT_LGKM0 == 0xC07F, "s_waitcnt encoding");

// A workgroup barrier for the step loop.  __syncthreads() would also fence memory, which makes every thread
// wait for all of its outstanding loads -- the activation tiles of the next steps included -- so the
// loop takes its waits explicitly: this thread's LDS writes (lgkmcnt 0) before the barrier, and the loads a
// step reads (a vmcnt wait at the top of the step).  The empty asm statements keep the compiler from moving
// LDS accesses across the barrier.
__device__ __forceinline__ void step_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct __attribute__((aligned(16))) Lds {
    uint32_t w[2][TN * WROW];   // unpacked int8 weight tiles, padded rows
    float dw[2][4 * TN];        // weight block scales: [block within step][row]
    float dx[2][4 * TM];        // activation scales: [block within step][row]
};
constexpr int XTILE = TM * KS / 4; // dwords of an activation tile, swizzled 16-byte chunks (x_slot)

template <int FMT>
__device__ __forceinline__ void store_step(Lds &lds, int buf, const StepRegs &r, int K, int kk, int tid)
{
    // On the half step that ends a row of an odd number of 64-column blocks, blocks 2 and 3 of the step get
    // zero weights and zero scales: every step then runs the same four-block compute, and the missing blocks
    // add exactly +0 (the MFMA gives the bias, the rescale 0 * bias - 0 * bias = +0, times a zero scale).
    const int kab = min(KS, K - kk) / QK8;
    if (FMT != LB_TERNARY_PLANAR && tid < TM) {
        const uint32_t hi = kab == 4 ? r.c.y : 0u;
        lds.dx[buf][0 * TM + tid] = half_bits_to_float((uint16_t)(r.c.x & 0xffffu));
        lds.dx[buf][1 * TM + tid] = half_bits_to_float((uint16_t)(r.c.x >> 16));
        lds.dx[buf][2 * TM + tid] = half_bits_to_float((uint16_t)(hi & 0xffffu));
        lds.dx[buf][3 * TM + tid] = half_bits_to_float((uint16_t)(hi >> 16));
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
            lds.dw[buf][rr] = half_bits_to_float((uint16_t)(r.sc >> r.sh));
    } else if (FMT == LB_Q8_0) {
        // the weights are int8 already: copied as they are
        const int j = p >> 1;
        *reinterpret_cast<uint4 *>(wrow + 8 * j + 4 * (p & 1)) = r.a;
        if ((p & 1) == 0)
            lds.dw[buf][j * TN + rr] = half_bits_to_float((uint16_t)(r.sc >> r.sh));
    } else if (FMT == LB_Q2_0_G64) {
        const int bb = p >> 2, d = p & 3;
        const bool live = 2 * bb < kab;
        uint32_t o[4];
        unpack_q2_dword(live ? r.a.x : 0x55555555u, o); // code 1 = weight 0
        *reinterpret_cast<uint4 *>(wrow + 16 * bb + 4 * d) = make_uint4(o[0], o[1], o[2], o[3]);
        if (d == 0)
            lds.dw[buf][bb * TN + rr] = live ? half_bits_to_float((uint16_t)(r.sc >> r.sh)) : 0.0f;
    } else {
        const int bb = p >> 2, hh = (p >> 1) & 1, sub = p & 1;
        const bool live = 2 * bb < kab;
        const uint32_t pos = live ? r.a.x : 0u, neg = live ? r.a.y : 0u;
        // bits 4 sub .. 4 sub + 3 of each byte: weights 8 t + 4 sub + s of the dword pair's 32
        const uint32_t lut = 0x00FF0100u; // (pos, neg): 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0
        uint32_t e[4];
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int rb = 4 * sub + s;
            e[s] = __builtin_amdgcn_perm(0u, lut, ((pos >> rb) & 0x01010101u) | (((neg >> rb) & 0x01010101u) << 1));
        }
        uint32_t t[4];
        transpose4(e[0], e[1], e[2], e[3], t);
        uint32_t *dst = wrow + 16 * bb + 8 * hh;
#pragma unroll
        for (int q = 0; q < 4; q++)
            dst[2 * q + sub] = t[q];
    }
}

// One wave's share of a K-step: its 32 x 32 output tile over the step's KAB = 4 q8_0 blocks (on a half step
// the last two carry zero weights and scales).  Each block's result is scaled as soon as it is ready; the
// next block's MFMA runs meanwhile (Q1_0, Q2_0), and the other waves of the SIMD fill the rest.
template <int FMT, bool EMIT, int KAB>
__device__ __forceinline__ void step_compute(const Lds &lds, int buf, const uint32_t *xt, const uint32_t (&xb)[4], int h,
                                             int l32, int wn, int wm, int m0, int n0, int M, int N, int nab, int kk,
                                             float (&acc)[16], v16i &iacc, const v16i &cbias,
                                             int32_t *__restrict__ sums)
{
    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    constexpr int JW = FMT == LB_Q1_0 ? 4 : FMT == LB_Q8_0 ? 1 : 2; // activation blocks per weight block
    const uint32_t *wl = lds.w[buf] + (32 * wn + l32) * WROW + 4 * h;
    auto mfma = [&](int j, const v16i &c) {
        const uint4 a4 = *reinterpret_cast<const uint4 *>(wl + 8 * j);
        const uint4 b4 = *reinterpret_cast<const uint4 *>(xt + xb[j]); // chunk 2 j + h of the lane's row
        const v4i A = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
        const v4i B = {(int)b4.x, (int)b4.y, (int)b4.z, (int)b4.w};
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, c, 0, 0, 0);
    };
    if (PLANAR) {
#pragma unroll
        for (int j = 0; j < KAB; j++)
            iacc = mfma(j, iacc);
        return;
    }
    // the step's activation scales of this lane's activation row
    float dx[KAB];
#pragma unroll
    for (int j = 0; j < KAB; j++)
        dx[j] = lds.dx[buf][j * TM + 32 * wm + l32];
    // every result is read as fp32 through the bias: 1.5 * 2^23 + isum exactly (|isum| < 2^22).  Q1_0 and
    // Q2_0 issue each block's MFMA before the previous block's rescale, so the wave's own rescale covers the
    // MFMA latency (Q8_0, whose weight scales change with every block, measured slower that way).
    constexpr bool AHEAD = FMT != LB_Q8_0;
    v16i Dn;
    if (AHEAD)
        Dn = mfma(0, cbias);
#pragma unroll
    for (int j = 0; j < KAB; j++) {
        const v16i Dj = AHEAD ? Dn : mfma(j, cbias);
        if (AHEAD && j + 1 < KAB)
            Dn = mfma(j + 1, cbias);
        // the weight block's scales of this lane's 16 weight rows
        float dwv[16];
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const float4 dw = *reinterpret_cast<const float4 *>(lds.dw[buf] + (j / JW) * TN + 32 * wn + 8 * g + 4 * h);
            dwv[4 * g] = dw.x, dwv[4 * g + 1] = dw.y, dwv[4 * g + 2] = dw.z, dwv[4 * g + 3] = dw.w;
        }
        const float c = -dx[j] * BIASF; // exact: an 11-bit significand times 3 * 2^22
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float v = fmaf(dx[j], __int_as_float(Dj[i]), c); // round(d_x * isum)
            acc[i] = fmaf(dwv[i], v, acc[i]);
        }
        if (EMIT) {
            const int m = m0 + 32 * wm + l32, kb = kk / QK8 + j;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int n = n0 + 32 * wn + 8 * (i >> 2) + 4 * h + (i & 3);
                if (m < M && n < N && kb < nab) // (the zero blocks of a half step have no sums)
                    sums[((int64_t)m * N + n) * nab + kb] = Dj[i] - (int)BIAS;
            }
        }
    }
}

// KSPLIT = 2 (grids of fewer than two workgroups per CU): a workgroup of 16 waves, whose two 8-wave halves
// walk alternate K-steps of the same output tile with their own LDS buffers and add their partial sums
// at the end, so a CU holds 16 waves where the tile count alone would give it 8.
template <int FMT, bool EMIT, int KSPLIT>
__global__ __launch_bounds__(GT * KSPLIT, EMIT ? 2 * KSPLIT : 4) void gemm_kernel(const uint8_t *__restrict__ W, int N, int K,
                                                                       float w_scale, const int8_t *__restrict__ X,
                                                                       const void *__restrict__ Xscale, int M,
                                                                       float *__restrict__ Y, int32_t *__restrict__ sums,
                                                                       int ntn)
{
    __shared__ Lds lds[KSPLIT];
    __shared__ uint32_t xt0[KSPLIT][XTILE], xt1[KSPLIT][XTILE];

    constexpr bool PLANAR = FMT == LB_TERNARY_PLANAR;
    // (uniform per wave: readfirstlane keeps the step bookkeeping in scalar registers)
    const int half = KSPLIT == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / GT);
    const int tid = (int)threadIdx.x % GT, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    // this wave's 32 x 32 output tile inside the 64 x 128 workgroup tile
    const int wn = wave & 1, wm = wave >> 1;
    const int bn = blockIdx.x % ntn, bm = blockIdx.x / ntn; // weight tiles vary fastest
    const int n0 = bn * TN, m0 = bm * TM;
    const int64_t rowcode = FMT == LB_Q1_0 ? K / 8 : FMT == LB_Q8_0 ? K : K / 4; // code bytes per weight row
    const int nab = K / QK8;                                                  // activation blocks per row
    const uint8_t *wsc = W + (int64_t)N * rowcode;
    const uint8_t *xsc = reinterpret_cast<const uint8_t *>(Xscale);

    // 16 registers of the bias, each made opaque to the compiler: a tile it knows to be uniform it rebuilds
    // before every MFMA (16 moves each) instead of keeping it live.  Planar: a zero accumulator.
    v16i cbias;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        int b = (int)BIAS;
        if (FMT != LB_TERNARY_PLANAR)
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
    const int kend = nsteps * KS;                   // the walk's K offsets are taken modulo this
    const int kfirst = ((bn % nsteps + half) % nsteps) * KS;

    const LaneOffs lo = lane_offsets<FMT>(N, K, M, n0, m0, tid);
    uint32_t xb[4]; // dword offsets in a tile of chunk 2 j + h of activation row 32 wm + l32
#pragma unroll
    for (int j = 0; j < 4; j++)
        xb[j] = 4u * (uint32_t)x_slot(32 * wm + l32, 2 * j + h);

    // Step j's weight codes and scales are loaded into registers, and its activation tile into LDS, while
    // step j - 1 computes; at the top of step j the thread waits for its own loads, unpacks the weights into
    // LDS, and a barrier makes every thread's share visible.  The step loop is unrolled by two so that the
    // LDS tiles of every step are fixed objects.
    StepRegs ring;
    int kk = kfirst;
    load_step<FMT>(ring, lo, W, wsc, xsc, kk, K - kk < KS, tid, m0, M, K);
    issue_x(xt0[half], X, lo, kk, K - kk < KS, wave, lane);

    for (int j0 = 0; j0 < nsh; j0 += 2)
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int j = j0 + q;
        if (j >= nsh) // uniform
            break;
        // the second half of a split workgroup may run one step short: it still meets every barrier
        const bool active = KSPLIT == 1 || j * KSPLIT + half < nsteps; // uniform per half
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(0)); // this thread's loads of step j have landed
        if (active)
            store_step<FMT>(lds[half], q, ring, K, kk, tid);
        step_barrier();
        // the next step's loads (past the last step the walk wraps: valid addresses, unused).  With one
        // step in all and two halves, the stride is twice the walk, so the offset may need two wraps.
        int kn = kk + KSPLIT * KS;
        kn = kn >= kend ? kn - kend : kn;
        kn = kn >= kend ? kn - kend : kn;
        load_step<FMT>(ring, lo, W, wsc, xsc, kn, K - kn < KS, tid, m0, M, K);
        issue_x(q ? xt0[half] : xt1[half], X, lo, kn, K - kn < KS, wave, lane);
        if (active)
            step_compute<FMT, EMIT, 4>(lds[half], q, q ? xt1[half] : xt0[half], xb, h, l32, wn, wm, m0, n0, M, N, nab,
                                       kk, acc, iacc, cbias, sums);
        kk = kn;
    }
    // the last (unused) activation loads must land before the workgroup's LDS is reused or released
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    if constexpr (KSPLIT == 2) {
        // the second half hands its partial sums to the first through LDS: 8 waves x 16 x 64 dwords = 32 KiB
        // over both halves' first activation tiles, free once every wave has passed this barrier
        static_assert(KSPLIT * sizeof(uint32_t) * XTILE >= 8 * 16 * 64 * 4, "reduction area");
        __syncthreads();
        uint32_t *red = xt0[0];
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

    // The wave's 32 x 32 tile of Y.  Lane (h, l32) holds weight rows n = 32 wn + 8 (i / 4) + 4 h + i % 4 of
    // activation row m = 32 wm + l32; the tile goes through LDS (a 32 x 32 fp32 area per wave, element
    // [m][n] at m * 32 + (n ^ m): the XOR keeps the column writes and the row reads free of bank conflicts)
    // so that every store writes two whole 128-byte row segments of Y.
    const int m = m0 + 32 * wm + l32;
    float out[16];
    if (PLANAR) {
        const float sx = reinterpret_cast<const float *>(Xscale)[min(m, M - 1)];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int n = n0 + 32 * wn + 8 * (i >> 2) + 4 * h + (i & 3);
            if (EMIT && m < M && n < N)
                sums[(int64_t)m * N + n] = iacc[i];
            out[i] = ((float)iacc[i] * sx) * w_scale;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++)
            out[i] = acc[i];
    }
    if (EMIT && Y == nullptr)
        return;
    if constexpr (KSPLIT == 1)
        __syncthreads(); // every wave is done with the activation tiles
    uint32_t *t = (wave < 4 ? xt0[0] : xt1[0]) + 1024 * (wave & 3);
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int nl = 8 * (i >> 2) + 4 * h + (i & 3);
        t[32 * l32 + (nl ^ l32)] = __float_as_uint(out[i]);
    }
    const int nc = lane & 31, n = n0 + 32 * wn + nc;
#pragma unroll
    for (int k = 0; k < 16; k++) {
        const int r = 2 * k + (lane >> 5), mm = m0 + 32 * wm + r;
        const float v = __uint_as_float(t[32 * r + (nc ^ r)]);
        if (mm < M && n < N)
            Y[(int64_t)mm * N + n] = v;
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
