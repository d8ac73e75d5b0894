// Batch-1 decode products for the three packed formats (Q1_0, Q2_0_g64, planar ternary) on gfx950.
//
// Arithmetic (bankml technical report, section III.8 "Operation"; tritium "Architecture", sections 1-2):
// every weight is a small integer, so each row's sum over a 32-activation block is an exact integer
// select-accumulate, and only the block scales are floating point.
//
// Mapping to CDNA4:
//  * The unit of work is a "slice": one 16-byte code record of one row -- a Q2_0_g64 block (64 weights,
//    two q8_0 activation blocks), a Q1_0 block (128 weights, four activation blocks) or a planar beat
//    (64 weights).
//  * A workgroup owns a tile of rows of one product.  It first stages the activation vector into LDS,
//    once, in the order the unpack needs (the activation, not the weights, is rearranged -- the bankml
//    report's ternary kernel does the same once per token).  Each int8 activation q is split into a
//    signed high nibble h = q >> 4 and an unsigned low nibble l = q & 15 (q = 16h + l), packed eight to
//    a dword in the order in which a shift-and-mask of a code word lays the weights out.
//  * A row is split over L lanes; a lane owns S slices (strided by L so each wave-wide 16-byte load is
//    contiguous) and keeps their staged activations in VGPRs across all the rows it streams.
//  * Per code dword, one mask (Q2_0: and at most one shift) isolates 8 codes or 8 sign bits as nibbles,
//    and one v_dot8_i32_i4 against the h nibbles plus one v_dot8_u32_u4 against the l nibbles accumulate
//    sum(code * q) = 16 * sum(code * h) + sum(code * l).  A masked bit that stays in place has nibble
//    value 2^r; that power of two is carried by the block scale (Q1_0, whose device records group each
//    activation block under one mask position) or recombined once per row (planar).  The offset forms of the pages give the exact
//    block sums: Q2_0  isum = sum(c q) - sum(q)  (code c = w + 1);  Q1_0  isum = 2 sum_{bit=1} q - sum(q);
//    planar  acc = sum_pos q - sum_neg q.
//  * Block scaling is one fp32 multiply-add per activation block and one per weight block (bankml
//    report, section III.3), then a cross-lane tree over the L lanes of the row.  Rows are never split
//    across workgroups, so results do not depend on the launch geometry (tritium "Architecture",
//    section 7: split rows, never a reduction).
#include "lowbit_internal.h"

namespace lb {

template <int FMT> struct F;
// SW: weights per slice; NAB: q8_0 blocks per slice; REC: dwords of staged activation per slice
// (SW/4 nibble words, then, for the ggml formats, d_x[NAB] (2 d_x / 2^j for Q1_0 block j) and
// -sum(q)[NAB])
template <> struct F<LB_Q2_0_G64> { enum { SW = 64, NAB = 2, REC = 20 }; };
template <> struct F<LB_Q1_0> { enum { SW = 128, NAB = 4, REC = 40 }; };
template <> struct F<LB_TERNARY_PLANAR> { enum { SW = 64, NAB = 0, REC = 16 }; };

constexpr int CODE_BYTES = 16; // every slice is one 16-byte record

// ------------------------------------------------------------------------------------------------
// Activation staging.  Nibble word (a, b) holds, at bits 4n..4n+3, the low (b = 0) or high (b = 1)
// nibble of activation e(a, n) of the slice, where e() is the position of the n-th code that the
// a-th mask extraction isolates:
//   Q2_0  a = 2k + s   (code dword k = weights 16k..16k+15; s = 0: mask 0x33333333, s = 1: shift 2
//                       first):  e = 16k + 2n + s
//   Q1_0  a = 4m + r   (device sign dword m, mask 0x11111111 << r; the device record puts the sign of
//                       weight 32r + 8m + n at bit 4n + r of dword m):  e = 32r + 8m + n
//   planar  a = 4k + r  (32-bit word k of plane bits; r = the bit within each nibble):  e = 32k + 4n + r
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nibbles16(uint32_t x) // low nibbles of 4 bytes -> 16 bits, in order
{
    x &= 0x0F0F0F0Fu;
    x = (x | (x >> 4)) & 0x00FF00FFu;
    return (x | (x >> 8)) & 0x0000FFFFu;
}

// The whole activation vector, staged by all threads of the workgroup as independent items: one item
// per nibble-word pair (the 8 activation bytes it covers, one 8/16/32-byte load, gathered with byte
// permutes where they are strided) and one per (slice, q8_0 block) for d_x and -sum(q).  Item loads are
// issued four at a time.
// The source sits in global memory (AS = 1) or, when the launch quantised it, in LDS (AS = 3); an explicit
// address space gives global or LDS loads instead of flat ones.
template <int AS, typename T> using src_t = __attribute__((address_space(AS))) const T;
typedef unsigned sv2u __attribute__((ext_vector_type(2))); // native vectors: loadable from any address space
typedef unsigned sv4u __attribute__((ext_vector_type(4)));
typedef float sv4f __attribute__((ext_vector_type(4)));
template <int AS> __device__ __forceinline__ uint2 ld2(src_t<AS, int8_t> *p)
{
    const sv2u t = *(src_t<AS, sv2u> *)p;
    return make_uint2(t.x, t.y);
}
template <int AS> __device__ __forceinline__ uint4 ld4(src_t<AS, int8_t> *p)
{
    const sv4u t = *(src_t<AS, sv4u> *)p;
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Loads of one item (one nibble-word pair: 8, 16 or 32 activation bytes) and of one (slice, q8_0 block)
// item (its 32 bytes and binary16 scale).
template <int FMT, int AS> struct StageLoads {
    uint4 v[FMT == LB_TERNARY_PLANAR ? 2 : 1];
};
template <int FMT, int AS>
__device__ __forceinline__ StageLoads<FMT, AS> stage_load_item(src_t<AS, int8_t> *xq, int it)
{
    constexpr int SW = F<FMT>::SW, WPS = SW / 8;
    StageLoads<FMT, AS> r;
    const int sl = it / WPS, a = it % WPS;
    src_t<AS, int8_t> *sb = xq + sl * SW;
    if (FMT == LB_Q1_0) { // 8 consecutive bytes
        const uint2 t = ld2<AS>(sb + 32 * (a & 3) + 8 * (a >> 2));
        r.v[0] = make_uint4(t.x, t.y, 0u, 0u);
    } else if (FMT == LB_Q2_0_G64) { // every other byte of 16
        r.v[0] = ld4<AS>(sb + 16 * (a >> 1));
    } else { // every fourth byte of 32
        r.v[0] = ld4<AS>(sb + 32 * (a >> 2));
        r.v[FMT == LB_TERNARY_PLANAR ? 1 : 0] = ld4<AS>(sb + 32 * (a >> 2) + 16);
    }
    return r;
}
template <int FMT, int AS>
__device__ __forceinline__ void stage_store_item(const StageLoads<FMT, AS> &t, int it, uint32_t *__restrict__ lds)
{
    constexpr int WPS = F<FMT>::SW / 8, REC = F<FMT>::REC;
    const int sl = it / WPS, a = it % WPS;
    uint32_t u0, u1;
    if (FMT == LB_Q1_0) {
        u0 = t.v[0].x;
        u1 = t.v[0].y;
    } else if (FMT == LB_Q2_0_G64) {
        const uint32_t sel = (a & 1) ? 0x07050301u : 0x06040200u;
        u0 = __builtin_amdgcn_perm(t.v[0].y, t.v[0].x, sel);
        u1 = __builtin_amdgcn_perm(t.v[0].w, t.v[0].z, sel);
    } else {
        const uint32_t r = (uint32_t)(a & 3), sel = r | ((4u + r) << 8);
        const uint4 lo4 = t.v[0], hi4 = t.v[FMT == LB_TERNARY_PLANAR ? 1 : 0];
        u0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(lo4.w, lo4.z, sel), __builtin_amdgcn_perm(lo4.y, lo4.x, sel),
                                   0x05040100u);
        u1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(hi4.w, hi4.z, sel), __builtin_amdgcn_perm(hi4.y, hi4.x, sel),
                                   0x05040100u);
    }
    uint32_t *rec = lds + sl * REC;
    rec[2 * a + 0] = nibbles16(u0) | (nibbles16(u1) << 16);
    rec[2 * a + 1] = nibbles16(u0 >> 4) | (nibbles16(u1 >> 4) << 16);
}
struct BlockLoads {
    uint4 b0, b1;
    uint32_t sc;
};
template <int FMT, int AS>
__device__ __forceinline__ BlockLoads stage_load_block(src_t<AS, int8_t> *xq, src_t<AS, uint16_t> *xscale, int it)
{
    constexpr int SW = F<FMT>::SW, NAB = F<FMT>::NAB > 0 ? F<FMT>::NAB : 1;
    const int sl = it / NAB, j = it % NAB;
    return {ld4<AS>(xq + sl * SW + 32 * j), ld4<AS>(xq + sl * SW + 32 * j + 16), (uint32_t)xscale[it]};
}
template <int FMT>
__device__ __forceinline__ void stage_store_block(const BlockLoads &t, int it, uint32_t *__restrict__ lds)
{
    constexpr int SW = F<FMT>::SW, NAB = F<FMT>::NAB > 0 ? F<FMT>::NAB : 1, REC = F<FMT>::REC;
    const int sl = it / NAB, j = it % NAB;
    int sq = 0;
    const uint32_t w[8] = {t.b0.x, t.b0.y, t.b0.z, t.b0.w, t.b1.x, t.b1.y, t.b1.z, t.b1.w};
#pragma unroll
    for (int k = 0; k < 8; k++)
        sq = __builtin_amdgcn_sdot4((int)w[k], 0x01010101, sq, false);
    // Q1_0 keeps 2 d_x / 2^j (exact): its block sums are 2 S - sum(q), S = the sum of q where the bit is 1,
    // and its products deliver 2^j S (the nibble value of mask position j)
    const float dx = half_bits_to_float((uint16_t)t.sc);
    const float q1f = j == 0 ? 2.0f : j == 1 ? 1.0f : j == 2 ? 0.5f : 0.25f;
    uint32_t *rec = lds + sl * REC;
    rec[SW / 4 + j] = __float_as_uint(FMT == LB_Q1_0 ? q1f * dx : dx);
    rec[SW / 4 + F<FMT>::NAB + j] = (uint32_t)(-sq);
}

// The whole activation vector, staged by all threads of the workgroup as independent items: one item
// per nibble-word pair (the 8 activation bytes it covers, one 8/16/32-byte load, gathered with byte
// permutes where they are strided) and one per (slice, q8_0 block) for d_x and -sum(q).  A thread's
// first items (UNR0 of the first kind, covering K up to 12288 for the ggml formats, and two of the
// second) are loaded before pre() runs -- the caller issues its first weight rows there -- so the waits
// for these loads never include the weights.  The source sits in global memory (AS = 1) or, when the
// launch quantised it, in LDS (AS = 3); an explicit address space gives global or LDS loads instead of
// flat ones.
template <int FMT, int AS, typename Pre>
__device__ __forceinline__ void stage_activation(const int8_t *__restrict__ xq_g, const void *__restrict__ xscale_g,
                                                 int ns, uint32_t *__restrict__ lds, Pre &&pre)
{
    src_t<AS, int8_t> *xq = (src_t<AS, int8_t> *)xq_g;
    src_t<AS, uint16_t> *xscale = (src_t<AS, uint16_t> *)xscale_g;
    constexpr int SW = F<FMT>::SW, NAB = F<FMT>::NAB;
    constexpr int WPS = SW / 8; // nibble-word pairs per slice
    constexpr int UNR0 = 6, NB0 = 2, UNR = 4;
    const int nw = ns * WPS, nblk = ns * NAB;
    const int t = threadIdx.x;
    StageLoads<FMT, AS> v0[UNR0];
#pragma unroll
    for (int q = 0; q < UNR0; q++)
        if (t + q * WG < nw)
            v0[q] = stage_load_item<FMT, AS>(xq, t + q * WG);
    // (unconditional, the index clamped to the last block: the scale's conversion then stays with its use,
    // after the weight rows, instead of joining the load under a branch and waiting for it here)
    BlockLoads k0[NB0];
#pragma unroll
    for (int q = 0; q < NB0; q++)
        if (NAB > 0)
            k0[q] = stage_load_block<FMT, AS>(xq, xscale, min(t + q * WG, nblk - 1));
    __builtin_amdgcn_sched_barrier(0);
    pre();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < UNR0; q++)
        if (t + q * WG < nw)
            stage_store_item<FMT, AS>(v0[q], t + q * WG, lds);
#pragma unroll
    for (int q = 0; q < NB0; q++)
        if (NAB > 0 && t + q * WG < nblk)
            stage_store_block<FMT>(k0[q], t + q * WG, lds);
    for (int base = t + UNR0 * WG; base < nw; base += UNR * WG) {
        StageLoads<FMT, AS> v[UNR];
#pragma unroll
        for (int q = 0; q < UNR; q++)
            if (base + q * WG < nw)
                v[q] = stage_load_item<FMT, AS>(xq, base + q * WG);
#pragma unroll
        for (int q = 0; q < UNR; q++)
            if (base + q * WG < nw)
                stage_store_item<FMT, AS>(v[q], base + q * WG, lds);
    }
    if (NAB > 0)
        for (int it = t + NB0 * WG; it < nblk; it += WG)
            stage_store_block<FMT>(stage_load_block<FMT, AS>(xq, xscale, it), it, lds);
}

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
__device__ __forceinline__ int udot8(uint32_t a, uint32_t b, int c)
{
    return (int)__builtin_amdgcn_udot8(a, b, (uint32_t)c, false);
}
// The first signed product of an accumulator chain, with the zero accumulator as an inline constant.  (The
// compiler would start the chain in the two-operand form that accumulates into its destination, which
// costs a move of zero into that register first: one VALU instruction per chain.)
__device__ __forceinline__ int sdot8z(uint32_t a, uint32_t b)
{
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// l - 16 h in one instruction (|h| < 2^23): the block whose mask bit reads as -8 in the signed product
__device__ __forceinline__ int sub16(int l, int h)
{
    int r;
    asm("v_mad_i32_i24 %0, %1, -16, %2" : "=v"(r) : "v"(h), "v"(l));
    return r;
}

// ------------------------------------------------------------------------------------------------
// Per-slice arithmetic.  Q formats return the slice's scaled contribution and (EMIT) its two exact
// block sums; planar accumulates its 16 integer partials.
// ------------------------------------------------------------------------------------------------

// Q2_0_g64: 4 code dwords, 16 2-bit codes each.
__device__ __forceinline__ void q2_isums(uint4 c, const uint32_t *A, int &i0, int &i1)
{
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    // the low-nibble accumulators start at -sum(q) (modular), so each block sum is one shift-add
    int h[2], l[2] = {(int)A[18], (int)A[19]};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t e0 = cw[k] & 0x33333333u;
        const uint32_t e1 = (cw[k] >> 2) & 0x33333333u;
        const int j = k >> 1;
        h[j] = (k & 1) ? sdot8(e0, A[(2 * k + 0) * 2 + 1], h[j]) : sdot8z(e0, A[(2 * k + 0) * 2 + 1]);
        l[j] = udot8(e0, A[(2 * k + 0) * 2 + 0], l[j]);
        h[j] = sdot8(e1, A[(2 * k + 1) * 2 + 1], h[j]);
        l[j] = udot8(e1, A[(2 * k + 1) * 2 + 0], l[j]);
    }
    i0 = h[0] * 16 + l[0];
    i1 = h[1] * 16 + l[1];
}

// Q1_0: 4 device sign dwords; mask 0x11111111 << r of each holds 8 weights of q8_0 block r at nibble
// value 2^r (read as -8 by the signed product when r = 3).  Returns C[r] = 2^r S_r, S_r = the sum of q
// over the weights of block r whose bit is 1; the block sum is 2 S_r - sum(q).
__device__ __forceinline__ void q1_group_sums(uint4 b, const uint32_t *A, int (&C)[4])
{
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
    // the eight accumulator chains advance together (dword by dword), so consecutive dot products are
    // independent
    int h[4], l[4];
#pragma unroll
    for (int m = 0; m < 4; m++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const uint32_t e = bw[m] & (0x11111111u << r);
            h[r] = m ? sdot8(e, A[(4 * m + r) * 2 + 1], h[r]) : sdot8z(e, A[(4 * m + r) * 2 + 1]);
            l[r] = udot8(e, A[(4 * m + r) * 2 + 0], m ? l[r] : 0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; r++)
        C[r] = r < 3 ? h[r] * 16 + l[r] : sub16(l[r], h[r]);
}

// Planar: plane words {pos0, pos1, neg0, neg1}.  Masking without a shift leaves bit r of a nibble in
// place, so nibble value = 2^r * bit; each r keeps its own accumulators and the row total is
// recombined exactly at the end (r = 3 reads as -8 in the signed product).
struct PlanarAcc {
    int ph[4], pl[4], nh[4], nl[4];
};

__device__ __forceinline__ void planar_accumulate(uint4 bt, const uint32_t *A, PlanarAcc &acc)
{
    const uint32_t pw[2] = {bt.x, bt.y}, nw[2] = {bt.z, bt.w};
#pragma unroll
    for (int k = 0; k < 2; k++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const uint32_t m = 0x11111111u << r;
            const uint32_t ep = pw[k] & m, en = nw[k] & m;
            acc.ph[r] = sdot8(ep, A[(4 * k + r) * 2 + 1], acc.ph[r]);
            acc.pl[r] = udot8(ep, A[(4 * k + r) * 2 + 0], acc.pl[r]);
            acc.nh[r] = sdot8(en, A[(4 * k + r) * 2 + 1], acc.nh[r]);
            acc.nl[r] = udot8(en, A[(4 * k + r) * 2 + 0], acc.nl[r]);
        }
    }
}

// 8 * (sum_pos q - sum_neg q) over what this lane accumulated.
__device__ __forceinline__ int planar_total8(const PlanarAcc &a)
{
    int t = 0;
#pragma unroll
    for (int r = 0; r < 3; r++)
        t += ((a.ph[r] - a.nh[r]) * 16 + (a.pl[r] - a.nl[r])) << (3 - r);
    t += -(a.ph[3] - a.nh[3]) * 16 + (a.pl[3] - a.nl[3]);
    return t;
}

// ------------------------------------------------------------------------------------------------
// One workgroup, one tile of rows [row0, row0 + nrows) of one product.
//
// Loads are unconditional: a lane past the tile's last row re-reads that row and a lane past the row's
// last slice re-reads that slice (its staged activations are zero, so it adds nothing and its result
// is never stored).  Offsets are 32-bit byte offsets from the tensor's base (the ABI keeps tensors
// under 4 GiB), advanced by one add per row and clamped by one min to the tile's last row, so every
// load stays inside the tensor.  A ring of NB register buffers keeps NB - 1 rows' loads in flight
// while a row is computed, and the first rows are requested before the activation is staged, so the
// weight stream never waits on the staging.
// ------------------------------------------------------------------------------------------------
template <int FMT, int S> struct RowRegs {
    uint4 code[S];
    uint32_t sc[S];
};

// Register buffers in the ring (rows in flight + 1).
constexpr int kRing = 2;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
// Tensors are in device global memory: loads through global-address-space pointers take a scalar base
// and a 32-bit per-lane offset (no 64-bit address arithmetic, no flat-address checks).
typedef __attribute__((address_space(1))) const v4u gv4u;
typedef __attribute__((address_space(1))) const uint16_t gu16;
typedef __attribute__((address_space(1))) const uint8_t gu8;
typedef __attribute__((address_space(1))) float gf32;

// One row's S slices.  off: byte offset of the row's first record; slo[i] / sls[i]: byte offset of
// this lane's i-th record / its scale within a row.  The code records are read exactly once:
// non-temporal loads keep the stream from displacing the activations and scales in the caches.
// FULL (a row has exactly L * S slices): slice i sits a constant L * 16 * i bytes after slice 0, which
// the loads take as an immediate offset.
template <int FMT, int L, int S, bool FULL>
__device__ __forceinline__ void issue_row(RowRegs<FMT, S> &r, const uint8_t *__restrict__ W,
                                          const uint8_t *__restrict__ scales, uint32_t off, const uint32_t (&slo)[S],
                                          const uint32_t (&sls)[S])
{
    const uint32_t soff = off >> 3; // record idx at byte 16 idx, its binary16 scale at byte 2 idx
    const gu8 *pc = (gu8 *)W + (off + slo[0]);
    const gu8 *ps = (gu8 *)scales + (soff + sls[0]);
#pragma unroll
    for (int i = 0; i < S; i++) {
        const v4u t = __builtin_nontemporal_load(
            (gv4u *)(FULL ? pc + i * L * CODE_BYTES : (gu8 *)W + (off + slo[i])));
        r.code[i] = make_uint4(t.x, t.y, t.z, t.w);
        if (FMT != LB_TERNARY_PLANAR) // small, shared by neighbouring lanes: left cacheable
            r.sc[i] = *(gu16 *)(FULL ? ps + i * L * 2 : (gu8 *)scales + (soff + sls[i]));
    }
}

// The row result of the product instantiations (no sums): every lane issues the store, and a lane that
// does not hold a stored result (not the row's last lane, or a row past the tile) addresses past the
// end of the tile's output range, where the buffer unit drops it.  No branch surrounds the store, so the
// compiler can count the loads still in flight exactly and waits only for the row it computes next.
__device__ __forceinline__ void store_row_result(__amdgpu_buffer_rsrc_t yt, bool keep, int rl, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yt, keep ? (uint32_t)rl * 4u : 0x80000000u, 0, 0);
}

template <int FMT, int L, int S, bool EMIT, bool FULL>
__device__ __forceinline__ void compute_row(const uint4 (&code)[S], const uint32_t (&sc)[S],
                                            const uint32_t (&act)[S][F<FMT>::REC], const float (&cfold)[S], int ns, int li,
                                            bool valid, int row, float w_scale, float sx, float *__restrict__ y,
                                            int32_t *__restrict__ sums, __amdgpu_buffer_rsrc_t yt, int rl)
{
    constexpr int NAB = F<FMT>::NAB, DX = F<FMT>::SW / 4;
    if (FMT == LB_TERNARY_PLANAR) {
        PlanarAcc acc = {};
#pragma unroll
        for (int i = 0; i < S; i++)
            planar_accumulate(code[i], act[i], acc);
        const int t = group_sum_i<L>(planar_total8(acc));
        const int a = t >> 3; // exact: the total is a multiple of 8
        // tritium "Architecture", section 5: activation scale and weight scale are applied as two fp32
        // multiplies, in that order
        const float ys = (float)a * sx;
        if constexpr (EMIT) {
            if (valid && li == L - 1) {
                sums[row] = a;
                if (y != nullptr) // the sums instantiation may be called without an output vector
                    y[row] = ys * w_scale;
            }
        } else {
            store_row_result(yt, valid && li == L - 1, rl, ys * w_scale);
        }
    } else {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < S; i++) {
            const int sl = li + i * L;
            float t;
            int is[NAB > 0 ? NAB : 1];
            if (FMT == LB_Q2_0_G64) {
                q2_isums(code[i], act[i], is[0], is[1]);
                // bankml report, section III.3: one multiply-add per q8_0 block, then one per weight block
                t = fmaf(__uint_as_float(act[i][DX + 1]), (float)is[1], __uint_as_float(act[i][DX]) * (float)is[0]);
            } else {
                // t = sum_j d_x[j] (2 S_j - sum q_j): the -sum_j d_x[j] sum q_j part is the slice constant
                // cfold (computed once per lane), then one multiply-add per q8_0 block of (2 d_x[j] / 2^j)
                // by 2^j S_j -- the same exact product 2 d_x[j] S_j
                int C[4];
                q1_group_sums(code[i], act[i], C);
                t = cfold[i];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    t = fmaf(__uint_as_float(act[i][DX + j]), (float)C[j], t);
                    is[j] = ((C[j] * 2) >> j) + (int)act[i][DX + NAB + j];
                }
            }
            const float c = fmaf(half_bits_to_float((uint16_t)sc[i]), t, part);
            part = (FULL || sl < ns) ? c : part;
            if (EMIT && valid && (FULL || sl < ns)) {
                int32_t *o = sums + (int64_t)row * (ns * NAB) + NAB * sl;
#pragma unroll
                for (int j = 0; j < NAB; j++)
                    o[j] = is[j];
            }
        }
        part = group_sum_f<L>(part);
        if constexpr (EMIT) {
            if (valid && li == L - 1 && y != nullptr)
                *(gf32 *)((gu8 *)y + (uint32_t)row * 4u) = part;
        } else {
            store_row_result(yt, valid && li == L - 1, rl, part);
        }
    }
}

template <int FMT, int L, int S, bool EMIT, bool FULL, bool QIN = false>
__device__ __forceinline__ void matvec_tile(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                            const int8_t *__restrict__ xq, const void *__restrict__ xscale,
                                            float *__restrict__ y, int32_t *__restrict__ sums, int row0, int nrows,
                                            uint32_t *__restrict__ lds, const float *__restrict__ x = nullptr)
{
    constexpr int REC = F<FMT>::REC;
    constexpr int GROUPS = 64 / L;           // rows per wave per iteration
    constexpr int STEP = GROUPS * (WG / 64); // rows per workgroup per iteration
    constexpr int NB = kRing;
    const int ns = K / F<FMT>::SW; // slices per row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, li = lane % L;
    const uint8_t *scales = W + (int64_t)N * ns * CODE_BYTES;
    const int rbase = wave * GROUPS + g; // this lane's row within an iteration

    const uint32_t rowbytes = (uint32_t)ns * CODE_BYTES;
    const uint32_t stepb = (uint32_t)STEP * rowbytes;
    const uint32_t last = (uint32_t)(row0 + nrows - 1) * rowbytes; // the tile's last row
    uint32_t slo[S], sls[S];
#pragma unroll
    for (int i = 0; i < S; i++) {
        // FULL: the row has exactly L * S slices (no lane past its end), so no clamp
        slo[i] = (uint32_t)(FULL ? li + i * L : min(li + i * L, ns - 1)) * CODE_BYTES;
        sls[i] = slo[i] >> 3;
    }
    // Offset of the row this lane requests next, before clamping.  Past the tile's end it may grow
    // (or wrap) freely: min(., last) keeps every load in bounds, and such rows are never stored.
    uint32_t onext = (uint32_t)(row0 + min(rbase, nrows - 1)) * rowbytes;

    RowRegs<FMT, S> buf[NB];
    // the first weight rows, requested once the activation's first loads are out (see stage_activation)
    auto first_rows = [&]() {
#pragma unroll
        for (int b = 0; b < NB - 1; b++) {
            issue_row<FMT, L, S, FULL>(buf[b], W, scales, min(onext, last), slo, sls);
            onext += stepb;
        }
    };

    if (QIN) {
        // fp32 activations (LB_ACT_F32_Q8_0): quantised to q8_0 into LDS past the staged records with the
        // arithmetic of the quantise kernel, then staged from there like quantised ones.  K / 4 float4
        // chunks, eight per block; WG is a multiple of 8, so a block's eight lanes are all in range or all
        // out.  A thread's first QPRE chunks (K up to 12288) are loaded before the first weight rows.
        int8_t *qb = reinterpret_cast<int8_t *>(lds + ns * REC);
        uint16_t *qs = reinterpret_cast<uint16_t *>(qb + K);
        constexpr int QPRE = 12, QU = 4;
        const int nc = K / 4;
        const int npre = min((nc + WG - 1) / WG, QPRE); // uniform
        auto ldx = [&](int c) {
            const sv4f t = ((src_t<1, sv4f> *)x)[min(c, nc - 1)];
            return make_float4(t.x, t.y, t.z, t.w);
        };
        auto quant = [&](float4 v, int c) {
            const float amax = q8_0_block_amax8(v);
            if (c < nc) {
                reinterpret_cast<uint32_t *>(qb)[c] = q8_0_pack4(v, amax);
                if ((c & 7) == 0)
                    qs[c >> 3] = q8_0_scale_bits(amax);
            }
        };
        float4 v[QPRE];
#pragma unroll
        for (int u = 0; u < QPRE; u++)
            if (u < npre)
                v[u] = ldx(threadIdx.x + u * WG);
        first_rows();
#pragma unroll
        for (int u = 0; u < QPRE; u++)
            if (u < npre)
                quant(v[u], threadIdx.x + u * WG);
        for (int c0 = threadIdx.x + QPRE * WG; c0 < nc; c0 += QU * WG) {
            float4 w[QU];
#pragma unroll
            for (int u = 0; u < QU; u++)
                w[u] = ldx(c0 + u * WG);
#pragma unroll
            for (int u = 0; u < QU; u++)
                quant(w[u], c0 + u * WG);
        }
        __syncthreads();
        stage_activation<FMT, 3>(qb, qs, ns, lds, [] {});
    } else {
        stage_activation<FMT, 1>(xq, xscale, ns, lds, first_rows);
    }
    __syncthreads();

    uint32_t act[S][REC];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int sl = li + i * L;
        if (FULL || sl < ns) {
            const uint4 *p = reinterpret_cast<const uint4 *>(lds + sl * REC);
#pragma unroll
            for (int q = 0; q < REC / 4; q++) {
                const uint4 t = p[q];
                act[i][4 * q + 0] = t.x;
                act[i][4 * q + 1] = t.y;
                act[i][4 * q + 2] = t.z;
                act[i][4 * q + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < REC; q++)
                act[i][q] = 0;
        }
    }
    const float sx = FMT == LB_TERNARY_PLANAR ? *reinterpret_cast<const float *>(xscale) : 0.0f;
    float cfold[S]; // Q1_0: -sum_j d_x[j] sum(q_j) of each slice (the staged words hold 2 d_x[j] / 2^j, -sum(q_j))
#pragma unroll
    for (int i = 0; i < S; i++) {
        float c = 0.0f;
        if (FMT == LB_Q1_0) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float back = j == 0 ? 0.5f : j == 1 ? 1.0f : j == 2 ? 2.0f : 4.0f; // exact
                c = fmaf(back * __uint_as_float(act[i][32 + j]), (float)(int)act[i][36 + j], c);
            }
        }
        cfold[i] = c;
    }

    // the tile's outputs y[row0, row0 + nrows) as a buffer range (the sums instantiation may run without y)
    const __amdgpu_buffer_rsrc_t yt =
        __builtin_amdgcn_make_buffer_rsrc(EMIT ? nullptr : y + row0, 0, EMIT ? 0 : nrows * 4, 0x00020000);
    // A tile of at most NB - 1 passes has all its rows' loads in flight already (the first passes were
    // requested before the staging): compute exactly its passes, no ring.  Such tiles are what a small
    // batch (one dependency phase of a token, fp32 inputs) is cut into; the instantiations for quantised
    // inputs leave the path out (a second copy of the row arithmetic costs them registers).
    if (QIN && nrows <= (NB - 1) * STEP) { // uniform
#pragma unroll
        for (int b = 0; b < NB - 1; b++) {
            const int rl = b * STEP + rbase;
            if (b == 0 || b * STEP < nrows) // uniform
                compute_row<FMT, L, S, EMIT, FULL>(buf[b].code, buf[b].sc, act, cfold, ns, li, rl < nrows, row0 + rl,
                                                   w_scale, sx, y, sums, yt, rl);
        }
        return;
    }
    for (int it = 0; it < nrows; it += NB * STEP) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            // No branch inside the ring: a row past the tile's end is computed from the clamped loads
            // and never stored.  With a branch here the compiler would sink each half's loads into the
            // half that uses them, after this row's arithmetic, and that half would wait for loads only
            // just issued.
            const int cur = it + b * STEP;
            issue_row<FMT, L, S, FULL>(buf[(b + NB - 1) % NB], W, scales, min(onext, last), slo, sls);
            __builtin_amdgcn_sched_barrier(0); // the next row's loads go out before this row's arithmetic
            onext += stepb;
            const int rl = cur + rbase;
            compute_row<FMT, L, S, EMIT, FULL>(buf[b].code, buf[b].sc, act, cfold, ns, li, rl < nrows, row0 + rl, w_scale,
                                               sx, y, sums, yt, rl);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Configurations (L lanes per row, S slices per lane), each compiled as its own kernel; the staged
// activations of a lane (S * REC dwords) must fit a budget of 160 registers.
// ------------------------------------------------------------------------------------------------
#define LB_CFGS(X)                                                                                            \
    X(0, 1, 1) X(1, 1, 2) X(2, 2, 2) X(3, 4, 1) X(4, 4, 2) X(5, 4, 4) X(6, 8, 2) X(7, 8, 4) X(8, 8, 5)        \
    X(9, 16, 1) X(10, 16, 2) X(11, 16, 4) X(12, 32, 2) X(13, 32, 3) X(14, 32, 4) X(15, 64, 2) X(16, 64, 3)    \
    X(17, 64, 4) X(18, 64, 8) X(19, 32, 1) X(20, 64, 1) X(21, 8, 8) X(22, 16, 3) X(23, 32, 6) X(24, 16, 7)

struct CfgLS {
    int L, S;
};
#define LB_CFG_ENTRY(i, l, s) {l, s},
static constexpr CfgLS kCfgs[] = {LB_CFGS(LB_CFG_ENTRY)};
#undef LB_CFG_ENTRY
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

constexpr int rec_of(int fmt) { return fmt == LB_Q1_0 ? F<LB_Q1_0>::REC : fmt == LB_Q2_0_G64 ? F<LB_Q2_0_G64>::REC
                                                                                            : F<LB_TERNARY_PLANAR>::REC; }
constexpr int sw_of(int fmt) { return fmt == LB_Q1_0 ? 128 : 64; }
constexpr bool cfg_allowed(int fmt, int S) { return S * rec_of(fmt) <= 160; }

// Choice (measured on the 8B- and 2B-shape products): fewest idle lane slots; among equals, a light
// register footprint (at most 80 staged dwords per lane, which keeps 3-4 waves per SIMD) before a
// heavy one; then fewer lanes per row (a shorter cross-lane reduction per row).
static int pick_cfg(int fmt, int64_t ns)
{
    int best = -1;
    int64_t best_waste = 0;
    bool best_light = false;
    for (int c = 0; c < kNumCfgs; c++) {
        if (!cfg_allowed(fmt, kCfgs[c].S))
            continue;
        const int64_t slots = (int64_t)kCfgs[c].L * kCfgs[c].S;
        if (slots < ns)
            continue;
        const int64_t waste = slots - ns;
        const bool light = kCfgs[c].S * rec_of(fmt) <= 80;
        const bool better = best < 0 || waste < best_waste ||
                            (waste == best_waste && light && !best_light) ||
                            (waste == best_waste && light == best_light && kCfgs[c].L < kCfgs[best].L);
        if (better) {
            best = c;
            best_waste = waste;
            best_light = light;
        }
    }
    return best;
}

int matvec_config(int fmt, int64_t K)
{
    if (fmt == LB_Q8_0)
        return q8_config(K);
    if (fmt == LB_TERNARY_B3)
        return b3_config(K);
    if (K <= 0 || K % sw_of(fmt))
        return -1;
    return pick_cfg(fmt, K / sw_of(fmt));
}

bool matvec_supported_k(int fmt, int64_t K) { return matvec_config(fmt, K) >= 0; }

bool matvec_config_full(int fmt, int cfg, int64_t K)
{
    if (fmt == LB_Q8_0 || fmt == LB_TERNARY_B3)
        return true; // one kernel per configuration; idle lanes are clamped inside it
    return (int64_t)kCfgs[cfg].L * kCfgs[cfg].S == K / sw_of(fmt);
}

int matvec_config_rows_per_iter(int fmt, int cfg)
{
    if (fmt == LB_Q8_0)
        return q8_rows_per_iter(cfg);
    if (fmt == LB_TERNARY_B3)
        return b3_rows_per_iter(cfg);
    return (64 / kCfgs[cfg].L) * (WG / 64);
}

int matvec_stage_bytes(int fmt, int64_t K)
{
    if (fmt == LB_Q8_0)
        return (int)q8_stage_bytes(K);
    if (fmt == LB_TERNARY_B3)
        return (int)b3_stage_bytes(K);
    return (int)((K / sw_of(fmt)) * rec_of(fmt) * 4);
}

template <int FMT, int L, int S, bool EMIT>
__global__ __launch_bounds__(WG) void matvec_kernel(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                                    const int8_t *__restrict__ xq, const void *__restrict__ xscale,
                                                    float *__restrict__ y, int32_t *__restrict__ sums, int tile_rows)
{
    extern __shared__ uint32_t lds[];
    const int row0 = blockIdx.x * tile_rows;
    const int nrows = min(tile_rows, N - row0);
    matvec_tile<FMT, L, S, EMIT, false>(W, N, K, w_scale, xq, xscale, y, sums, row0, nrows, lds);
}

template <int FMT, bool EMIT>
static hipError_t launch_single(int cfg, const uint8_t *W, int N, int K, float w_scale, const int8_t *xq,
                                const void *xscale, float *y, int32_t *sums, int tile_rows, hipStream_t stream)
{
    const int ntiles = (N + tile_rows - 1) / tile_rows;
    const size_t lds = (size_t)matvec_stage_bytes(FMT, K);
    switch (cfg) {
#define LB_CASE(i, l, s)                                                                                      \
    case i:                                                                                                   \
        if constexpr (cfg_allowed(FMT, s))                                                                    \
            hipLaunchKernelGGL((matvec_kernel<FMT, l, s, EMIT>), dim3(ntiles), dim3(WG), lds, stream, W, N, K,   \
                               w_scale, xq, xscale, y, sums, tile_rows);                                       \
        break;
        LB_CFGS(LB_CASE)
#undef LB_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_matvec(int fmt, const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *xq,
                         const void *xscale, float *y, int32_t *sums, hipStream_t s)
{
    if (fmt == LB_Q8_0)
        return launch_q8(W, N, K, xq, static_cast<const uint16_t *>(xscale), y, sums, s);
    if (fmt == LB_TERNARY_B3)
        return launch_b3(W, N, K, w_scale, xq, static_cast<const float *>(xscale), y, sums, s);
    const int cfg = matvec_config(fmt, K);
    if (cfg < 0)
        return hipErrorInvalidValue;
    // enough workgroups to cover the device when the product allows it, whole iterations per tile
    const int rpi = matvec_config_rows_per_iter(fmt, cfg);
    int64_t tile = (N + 1023) / 1024;
    tile = ((tile + rpi - 1) / rpi) * rpi;
    if (tile < rpi)
        tile = rpi;
    if (tile > 32 * rpi)
        tile = 32 * rpi;
    const bool emit = sums != nullptr;
    const int n = (int)N, k = (int)K, t = (int)tile;
    switch (fmt) {
    case LB_Q1_0:
        return emit ? launch_single<LB_Q1_0, true>(cfg, W, n, k, w_scale, xq, xscale, y, sums, t, s)
                    : launch_single<LB_Q1_0, false>(cfg, W, n, k, w_scale, xq, xscale, y, sums, t, s);
    case LB_Q2_0_G64:
        return emit ? launch_single<LB_Q2_0_G64, true>(cfg, W, n, k, w_scale, xq, xscale, y, sums, t, s)
                    : launch_single<LB_Q2_0_G64, false>(cfg, W, n, k, w_scale, xq, xscale, y, sums, t, s);
    case LB_TERNARY_PLANAR:
        return emit ? launch_single<LB_TERNARY_PLANAR, true>(cfg, W, n, k, w_scale, xq, xscale, y, sums, t, s)
                    : launch_single<LB_TERNARY_PLANAR, false>(cfg, W, n, k, w_scale, xq, xscale, y, sums, t, s);
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------------
// Batched: one launch per (format, configuration) group of a work list.  Each workgroup looks up its
// product (a uniform, scalar-cached read); every instantiation is compiled for one configuration, so
// each gets the registers it needs and no more.
// ------------------------------------------------------------------------------------------------
template <int FMT, int L, int S, bool FULL, bool QIN>
__global__ __launch_bounds__(WG) void matvec_batched_kernel(const DevDesc *__restrict__ desc,
                                                            const TileRef *__restrict__ tiles)
{
    extern __shared__ uint32_t lds[];
    const TileRef tr = tiles[blockIdx.x];
    const DevDesc d = desc[tr.prod];
    const int row0 = tr.row0;
    const int nrows = min(d.tile_rows, d.N - row0);
    matvec_tile<FMT, L, S, false, FULL, QIN>(d.W, d.N, d.K, d.w_scale, d.xq, d.xscale, d.y, nullptr, row0, nrows, lds,
                                             d.x);
}

// fp32 activations quantised in the launch: the ggml formats (q8_0 activations) only
constexpr bool qin_allowed(int fmt) { return fmt == LB_Q1_0 || fmt == LB_Q2_0_G64; }

template <int FMT>
static hipError_t launch_batched_fmt(const BatchGroup &g, hipStream_t stream, size_t lds_bytes)
{
    switch (g.cfg_a) {
#define LB_BCASE(i, l, s)                                                                                     \
    case i:                                                                                                   \
        if constexpr (cfg_allowed(FMT, s)) {                                                                  \
            if (g.qin) {                                                                                      \
                if constexpr (qin_allowed(FMT)) {                                                             \
                    if (g.full)                                                                               \
                        hipLaunchKernelGGL((matvec_batched_kernel<FMT, l, s, true, true>), dim3(g.ntiles),    \
                                           dim3(WG), lds_bytes, stream, g.desc, g.tiles);                     \
                    else                                                                                      \
                        hipLaunchKernelGGL((matvec_batched_kernel<FMT, l, s, false, true>), dim3(g.ntiles),   \
                                           dim3(WG), lds_bytes, stream, g.desc, g.tiles);                     \
                } else {                                                                                      \
                    return hipErrorInvalidValue;                                                              \
                }                                                                                             \
            } else if (g.full) {                                                                              \
                hipLaunchKernelGGL((matvec_batched_kernel<FMT, l, s, true, false>), dim3(g.ntiles), dim3(WG),    \
                                   lds_bytes, stream, g.desc, g.tiles);                                       \
            } else {                                                                                          \
                hipLaunchKernelGGL((matvec_batched_kernel<FMT, l, s, false, false>), dim3(g.ntiles), dim3(WG),   \
                                   lds_bytes, stream, g.desc, g.tiles);                                       \
            }                                                                                                 \
        }                                                                                                     \
        break;
        LB_CFGS(LB_BCASE)
#undef LB_BCASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int FMT> static int blocks_per_cu_fmt(int cfg, bool full, bool qin, size_t lds_bytes)
{
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (cfg) {
#define LB_OCASE(i, l, s)                                                                                     \
    case i:                                                                                                   \
        if constexpr (cfg_allowed(FMT, s)) {                                                                  \
            if (qin) {                                                                                        \
                if constexpr (qin_allowed(FMT))                                                               \
                    e = full ? hipOccupancyMaxActiveBlocksPerMultiprocessor(                                  \
                                   &n, matvec_batched_kernel<FMT, l, s, true, true>, WG, lds_bytes)           \
                             : hipOccupancyMaxActiveBlocksPerMultiprocessor(                                  \
                                   &n, matvec_batched_kernel<FMT, l, s, false, true>, WG, lds_bytes);         \
            } else {                                                                                          \
                e = full ? hipOccupancyMaxActiveBlocksPerMultiprocessor(                                      \
                               &n, matvec_batched_kernel<FMT, l, s, true, false>, WG, lds_bytes)              \
                         : hipOccupancyMaxActiveBlocksPerMultiprocessor(                                      \
                               &n, matvec_batched_kernel<FMT, l, s, false, false>, WG, lds_bytes);            \
            }                                                                                                 \
        }                                                                                                     \
        break;
        LB_CFGS(LB_OCASE)
#undef LB_OCASE
    default:
        break;
    }
    return e == hipSuccess && n > 0 ? n : 1;
}

int matvec_batched_blocks_per_cu(int fmt, int cfg, bool full, bool qin, size_t lds_bytes)
{
    switch (fmt) {
    case LB_Q1_0:
        return blocks_per_cu_fmt<LB_Q1_0>(cfg, full, qin, lds_bytes);
    case LB_Q2_0_G64:
        return blocks_per_cu_fmt<LB_Q2_0_G64>(cfg, full, qin, lds_bytes);
    case LB_TERNARY_PLANAR:
        return blocks_per_cu_fmt<LB_TERNARY_PLANAR>(cfg, full, false, lds_bytes);
    case LB_Q8_0:
        return q8_blocks_per_cu(cfg, lds_bytes);
    case LB_TERNARY_B3:
        return b3_blocks_per_cu(cfg, lds_bytes);
    }
    return 1;
}

hipError_t launch_matvec_batched(const BatchGroup &g, hipStream_t s, size_t lds_bytes)
{
    switch (g.fmt) {
    case LB_Q1_0:
        return launch_batched_fmt<LB_Q1_0>(g, s, lds_bytes);
    case LB_Q2_0_G64:
        return launch_batched_fmt<LB_Q2_0_G64>(g, s, lds_bytes);
    case LB_TERNARY_PLANAR:
        return launch_batched_fmt<LB_TERNARY_PLANAR>(g, s, lds_bytes);
    case LB_Q8_0:
        return launch_q8_batched(g, lds_bytes, s);
    case LB_TERNARY_B3:
        return launch_b3_batched(g, lds_bytes, s);
    }
    return hipErrorInvalidValue;
}

} // namespace lb
