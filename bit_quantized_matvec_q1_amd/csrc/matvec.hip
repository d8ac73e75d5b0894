// Batch-1 decode products for the three packed formats (Q1_0, Q2_0_g64, planar ternary) on gfx950.
//
// Arithmetic (bankml technical report, section III.8 "Operation"; tritium "Architecture", sections 1-2):
// every weight is a small integer, so each row's sum over a 32-activation block is an exact integer
// select-accumulate, and only the block scales are floating point.
//
// Mapping to CDNA4:
//  * The unit of work is a "slice" of 64 consecutive weights of one row: one Q2_0_g64 code record
//    (16 B), half a Q1_0 block's sign bits (8 B), or one planar beat (16 B).  A slice meets exactly two
//    q8_0 activation blocks.
//  * A workgroup owns a tile of rows of one product.  It first stages the activation vector into LDS,
//    once, in the order the unpack needs (the activation, not the weights, is rearranged -- the bankml
//    report's ternary kernel does the same once per token).  Each int8 activation q is split into a
//    signed high nibble h = q >> 4 and an unsigned low nibble l = q & 15 (q = 16h + l), packed eight to
//    a dword in the order in which a shift-and-mask of a code word lays the weights out.
//  * A row is split over L lanes; a lane owns S slices (strided by L so each wave-wide 16-byte load is
//    contiguous) and keeps their staged activations in VGPRs across all the rows it streams.
//  * Per code dword, one mask (and at most one shift) isolates 8 codes or 8 sign bits as nibbles, and
//    one v_dot8_i32_i4 against the h nibbles plus one v_dot8_u32_u4 against the l nibbles accumulate
//    sum(code * q) = 16 * sum(code * h) + sum(code * l).  The offset forms of the pages give the exact
//    block sums: Q2_0  isum = sum(c q) - sum(q)  (code c = w + 1);  Q1_0  isum = 2 sum_{bit=1} q - sum(q);
//    planar  acc = sum_pos q - sum_neg q.
//  * Block scaling is one fp32 multiply-add per activation block and one per weight block (bankml
//    report, section III.3), then a cross-lane tree over the L lanes of the row.  Rows are never split
//    across workgroups, so results do not depend on the launch geometry (tritium "Architecture",
//    section 7: split rows, never a reduction).
#include "lowbit_internal.h"

namespace lb {

template <int FMT> struct F;
// REC: dwords of staged activation per slice: 16 nibble words, then (ggml formats) dx[2] and sum(q)[2]
template <> struct F<LB_Q2_0_G64> { enum { REC = 20, CODE_BYTES = 16 }; };
template <> struct F<LB_Q1_0> { enum { REC = 20, CODE_BYTES = 8 }; };
template <> struct F<LB_TERNARY_PLANAR> { enum { REC = 16, CODE_BYTES = 16 }; };

constexpr int SLICE = 64; // weights per slice

// ------------------------------------------------------------------------------------------------
// Activation staging.  Nibble word (a, b) holds, at bits 4n..4n+3, the low (b = 0) or high (b = 1)
// nibble of activation e(a, n) of the slice, where e() is the position of the n-th code that the
// a-th mask extraction isolates:
//   Q2_0  a = 2k + s   (code dword k = weights 16k..16k+15; s = 0: mask 0x33333333, s = 1: shift 2
//                       first):  e = 16k + 2n + s
//   Q1_0 / planar  a = 4k + r  (32-bit word k of signs / plane bits; r = the bit within each nibble):
//                       e = 32k + 4n + r
// ------------------------------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ void stage_slice(const int8_t *__restrict__ xq, const void *__restrict__ xscale, int sl,
                                            uint32_t *__restrict__ rec)
{
    const uint4 *src = reinterpret_cast<const uint4 *>(xq + (int64_t)sl * SLICE);
    uint32_t wb[SLICE / 4];
#pragma unroll
    for (int i = 0; i < SLICE / 16; i++) {
        const uint4 t = src[i];
        wb[4 * i + 0] = t.x;
        wb[4 * i + 1] = t.y;
        wb[4 * i + 2] = t.z;
        wb[4 * i + 3] = t.w;
    }
#define LB_BYTE(i) ((wb[(i) >> 2] >> (8 * ((i)&3))) & 0xffu)
#pragma unroll
    for (int a = 0; a < 8; a++) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int n = 0; n < 8; n++) {
            const int e = FMT == LB_Q2_0_G64 ? 16 * (a >> 1) + 2 * n + (a & 1) : 32 * (a >> 2) + 4 * n + (a & 3);
            const uint32_t v = LB_BYTE(e);
            lo |= (v & 15u) << (4 * n);
            hi |= (v >> 4) << (4 * n);
        }
        rec[2 * a + 0] = lo;
        rec[2 * a + 1] = hi;
    }
    if (FMT != LB_TERNARY_PLANAR) {
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(xscale);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            rec[16 + j] = __float_as_uint(half_bits_to_float(xs[2 * sl + j]));
            int sq = 0;
#pragma unroll
            for (int i = 0; i < 32; i++)
                sq += (int)(int8_t)LB_BYTE(32 * j + i);
            rec[18 + j] = (uint32_t)sq;
        }
    }
#undef LB_BYTE
}

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
__device__ __forceinline__ int udot8(uint32_t a, uint32_t b, int c)
{
    return (int)__builtin_amdgcn_udot8(a, b, (uint32_t)c, false);
}

// ------------------------------------------------------------------------------------------------
// Per-slice arithmetic.  Q formats return the slice's scaled contribution and (EMIT) its two exact
// block sums; planar accumulates its 16 integer partials.
// ------------------------------------------------------------------------------------------------

// Q2_0_g64: 4 code dwords, 16 2-bit codes each.
__device__ __forceinline__ void q2_isums(uint4 c, const uint32_t *A, int &i0, int &i1)
{
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    int h[2] = {0, 0}, l[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t e0 = cw[k] & 0x33333333u;
        const uint32_t e1 = (cw[k] >> 2) & 0x33333333u;
        const int j = k >> 1;
        h[j] = sdot8(e0, A[(2 * k + 0) * 2 + 1], h[j]);
        l[j] = udot8(e0, A[(2 * k + 0) * 2 + 0], l[j]);
        h[j] = sdot8(e1, A[(2 * k + 1) * 2 + 1], h[j]);
        l[j] = udot8(e1, A[(2 * k + 1) * 2 + 0], l[j]);
    }
    i0 = h[0] * 16 + l[0] - (int)A[18];
    i1 = h[1] * 16 + l[1] - (int)A[19];
}

// Q1_0 (half a block): 2 sign dwords, 32 bits each; bit r of nibble n is weight 4n + r.
__device__ __forceinline__ void q1_isums(uint2 b, const uint32_t *A, int &i0, int &i1)
{
    const uint32_t bw[2] = {b.x, b.y};
    int s[2];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        int h = 0, l = 0;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const uint32_t e = (bw[k] >> r) & 0x11111111u;
            h = sdot8(e, A[(4 * k + r) * 2 + 1], h);
            l = udot8(e, A[(4 * k + r) * 2 + 0], l);
        }
        s[k] = h * 16 + l; // sum of q where the sign bit is 1
    }
    i0 = 2 * s[0] - (int)A[18];
    i1 = 2 * s[1] - (int)A[19];
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
// Cross-lane sum over aligned groups of L lanes with DPP (no LDS round trip).  The total ends up in the
// group's last lane (li == L - 1); for L <= 16 every lane of the group holds it.
// ------------------------------------------------------------------------------------------------
template <int L> __device__ __forceinline__ int group_sum_i(int v)
{
    if (L >= 2)
        v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); // quad_perm [1,0,3,2]
    if (L >= 4)
        v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); // quad_perm [2,3,0,1]
    if (L >= 8)
        v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); // row_half_mirror
    if (L >= 16)
        v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // row_mirror
    if (L >= 32)
        v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
    if (L >= 64)
        v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
    return v;
}

template <int L> __device__ __forceinline__ float group_sum_f(float v)
{
    if (L >= 2)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if (L >= 4)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if (L >= 8)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if (L >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    if (L >= 32)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    if (L >= 64)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

// ------------------------------------------------------------------------------------------------
// One workgroup, one tile of rows [row0, row0 + nrows) of one product.
//
// Loads are unconditional: a lane past the tile's last row re-reads that row and a lane past the row's
// last slice re-reads that slice (its staged activations are zero, so it adds nothing and its result
// is never stored).  Offsets are 32-bit from the tensor's base (the ABI keeps tensors under 4 GiB).
// The next rows' loads are issued before the current rows are computed (ping-pong registers), and the
// first rows' loads before the activation is staged, so the weight stream never waits on the staging.
// ------------------------------------------------------------------------------------------------
template <int FMT, int L, int S> struct RowRegs {
    uint4 code[S];
    uint32_t sc[S];
};

template <int FMT, int L, int S>
__device__ __forceinline__ void issue_row(RowRegs<FMT, L, S> &r, const uint8_t *__restrict__ W,
                                          const uint16_t *__restrict__ scales, uint32_t row, int ns, int li)
{
    constexpr int CB = F<FMT>::CODE_BYTES;
    const uint32_t nsr = FMT == LB_Q1_0 ? (uint32_t)ns / 2 : (uint32_t)ns;
#pragma unroll
    for (int i = 0; i < S; i++) {
        const uint32_t sl = (uint32_t)min(li + i * L, ns - 1);
        const uint32_t off = (row * (uint32_t)ns + sl) * CB;
        if (CB == 16) {
            r.code[i] = *reinterpret_cast<const uint4 *>(W + off);
        } else {
            const uint2 t = *reinterpret_cast<const uint2 *>(W + off);
            r.code[i] = make_uint4(t.x, t.y, 0, 0);
        }
        if (FMT != LB_TERNARY_PLANAR)
            r.sc[i] = scales[row * nsr + (FMT == LB_Q1_0 ? sl >> 1 : sl)];
    }
}

template <int FMT, int L, int S, bool EMIT>
__device__ __forceinline__ void compute_row(const RowRegs<FMT, L, S> &r, const uint32_t (&act)[S][F<FMT>::REC],
                                            int ns, int li, bool valid, int row, float w_scale, float sx,
                                            float *__restrict__ y, int32_t *__restrict__ sums)
{
    if (FMT == LB_TERNARY_PLANAR) {
        PlanarAcc acc = {};
#pragma unroll
        for (int i = 0; i < S; i++)
            planar_accumulate(r.code[i], act[i], acc);
        const int t = group_sum_i<L>(planar_total8(acc));
        if (valid && li == L - 1) {
            const int a = t >> 3; // exact: the total is a multiple of 8
            if (EMIT)
                sums[row] = a;
            // tritium "Architecture", section 5: activation scale and weight scale are applied as two
            // fp32 multiplies, in that order
            const float ys = (float)a * sx;
            if (!EMIT || y != nullptr) // the sums instantiation may be called without an output vector
                y[row] = ys * w_scale;
        }
    } else {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < S; i++) {
            const int sl = li + i * L;
            int i0, i1;
            if (FMT == LB_Q2_0_G64)
                q2_isums(r.code[i], act[i], i0, i1);
            else
                q1_isums(make_uint2(r.code[i].x, r.code[i].y), act[i], i0, i1);
            const float dx0 = __uint_as_float(act[i][16]), dx1 = __uint_as_float(act[i][17]);
            const float t = fmaf(dx1, (float)i1, dx0 * (float)i0);
            const float c = fmaf(half_bits_to_float((uint16_t)r.sc[i]), t, part);
            part = sl < ns ? c : part;
            if (EMIT && valid && sl < ns) {
                int32_t *o = sums + (int64_t)row * (ns * 2) + 2 * sl;
                o[0] = i0;
                o[1] = i1;
            }
        }
        part = group_sum_f<L>(part);
        if (valid && li == L - 1 && (!EMIT || y != nullptr))
            y[row] = part;
    }
}

template <int FMT, int L, int S, bool EMIT>
__device__ __forceinline__ void matvec_tile(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                            const int8_t *__restrict__ xq, const void *__restrict__ xscale,
                                            float *__restrict__ y, int32_t *__restrict__ sums, int row0, int nrows,
                                            uint32_t *__restrict__ lds)
{
    constexpr int REC = F<FMT>::REC;
    constexpr int CB = F<FMT>::CODE_BYTES;
    constexpr int GROUPS = 64 / L;              // rows per wave per iteration
    constexpr int ROWS_IT = GROUPS * (WG / 64); // rows per workgroup per iteration
    const int ns = K / SLICE;                   // slices per row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, li = lane % L;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(W + (int64_t)N * ns * CB);
    const int rbase = wave * GROUPS + g; // this lane's row within an iteration

    auto row_at = [&](int it) -> uint32_t { return (uint32_t)(row0 + min(it + rbase, nrows - 1)); };

    RowRegs<FMT, L, S> ra, rb;
    issue_row<FMT, L, S>(ra, W, scales, row_at(0), ns, li);

    for (int sl = threadIdx.x; sl < ns; sl += WG)
        stage_slice<FMT>(xq, xscale, sl, lds + sl * REC);
    __syncthreads();

    uint32_t act[S][REC];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int sl = li + i * L;
        if (sl < ns) {
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

    for (int it = 0; it < nrows; it += 2 * ROWS_IT) {
        const bool more1 = it + ROWS_IT < nrows; // uniform across the workgroup
        if (more1)
            issue_row<FMT, L, S>(rb, W, scales, row_at(it + ROWS_IT), ns, li);
        compute_row<FMT, L, S, EMIT>(ra, act, ns, li, it + rbase < nrows, row0 + it + rbase, w_scale, sx, y, sums);
        if (!more1)
            break;
        if (it + 2 * ROWS_IT < nrows)
            issue_row<FMT, L, S>(ra, W, scales, row_at(it + 2 * ROWS_IT), ns, li);
        compute_row<FMT, L, S, EMIT>(rb, act, ns, li, it + ROWS_IT + rbase < nrows, row0 + it + ROWS_IT + rbase,
                                     w_scale, sx, y, sums);
    }
}

// ------------------------------------------------------------------------------------------------
// Configurations (L lanes per row, S slices per lane).  The host picks, per product, the entry that
// wastes the fewest lane slots for K/64 slices, then the one with fewer lanes per row.
// ------------------------------------------------------------------------------------------------
#define LB_CFGS(X)                                                                                            \
    X(0, 1, 1) X(1, 1, 2) X(2, 2, 2) X(3, 4, 1) X(4, 4, 2) X(5, 4, 4) X(6, 8, 2) X(7, 8, 4) X(8, 8, 5)        \
    X(9, 16, 1) X(10, 16, 2) X(11, 16, 4) X(12, 32, 2) X(13, 32, 4) X(14, 64, 2) X(15, 64, 3) X(16, 64, 4)    \
    X(17, 64, 8)

struct CfgLS {
    int L, S;
};
#define LB_CFG_ENTRY(i, l, s) {l, s},
static const CfgLS kCfgs[] = {LB_CFGS(LB_CFG_ENTRY)};
#undef LB_CFG_ENTRY
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr int kBigCfg = 17; // the only entry kept out of the batched kernel (160 VGPRs of activations)

static int pick_cfg(int64_t ns, bool batched)
{
    int best = -1;
    int64_t best_waste = 0;
    for (int c = 0; c < kNumCfgs; c++) {
        if (batched && c == kBigCfg)
            continue;
        const int64_t slots = (int64_t)kCfgs[c].L * kCfgs[c].S;
        if (slots < ns)
            continue;
        const int64_t waste = slots - ns;
        if (best < 0 || waste < best_waste || (waste == best_waste && kCfgs[c].L < kCfgs[best].L)) {
            best = c;
            best_waste = waste;
        }
    }
    return best;
}

int matvec_config(int fmt, int64_t K)
{
    (void)fmt;
    if (K <= 0 || K % SLICE)
        return -1;
    return pick_cfg(K / SLICE, true);
}

bool matvec_supported_k(int fmt, int64_t K)
{
    (void)fmt;
    return K > 0 && K % SLICE == 0 && pick_cfg(K / SLICE, false) >= 0;
}

int matvec_config_rows_per_iter(int fmt, int cfg)
{
    (void)fmt;
    return (64 / kCfgs[cfg].L) * (WG / 64);
}

template <int FMT, int L, int S, bool EMIT>
__global__ __launch_bounds__(WG) void matvec_kernel(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                                    const int8_t *__restrict__ xq, const void *__restrict__ xscale,
                                                    float *__restrict__ y, int32_t *__restrict__ sums, int tile_rows)
{
    extern __shared__ uint32_t lds[];
    const int row0 = blockIdx.x * tile_rows;
    const int nrows = min(tile_rows, N - row0);
    matvec_tile<FMT, L, S, EMIT>(W, N, K, w_scale, xq, xscale, y, sums, row0, nrows, lds);
}

template <int FMT, bool EMIT>
static hipError_t launch_single(int cfg, const uint8_t *W, int N, int K, float w_scale, const int8_t *xq,
                                const void *xscale, float *y, int32_t *sums, int tile_rows, hipStream_t stream)
{
    const int ntiles = (N + tile_rows - 1) / tile_rows;
    const size_t lds = (size_t)(K / SLICE) * F<FMT>::REC * 4;
    switch (cfg) {
#define LB_CASE(i, l, s)                                                                                      \
    case i:                                                                                                   \
        hipLaunchKernelGGL((matvec_kernel<FMT, l, s, EMIT>), dim3(ntiles), dim3(WG), lds, stream, W, N, K,       \
                           w_scale, xq, xscale, y, sums, tile_rows);                                           \
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
    const int cfg = pick_cfg(K / SLICE, false);
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
// Batched: one launch over a device table of products of one format.  Each workgroup looks up its
// product (a uniform, scalar-cached read) and runs the configuration the host chose for it.
// ------------------------------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(WG) void matvec_batched_kernel(const DevDesc *__restrict__ desc,
                                                            const int32_t *__restrict__ tile_prod)
{
    extern __shared__ uint32_t lds[];
    const int t = blockIdx.x;
    const DevDesc d = desc[tile_prod[t]];
    const int row0 = (t - d.tile_begin) * d.tile_rows;
    const int nrows = min(d.tile_rows, d.N - row0);
    switch (d.cfg) {
#define LB_BCASE(i, l, s)                                                                                     \
    case i:                                                                                                   \
        if (i != kBigCfg)                                                                                     \
            matvec_tile<FMT, l, (i == kBigCfg ? 1 : s), false>(d.W, d.N, d.K, d.w_scale, d.xq, d.xscale, d.y,  \
                                                               nullptr, row0, nrows, lds);                     \
        break;
        LB_CFGS(LB_BCASE)
#undef LB_BCASE
    }
}

hipError_t launch_matvec_batched(const BatchGroup &g, hipStream_t s, size_t lds_bytes)
{
    switch (g.fmt) {
    case LB_Q1_0:
        hipLaunchKernelGGL(matvec_batched_kernel<LB_Q1_0>, dim3(g.ntiles), dim3(WG), lds_bytes, s, g.desc, g.tile_prod);
        break;
    case LB_Q2_0_G64:
        hipLaunchKernelGGL(matvec_batched_kernel<LB_Q2_0_G64>, dim3(g.ntiles), dim3(WG), lds_bytes, s, g.desc,
                           g.tile_prod);
        break;
    case LB_TERNARY_PLANAR:
        hipLaunchKernelGGL(matvec_batched_kernel<LB_TERNARY_PLANAR>, dim3(g.ntiles), dim3(WG), lds_bytes, s, g.desc,
                           g.tile_prod);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int matvec_stage_bytes(int fmt, int64_t K)
{
    return (int)((K / SLICE) * (fmt == LB_TERNARY_PLANAR ? F<LB_TERNARY_PLANAR>::REC : F<LB_Q2_0_G64>::REC) * 4);
}

} // namespace lb
