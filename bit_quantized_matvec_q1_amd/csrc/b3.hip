// Batch-1 decode product of base-3 ternary beats (five trits per byte) with per-token int8 activations.
//
// Arithmetic (bankml technical report, section III.8 "Information" and "Operation": five trits fit in a
// byte, 3^5 = 243 <= 256, and the ternary product is an exact signed sum; tritium "Architecture",
// sections 1, 2, 5 and 10: the planar body's select-accumulate, its output rule y = ((float)acc * s_x) * s_w,
// and base-3 packing at 1.6 bits per weight as the open question this kernel measures): with the stored code
// c = w + 1 of each trit, acc = sum c q - sum q, exactly.
//
// Decode on CDNA4.  The device layout (lowbit_pack_weights) keeps the beat stream but stores each base-3
// byte v as the 8-bit fraction b = ceil(256 v / 243) (v = 243 b >> 8).  A 16-byte record is four dwords of
// four bytes (20 trits each), decoded two ways so that the vector ALU and the LDS share the work:
//  * the first three dwords by table: per byte one 8-byte LDS entry indexed by b (one SDWA shift forms the
//    address), holding the byte's five codes c_t = w + 1 -- c_0 .. c_3 as the bytes of its first dword,
//    multiplied with v_dot4_i32_i8 against the activations of the byte's first four columns, and c_4 in
//    byte k (the byte's position in its dword) of the second, ORed over the dword's four bytes and
//    multiplied once against the four fifth columns: 11 operations and 4 LDS reads per 20 trits;
//  * the fourth dword arithmetically: the leading m base-3 digits of v are F_m = floor(3^m b / 256)
//    (F_5 = v), digit 5 - m is F_m - 3 F_(m-1), and for the five columns j0 .. j0 + 4 of a byte
//        sum_t c_t q_(j0+t) = sum_(m=1..4) F_m q_(j0+5-m) + d_0 q_j0 - 3 sum_(m=1..3) F_m q_(j0+4-m),
//    with d_0 = F_5 - 3 F_4.  The dword's bytes go to the 16-bit halves of two registers (two byte
//    permutes); per m both are multiplied by 3 (products below 2^16, so the halves never carry into each
//    other) and one permute gathers the four F_m into one int8 dword for v_dot4_i32_i8: 27 operations.
// All table reads alone left the LDS as the limit (most of its busy cycles bank conflicts), the arithmetic
// alone the vector ALU; three to one measured fastest.  The activations are staged once per workgroup in
// the order each form reads (five dwords per record dword either way).

// Work split as in the other decode kernels: a row over L lanes, S beats per lane (strided by L so a
// wave-wide 16-byte load is contiguous), the staged activation pairs held in registers for every row a
// lane streams, the next row's loads in flight, a DPP tree per row; rows never split across workgroups.
#include "lowbit_internal.h"

namespace lb {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u gv4u;
typedef __attribute__((address_space(1))) const uint8_t gu8;

constexpr int BCOLS = 80; // columns per beat
constexpr int REC = 20;   // staged dwords per beat: 4 record dwords x 5 column offsets

#define LB_B3_CFGS(X)                                                                                         \
    X(0, 16, 1) X(1, 16, 2) X(2, 32, 1) X(3, 32, 2) X(4, 32, 3) X(5, 64, 1) X(6, 64, 2) X(7, 32, 5) X(8, 64, 3)     \
    X(9, 64, 4) X(10, 64, 6)

struct CfgLS {
    int L, S;
};
#define LB_B3_ENTRY(i, l, s) {l, s},
constexpr CfgLS kB3Cfgs[] = {LB_B3_CFGS(LB_B3_ENTRY)};
#undef LB_B3_ENTRY
constexpr int kB3NumCfgs = sizeof(kB3Cfgs) / sizeof(kB3Cfgs[0]);

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// The LDS table: for each byte position k of a record dword and each stored byte b, the digits c_t (the
// codes w + 1, lowest digit first) of the base-3 value v = 243 b >> 8 -- c_0 .. c_3 as the four bytes of
// the entry's first dword, c_4 in byte k of its second (zero elsewhere), so that the second dwords of a
// record dword's four bytes combine by OR.  4 x 256 entries of 8 bytes, built by every workgroup.
__device__ __forceinline__ void b3_build_lut(uint2 *__restrict__ lut)
{
    // one stored byte per thread, its entry written for all four byte positions
    for (int b = threadIdx.x; b < 256; b += WG) {
        uint32_t v = (243u * (uint32_t)b) >> 8, lo = 0;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            lo |= (v % 3u) << (8 * t);
            v /= 3u;
        }
#pragma unroll
        for (int k = 0; k < 4; k++)
            lut[256 * k + b] = make_uint2(lo, v << (8 * k)); // v is digit 4 now
    }
}

// Byte k of d times 8, in one instruction (the byte selected by the operand's own SDWA field).
template <int k> __device__ __forceinline__ uint32_t byte_x8(uint32_t d)
{
    uint32_t r;
    if (k == 0)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(d));
    else if (k == 1)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(d));
    else if (k == 2)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(d));
    else
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(d));
    return r;
}

// The four bytes of one record dword by table: per byte k one entry, whose first dword is multiplied against
// the activations of the byte's first four columns (A[k]) and whose second dwords, ORed over the four
// bytes, against those of their fifth columns (A[4]).
__device__ __forceinline__ void b3_dword(uint32_t d, const uint32_t *A, const uint2 *__restrict__ lut, int &acc)
{
    uint32_t hi = 0;
    const uint32_t a[4] = {byte_x8<0>(d), byte_x8<1>(d), byte_x8<2>(d), byte_x8<3>(d)};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint2 e = *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(lut + 256 * k) + a[k]);
        acc = dot4(e.x, A[k], acc);
        hi |= e.y;
    }
    acc = dot4(hi, A[4], acc);
}

// The four bytes of one record dword arithmetically: F_m of all four in one dword per m, int8 dot products
// against the staged activation columns P[o] (byte k of P[o]: the activation of column 5 k + o of the
// dword's 20).
__device__ __forceinline__ void b3_dword_arith(uint32_t d, const uint32_t *P, int &acc_a, int &acc_b)
{
    uint32_t ye = __builtin_amdgcn_perm(0u, d, 0x0C020C00u); // bytes 0 and 2 in the low bytes of the halves
    uint32_t yo = __builtin_amdgcn_perm(0u, d, 0x0C030C01u); // bytes 1 and 3
    uint32_t f4 = 0;
#pragma unroll
    for (int m = 1; m <= 5; m++) {
        ye *= 3u; // 3^m b per half: below 2^16, so the halves never carry into each other
        yo *= 3u;
        const uint32_t f = __builtin_amdgcn_perm(yo, ye, 0x07030501u); // the high bytes: F_m of bytes 0..3
        if (m <= 4)
            acc_a = dot4(f, P[5 - m], acc_a);
        if (m <= 3)
            acc_b = dot4(f, P[4 - m], acc_b);
        if (m == 4)
            f4 = f;
        if (m == 5) // digit 0 of each byte, F_5 - 3 F_4 in 0..2: no byte borrows or carries
            acc_a = dot4(f - 3u * f4, P[0], acc_a);
    }
}

// Stage the activation once per workgroup: per beat and record dword five dwords (columns past K read
// q = 0) -- for the table-decoded dwords 0..2, per byte k (columns c0 + 5 k .. c0 + 5 k + 4) the activations
// of its first four columns, then one dword whose byte k is that of its fifth column; for dword 3 the
// transposed columns P[o], byte k = column 5 k + o.  One item per record dword: its 20 columns as five
// dword loads (K is a multiple of 64, so a dword is wholly in or past the row), rearranged with byte
// selects.  The row's sum of q comes from the same loads: each wave's total at sumq[wave], summed by the
// reader after the workgroup's barrier.
template <int i> __device__ __forceinline__ uint32_t qbyte(const uint32_t (&s)[5])
{
    return (s[i / 4] >> (8 * (i % 4))) & 0xFFu;
}
template <int a, int b, int c, int d> __device__ __forceinline__ uint32_t gather4(const uint32_t (&s)[5])
{
    return qbyte<a>(s) | qbyte<b>(s) << 8 | qbyte<c>(s) << 16 | qbyte<d>(s) << 24;
}

__device__ __forceinline__ void b3_stage(const int8_t *__restrict__ xq, int K, int nbt, uint32_t *__restrict__ lds,
                                         int *__restrict__ sumq)
{
    int part = 0;
    for (int it = threadIdx.x; it < nbt * 4; it += WG) {
        const int bt = it >> 2, dd = it & 3;
        const int c0 = bt * BCOLS + 20 * dd;
        uint32_t s[5];
#pragma unroll
        for (int u = 0; u < 5; u++)
            s[u] = c0 + 4 * u < K ? *reinterpret_cast<const uint32_t *>(xq + c0 + 4 * u) : 0u;
#pragma unroll
        for (int u = 0; u < 5; u++)
            part = __builtin_amdgcn_sdot4((int)s[u], 0x01010101, part, false);
        uint4 o03;
        uint32_t o4;
        if (dd == 3) {
            o03 = make_uint4(gather4<0, 5, 10, 15>(s), gather4<1, 6, 11, 16>(s), gather4<2, 7, 12, 17>(s),
                             gather4<3, 8, 13, 18>(s));
            o4 = gather4<4, 9, 14, 19>(s);
        } else {
            o03 = make_uint4(gather4<0, 1, 2, 3>(s), gather4<5, 6, 7, 8>(s), gather4<10, 11, 12, 13>(s),
                             gather4<15, 16, 17, 18>(s));
            o4 = gather4<4, 9, 14, 19>(s);
        }
        uint32_t *dst = lds + bt * REC + 5 * dd;
        dst[0] = o03.x;
        dst[1] = o03.y;
        dst[2] = o03.z;
        dst[3] = o03.w;
        dst[4] = o4;
    }
    static_assert(WG == 256, "four per-wave partial sums (the 16 bytes past the staged activation)");
    part = group_sum_i<64>(part);
    if ((threadIdx.x & 63) == 63)
        sumq[threadIdx.x >> 6] = part;
}

template <int S> struct B3Row {
    uint4 code[S];
};

template <int L, int S, bool EMIT>
__device__ __forceinline__ void b3_tile(const uint8_t *__restrict__ W, int K, float w_scale, const int8_t *__restrict__ xq,
                                        float sx, float *__restrict__ y, int32_t *__restrict__ sums, int row0, int nrows,
                                        uint32_t *__restrict__ lds)
{
    constexpr int GROUPS = 64 / L;
    constexpr int STEP = GROUPS * (WG / 64);
    const int nbt = (K + BCOLS - 1) / BCOLS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, li = lane % L;
    const int rbase = wave * GROUPS + g;
    const uint32_t rowbytes = (uint32_t)nbt * 16u;
    const uint32_t stepb = (uint32_t)STEP * rowbytes;
    const uint32_t last = (uint32_t)(row0 + nrows - 1) * rowbytes;
    uint32_t bo[S];
#pragma unroll
    for (int i = 0; i < S; i++)
        bo[i] = (uint32_t)min(li + i * L, nbt - 1) * 16u; // a lane past the row's end re-reads its last beat
    uint32_t onext = (uint32_t)(row0 + min(rbase, nrows - 1)) * rowbytes;

    auto issue = [&](B3Row<S> &r, uint32_t off) {
#pragma unroll
        for (int i = 0; i < S; i++) {
            const v4u t = __builtin_nontemporal_load((gv4u *)((gu8 *)W + (off + bo[i])));
            r.code[i] = make_uint4(t.x, t.y, t.z, t.w);
        }
    };
    B3Row<S> buf[2];
    issue(buf[0], min(onext, last));
    onext += stepb;
    // the tile's outputs y[row0, row0 + nrows) as a buffer range (the sums instantiation may run without y)
    const __amdgpu_buffer_rsrc_t yt =
        __builtin_amdgcn_make_buffer_rsrc(EMIT ? nullptr : y + row0, 0, EMIT ? 0 : nrows * 4, 0x00020000);

    __shared__ uint2 lut_s[4 * 256]; // (static: its address is a constant, folded into the reads' offsets)
    const uint2 *lut = lut_s;
    b3_build_lut(lut_s);
    int *sumq = reinterpret_cast<int *>(lds + nbt * REC);
    b3_stage(xq, K, nbt, lds, sumq);
    __syncthreads();

    uint32_t act[S][REC];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int bt = li + i * L;
        const uint4 *p = reinterpret_cast<const uint4 *>(lds + min(bt, nbt - 1) * REC);
#pragma unroll
        for (int q = 0; q < REC / 4; q++) {
            const uint4 t = p[q];
            const bool in = bt < nbt; // a lane past the row's end multiplies by zero
            act[i][4 * q + 0] = in ? t.x : 0u;
            act[i][4 * q + 1] = in ? t.y : 0u;
            act[i][4 * q + 2] = in ? t.z : 0u;
            act[i][4 * q + 3] = in ? t.w : 0u;
        }
    }
    const int sq = sumq[0] + sumq[1] + sumq[2] + sumq[3];

    for (int it = 0; it < nrows; it += 2 * STEP) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            // no branch inside the pair: a row past the tile's end is computed from the clamped loads and
            // never stored, so the next row's loads are issued every time, ahead of this row's arithmetic,
            // and the load counter waits only for the row computed next
            const int cur = it + p * STEP;
            issue(buf[p ^ 1], min(onext, last));
            __builtin_amdgcn_sched_barrier(0);
            onext += stepb;
            int acc = 0, acc_a = 0, acc_b = 0;
#pragma unroll
            for (int i = 0; i < S; i++) {
                b3_dword(buf[p].code[i].x, act[i] + 0, lut, acc);
                b3_dword(buf[p].code[i].y, act[i] + 5, lut, acc);
                b3_dword(buf[p].code[i].z, act[i] + 10, lut, acc);
                b3_dword_arith(buf[p].code[i].w, act[i] + 15, acc_a, acc_b);
            }
            acc = group_sum_i<L>(acc + acc_a - 3 * acc_b);
            const int rl = cur + rbase;
            const int a = acc - sq; // sum (w + 1) q - sum q
            // tritium "Architecture", section 5: activation scale, then weight scale, in fp32
            const float ys = (float)a * sx;
            if constexpr (EMIT) {
                if (rl < nrows && li == L - 1) {
                    sums[row0 + rl] = a;
                    if (y != nullptr)
                        y[row0 + rl] = ys * w_scale;
                }
            } else {
                // every lane stores; a lane without a result addresses past the tile's output range, where
                // the buffer unit drops it (no branch around the store)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ys * w_scale), yt,
                                                      rl < nrows && li == L - 1 ? (uint32_t)rl * 4u : 0x80000000u,
                                                      0, 0);
            }
        }
    }
}

template <int L, int S, bool EMIT>
__global__ __launch_bounds__(WG) void b3_kernel(const uint8_t *__restrict__ W, int N, int K, float w_scale,
                                                 const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                 float *__restrict__ y, int32_t *__restrict__ sums, int tile_rows)
{
    extern __shared__ uint4 lds4[];
    const int row0 = blockIdx.x * tile_rows;
    b3_tile<L, S, EMIT>(W, K, w_scale, xq, xs[0], y, sums, row0, min(tile_rows, N - row0),
                        reinterpret_cast<uint32_t *>(lds4));
}

template <int L, int S>
__global__ __launch_bounds__(WG) void b3_batched_kernel(const DevDesc *__restrict__ desc, const TileRef *__restrict__ tiles)
{
    extern __shared__ uint4 lds4[];
    const TileRef tr = tiles[blockIdx.x];
    const DevDesc d = desc[tr.prod];
    b3_tile<L, S, false>(d.W, d.K, d.w_scale, d.xq, *static_cast<const float *>(d.xscale), d.y, nullptr, tr.row0,
                         min(d.tile_rows, d.N - tr.row0), reinterpret_cast<uint32_t *>(lds4));
}

} // namespace

// Choice: the fewest idle lane slots among the configurations (their staged activation fits 120 registers
// per lane: at most 6 beats, so K up to 64 x 6 x 80 = 30720); then fewer lanes per row.
int b3_config(int64_t K)
{
    if (K <= 0 || K % 64)
        return -1;
    const int64_t nbt = (K + BCOLS - 1) / BCOLS;
    int best = -1;
    int64_t bw = 0;
    for (int c = 0; c < kB3NumCfgs; c++) {
        const int64_t slots = (int64_t)kB3Cfgs[c].L * kB3Cfgs[c].S;
        if (slots < nbt)
            continue;
        const int64_t waste = slots - nbt;
        if (best < 0 || waste < bw || (waste == bw && kB3Cfgs[c].L < kB3Cfgs[best].L)) {
            best = c;
            bw = waste;
        }
    }
    return best;
}

int b3_rows_per_iter(int cfg) { return (64 / kB3Cfgs[cfg].L) * (WG / 64); }
size_t b3_stage_bytes(int64_t K) { return (size_t)((K + BCOLS - 1) / BCOLS) * REC * 4 + 16; }

hipError_t launch_b3(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *xq, const float *xs, float *y,
                     int32_t *sums, hipStream_t stream)
{
    const int cfg = b3_config(K);
    if (cfg < 0)
        return hipErrorInvalidValue;
    const int rpi = b3_rows_per_iter(cfg);
    int64_t tile = (N + 1023) / 1024;
    tile = (tile + rpi - 1) / rpi * rpi;
    tile = tile < rpi ? rpi : tile > 32 * rpi ? 32 * rpi : tile;
    const int ntiles = (int)((N + tile - 1) / tile);
    const size_t lds = b3_stage_bytes(K);
    const int n = (int)N, k = (int)K, t = (int)tile;
    switch (cfg) {
#define LB_B3_CASE(i, l, s)                                                                                   \
    case i:                                                                                                   \
        if (sums)                                                                                             \
            hipLaunchKernelGGL((b3_kernel<l, s, true>), dim3(ntiles), dim3(WG), lds, stream, W, n, k, w_scale,  \
                               xq, xs, y, sums, t);                                                           \
        else                                                                                                  \
            hipLaunchKernelGGL((b3_kernel<l, s, false>), dim3(ntiles), dim3(WG), lds, stream, W, n, k, w_scale, \
                               xq, xs, y, sums, t);                                                           \
        break;
        LB_B3_CFGS(LB_B3_CASE)
#undef LB_B3_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_b3_batched(const BatchGroup &g, size_t lds, hipStream_t stream)
{
    switch (g.cfg_a) {
#define LB_B3_BCASE(i, l, s)                                                                                  \
    case i:                                                                                                   \
        hipLaunchKernelGGL((b3_batched_kernel<l, s>), dim3(g.ntiles), dim3(WG), lds, stream, g.desc, g.tiles);  \
        break;
        LB_B3_CFGS(LB_B3_BCASE)
#undef LB_B3_BCASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int b3_blocks_per_cu(int cfg, size_t lds)
{
    int nb = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (cfg) {
#define LB_B3_OCASE(i, l, s)                                                                                  \
    case i:                                                                                                   \
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, b3_batched_kernel<l, s>, WG, lds);             \
        break;
        LB_B3_CFGS(LB_B3_OCASE)
#undef LB_B3_OCASE
    default:
        break;
    }
    return e == hipSuccess && nb > 0 ? nb : 1;
}

} // namespace lb
