// Batch-1 decode product of Q8_0 weights with q8_0 activations (vec_dot_q8_0_q8_0) on gfx950.
//
// Arithmetic (bankml technical report, section III.2 "The Q1_0 format and its arithmetic" for the q8_0
// block -- a binary16 scale, then 32 signed bytes -- and section III.3 for the float chain; the build
// history's 0.3.9 entry names the same product for the q8_0 KV cache, and "Q8_0 weights" as work left):
// per row, isum_b = sum over the 32 weights of block b of w_i * q_i, an exact integer, then
// y = sum_b d_w[b] * (d_x[b] * isum_b) in fp32.
//
// Mapping to CDNA4: the weight stream is one byte per weight, so the kernel is HBM-bound with a wide
// margin (8 v_dot4_i32_i8 and three float operations per 34 bytes).  The device layout keeps the 32
// weight bytes of a block as one 32-byte record ([N][K/32][32], then the binary16 scales [N][K/32]), so
// a lane streams two 16-byte beats per block.  A row is split over L lanes, each owning S blocks (lane li
// takes blocks li, li + L, ... so a wave-wide load is contiguous); the activation bytes and scales of a
// lane's blocks are staged through LDS once per workgroup and then held in registers for every row the
// lane streams, with the next row's loads in flight while a row is computed.  The L lanes of a row are
// summed with DPP; rows never split across workgroups (tritium "Architecture", section 7).
#include "lowbit_internal.h"

namespace lb {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u gv4u;
typedef __attribute__((address_space(1))) const uint8_t gu8;
typedef __attribute__((address_space(1))) const uint16_t gu16;

constexpr int QB = 32; // bytes per Q8_0 record (and weights per block)
constexpr int UB = 16; // bytes per unit: half a record, one 16-byte beat

// Configurations (L lanes per row, S units per lane).  The unit of work is half a block (16 weights):
// lane li takes units li, li + L, ..., so one wave-wide load is 64 consecutive beats, and L is even, so
// the two halves of a block sit in lanes li and li ^ 1 of the same row.
#define LB_Q8_CFGS(X)                                                                                         \
    X(0, 8, 1) X(1, 8, 2) X(2, 8, 4) X(3, 8, 6) X(4, 8, 8) X(5, 16, 1) X(6, 16, 2) X(7, 16, 4) X(8, 16, 6)      \
    X(9, 16, 8) X(10, 32, 2) X(11, 32, 3) X(12, 32, 4) X(13, 32, 6) X(14, 32, 8) X(15, 64, 2) X(16, 64, 3)    \
    X(17, 64, 4) X(18, 64, 5) X(19, 64, 6) X(20, 64, 8) X(21, 64, 10) X(22, 64, 12) X(23, 64, 16)

struct CfgLS {
    int L, S;
};
#define LB_Q8_ENTRY(i, l, s) {l, s},
constexpr CfgLS kQ8Cfgs[] = {LB_Q8_CFGS(LB_Q8_ENTRY)};
#undef LB_Q8_ENTRY
constexpr int kQ8NumCfgs = sizeof(kQ8Cfgs) / sizeof(kQ8Cfgs[0]);

template <int S> struct Q8Row {
    uint4 w[S];     // the unit's 16 weight bytes
    uint32_t sc[S]; // its block's binary16 scale
};

template <int L, int S>
__device__ __forceinline__ void q8_issue(Q8Row<S> &r, const uint8_t *__restrict__ W, const uint8_t *__restrict__ scales,
                                         uint32_t off, const uint32_t (&uo)[S])
{
    // off: byte offset of the row's first record; uo[i]: byte offset of this lane's i-th unit in a row
    const uint32_t soff = off >> 4; // record index at byte 32 idx, its scale at byte 2 idx
#pragma unroll
    for (int i = 0; i < S; i++) {
        const v4u a = __builtin_nontemporal_load((gv4u *)((gu8 *)W + (off + uo[i])));
        r.w[i] = make_uint4(a.x, a.y, a.z, a.w);
        r.sc[i] = *(gu16 *)((gu8 *)scales + (soff + ((uo[i] >> 5) << 1)));
    }
}

__device__ __forceinline__ int dot16(uint4 w, uint4 x, int acc)
{
    acc = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, acc, false);
    return __builtin_amdgcn_sdot4((int)w.w, (int)x.w, acc, false);
}

template <int L, int S, bool EMIT>
__device__ __forceinline__ void q8_tile(const uint8_t *__restrict__ W, int N, int K, const int8_t *__restrict__ xq,
                                        const uint16_t *__restrict__ xs, float *__restrict__ y, int32_t *__restrict__ sums,
                                        int row0, int nrows, uint32_t *__restrict__ lds)
{
    constexpr int GROUPS = 64 / L;
    constexpr int STEP = GROUPS * (WG / 64);
    const int nb = K / QB, nu = K / UB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, li = lane % L;
    const uint8_t *scales = W + (size_t)N * nb * QB;
    const int rbase = wave * GROUPS + g;
    const uint32_t rowbytes = (uint32_t)nb * QB;
    const uint32_t stepb = (uint32_t)STEP * rowbytes;
    const uint32_t last = (uint32_t)(row0 + nrows - 1) * rowbytes;
    uint32_t uo[S];
#pragma unroll
    for (int i = 0; i < S; i++)
        uo[i] = (uint32_t)min(li + i * L, nu - 1) * UB; // a lane past the row's end re-reads its last unit
    uint32_t onext = (uint32_t)(row0 + min(rbase, nrows - 1)) * rowbytes;

    Q8Row<S> buf[2];
    q8_issue<L, S>(buf[0], W, scales, min(onext, last), uo);
    onext += stepb;

    // stage the activation bytes and the scales (as floats) once for the workgroup
    uint4 *xl = reinterpret_cast<uint4 *>(lds);
    float *dl = reinterpret_cast<float *>(lds + K / 4);
    for (int i = threadIdx.x; i < nu; i += WG)
        xl[i] = reinterpret_cast<const uint4 *>(xq)[i];
    for (int i = threadIdx.x; i < nb; i += WG)
        dl[i] = half_bits_to_float(xs[i]);
    __syncthreads();

    uint4 xu[S];
    float dx[S];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int u = li + i * L;
        const bool in = u < nu;
        xu[i] = in ? xl[u] : make_uint4(0u, 0u, 0u, 0u);
        dx[i] = in ? dl[u >> 1] : 0.0f;
    }

    // the tile's outputs y[row0, row0 + nrows) as a buffer range (the sums instantiation may run without y)
    const __amdgpu_buffer_rsrc_t yt =
        __builtin_amdgcn_make_buffer_rsrc(EMIT ? nullptr : y + row0, 0, EMIT ? 0 : nrows * 4, 0x00020000);
    for (int it = 0; it < nrows; it += 2 * STEP) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            // no branch inside the pair: a row past the tile's end is computed from the clamped loads and
            // never stored, so the next row's loads are issued every time, ahead of this row's arithmetic,
            // and the load counter waits only for the row computed next
            const int cur = it + p * STEP;
            q8_issue<L, S>(buf[p ^ 1], W, scales, min(onext, last), uo);
            __builtin_amdgcn_sched_barrier(0);
            onext += stepb;
            const int rl = cur + rbase;
            const bool valid = rl < nrows;
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < S; i++) {
                const int ih = dot16(buf[p].w[i], xu[i], 0); // half a block's sum
                // bankml report, section III.3: a multiply-add by d_x, then one by the block's weight scale;
                // the two halves of a block are scaled separately and meet in the row sum
                const float t = dx[i] * (float)ih;
                part = fmaf(half_bits_to_float((uint16_t)buf[p].sc[i]), t, part);
                if (EMIT) {
                    // the block's exact sum: this half plus its neighbour lane's (li ^ 1)
                    const int isum = ih + __builtin_amdgcn_update_dpp(0, ih, 0xB1, 0xF, 0xF, false);
                    const int u = li + i * L;
                    if (valid && (li & 1) == 0 && u < nu)
                        sums[(size_t)(row0 + rl) * nb + (u >> 1)] = isum;
                }
            }
            part = group_sum_f<L>(part);
            if constexpr (EMIT) {
                if (valid && li == L - 1 && y != nullptr)
                    y[row0 + rl] = part;
            } else {
                // every lane stores; a lane without a result addresses past the tile's output range, where
                // the buffer unit drops it (no branch around the store)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), yt,
                                                      valid && li == L - 1 ? (uint32_t)rl * 4u : 0x80000000u, 0, 0);
            }
        }
    }
}

template <int L, int S, bool EMIT>
__global__ __launch_bounds__(WG) void q8_kernel(const uint8_t *__restrict__ W, int N, int K, const int8_t *__restrict__ xq,
                                                 const uint16_t *__restrict__ xs, float *__restrict__ y,
                                                 int32_t *__restrict__ sums, int tile_rows)
{
    extern __shared__ uint4 lds4[];
    const int row0 = blockIdx.x * tile_rows;
    q8_tile<L, S, EMIT>(W, N, K, xq, xs, y, sums, row0, min(tile_rows, N - row0), reinterpret_cast<uint32_t *>(lds4));
}

template <int L, int S>
__global__ __launch_bounds__(WG) void q8_batched_kernel(const DevDesc *__restrict__ desc, const TileRef *__restrict__ tiles)
{
    extern __shared__ uint4 lds4[];
    const TileRef tr = tiles[blockIdx.x];
    const DevDesc d = desc[tr.prod];
    q8_tile<L, S, false>(d.W, d.N, d.K, d.xq, static_cast<const uint16_t *>(d.xscale), d.y, nullptr, tr.row0,
                         min(d.tile_rows, d.N - tr.row0), reinterpret_cast<uint32_t *>(lds4));
}

} // namespace

// Choice: the fewest idle lane slots; then S nearest 4 (a light register load with enough units per lane
// to amortise the row's reduction); then more lanes per row.
int q8_config(int64_t K)
{
    if (K <= 0 || K % QB)
        return -1;
    const int64_t nb = K / UB; // units per row
    int best = -1;
    int64_t bw = 0;
    int bd = 0;
    for (int c = 0; c < kQ8NumCfgs; c++) {
        const int64_t slots = (int64_t)kQ8Cfgs[c].L * kQ8Cfgs[c].S;
        if (slots < nb)
            continue;
        const int64_t waste = slots - nb;
        const int dist = kQ8Cfgs[c].S > 4 ? kQ8Cfgs[c].S - 4 : 4 - kQ8Cfgs[c].S;
        if (best < 0 || waste < bw || (waste == bw && (dist < bd || (dist == bd && kQ8Cfgs[c].L > kQ8Cfgs[best].L)))) {
            best = c;
            bw = waste;
            bd = dist;
        }
    }
    return best;
}

int q8_rows_per_iter(int cfg) { return (64 / kQ8Cfgs[cfg].L) * (WG / 64); }
size_t q8_stage_bytes(int64_t K) { return (size_t)K + (size_t)(K / QB) * 4; }

hipError_t launch_q8(const uint8_t *W, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xs, float *y,
                     int32_t *sums, hipStream_t stream)
{
    const int cfg = q8_config(K);
    if (cfg < 0)
        return hipErrorInvalidValue;
    const int rpi = q8_rows_per_iter(cfg);
    int64_t tile = (N + 1023) / 1024;
    tile = (tile + rpi - 1) / rpi * rpi;
    tile = tile < rpi ? rpi : tile > 32 * rpi ? 32 * rpi : tile;
    const int ntiles = (int)((N + tile - 1) / tile);
    const size_t lds = q8_stage_bytes(K);
    const int n = (int)N, k = (int)K, t = (int)tile;
    switch (cfg) {
#define LB_Q8_CASE(i, l, s)                                                                                   \
    case i:                                                                                                   \
        if (sums)                                                                                             \
            hipLaunchKernelGGL((q8_kernel<l, s, true>), dim3(ntiles), dim3(WG), lds, stream, W, n, k, xq, xs, y,  \
                               sums, t);                                                                      \
        else                                                                                                  \
            hipLaunchKernelGGL((q8_kernel<l, s, false>), dim3(ntiles), dim3(WG), lds, stream, W, n, k, xq, xs, y, \
                               sums, t);                                                                      \
        break;
        LB_Q8_CFGS(LB_Q8_CASE)
#undef LB_Q8_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_q8_batched(const BatchGroup &g, size_t lds, hipStream_t stream)
{
    switch (g.cfg_a) {
#define LB_Q8_BCASE(i, l, s)                                                                                  \
    case i:                                                                                                   \
        hipLaunchKernelGGL((q8_batched_kernel<l, s>), dim3(g.ntiles), dim3(WG), lds, stream, g.desc, g.tiles);  \
        break;
        LB_Q8_CFGS(LB_Q8_BCASE)
#undef LB_Q8_BCASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int q8_blocks_per_cu(int cfg, size_t lds)
{
    int nb = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (cfg) {
#define LB_Q8_OCASE(i, l, s)                                                                                  \
    case i:                                                                                                   \
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, q8_batched_kernel<l, s>, WG, lds);             \
        break;
        LB_Q8_CFGS(LB_Q8_OCASE)
#undef LB_Q8_OCASE
    default:
        break;
    }
    return e == hipSuccess && nb > 0 ? nb : 1;
}

} // namespace lb
