// Dense bf16 head matvec: y[n] = sum_k f32(W[n][k]) * x[k] (tritium "Architecture", section 3: the
// tied output head is the largest single stream of a decode step, stored as bf16).
//
// Purely bandwidth-bound: each weight byte is read once with 16-byte loads (8 bf16), widened to fp32
// exactly (bf16 is the top half of a binary32), and multiply-added against x held in VGPRs.  A row is
// spread over one wave (each lane owns S chunks of 8 columns, strided so every wave-wide load is
// contiguous) and closed with a cross-lane tree.  Rows longer than the registers hold x for (4096 columns
// here, 8192 for the int8 head) run as column segments, one launch each in stream order: the first
// stores its partial sums, every later one adds its own to them (one atomic add per row and segment, in a
// fixed order, so the result does not depend on timing).
#include "lowbit_internal.h"

#include <algorithm>
#include <atomic>

namespace lb {

typedef unsigned hv4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const hv4u ghv4u;
typedef __attribute__((address_space(1))) const uint8_t ghu8;

// A workgroup owns a tile of rows; wave w takes rows w, w + 4, ... of it.  Loads are unconditional
// (chunk offsets clamped to the row's last chunk, row offsets to the tile's last row -- both in bounds,
// their results never stored or multiplied by a zero x), non-temporal (the weights are read once), and
// issued one row ahead into a second register buffer.
// The store of a row's total: the first segment writes it, later ones add to it.  Every lane issues it; a
// lane without the total addresses past the tile's output range, where the buffer unit drops it.
template <bool ADD> __device__ __forceinline__ void put_row(__amdgpu_buffer_rsrc_t yt, bool keep, int rl, float v)
{
    const uint32_t off = keep ? (uint32_t)rl * 4u : 0x80000000u;
    if constexpr (ADD)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, yt, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yt, off, 0, 0);
}

// One column segment [0, K) of the rows (W and x already offset to it); ldw: the full row length.
template <int S, bool ADD>
__global__ __launch_bounds__(WG) void head_kernel(const uint16_t *__restrict__ W, int N, int K, int ldw,
                                                  const float *__restrict__ x, float *__restrict__ y, int tile_rows)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nch = K / 8; // chunks of 8 columns per row
    float xr[S][8];
    uint32_t co[S]; // byte offset of this lane's chunks within a row
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int ch = lane + 64 * i;
        co[i] = (uint32_t)min(ch, nch - 1) * 16u;
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
    const bool ragged = nch != 64 * S; // some lanes' last chunk lies past the row: zero its weights too
    const int row0 = blockIdx.x * tile_rows;
    const int nrows = min(tile_rows, N - row0);
    constexpr int STEP = WG / 64;
    const uint32_t rowb = (uint32_t)ldw * 2u;
    const uint32_t last = (uint32_t)(row0 + nrows - 1) * rowb;
    uint32_t onext = (uint32_t)(row0 + min(wave, nrows - 1)) * rowb;
    uint4 buf[2][S];
    auto issue = [&](uint4 (&w)[S], uint32_t off) {
#pragma unroll
        for (int i = 0; i < S; i++) {
            const hv4u t = __builtin_nontemporal_load((ghv4u *)((ghu8 *)W + (off + co[i])));
            w[i] = make_uint4(t.x, t.y, t.z, t.w);
        }
    };
    issue(buf[0], min(onext, last));
    onext += STEP * rowb;
    const __amdgpu_buffer_rsrc_t yt = __builtin_amdgcn_make_buffer_rsrc(y + row0, 0, nrows * 4, 0x00020000);
    for (int it = 0; it < nrows; it += 2 * STEP) {
#pragma unroll
        for (int b = 0; b < 2; b++) {
            // no branch inside the pair: a row past the tile's end is computed from the clamped loads and
            // never stored, so the next row's loads are issued every time, ahead of this row's arithmetic,
            // and the load counter waits only for the row computed next
            const int cur = it + b * STEP;
            issue(buf[b ^ 1], min(onext, last));
            __builtin_amdgcn_sched_barrier(0);
            onext += STEP * rowb;
            if (ragged && lane + 64 * (S - 1) >= nch)
                buf[b][S - 1] = make_uint4(0u, 0u, 0u, 0u);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < S; i++) {
                const uint32_t v[4] = {buf[b][i].x, buf[b][i].y, buf[b][i].z, buf[b][i].w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    acc = fmaf(__uint_as_float(v[j] << 16), xr[i][2 * j], acc);
                    acc = fmaf(__uint_as_float(v[j] & 0xffff0000u), xr[i][2 * j + 1], acc);
                }
            }
            acc = group_sum_f<64>(acc);
            const int rl = cur + wave;
            put_row<ADD>(yt, rl < nrows && lane == 63, rl, acc); // no branch around the store
        }
    }
}

// int8 head: y[n] = s_w[n] * sum_k W[n][k] * x[k] (tritium "Architecture", section 10: int8 as the obvious
// move for the head; one fp32 scale per row).  Half the bytes of the bf16 head: the same streaming
// structure with 16-byte loads of 16 weights, each widened to fp32 exactly (a signed byte) and
// multiply-added against x held in VGPRs; the row's scale multiplies the finished sum.  A row takes L
// lanes (64 / L rows per wave) and each lane S chunks, L chosen so that L * S covers the row's chunks with
// the fewest idle lane slots (K = 2560: 160 chunks = 32 lanes x 5).
template <int L, int S, bool ADD>
__global__ __launch_bounds__(WG) void head_i8_kernel(const int8_t *__restrict__ W, const float *__restrict__ sw, int N,
                                                     int K, int ldw, const float *__restrict__ x,
                                                     float *__restrict__ y, int tile_rows)
{
    constexpr int G = 64 / L;            // rows per wave
    constexpr int STEP = G * (WG / 64);  // rows per workgroup iteration
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, li = lane % L;
    const int nch = K / 16; // chunks of 16 columns per row
    uint32_t co[S];         // byte offset of this lane's chunks within a row
#pragma unroll
    for (int i = 0; i < S; i++)
        co[i] = (uint32_t)min(li + L * i, nch - 1) * 16u;
    const int row0 = blockIdx.x * tile_rows;
    const int nrows = min(tile_rows, N - row0);
    const int rbase = wave * G + g; // this lane's row within an iteration
    const uint32_t rowb = (uint32_t)ldw;
    const uint32_t last = (uint32_t)(row0 + nrows - 1) * rowb;
    uint32_t onext = (uint32_t)(row0 + min(rbase, nrows - 1)) * rowb;
    // a ring of NB register buffers: NB - 1 rows' loads in flight while a row is computed (3 measured
    // fastest: 2 leaves HBM idle, 4 costs occupancy)
    constexpr int NB = 3;
    uint4 buf[NB][S];
    float sbuf[NB]; // the row's scale travels with its weights
    const int rlast = row0 + nrows - 1;
    int rnext = row0 + min(rbase, nrows - 1);
    auto issue = [&](uint4 (&w)[S], float &s, uint32_t off, int row) {
#pragma unroll
        for (int i = 0; i < S; i++) {
            const hv4u t = __builtin_nontemporal_load((ghv4u *)((ghu8 *)W + (off + co[i])));
            w[i] = make_uint4(t.x, t.y, t.z, t.w);
        }
        s = sw[row];
    };
#pragma unroll
    for (int b = 0; b < NB - 1; b++) {
        issue(buf[b], sbuf[b], min(onext, last), min(rnext, rlast));
        onext += STEP * rowb;
        rnext += STEP;
    }
    // x into registers while the first rows stream in (columns past K read zero)
    float xr[S][16];
#pragma unroll
    for (int i = 0; i < S; i++) {
        const int ch = li + L * i;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 a = ch < nch ? reinterpret_cast<const float4 *>(x)[4 * ch + q] : make_float4(0.f, 0.f, 0.f, 0.f);
            xr[i][4 * q + 0] = a.x, xr[i][4 * q + 1] = a.y, xr[i][4 * q + 2] = a.z, xr[i][4 * q + 3] = a.w;
        }
    }
    const __amdgpu_buffer_rsrc_t yt = __builtin_amdgcn_make_buffer_rsrc(y + row0, 0, nrows * 4, 0x00020000);
    for (int it = 0; it < nrows; it += NB * STEP) {
#pragma unroll
        for (int b = 0; b < NB; b++) {
            // no branch inside the ring: a row past the tile's end is computed from the clamped loads and
            // never stored, so the next row's loads are issued every time, ahead of this row's arithmetic,
            // and the load counter waits only for the row computed next
            const int cur = it + b * STEP;
            issue(buf[(b + NB - 1) % NB], sbuf[(b + NB - 1) % NB], min(onext, last), min(rnext, rlast));
            __builtin_amdgcn_sched_barrier(0);
            onext += STEP * rowb;
            rnext += STEP;
            // a lane's chunk past the row's end re-read the last chunk; its x is zero, so it adds nothing;
            // a lane past the tile's last row re-read that row, and its sum is not stored
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < S; i++) {
                const uint32_t v[4] = {buf[b][i].x, buf[b][i].y, buf[b][i].z, buf[b][i].w};
#pragma unroll
                for (int j = 0; j < 4; j++)
#pragma unroll
                    for (int t = 0; t < 4; t++)
                        acc = fmaf((float)(int)(int8_t)(v[j] >> (8 * t)), xr[i][4 * j + t], acc);
            }
            acc = group_sum_f<L>(acc);
            const int rl = cur + rbase;
            put_row<ADD>(yt, rl < nrows && li == L - 1, rl, sbuf[b] * acc); // no branch around the store
        }
    }
}

// Resident workgroups of one int8-head configuration on the current device, cached per device.
template <int L, int S> static int head_i8_slots()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, nb = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, head_i8_kernel<L, S, false>, WG, 0) != hipSuccess ||
            nb < 1)
            nb = 1;
        v = cus * nb;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int L, int S>
static hipError_t launch_head_i8_cfg(const int8_t *W, const float *sw, int N, int K, int ldw, bool add,
                                     const float *x, float *y, hipStream_t s)
{
    // one workgroup per resident slot, each streaming one contiguous range of rows with x loaded once:
    // no second, partly filled round of workgroups, and x is read from L2 once per slot
    constexpr int PASS = 3 * (64 / L) * (WG / 64); // rows of one pass of the three-row ring
    const int slots = head_i8_slots<L, S>();
    int tile = (N + slots - 1) / slots;
    tile = (tile + PASS - 1) / PASS * PASS;
    const int grid = (N + tile - 1) / tile;
    if (add)
        hipLaunchKernelGGL((head_i8_kernel<L, S, true>), dim3(grid), dim3(WG), 0, s, W, sw, N, K, ldw, x, y, tile);
    else
        hipLaunchKernelGGL((head_i8_kernel<L, S, false>), dim3(grid), dim3(WG), 0, s, W, sw, N, K, ldw, x, y, tile);
    return hipGetLastError();
}

// One column segment (at most 8192 columns) of the int8 head.
static hipError_t launch_head_i8_seg(const int8_t *W, const float *sw, int64_t N, int64_t K, int64_t ldw, bool add,
                                     const float *x, float *y, hipStream_t s)
{
    const int nch = (int)(K / 16);
    // lanes per row: the fewest idle lane slots (L * S - nch) with S <= 8, then the most lanes
    int L = 64, S = (nch + 63) / 64;
    for (int l : {32, 16}) {
        const int sl = (nch + l - 1) / l;
        if (sl <= 8 && l * sl - nch < L * S - nch) {
            L = l;
            S = sl;
        }
    }
    const int n = (int)N, k = (int)K, ld = (int)ldw;
    switch (L * 16 + S) {
#define LB_HEAD_I8(l, sv)                                                                                     \
    case l * 16 + sv:                                                                                         \
        return launch_head_i8_cfg<l, sv>(W, sw, n, k, ld, add, x, y, s);
#define LB_HEAD_I8_L(l)                                                                                       \
    LB_HEAD_I8(l, 1) LB_HEAD_I8(l, 2) LB_HEAD_I8(l, 3) LB_HEAD_I8(l, 4) LB_HEAD_I8(l, 5) LB_HEAD_I8(l, 6)       \
    LB_HEAD_I8(l, 7) LB_HEAD_I8(l, 8)
        LB_HEAD_I8_L(16) LB_HEAD_I8_L(32) LB_HEAD_I8_L(64)
#undef LB_HEAD_I8_L
#undef LB_HEAD_I8
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_head_i8(const int8_t *W, const float *sw, int64_t N, int64_t K, const float *x, float *y, hipStream_t s)
{
    constexpr int64_t SEG = 8192; // the columns one launch holds x for
    for (int64_t k0 = 0; k0 < K; k0 += SEG) {
        const hipError_t e = launch_head_i8_seg(W + k0, sw, N, std::min(SEG, K - k0), K, k0 > 0, x + k0, y, s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_head(const uint16_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s)
{
    constexpr int64_t SEG = 4096; // the columns one launch holds x for
    const int tile = 64;
    const int grid = (int)((N + tile - 1) / tile);
    for (int64_t k0 = 0; k0 < K; k0 += SEG) {
        const int kseg = (int)std::min(SEG, K - k0);
        const int S = (kseg / 8 + 63) / 64;
        const bool add = k0 > 0;
        switch (S) {
#define LB_HEAD(n)                                                                                            \
    case n:                                                                                                   \
        if (add)                                                                                              \
            hipLaunchKernelGGL((head_kernel<n, true>), dim3(grid), dim3(WG), 0, s, W + k0, (int)N, kseg, (int)K,   \
                               x + k0, y, tile);                                                              \
        else                                                                                                  \
            hipLaunchKernelGGL((head_kernel<n, false>), dim3(grid), dim3(WG), 0, s, W + k0, (int)N, kseg, (int)K,  \
                               x + k0, y, tile);                                                              \
        break;
            LB_HEAD(1) LB_HEAD(2) LB_HEAD(3) LB_HEAD(4) LB_HEAD(5) LB_HEAD(6) LB_HEAD(7) LB_HEAD(8)
#undef LB_HEAD
        default:
            return hipErrorInvalidValue;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace lb
