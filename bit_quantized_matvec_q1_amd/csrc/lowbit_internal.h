// Internal declarations shared by the HIP translation units of liblowbit.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/lowbit.h"

namespace lb {

constexpr int QK8 = 32;   // activations per q8_0 block
constexpr int WG = 256;   // threads per workgroup for the streaming kernels (4 wave64)

// Weights per 16-byte code record ("slice"): one Q2_0_g64 block, one Q1_0 block's sign bits, one
// planar beat.  The device layout of the ggml formats is [N][K/QK][16 B] code records followed by
// [N][K/QK] binary16 scales.
constexpr int slice_weights(int fmt) { return fmt == LB_Q1_0 ? 128 : fmt == LB_Q8_0 ? 32 : 64; }

inline __device__ float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// --- cross-lane sum over aligned groups of L lanes with DPP (no LDS round trip).  The total ends up in
// the group's last lane (li == L - 1); for L <= 16 every lane of the group holds it.
// q8_0 (bankml technical report, section III.2: blocks of 32 signed bytes with their own half-precision
// scale, 127 / max|x| with round-half-to-even), as computed by eight lanes per block, one float4 each:
// the block's amax is the maximum over the eight lanes (exact in any order), the multiplier 127 / amax a
// correctly rounded fp32 quotient (0 when amax = 0), each q round-half-even of the fp32 product, and the
// stored scale fp16_rne(amax / 127) of the correctly rounded fp32 quotient.  Every quantiser of the
// library goes through these two functions, so they all give the same bytes.
inline __device__ float q8_0_block_amax8(float4 v)
{
    // maximum over the 8 lanes by DPP: swap neighbours, swap pairs (each quad then holds its maximum), then
    // mirror within the 8 (lane i meets lane 7 - i of the other quad)
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1, 0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E, 0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x141, 0xF, 0xF, false)));
    return amax;
}
inline __device__ uint32_t q8_0_pack4(float4 v, float amax)
{
    const float id = amax > 0.0f ? 127.0f / amax : 0.0f;
    return (uint32_t)((int)rintf(v.x * id) & 0xff) | (uint32_t)((int)rintf(v.y * id) & 0xff) << 8 |
           (uint32_t)((int)rintf(v.z * id) & 0xff) << 16 | (uint32_t)((int)rintf(v.w * id) & 0xff) << 24;
}
inline __device__ uint16_t q8_0_scale_bits(float amax) { return __half_as_ushort(__float2half_rn(amax / 127.0f)); }

template <int L> inline __device__ int group_sum_i(int v)
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

template <int L> inline __device__ float group_sum_f(float v)
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

// --- launchers (each validates nothing: the ABI layer has done it) ------------------------------

hipError_t launch_quantize_q8_0(const float *x, int64_t M, int64_t K, int8_t *xq, uint16_t *xs, hipStream_t s);
hipError_t launch_quantize_i8_row(const float *x, int64_t M, int64_t K, int8_t *xq, float *xs, hipStream_t s);
hipError_t launch_pack(int fmt, const uint8_t *blocks, int64_t N, int64_t K, uint8_t *packed, bool unpack,
                       hipStream_t s);
hipError_t launch_fill_zero(float *y, int64_t n, hipStream_t s);
hipError_t launch_fill_zero_i32(int32_t *y, int64_t n, hipStream_t s);

// decode products; sums != nullptr selects the instantiation that also stores the integer sums
hipError_t launch_matvec(int fmt, const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *xq,
                         const void *xscale, float *y, int32_t *sums, hipStream_t s);
bool matvec_supported_k(int fmt, int64_t K);

hipError_t launch_gemm(int fmt, const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *Xq,
                       const void *Xscale, int64_t M, float *Y, int32_t *sums, hipStream_t s);

hipError_t launch_read_probe(const void *buf, int64_t nbytes, uint32_t *sink, hipStream_t s);

hipError_t launch_head(const uint16_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s);
hipError_t launch_head_i8(const int8_t *W, const float *sw, int64_t N, int64_t K, const float *x, float *y,
                          hipStream_t s);

// batched decode: a device table of products, grouped by kernel configuration
struct DevDesc {
    const uint8_t *W;
    const int8_t *xq;
    const void *xscale;
    float *y;
    int32_t N, K;
    float w_scale;
    int32_t cfg;        // index into the format's configuration table
    int32_t tile_rows;  // rows per tile
    const float *x;     // fp32 activations quantised in the launch (LB_ACT_F32_Q8_0), else null
};

struct TileRef {        // one workgroup of a batched launch: its product and first row
    int32_t prod, row0;
};

struct BatchGroup {
    int fmt;
    int cfg_a;               // the kernel configuration of this launch group
    int full;                // every product's row has exactly L * S slices of the configuration
    int qin;                 // the products' activations are fp32, quantised to q8_0 in the launch
    int32_t ntiles;          // workgroups in the launch
    const DevDesc *desc;     // device
    const TileRef *tiles;    // device, one per workgroup
};

int matvec_config(int fmt, int64_t K);           // configuration index for a product, -1 if none
int matvec_config_rows_per_iter(int fmt, int cfg); // rows one workgroup covers per iteration
bool matvec_config_full(int fmt, int cfg, int64_t K); // a row of K has exactly L * S slices
hipError_t launch_matvec_batched(const BatchGroup &g, hipStream_t s, size_t lds_bytes);
int matvec_batched_blocks_per_cu(int fmt, int cfg, bool full, bool qin, size_t lds_bytes); // resident per CU
// LDS bytes of one row of K activations quantised to q8_0 in a launch (int8 [K], then binary16 [K/32])
inline int64_t q8_0_lds_bytes(int64_t K) { return (K + K / 16 + 15) / 16 * 16; }
int matvec_stage_bytes(int fmt, int64_t K); // LDS bytes of one product's staged activation

// Q8_0 weights x q8_0 activations (q8.hip): configurations in their own index space
int q8_config(int64_t K);
int q8_rows_per_iter(int cfg);
size_t q8_stage_bytes(int64_t K);
hipError_t launch_q8(const uint8_t *W, int64_t N, int64_t K, const int8_t *xq, const uint16_t *xs, float *y,
                     int32_t *sums, hipStream_t s);
hipError_t launch_q8_batched(const BatchGroup &g, size_t lds, hipStream_t s);
int q8_blocks_per_cu(int cfg, size_t lds);

// the planar product by bit-serial popcounts (popcount.hip): a third implementation for differential tests
hipError_t launch_popcount(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *xq, const float *xs,
                           float *y, int32_t *sums, hipStream_t s);

// base-3 ternary beats x per-token int8 activations (b3.hip)
int b3_config(int64_t K);
int b3_rows_per_iter(int cfg);
size_t b3_stage_bytes(int64_t K);
hipError_t launch_b3(const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *xq, const float *xs, float *y,
                     int32_t *sums, hipStream_t s);
hipError_t launch_b3_batched(const BatchGroup &g, size_t lds, hipStream_t s);
int b3_blocks_per_cu(int cfg, size_t lds);

} // namespace lb
