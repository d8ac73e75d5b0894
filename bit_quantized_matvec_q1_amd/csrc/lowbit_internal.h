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
constexpr int slice_weights(int fmt) { return fmt == LB_Q1_0 ? 128 : 64; }

inline __device__ float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

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

hipError_t launch_head(const uint16_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s);

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
};

struct TileRef {        // one workgroup of a batched launch: its product and first row
    int32_t prod, row0;
};

struct BatchGroup {
    int fmt;
    int cfg_a;               // the kernel configuration of this launch group
    int full;                // every product's row has exactly L * S slices of the configuration
    int32_t ntiles;          // workgroups in the launch
    const DevDesc *desc;     // device
    const TileRef *tiles;    // device, one per workgroup
};

int matvec_config(int fmt, int64_t K);           // configuration index for a product, -1 if none
int matvec_config_rows_per_iter(int fmt, int cfg); // rows one workgroup covers per iteration
bool matvec_config_full(int fmt, int cfg, int64_t K); // a row of K has exactly L * S slices
hipError_t launch_matvec_batched(const BatchGroup &g, hipStream_t s, size_t lds_bytes);
int matvec_batched_blocks_per_cu(int fmt, int cfg, bool full, size_t lds_bytes); // resident workgroups per CU
int matvec_stage_bytes(int fmt, int64_t K); // LDS bytes of one product's staged activation

} // namespace lb
