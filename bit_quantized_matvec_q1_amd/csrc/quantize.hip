// Activation quantisers, the one-time weight layout conversion and small fills.
#include "lowbit_internal.h"

namespace lb {

// q8_0 (bankml technical report, section III.2: blocks of 32 signed bytes with their own half-precision
// scale, 127 / max|x| with round-half-to-even): amax is exact, the stored scale is fp16_rne(amax / 127)
// of the correctly rounded fp32 quotient, the multiplier 127 / amax a correctly rounded fp32 quotient
// (0 when amax = 0), and each q round-half-even of the fp32 product.
//
// Eight lanes per block, one float4 each, so a wave reads 1 KiB of consecutive activations and writes
// 256 consecutive bytes of q; the block's amax is the maximum over its eight lanes (exact in any order).
// Workgroups hold whole blocks (WG is a multiple of 8), so a block's lanes are all in range or all out.
__global__ __launch_bounds__(WG) void quantize_q8_0_kernel(const float *__restrict__ x, int64_t nblocks,
                                                           int8_t *__restrict__ xq, uint16_t *__restrict__ xs)
{
    const int64_t c = (int64_t)blockIdx.x * WG + threadIdx.x; // float4 chunk: block c / 8, values 4 (c % 8) ..
    const bool in = (c >> 3) < nblocks;
    const float4 v = in ? reinterpret_cast<const float4 *>(x)[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const float amax = q8_0_block_amax8(v);
    if (!in)
        return;
    reinterpret_cast<uint32_t *>(xq)[c] = q8_0_pack4(v, amax);
    if ((c & 7) == 0)
        xs[c >> 3] = q8_0_scale_bits(amax);
}

hipError_t launch_quantize_q8_0(const float *x, int64_t M, int64_t K, int8_t *xq, uint16_t *xs, hipStream_t s)
{
    const int64_t nblocks = M * (K / QK8);
    const int64_t grid = (nblocks * 8 + WG - 1) / WG;
    hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)grid), dim3(WG), 0, s, x, nblocks, xq, xs);
    return hipGetLastError();
}

// Per-token int8 (tritium "Architecture", section 1): with the row's amax, s = amax / 127 and
// q = clamp(rne(x * (127 / amax)), -128, 127); these give the multiplier and one q.
inline __device__ float i8_row_multiplier(float amax) { return amax > 0.0f ? 127.0f / amax : 0.0f; }
inline __device__ float i8_row_scale(float amax) { return amax / 127.0f; }
inline __device__ int quantize_i8(float x, float id)
{
    return (int)fminf(fmaxf(rintf(x * id), -128.0f), 127.0f);
}

// Per-token int8 (tritium "Architecture", section 1: int8 activations; one absmax scale per token).
// One workgroup per row: amax over the row, s = amax / 127, q = clamp(rne(x * (127 / amax)), -128, 127).
__device__ __forceinline__ float block_max(float v, float *red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])); // max is exact in any order
}

// Rows whose K is a multiple of 4 and at most 4 * WG * NC: each thread holds NC float4 chunks of the row
// in registers (all loads in flight together), so the row is read once; q leaves as packed dwords.
template <int NC>
__global__ __launch_bounds__(WG) void quantize_i8_row_vec_kernel(const float *__restrict__ x, int64_t K,
                                                                 int8_t *__restrict__ xq, float *__restrict__ xs)
{
    __shared__ float red[WG / 64];
    const int64_t m = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + m * K);
    const int nch = (int)(K / 4);
    float4 v[NC];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int i = (int)threadIdx.x + c * WG;
        v[c] = i < nch ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[c].x), fabsf(v[c].y)), fmaxf(fabsf(v[c].z), fabsf(v[c].w))));
    }
    amax = block_max(amax, red);
    const float id = i8_row_multiplier(amax);
    if (threadIdx.x == 0)
        xs[m] = i8_row_scale(amax);
    uint32_t *qr = reinterpret_cast<uint32_t *>(xq + m * K);
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int i = (int)threadIdx.x + c * WG;
        if (i < nch)
            qr[i] = (uint32_t)(quantize_i8(v[c].x, id) & 0xff) | (uint32_t)(quantize_i8(v[c].y, id) & 0xff) << 8 |
                    (uint32_t)(quantize_i8(v[c].z, id) & 0xff) << 16 | (uint32_t)(quantize_i8(v[c].w, id) & 0xff) << 24;
    }
}

// Any K: two passes over the row.
__global__ __launch_bounds__(WG) void quantize_i8_row_kernel(const float *__restrict__ x, int64_t K,
                                                             int8_t *__restrict__ xq, float *__restrict__ xs)
{
    __shared__ float red[WG / 64];
    const int64_t m = blockIdx.x;
    const float *xr = x + m * K;
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += WG)
        amax = fmaxf(amax, fabsf(xr[k]));
    amax = block_max(amax, red);
    const float id = i8_row_multiplier(amax);
    if (threadIdx.x == 0)
        xs[m] = i8_row_scale(amax);
    int8_t *qr = xq + m * K;
    for (int64_t k = threadIdx.x; k < K; k += WG)
        qr[k] = (int8_t)quantize_i8(xr[k], id);
}

hipError_t launch_quantize_i8_row(const float *x, int64_t M, int64_t K, int8_t *xq, float *xs, hipStream_t s)
{
    const dim3 grid((unsigned)M), block(WG);
    const int64_t nch = K / 4;
    if (K % 4 == 0 && nch <= WG)
        hipLaunchKernelGGL(quantize_i8_row_vec_kernel<1>, grid, block, 0, s, x, K, xq, xs);
    else if (K % 4 == 0 && nch <= 2 * WG)
        hipLaunchKernelGGL(quantize_i8_row_vec_kernel<2>, grid, block, 0, s, x, K, xq, xs);
    else if (K % 4 == 0 && nch <= 4 * WG)
        hipLaunchKernelGGL(quantize_i8_row_vec_kernel<4>, grid, block, 0, s, x, K, xq, xs);
    else if (K % 4 == 0 && nch <= 8 * WG)
        hipLaunchKernelGGL(quantize_i8_row_vec_kernel<8>, grid, block, 0, s, x, K, xq, xs);
    else
        hipLaunchKernelGGL(quantize_i8_row_kernel, grid, block, 0, s, x, K, xq, xs);
    return hipGetLastError();
}

// ggml blocks [N][nb][2 + 16] <-> device layout [N][nb][16] code records, then [N][nb] binary16 scales.
// Planar beats are copied unchanged.  One thread per block; byte accesses (the ggml stream has 18-byte
// records, so nothing in it is aligned).
// Q1_0 sign bits in the device layout.  In a ggml block, dword r (bytes 4r..4r+3) holds the signs of
// weights 32r..32r+31, weight 32r + 8m + k at bit 8m + k.  The device record moves that bit to bit 4k + r
// of dword m, so that masking any device dword with 0x11111111 << r isolates eight weights of q8_0
// activation block r, one per nibble, already in place for a nibble dot product.
__device__ __forceinline__ uint32_t spread8_nibbles(uint32_t x) // bit k of an 8-bit value -> bit 4k
{
    x = (x | (x << 12)) & 0x000F000Fu;
    x = (x | (x << 6)) & 0x03030303u;
    x = (x | (x << 3)) & 0x11111111u;
    return x;
}

__device__ __forceinline__ uint32_t gather8_nibbles(uint32_t x) // bit 4k -> bit k (other bits zero)
{
    x &= 0x11111111u;
    x = (x | (x >> 3)) & 0x03030303u;
    x = (x | (x >> 6)) & 0x000F000Fu;
    x = (x | (x >> 12)) & 0x000000FFu;
    return x;
}

__device__ __forceinline__ void q1_to_device(const uint32_t (&nat)[4], uint32_t (&dev)[4])
{
    for (int m = 0; m < 4; m++) {
        uint32_t v = 0;
        for (int r = 0; r < 4; r++)
            v |= spread8_nibbles((nat[r] >> (8 * m)) & 0xFFu) << r;
        dev[m] = v;
    }
}

__device__ __forceinline__ void q1_from_device(const uint32_t (&dev)[4], uint32_t (&nat)[4])
{
    for (int r = 0; r < 4; r++) {
        uint32_t v = 0;
        for (int m = 0; m < 4; m++)
            v |= gather8_nibbles(dev[m] >> r) << (8 * m);
        nat[r] = v;
    }
}

__global__ __launch_bounds__(WG) void pack_kernel(int fmt, const uint8_t *__restrict__ src, int64_t nblk,
                                                  uint8_t *__restrict__ dst, int unpack)
{
    const int64_t b = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (b >= nblk)
        return;
    if (fmt == LB_TERNARY_PLANAR) {
        for (int i = 0; i < 16; i++)
            dst[b * 16 + i] = src[b * 16 + i];
        return;
    }
    if (fmt == LB_TERNARY_B3) {
        // base-3 byte v <-> the 8-bit fraction b = ceil(256 v / 243) the decode kernel reads (v = 243 b >> 8)
        for (int i = 0; i < 16; i++) {
            const uint32_t v = src[b * 16 + i];
            dst[b * 16 + i] = (uint8_t)(unpack ? (243u * v) >> 8 : (256u * v + 242u) / 243u);
        }
        return;
    }
    if (fmt == LB_Q8_0) {
        // 34-byte block (binary16 scale, 32 weight bytes) <-> a 32-byte record + the scale in the scale array
        if (!unpack) {
            for (int i = 0; i < 32; i++)
                dst[b * 32 + i] = src[b * 34 + 2 + i];
            dst[nblk * 32 + b * 2 + 0] = src[b * 34 + 0];
            dst[nblk * 32 + b * 2 + 1] = src[b * 34 + 1];
        } else {
            for (int i = 0; i < 32; i++)
                dst[b * 34 + 2 + i] = src[b * 32 + i];
            dst[b * 34 + 0] = src[nblk * 32 + b * 2 + 0];
            dst[b * 34 + 1] = src[nblk * 32 + b * 2 + 1];
        }
        return;
    }
    // 16 code bytes of an 18-byte ggml block <-> one 16-byte device record (+ the binary16 scale in the
    // scale array); Q1_0 records also permute their bits (above), Q2_0_g64 records keep them as they are
    const uint8_t *in = unpack ? src + b * 16 : src + b * 18 + 2;
    uint8_t *out = unpack ? dst + b * 18 + 2 : dst + b * 16;
    uint32_t w[4], o[4];
    for (int d = 0; d < 4; d++)
        w[d] = (uint32_t)in[4 * d] | ((uint32_t)in[4 * d + 1] << 8) | ((uint32_t)in[4 * d + 2] << 16) |
               ((uint32_t)in[4 * d + 3] << 24);
    if (fmt == LB_Q1_0) {
        if (unpack)
            q1_from_device(w, o);
        else
            q1_to_device(w, o);
    } else {
        for (int d = 0; d < 4; d++)
            o[d] = w[d];
    }
    for (int d = 0; d < 4; d++)
        for (int i = 0; i < 4; i++)
            out[4 * d + i] = (uint8_t)(o[d] >> (8 * i));
    if (!unpack) {
        dst[nblk * 16 + b * 2 + 0] = src[b * 18 + 0];
        dst[nblk * 16 + b * 2 + 1] = src[b * 18 + 1];
    } else {
        dst[b * 18 + 0] = src[nblk * 16 + b * 2 + 0];
        dst[b * 18 + 1] = src[nblk * 16 + b * 2 + 1];
    }
}

hipError_t launch_pack(int fmt, const uint8_t *blocks, int64_t N, int64_t K, uint8_t *packed, bool unpack,
                       hipStream_t s)
{
    const int64_t nblk = fmt == LB_TERNARY_B3 ? N * ((K + 79) / 80) // beats of 16 bytes
                                              : N * (K / (fmt == LB_Q1_0 ? 128 : fmt == LB_Q8_0 ? 32 : 64));
    const int64_t grid = (nblk + WG - 1) / WG;
    if (unpack)
        hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(WG), 0, s, fmt, (const uint8_t *)packed, nblk,
                           (uint8_t *)blocks, 1);
    else
        hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(WG), 0, s, fmt, blocks, nblk, packed, 0);
    return hipGetLastError();
}

template <typename T> __global__ __launch_bounds__(WG) void fill_zero_kernel(T *__restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i < n)
        y[i] = T(0);
}

hipError_t launch_fill_zero(float *y, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(fill_zero_kernel<float>, dim3((unsigned)((n + WG - 1) / WG)), dim3(WG), 0, s, y, n);
    return hipGetLastError();
}

hipError_t launch_fill_zero_i32(int32_t *y, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(fill_zero_kernel<int32_t>, dim3((unsigned)((n + WG - 1) / WG)), dim3(WG), 0, s, y, n);
    return hipGetLastError();
}

} // namespace lb
