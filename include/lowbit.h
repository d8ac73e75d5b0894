/*
 * lowbit.h -- C ABI of liblowbit.so: products of packed low-bit weights with int8 activations on one
 * AMD Instinct MI355X (gfx950).
 *
 * Weight formats:
 *   LB_Q1_0           ggml Q1_0: 18-byte blocks of 128 weights, binary16 scale d then 16 bytes of sign
 *                     bits, least-significant bit first; weight = d * (bit ? +1 : -1).
 *                     (bankml technical report, section III.2 "The Q1_0 format and its arithmetic".)
 *   LB_Q2_0_G64       ggml Q2_0 with group 64: 18-byte blocks of 64 weights, binary16 d then 16 bytes of
 *                     2-bit codes, lowest bits first; weight = (code - 1) * d, code in {0,1,2,3}.
 *                     (bankml technical report, section III.5 "The Q2_0_g64 (ternary) kernel".)
 *   LB_TERNARY_PLANAR the planar ternary beat: 16 bytes per 64 consecutive columns of one row,
 *                     {u64 pos, u64 neg}, column c at bit c; weight = pos_c - neg_c, times one fp32
 *                     per-tensor scale.  (tritium "Architecture", section 2 "bit planes".)
 *   LB_Q8_0           ggml Q8_0 weights: 34-byte blocks of 32 weights, binary16 scale d then 32 signed
 *                     bytes; weight = d * byte.  The q8_0 block of the bankml technical report, section
 *                     III.2, used for weights ("Q8_0 weights" and vec_dot_q8_0_q8_0 for the KV cache in
 *                     the bankml build history's 0.3.9 entry).  Decode takes K up to 16384; prefill
 *                     (lowbit_gemm, lowbit_block_sums with M > 1) also needs K % 128 == 0 (LB_ESHAPE).
 *   LB_TERNARY_B3     base-3 ternary beats: 16 bytes per 80 consecutive columns of one row, byte j holding
 *                     columns 5j..5j+4 as the integer sum_t (w + 1) * 3^t, lowest digit first (0..242);
 *                     a row of K columns (K % 64 == 0) takes ceil(K/80) beats, the columns past K coded 0.
 *                     Weight = w times one fp32 per-tensor scale, with per-token int8 activations and the
 *                     planar output rule.  Five trits per byte (bankml technical report, section III.8
 *                     "Information"); base-3 packing of the planar body at 1.6 bits per weight (tritium
 *                     "Architecture", section 10).  Decode only; bytes above 242 are not base-3 bytes.
 *
 * Activation formats:
 *   LB_ACT_Q8_0       ggml q8_0: int8 xq[M][K] plus binary16 scales xscale[M][K/32]; one block of 32
 *                     activations per scale (bankml technical report, section III.2).  Used with the
 *                     two ggml weight formats.
 *   LB_ACT_I8_ROW     int8 xq[M][K] plus one fp32 scale per row (per token), xscale[M] (tritium
 *                     "Architecture", section 1: activations are int8).  Used with the planar format.
 *   LB_ACT_F32_Q8_0   fp32 x[K], quantised to q8_0 by the batch itself, with exactly the arithmetic of
 *                     lowbit_quantize_act(LB_ACT_Q8_0) (so the results are bit-identical to quantising
 *                     first).  Batched decode of LB_Q1_0 and LB_Q2_0_G64 only: a product that depends on the
 *                     previous one's output then needs no quantise call of its own.  Rows of at most 8192
 *                     columns are quantised inside the products' own launch (every workgroup quantises
 *                     the row it stages); a batch from lowbit_batch_create quantises longer rows with one
 *                     launch per distinct (x, K) ahead of its products, into device memory it owns.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated otherwise; the caller owns every buffer.  No
 *     entry point below allocates, frees or synchronises, except lowbit_batch_create/destroy, which
 *     are set-up calls.
 *   - Work is enqueued asynchronously on the caller's HIP stream `s` (NULL = the null stream).
 *   - Arguments are validated on the host before anything is launched; an error launches nothing.
 *     There is no fallback path: an unsupported device or shape is an error, never a slower kernel.
 *   - Outputs are row-major fp32.  Integer per-block sums are exact; fp32 outputs follow the
 *     definition  y = sum_b d_w[b] * sum_{j in b} d_x[j] * isum[j]  up to fp32 rounding order.
 *   - N == 0 or M == 0 is an empty product: LB_OK, nothing launched.  K == 0 writes zeros.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LB_Q1_0 = 1, LB_Q2_0_G64 = 2, LB_TERNARY_PLANAR = 3, LB_Q8_0 = 4, LB_TERNARY_B3 = 5 } lb_wfmt;
typedef enum { LB_ACT_Q8_0 = 1, LB_ACT_I8_ROW = 2, LB_ACT_F32_Q8_0 = 3 } lb_afmt;

typedef enum {
    LB_OK = 0,
    LB_EINVAL = 1,       /* null pointer, unknown enum, or a weight/activation format pairing that is not defined */
    LB_ESHAPE = 2,       /* negative size, K not a multiple of the weight block (128, 64, 64, 32, 64), or over a limit */
    LB_EALIGN = 3,       /* a pointer is not aligned as its argument requires */
    LB_EUNSUPPORTED = 4, /* the current device is not gfx950, or the entry point has no kernel for the format */
    LB_EDEVICE = 5,      /* a HIP call failed; lowbit_last_error() holds the runtime's message */
    LB_ENOMEM = 6        /* host memory for a set-up object (lowbit_batch_create) could not be allocated */
} lb_status;

/* Human-readable name of a status code (static string). */
const char *lowbit_status_str(lb_status st);

/* Message of the last error raised by this library on the calling thread ("" if none; at most 511
 * characters, valid until the thread's next failing call). */
const char *lowbit_last_error(void);

/*
 * Bytes of the device layout of an N x K weight tensor in format `fmt`: 18 per Q1_0 / Q2_0_g64 block (128
 * or 64 weights), 34 per Q8_0 block (32 weights), 16 per planar beat (64 columns) or base-3 beat (80
 * columns, ceil(K/80) per row) -- the same count as the on-disk format (1.125, 2.25, 8.5, 2 and 1.6 bits
 * per weight; bankml technical report sections III.2, III.5 and III.8).
 * Returns -1 for a bad format or shape.
 */
int64_t lowbit_weight_bytes(int fmt, int64_t N, int64_t K);

/*
 * One-time conversion of a ggml block stream into the device layout the kernels read.
 *   blocks: device, N rows x K/QK blocks of 18 bytes (34 for Q8_0), row-major, no alignment requirement.
 *   packed: device, lowbit_weight_bytes(fmt, N, K) bytes, 16-byte aligned.  Layout: all 16-byte code
 *           records row-major ([N][K/QK][16]; Q8_0: 32-byte records of the block's weight bytes,
 *           [N][K/32][32]), then all binary16 scales row-major ([N][K/QK]).
 *           A Q2_0_g64 record is the block's 16 code bytes as they are.  A Q1_0 record permutes the
 *           block's 128 sign bits: the sign of weight 32r + 8m + k (r, m in 0..3, k in 0..7), at bit
 *           8m + k of little-endian dword r in the ggml block, sits at bit 4k + r of dword m, so one
 *           mask (0x11111111 << r) isolates eight weights of activation block r as nibbles.
 * Lossless (lowbit_unpack_weights is its inverse).  For LB_TERNARY_PLANAR the beat stream already is
 * the device layout (tritium "Architecture", section 2: the file layout is the beat stream) and pack
 * copies it unchanged.  For LB_TERNARY_B3 pack keeps the beat stream and writes each base-3 byte v as
 * b = ceil(256 v / 243), whose leading m base-3 digits are floor(3^m b / 256) (unpack: v = 243 b >> 8).
 */
lb_status lowbit_pack_weights(int fmt, const void *blocks, int64_t N, int64_t K, void *packed, hipStream_t s);
lb_status lowbit_unpack_weights(int fmt, const void *packed, int64_t N, int64_t K, void *blocks, hipStream_t s);

/*
 * Quantise fp32 activation rows x[M][K] (device, 16-byte aligned).
 *   LB_ACT_Q8_0:  per block of 32, amax = max|x|; xscale (uint16 binary16, [M][K/32]) = fp16_rne(amax/127);
 *                 xq = round_half_even(x * (127/amax)) in fp32, 0 when amax = 0.  K % 32 == 0.
 *                 (bankml technical report, section III.2: 127 / max|x| with round-half-to-even.)
 *   LB_ACT_I8_ROW: per row, amax over the row; xscale (fp32, [M]) = amax/127;
 *                 xq = clamp(round_half_even(x * (127/amax)), -128, 127).
 *   xq: device int8 [M][K], 16-byte aligned.  xscale: device, 4-byte aligned.
 */
lb_status lowbit_quantize_act(int afmt, const float *x, int64_t M, int64_t K, int8_t *xq, void *xscale,
                              hipStream_t s);

/*
 * Batch-1 decode product y[N] = W . dequant(xq): the select-accumulate of the weights over the int8
 * activations, exact integer sums per activation block, scaled per block in fp32
 * (bankml technical report, sections III.2, III.5 and III.8; tritium "Architecture", sections 1-2).
 *   W:      device layout of the N x K tensor (lowbit_pack_weights; planar beats as they are), 16-byte aligned.
 *   w_tensor_scale: planar and base-3 per-tensor scale s_w (y = ((float)acc * s_x) * s_w); ignored otherwise.
 *   afmt:   LB_ACT_Q8_0 for the ggml formats, LB_ACT_I8_ROW for planar and base-3 beats.
 *   xq:     device int8 [K], 16-byte aligned.  xscale: binary16 [K/32] or one fp32, 4-byte aligned.
 *   y:      device fp32 [N], 4-byte aligned.
 * Limits: K <= 32768 (16384 for LB_Q8_0, 30720 for LB_TERNARY_B3) and N <= 2^31 - 1; the weight tensor must
 * be smaller than 4 GiB.
 */
lb_status lowbit_matvec(int fmt, const void *W, int64_t N, int64_t K, float w_tensor_scale, int afmt,
                        const int8_t *xq, const void *xscale, float *y, hipStream_t s);

/*
 * Prefill product Y[M][N] = dequant(Xq) . W^T for M activation rows: the same per-block integer sums
 * as lowbit_matvec, computed as int8 matrix-core products over weight tiles unpacked to int8 in LDS,
 * then scaled per block in fp32 (bankml technical report, section III.3: a tile that loads each weight
 * block once and applies it to several activation columns; tritium "Architecture", section 3:
 * prefill runs compute-bound).
 *   Xq: device int8 [M][K], 16-byte aligned; Xscale: binary16 [M][K/32] (ggml formats) or fp32 [M].
 *   Y:  device fp32 [M][N], 4-byte aligned.
 * Limits (else LB_ESHAPE): those of lowbit_matvec, M * N < 2^31 outputs, M * K < 2^32 activation bytes,
 * and K % 128 == 0 for LB_Q8_0.  LB_TERNARY_B3 has no prefill kernel (LB_EUNSUPPORTED).
 */
lb_status lowbit_gemm(int fmt, const void *W, int64_t N, int64_t K, float w_tensor_scale, int afmt,
                      const int8_t *Xq, const void *Xscale, int64_t M, float *Y, hipStream_t s);

/*
 * The exact integer sums the products above are built from, written by the same kernels (M == 1: the
 * decode kernel; M > 1: the prefill kernel) instantiated with one extra store:
 *   ggml formats: sums int32 [M][N][K/32], sums[m][n][j] = sum over activation block j of w * q;
 *   planar:       sums int32 [M][N], the whole row's select-accumulate.
 */
lb_status lowbit_block_sums(int fmt, const void *W, int64_t N, int64_t K, int afmt, const int8_t *Xq,
                            const void *Xscale, int64_t M, int32_t *sums, hipStream_t s);

/*
 * Dense bf16 head matvec y[N] = sum_k bf16_to_f32(W[n][k]) * x[k], accumulated in fp32
 * (tritium "Architecture", section 3: the dense head is the largest single stream; bf16 storage).
 *   W: device uint16 bf16 bits [N][K], 16-byte aligned, K % 8 == 0; x: device fp32 [K], 16-byte aligned;
 *   y: device fp32 [N].  K must be a multiple of 8 and at most 32768 and the weights smaller than 4 GiB;
 *   otherwise LB_ESHAPE.  Rows longer than 4096 columns run as column segments of 4096, one launch each on
 *   `s`: the first writes y, each later one adds its partial sums to it (in that fixed order).
 */
lb_status dense_head_matvec(const uint16_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s);

/*
 * The planar product computed by bit-serial popcounts: with q = sum_p t_p bit_p(q) (t_p = 2^p, t_7 = -128),
 * acc = sum_p t_p (popcount(pos & Q_p) - popcount(neg & Q_p)) over the activation bit planes Q_p (tritium
 * "Architecture", section 4.3 "About popcount": the formulation kept as a third independent implementation
 * for differential tests; section 5: the implementations must agree).  Same arguments and output rule as
 * lowbit_matvec for LB_TERNARY_PLANAR with LB_ACT_I8_ROW activations, plus row_sums (device int32 [N],
 * 4-byte aligned, may be NULL): the exact integer acc per row.  y may be NULL when row_sums is not.
 * Results are bit-identical to lowbit_matvec / lowbit_block_sums.  K <= 8192; otherwise LB_ESHAPE.
 */
lb_status lowbit_matvec_popcount(const void *W, int64_t N, int64_t K, float w_tensor_scale, const int8_t *xq,
                                 const float *xscale, float *y, int32_t *row_sums, hipStream_t s);

/*
 * int8 dense head matvec y[n] = row_scale[n] * sum_k W[n][k] * x[k], accumulated in fp32 (tritium
 * "Architecture", section 10: int8 is the obvious move for the head, at half the bf16 head's bytes; the
 * reading taken: symmetric int8 weights with one fp32 scale per row).
 *   W: device int8 [N][K], 16-byte aligned; row_scale: device fp32 [N], 4-byte aligned; x: device fp32 [K],
 *   16-byte aligned; y: device fp32 [N], 4-byte aligned.  K must be a multiple of 16 and at most 32768 and
 *   the weights smaller than 4 GiB; otherwise LB_ESHAPE.  Rows longer than 8192 columns run as column
 *   segments of 8192, one launch each on `s`: the first writes row_scale[n] times its partial sum, each
 *   later one adds its own (in that fixed order).
 */
lb_status dense_head_matvec_i8(const int8_t *W, const float *row_scale, int64_t N, int64_t K, const float *x, float *y,
                               hipStream_t s);

/*
 * Many independent decode products in ONE launch (a token's work list).  A batch is a set-up object:
 * lowbit_batch_create validates the host-side list, and copies it with its tile table into device
 * memory it allocates once; lowbit_matvec_batched then enqueues, on `s`, one kernel per (weight format,
 * kernel configuration) group of the list -- one or two for a model's token -- over every product.
 * (tritium "Architecture", section 7: handing each small matvec to a pool costs more than the matvec
 * itself -- dispatch, not arithmetic, is what a token's many products must amortise.)
 */
typedef struct {
    int32_t fmt;          /* lb_wfmt */
    int32_t afmt;         /* lb_afmt, paired with fmt as in lowbit_matvec */
    int64_t N, K;         /* rows, columns */
    const void *W;        /* device layout, 16-byte aligned */
    float w_tensor_scale; /* planar only */
    const int8_t *xq;     /* device int8 [K] (ignored for LB_ACT_F32_Q8_0) */
    const void *xscale;   /* device binary16 [K/32] or fp32 [1] (ignored for LB_ACT_F32_Q8_0) */
    float *y;             /* device fp32 [N] */
    const float *x;       /* LB_ACT_F32_Q8_0 only: device fp32 [K], 16-byte aligned; else ignored */
} lb_matvec_desc;

typedef struct lb_batch lb_batch;

/* list: HOST array of n descriptors (n >= 1).  On success *out owns device memory until destroyed;
 * lowbit_batch_destroy frees it (hipFree, which waits for the device), so no launch may use it after.
 * The buffers the descriptors point to must stay valid while the batch is used.  A descriptor with
 * afmt LB_ACT_F32_Q8_0 takes its activations from x and needs fmt LB_Q1_0 or LB_Q2_0_G64 (else
 * LB_EUNSUPPORTED); null x is LB_EINVAL, x not 16-byte aligned LB_EALIGN. */
lb_status lowbit_batch_create(const lb_matvec_desc *list, int32_t n, lb_batch **out);
lb_status lowbit_matvec_batched(const lb_batch *b, hipStream_t s);
/* Kernel launches one lowbit_matvec_batched call makes (the quantise launches of long fp32 rows plus one
 * per weight format and kernel configuration present); -1 for a null batch. */
int32_t lowbit_batch_launches(const lb_batch *b);
void lowbit_batch_destroy(lb_batch *b);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the work list of lowbit_batch_create run in one call, with its
 * descriptor and tile tables held in a fixed device array of LB_STATIC_TABLE_BYTES bytes inside the library
 * instead of memory the library allocates.  Calls no hipMalloc / hipFree; the tile plan is built in host
 * memory on every call.
 *   list: HOST array of n descriptors, validated exactly as by lowbit_batch_create (same status codes);
 *         the same products give bit-identical outputs as a batch of that list (here every fp32 row,
 *         however long, is quantised inside its products' launches).
 *   A list whose tables exceed LB_STATIC_TABLE_BYTES (64 bytes per product plus 8 per row tile: for
 *   example 14,000 single-tile products, or 130,000 tiles -- about 8 GB of Q1_0 / Q2_0 weights in their
 *   64 KiB tiles, 32 GB in 256 KiB tiles) is refused with LB_ESHAPE before anything is enqueued.
 * The tables are copied into the array on `s` (stream-ordered after earlier work on `s`), then the kernels
 * run on `s`.  Every call on one GPU shares that GPU's array, which keeps the last call's tables: calls
 * that overlap on one GPU -- on different streams, or from different host threads without ordering --
 * race and may compute with another call's tables.  Calls queued on one stream are safe.
 */
#define LB_STATIC_TABLE_BYTES (1 << 20)
lb_status lowbit_matvec_batched_static(const lb_matvec_desc *list, int32_t n, hipStream_t s);

/*
 * Measurement helper, not a product: a streaming read of `nbytes` (a multiple of 16, 16-byte aligned) of
 * device memory by 16-byte non-temporal loads, the access pattern of the decode kernels' weight stream,
 * so its rate bounds theirs (tritium "Architecture", section 3: the roofline is measured with a
 * streaming-read probe in the same run).  `sink` (device uint32, at least 65536 entries, 4-byte aligned) is
 * written only when a workgroup's checksum of the bytes equals a fixed constant, so the loads cannot be
 * removed and almost nothing is written.
 */
lb_status lowbit_read_probe(const void *buf, int64_t nbytes, uint32_t *sink, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
