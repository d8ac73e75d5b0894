// The C ABI of liblowbit.so: argument validation, the device check, and dispatch to the kernels.
// Every argument is checked on the host before anything is launched; an error launches nothing and
// there is no fallback path (tritium "Architecture", section 4.2: a pinned kernel errors rather than
// falling back, so a run never measures a different kernel than the one it names).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <queue>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <vector>

#include "lowbit_internal.h"

namespace {

// fixed storage: recording an error never allocates (nothing may throw through the C ABI)
thread_local char g_last_error[512];

lb_status fail(lb_status st, const char *fn, const char *what)
{
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", fn, what);
    return st;
}

lb_status hip_fail(const char *fn, hipError_t e)
{
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s: %s", fn, hipGetErrorName(e), hipGetErrorString(e));
    return LB_EDEVICE;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_wfmt(int f)
{
    return f == LB_Q1_0 || f == LB_Q2_0_G64 || f == LB_TERNARY_PLANAR || f == LB_Q8_0 || f == LB_TERNARY_B3;
}
// K must be a multiple of this (base-3 rows are whole planar widths; their beats hold 80 columns)
int64_t block_weights(int f) { return f == LB_Q1_0 ? 128 : f == LB_Q8_0 ? 32 : 64; }
int64_t block_bytes(int f) { return f == LB_TERNARY_PLANAR ? 16 : f == LB_Q8_0 ? 34 : 18; }
int paired_afmt(int f) { return f == LB_TERNARY_PLANAR || f == LB_TERNARY_B3 ? LB_ACT_I8_ROW : LB_ACT_Q8_0; }
// bytes of an N x K tensor (K a multiple of block_weights)
int64_t tensor_bytes(int f, int64_t N, int64_t K)
{
    if (f == LB_TERNARY_B3)
        return N * ((K + 79) / 80) * 16;
    return N * (K / block_weights(f)) * block_bytes(f);
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices]; // 0 unknown, 1 gfx950, 2 other

// The kernels are written for gfx950 only; any other device is refused.
lb_status check_device(const char *fn)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(LB_EUNSUPPORTED, fn, "no HIP device is available (a gfx950 GPU is required)");
    }
    int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(LB_EUNSUPPORTED, fn, "cannot query the current device");
        }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_relaxed);
    }
    if (st != 1)
        return fail(LB_EUNSUPPORTED, fn, "the current device is not gfx950");
    return LB_OK;
}

// Shared checks of a decode product's arguments (lowbit_matvec and each batch entry).
lb_status check_product(const char *fn, int fmt, const void *W, int64_t N, int64_t K, int afmt, const void *xq,
                        const void *xscale, const void *y)
{
    if (!is_wfmt(fmt) || (afmt != LB_ACT_Q8_0 && afmt != LB_ACT_I8_ROW))
        return fail(LB_EINVAL, fn, "unknown weight or activation format");
    if (afmt != paired_afmt(fmt))
        return fail(LB_EINVAL, fn, "activation format does not match the weight format "
                                   "(Q1_0/Q2_0_g64/Q8_0 take LB_ACT_Q8_0, planar takes LB_ACT_I8_ROW)");
    if (N < 0 || K < 0)
        return fail(LB_ESHAPE, fn, "negative size");
    if (K % block_weights(fmt))
        return fail(LB_ESHAPE, fn, "K is not a multiple of the weight block (128 for Q1_0, 32 for Q8_0, 64 otherwise)");
    if (fmt == LB_TERNARY_B3 && K > 30720) // a row is at most 64 lanes of six 80-column beats
        return fail(LB_ESHAPE, fn, "K above 30720 for base-3 beats");
    if (K > 32768 || N > INT32_MAX)
        return fail(LB_ESHAPE, fn, "K above 32768 or N above 2^31-1");
    if (fmt == LB_Q8_0 && K > 16384) // a row is at most one wave of lanes with 8 blocks each
        return fail(LB_ESHAPE, fn, "K above 16384 for Q8_0");
    if (tensor_bytes(fmt, N, K) >= (int64_t(1) << 32))
        return fail(LB_ESHAPE, fn, "weight tensor of 4 GiB or more");
    if (N == 0)
        return LB_OK;
    if (!W || !xq || !xscale || !y)
        return fail(LB_EINVAL, fn, "null pointer");
    if (!aligned(W, 16) || !aligned(xq, 16) || !aligned(xscale, 4) || !aligned(y, 4))
        return fail(LB_EALIGN, fn, "W and xq need 16-byte alignment, xscale and y 4-byte alignment");
    return LB_OK;
}

} // namespace

extern "C" {

const char *lowbit_status_str(lb_status st)
{
    switch (st) {
    case LB_OK:
        return "LB_OK";
    case LB_EINVAL:
        return "LB_EINVAL: invalid argument";
    case LB_ESHAPE:
        return "LB_ESHAPE: invalid shape";
    case LB_EALIGN:
        return "LB_EALIGN: misaligned pointer";
    case LB_EUNSUPPORTED:
        return "LB_EUNSUPPORTED: unsupported device or format";
    case LB_EDEVICE:
        return "LB_EDEVICE: HIP runtime error";
    case LB_ENOMEM:
        return "LB_ENOMEM: host memory exhausted";
    }
    return "unknown lb_status";
}

const char *lowbit_last_error(void) { return g_last_error; }

int64_t lowbit_weight_bytes(int fmt, int64_t N, int64_t K)
{
    if (!is_wfmt(fmt) || N < 0 || K < 0 || K % block_weights(fmt))
        return -1;
    return tensor_bytes(fmt, N, K);
}

static lb_status pack_common(const char *fn, int fmt, const void *src, int64_t N, int64_t K, void *dst,
                             bool unpack, hipStream_t s)
{
    if (!is_wfmt(fmt))
        return fail(LB_EINVAL, fn, "unknown weight format");
    if (N < 0 || K < 0 || K % block_weights(fmt))
        return fail(LB_ESHAPE, fn, "negative size or K not a multiple of the weight block");
    if (N == 0 || K == 0)
        return LB_OK;
    if (!src || !dst)
        return fail(LB_EINVAL, fn, "null pointer");
    const void *packed = unpack ? src : dst;
    if (!aligned(packed, 16))
        return fail(LB_EALIGN, fn, "the device layout needs 16-byte alignment");
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e = lb::launch_pack(fmt, static_cast<const uint8_t *>(unpack ? dst : src), N, K,
                                   static_cast<uint8_t *>(unpack ? const_cast<void *>(src) : dst), unpack, s);
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

lb_status lowbit_pack_weights(int fmt, const void *blocks, int64_t N, int64_t K, void *packed, hipStream_t s)
{
    return pack_common("lowbit_pack_weights", fmt, blocks, N, K, packed, false, s);
}

lb_status lowbit_unpack_weights(int fmt, const void *packed, int64_t N, int64_t K, void *blocks, hipStream_t s)
{
    return pack_common("lowbit_unpack_weights", fmt, packed, N, K, blocks, true, s);
}

lb_status lowbit_quantize_act(int afmt, const float *x, int64_t M, int64_t K, int8_t *xq, void *xscale,
                              hipStream_t s)
{
    const char *fn = "lowbit_quantize_act";
    if (afmt != LB_ACT_Q8_0 && afmt != LB_ACT_I8_ROW)
        return fail(LB_EINVAL, fn, "unknown activation format");
    if (M < 0 || K < 0 || M > INT32_MAX)
        return fail(LB_ESHAPE, fn, "negative size");
    if (afmt == LB_ACT_Q8_0 && K % lb::QK8)
        return fail(LB_ESHAPE, fn, "K is not a multiple of 32");
    if (M == 0 || K == 0)
        return LB_OK;
    if (!x || !xq || !xscale)
        return fail(LB_EINVAL, fn, "null pointer");
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xscale, 4))
        return fail(LB_EALIGN, fn, "x and xq need 16-byte alignment, xscale 4-byte alignment");
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e = afmt == LB_ACT_Q8_0
                       ? lb::launch_quantize_q8_0(x, M, K, xq, static_cast<uint16_t *>(xscale), s)
                       : lb::launch_quantize_i8_row(x, M, K, xq, static_cast<float *>(xscale), s);
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

static lb_status matvec_common(const char *fn, int fmt, const void *W, int64_t N, int64_t K, float w_scale,
                               int afmt, const int8_t *xq, const void *xscale, float *y, int32_t *sums,
                               hipStream_t s)
{
    lb_status st = check_product(fn, fmt, W, N, K, afmt, xq, xscale, sums ? (const void *)sums : (const void *)y);
    if (st != LB_OK || N == 0)
        return st;
    st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e;
    if (K == 0) {
        // an empty sum: y = 0 (and no per-block sums exist; planar and base-3 row sums are 0)
        if (sums)
            e = fmt == LB_TERNARY_PLANAR || fmt == LB_TERNARY_B3 ? lb::launch_fill_zero_i32(sums, N, s) : hipSuccess;
        else
            e = lb::launch_fill_zero(y, N, s);
    } else {
        e = lb::launch_matvec(fmt, static_cast<const uint8_t *>(W), N, K, w_scale, xq, xscale, y, sums, s);
    }
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

lb_status lowbit_matvec(int fmt, const void *W, int64_t N, int64_t K, float w_tensor_scale, int afmt,
                        const int8_t *xq, const void *xscale, float *y, hipStream_t s)
{
    return matvec_common("lowbit_matvec", fmt, W, N, K, w_tensor_scale, afmt, xq, xscale, y, nullptr, s);
}

static lb_status gemm_common(const char *fn, int fmt, const void *W, int64_t N, int64_t K, float w_scale,
                             int afmt, const int8_t *Xq, const void *Xscale, int64_t M, float *Y, int32_t *sums,
                             hipStream_t s)
{
    if (M < 0 || M > INT32_MAX)
        return fail(LB_ESHAPE, fn, "negative M");
    lb_status st = check_product(fn, fmt, W, N, K, afmt, Xq, Xscale, sums ? (const void *)sums : (const void *)Y);
    if (st != LB_OK || N == 0 || M == 0)
        return st;
    if (N * M >= (int64_t(1) << 31) / ((sums && fmt != LB_TERNARY_PLANAR) ? (K / 32 + 1) : 1))
        return fail(LB_ESHAPE, fn, "output of 2^31 elements or more");
    if (M * K >= (int64_t(1) << 32))
        return fail(LB_ESHAPE, fn, "activation matrix of 4 GiB or more");
    if (fmt == LB_Q8_0 && K % 128)
        return fail(LB_ESHAPE, fn, "Q8_0 prefill needs K to be a multiple of 128");
    st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e;
    if (K == 0) {
        if (sums)
            e = fmt == LB_TERNARY_PLANAR ? lb::launch_fill_zero_i32(sums, M * N, s) : hipSuccess;
        else
            e = lb::launch_fill_zero(Y, M * N, s);
    } else {
        e = lb::launch_gemm(fmt, static_cast<const uint8_t *>(W), N, K, w_scale, Xq, Xscale, M, Y, sums, s);
    }
    if (e == hipErrorNotSupported)
        return fail(LB_EUNSUPPORTED, fn, "this weight format has no prefill kernel yet");
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

lb_status lowbit_gemm(int fmt, const void *W, int64_t N, int64_t K, float w_tensor_scale, int afmt,
                      const int8_t *Xq, const void *Xscale, int64_t M, float *Y, hipStream_t s)
{
    return gemm_common("lowbit_gemm", fmt, W, N, K, w_tensor_scale, afmt, Xq, Xscale, M, Y, nullptr, s);
}

lb_status lowbit_block_sums(int fmt, const void *W, int64_t N, int64_t K, int afmt, const int8_t *Xq,
                            const void *Xscale, int64_t M, int32_t *sums, hipStream_t s)
{
    const char *fn = "lowbit_block_sums";
    if (!sums && N > 0 && M > 0)
        return fail(LB_EINVAL, fn, "null pointer");
    if (M == 1)
        return matvec_common(fn, fmt, W, N, K, 1.0f, afmt, Xq, Xscale, nullptr, sums, s);
    return gemm_common(fn, fmt, W, N, K, 1.0f, afmt, Xq, Xscale, M, nullptr, sums, s);
}

lb_status dense_head_matvec(const uint16_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s)
{
    const char *fn = "dense_head_matvec";
    if (N < 0 || K < 0 || N > INT32_MAX)
        return fail(LB_ESHAPE, fn, "negative size");
    if (K % 8 || K > 32768)
        return fail(LB_ESHAPE, fn, "K must be a multiple of 8 and at most 32768");
    if (N * K * 2 >= (int64_t(1) << 32))
        return fail(LB_ESHAPE, fn, "weight tensor of 4 GiB or more");
    if (N == 0)
        return LB_OK;
    if (!W || !x || !y)
        return fail(LB_EINVAL, fn, "null pointer");
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4))
        return fail(LB_EALIGN, fn, "W and x need 16-byte alignment, y 4-byte alignment");
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e = K == 0 ? lb::launch_fill_zero(y, N, s) : lb::launch_head(W, N, K, x, y, s);
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

lb_status lowbit_matvec_popcount(const void *W, int64_t N, int64_t K, float w_tensor_scale, const int8_t *xq,
                                 const float *xscale, float *y, int32_t *row_sums, hipStream_t s)
{
    const char *fn = "lowbit_matvec_popcount";
    lb_status st = check_product(fn, LB_TERNARY_PLANAR, W, N, K, LB_ACT_I8_ROW, xq, xscale,
                                 y ? (const void *)y : (const void *)row_sums);
    if (st != LB_OK || N == 0)
        return st;
    if (K > 8192)
        return fail(LB_ESHAPE, fn, "K above 8192 (the activation planes are held in registers)");
    if (row_sums && !aligned(row_sums, 4))
        return fail(LB_EALIGN, fn, "row_sums needs 4-byte alignment");
    st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e;
    if (K == 0) {
        e = y ? lb::launch_fill_zero(y, N, s) : hipSuccess;
        if (e == hipSuccess && row_sums)
            e = lb::launch_fill_zero_i32(row_sums, N, s);
    } else {
        e = lb::launch_popcount(static_cast<const uint8_t *>(W), N, K, w_tensor_scale, xq, xscale, y, row_sums, s);
    }
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

lb_status dense_head_matvec_i8(const int8_t *W, const float *row_scale, int64_t N, int64_t K, const float *x, float *y,
                               hipStream_t s)
{
    const char *fn = "dense_head_matvec_i8";
    if (N < 0 || K < 0 || N > INT32_MAX)
        return fail(LB_ESHAPE, fn, "negative size");
    if (K % 16 || K > 32768)
        return fail(LB_ESHAPE, fn, "K must be a multiple of 16 and at most 32768");
    if (N * K >= (int64_t(1) << 32))
        return fail(LB_ESHAPE, fn, "weight tensor of 4 GiB or more");
    if (N == 0)
        return LB_OK;
    if (!W || !row_scale || !x || !y)
        return fail(LB_EINVAL, fn, "null pointer");
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(row_scale, 4))
        return fail(LB_EALIGN, fn, "W and x need 16-byte alignment, row_scale and y 4-byte alignment");
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e = K == 0 ? lb::launch_fill_zero(y, N, s) : lb::launch_head_i8(W, row_scale, N, K, x, y, s);
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

lb_status lowbit_read_probe(const void *buf, int64_t nbytes, uint32_t *sink, hipStream_t s)
{
    const char *fn = "lowbit_read_probe";
    if (nbytes < 0 || nbytes % 16)
        return fail(LB_ESHAPE, fn, "nbytes must be a non-negative multiple of 16");
    if (nbytes == 0)
        return LB_OK;
    if (!buf || !sink)
        return fail(LB_EINVAL, fn, "null pointer");
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return fail(LB_EALIGN, fn, "buf needs 16-byte alignment, sink 4-byte alignment");
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;
    hipError_t e = lb::launch_read_probe(buf, nbytes, sink, s);
    return e == hipSuccess ? LB_OK : hip_fail(fn, e);
}

// ---- batched decode ------------------------------------------------------------------------------

// The tile size a large batch keeps, measured per format on whole tokens (the 8B shapes for Q1_0, Q2_0 and
// Q8_0, the 2B shapes for planar and base-3; launch times with every size from 32 to 384 KiB forced): the
// two nibble-product formats run fastest with small tiles, 64 KiB (96 KiB for rows above 8192 columns, which
// stage three times the activation per tile) -- 3 % faster than 256 KiB for both --, planar and Q8_0 with
// 256 KiB and base-3 with 224 KiB.
static int64_t default_tile_bytes(int fmt, int64_t K)
{
    if (fmt == LB_Q1_0 || fmt == LB_Q2_0_G64)
        return (K > 8192 ? 96 : 64) * 1024;
    return (fmt == LB_TERNARY_B3 ? 224 : 256) * 1024;
}

// Tile plan of one launch group.  Every product is cut into row tiles (whole row iterations of the
// configuration) of about the same weight bytes, between 16 and 384 KiB.  A large batch (four or more
// rounds of the group's resident workgroup slots at the default size -- a whole token's products) keeps
// the format's default size.  A smaller one -- one dependency phase of a token, a few tens of MB -- takes
// the size whose in-order dispatch onto the slots (CUs x workgroups per CU) has the shortest simulated
// makespan, each tile costing its weight bytes plus a fixed start-up share, if that beats the default by at
// least 5 % (among sizes within 0.5 % of the best, the largest): tiles small enough to occupy every CU
// instead of a few dozen workgroups.  Tiles are emitted largest first, so the partial tiles of every
// product fill the tail of the launch.
static void plan_tiles(int fmt, int cfg, std::vector<lb::DevDesc> &ds, int64_t slots, std::vector<lb::TileRef> &out)
{
    constexpr int64_t kStartup = 24 * 1024; // bytes-equivalent of one workgroup's staging and start-up
    int64_t maxk = 0;
    for (const lb::DevDesc &d : ds)
        maxk = std::max<int64_t>(maxk, d.K);
    const int64_t kDefault = default_tile_bytes(fmt, maxk);
    const int64_t rpi = lb::matvec_config_rows_per_iter(fmt, cfg);
    auto rows_for = [&](int64_t tb, const lb::DevDesc &d) {
        const int64_t rb = lowbit_weight_bytes(fmt, 1, d.K);
        const int64_t want = std::max<int64_t>(1, (tb + rb - 1) / rb);
        return rpi * ((want + rpi - 1) / rpi);
    };
    std::vector<int64_t> cand, span, ntiles;
    std::vector<int64_t> costs;
    std::vector<int64_t> sizes = {16 * 1024, 24 * 1024, 32 * 1024, 48 * 1024, 64 * 1024, 96 * 1024, 128 * 1024,
                                  160 * 1024};
    for (int64_t tb = 192 * 1024; tb <= 384 * 1024; tb += 16 * 1024)
        sizes.push_back(tb);
    for (int64_t tb : sizes) {
        costs.clear();
        for (const lb::DevDesc &d : ds) {
            const int64_t rows = rows_for(tb, d), rb = lowbit_weight_bytes(fmt, 1, d.K);
            for (int64_t r0 = 0; r0 < d.N; r0 += rows)
                costs.push_back(std::min<int64_t>(rows, d.N - r0) * rb + kStartup);
        }
        std::sort(costs.begin(), costs.end(), std::greater<int64_t>());
        std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> q;
        for (int64_t i = 0; i < std::min<int64_t>(slots, (int64_t)costs.size()); i++)
            q.push(0);
        int64_t make = 0;
        for (int64_t c : costs) {
            const int64_t t = q.top() + c;
            q.pop();
            q.push(t);
            make = std::max(make, t);
        }
        cand.push_back(tb);
        span.push_back(make);
        ntiles.push_back((int64_t)costs.size());
    }
    const int64_t best = *std::min_element(span.begin(), span.end());
    int64_t tb = kDefault, at_default = 0, tiles_default = 0;
    for (size_t i = 0; i < cand.size(); i++)
        if (cand[i] == kDefault)
            at_default = span[i], tiles_default = ntiles[i];
    // the model is coarse: leave the default unless the batch is small and it predicts >= 5 %
    if (tiles_default < 4 * slots && best * 100 < at_default * 95)
        for (size_t i = 0; i < cand.size(); i++)
            if (span[i] * 1000 <= best * 1005)
                tb = cand[i];
    struct T {
        int64_t cost;
        lb::TileRef ref;
    };
    std::vector<T> ts;
    for (size_t p = 0; p < ds.size(); p++) {
        const int64_t rows = rows_for(tb, ds[p]), rb = lowbit_weight_bytes(fmt, 1, ds[p].K);
        ds[p].tile_rows = (int32_t)std::min<int64_t>(rows, INT32_MAX);
        for (int64_t r0 = 0; r0 < ds[p].N; r0 += rows)
            ts.push_back({std::min<int64_t>(rows, ds[p].N - r0) * rb, {(int32_t)p, (int32_t)r0}});
    }
    std::stable_sort(ts.begin(), ts.end(), [](const T &a, const T &b) { return a.cost > b.cost; });
    out.clear();
    for (const T &t : ts)
        out.push_back(t.ref);
}

struct lb_batch {
    struct Group {
        lb::BatchGroup g;
        size_t lds;
    };
    // an fp32 activation row quantised to q8_0 by a launch of its own ahead of the groups, into the batch's
    // device memory
    struct Quant {
        const float *x;
        int64_t K;
        int8_t *xq;
        uint16_t *xs;
    };
    std::vector<Quant> quants;
    std::vector<Group> groups;
    void *dev = nullptr;
    int device = -1;
};

namespace {

// fp32 activation rows (LB_ACT_F32_Q8_0) longer than this are quantised by one launch of their own ahead of
// the products instead of inside every product workgroup: each workgroup would read and quantise the whole
// row for a tile of a few rows.  Measured on the dependency-ordered 8B token's down projection (K = 12288,
// 14 MB): 9.1 us per phase quantised in the launch, 7.5 us with a quantise launch first; at K = 4096 the
// in-launch form is 1.3-1.7 us faster per phase.
constexpr int64_t kQinMaxK = 8192;

// A validated work list cut into launch groups with their device tables, still in host memory.
struct BatchPlan {
    struct Key {
        int fmt, cfg, qin;
    };
    // an fp32 row quantised ahead of the groups; its q8_0 bytes then binary16 scales sit `off` bytes past the
    // tables, each part padded to 256 bytes
    struct PreQ {
        const float *x;
        int64_t K;
        size_t off;
    };
    std::vector<Key> keys;
    std::vector<std::vector<lb::DevDesc>> descs;
    std::vector<std::vector<int>> preq_of; // per descriptor: its row in preq, or -1
    std::vector<PreQ> preq;
    size_t preq_bytes = 0;
    std::vector<std::vector<lb::TileRef>> tiles;
    std::vector<int> full;
    std::vector<size_t> lds;
    int device = 0;

    static size_t padded(size_t b) { return (b + 255) / 256 * 256; }
    // bytes of the device tables: per group its descriptors, then its tiles, each padded to 256 bytes
    size_t table_bytes() const
    {
        size_t bytes = 0;
        for (size_t gi = 0; gi < keys.size(); gi++)
            bytes += padded(descs[gi].size() * sizeof(lb::DevDesc)) + padded(tiles[gi].size() * sizeof(lb::TileRef));
        return bytes;
    }
    static size_t q8_bytes(int64_t K) { return padded((size_t)K) + padded((size_t)(K / 32) * 2); }
    // Lay the tables out at `host` (table_bytes() bytes) for device address `dev`, and describe the launch
    // groups that read them there and the quantise launches that precede them (their q8_0 rows at
    // dev + table_bytes(), preq_bytes more bytes of device memory).
    void emit(char *host, char *dev, std::vector<lb_batch::Group> &groups, std::vector<lb_batch::Quant> &quants) const
    {
        size_t off = 0;
        groups.clear();
        quants.clear();
        char *const qbase = dev + table_bytes();
        for (const PreQ &q : preq)
            quants.push_back({q.x, q.K, reinterpret_cast<int8_t *>(qbase + q.off),
                              reinterpret_cast<uint16_t *>(qbase + q.off + padded((size_t)q.K))});
        for (size_t gi = 0; gi < keys.size(); gi++) {
            lb_batch::Group grp;
            grp.g.fmt = keys[gi].fmt;
            grp.g.cfg_a = keys[gi].cfg;
            grp.g.full = full[gi];
            grp.g.qin = keys[gi].qin;
            grp.g.ntiles = (int32_t)tiles[gi].size();
            grp.g.desc = reinterpret_cast<const lb::DevDesc *>(dev + off);
            std::memcpy(host + off, descs[gi].data(), descs[gi].size() * sizeof(lb::DevDesc));
            lb::DevDesc *hd = reinterpret_cast<lb::DevDesc *>(host + off);
            for (size_t j = 0; j < descs[gi].size(); j++)
                if (preq_of[gi][j] >= 0) { // reads the row its quantise launch writes
                    const lb_batch::Quant &q = quants[(size_t)preq_of[gi][j]];
                    hd[j].xq = q.xq;
                    hd[j].xscale = q.xs;
                }
            off += padded(descs[gi].size() * sizeof(lb::DevDesc));
            grp.g.tiles = reinterpret_cast<const lb::TileRef *>(dev + off);
            std::memcpy(host + off, tiles[gi].data(), tiles[gi].size() * sizeof(lb::TileRef));
            off += padded(tiles[gi].size() * sizeof(lb::TileRef));
            grp.lds = lds[gi];
            groups.push_back(grp);
        }
    }
};

// Validate a host work list and plan its launches (no device memory is touched).  prequant: fp32 rows above
// kQinMaxK columns get a quantise launch of their own (the batch object holds their q8_0 rows); without it
// every fp32 row is quantised inside its products' launches.
lb_status batch_plan(const char *fn, const lb_matvec_desc *list, int32_t n, BatchPlan &plan, bool prequant)
{
    if (!list || n < 1)
        return fail(LB_EINVAL, fn, "empty or null work list");
    for (int32_t i = 0; i < n; i++) {
        const lb_matvec_desc &d = list[i];
        lb_status st;
        if (d.afmt == LB_ACT_F32_Q8_0) {
            // fp32 activations quantised in the product's own launch
            if (is_wfmt(d.fmt) && d.fmt != LB_Q1_0 && d.fmt != LB_Q2_0_G64)
                return fail(LB_EUNSUPPORTED, fn, "LB_ACT_F32_Q8_0 is for Q1_0 and Q2_0_g64 weights only");
            if (d.N > 0 && !d.x)
                return fail(LB_EINVAL, fn, "null x for LB_ACT_F32_Q8_0");
            if (d.N > 0 && !aligned(d.x, 16))
                return fail(LB_EALIGN, fn, "x needs 16-byte alignment");
            // x stands in for xq and xscale in the shared checks
            st = check_product(fn, d.fmt, d.W, d.N, d.K, LB_ACT_Q8_0, d.x, d.x, d.y);
        } else {
            st = check_product(fn, d.fmt, d.W, d.N, d.K, d.afmt, d.xq, d.xscale, d.y);
        }
        if (st != LB_OK)
            return st;
        if (d.K == 0 && d.N > 0)
            return fail(LB_ESHAPE, fn, "K == 0 in a work list (use lowbit_matvec for empty sums)");
        if (d.N > 0 && lb::matvec_config(d.fmt, d.K) < 0)
            return fail(LB_ESHAPE, fn, "K above the decode kernel's limit");
    }
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;

    // one launch group per (weight format, kernel configuration) present, products in list order
    for (int32_t i = 0; i < n; i++) {
        const lb_matvec_desc &d = list[i];
        if (d.N == 0)
            continue;
        const int cfg = lb::matvec_config(d.fmt, d.K);
        const bool pre = prequant && d.afmt == LB_ACT_F32_Q8_0 && d.K > kQinMaxK;
        const int qin = d.afmt == LB_ACT_F32_Q8_0 && !pre ? 1 : 0;
        int pi = -1;
        if (pre) { // one quantise launch per distinct (x, K)
            for (size_t j = 0; j < plan.preq.size() && pi < 0; j++)
                if (plan.preq[j].x == d.x && plan.preq[j].K == d.K)
                    pi = (int)j;
            if (pi < 0) {
                pi = (int)plan.preq.size();
                plan.preq.push_back({d.x, d.K, plan.preq_bytes});
                plan.preq_bytes += BatchPlan::q8_bytes(d.K);
            }
        }
        size_t gi = 0;
        while (gi < plan.keys.size() &&
               !(plan.keys[gi].fmt == d.fmt && plan.keys[gi].cfg == cfg && plan.keys[gi].qin == qin))
            gi++;
        if (gi == plan.keys.size()) {
            plan.keys.push_back({d.fmt, cfg, qin});
            plan.descs.emplace_back();
            plan.preq_of.emplace_back();
            plan.lds.push_back(0);
        }
        lb::DevDesc dd;
        dd.W = static_cast<const uint8_t *>(d.W);
        dd.xq = d.xq;
        dd.xscale = d.xscale;
        dd.y = d.y;
        dd.N = (int32_t)d.N;
        dd.K = (int32_t)d.K;
        dd.w_scale = d.w_tensor_scale;
        dd.cfg = cfg;
        dd.tile_rows = 0; // set by the tile plan
        dd.x = qin ? d.x : nullptr;
        plan.descs[gi].push_back(dd);
        plan.preq_of[gi].push_back(pi);
        plan.lds[gi] = std::max(plan.lds[gi], (size_t)lb::matvec_stage_bytes(d.fmt, d.K) +
                                                  (qin ? (size_t)lb::q8_0_lds_bytes(d.K) : 0));
    }
    int cus = 0;
    (void)hipGetDevice(&plan.device); // succeeded in check_device
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, plan.device) != hipSuccess || cus < 1)
        cus = 1;
    plan.tiles.resize(plan.keys.size());
    plan.full.assign(plan.keys.size(), 1);
    for (size_t gi = 0; gi < plan.keys.size(); gi++) {
        const BatchPlan::Key &k = plan.keys[gi];
        for (const lb::DevDesc &dd : plan.descs[gi])
            plan.full[gi] &= lb::matvec_config_full(k.fmt, k.cfg, dd.K) ? 1 : 0;
        const int64_t slots =
            (int64_t)cus * lb::matvec_batched_blocks_per_cu(k.fmt, k.cfg, plan.full[gi] != 0, k.qin != 0, plan.lds[gi]);
        plan_tiles(k.fmt, k.cfg, plan.descs[gi], slots, plan.tiles[gi]);
    }
    return LB_OK;
}

lb_status launch_groups(const char *fn, const std::vector<lb_batch::Quant> &quants,
                        const std::vector<lb_batch::Group> &groups, hipStream_t s)
{
    for (const auto &q : quants) {
        hipError_t e = lb::launch_quantize_q8_0(q.x, 1, q.K, q.xq, q.xs, s);
        if (e != hipSuccess)
            return hip_fail(fn, e);
    }
    for (const auto &grp : groups) {
        hipError_t e = lb::launch_matvec_batched(grp.g, s, grp.lds);
        if (e != hipSuccess)
            return hip_fail(fn, e);
    }
    return LB_OK;
}

// ---- the allocation-free variant: its tables live in a fixed device array -------------------------

// The work-list tables of lowbit_matvec_batched_static, one copy per GPU (each device holds its own
// instance of a __device__ array).  Host code never names it as an address: its device address is looked
// up once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[LB_STATIC_TABLE_BYTES];

std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::atomic<int> g_scratch_state[kMaxDevices]; // 0 not looked up, 1 looked up, 2 lookup failed

lb_status scratch_address(const char *fn, int dev, char **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return fail(LB_EINVAL, fn, "device index out of range");
    int st = g_scratch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)); // the current device's copy
        if (e != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            g_scratch_state[dev].store(2, std::memory_order_release);
            return hip_fail(fn, e == hipSuccess ? hipErrorInvalidSymbol : e);
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_relaxed);
        g_scratch_state[dev].store(1, std::memory_order_release);
        st = 1;
    }
    if (st != 1)
        return fail(LB_EDEVICE, fn, "the device address of the static table could not be found");
    *out = static_cast<char *>(g_scratch_ptr[dev].load(std::memory_order_relaxed));
    return LB_OK;
}

lb_status batched_static(const lb_matvec_desc *list, int32_t n, hipStream_t s)
{
    const char *fn = "lowbit_matvec_batched_static";
    BatchPlan plan;
    lb_status st = batch_plan(fn, list, n, plan, false); // every fp32 row quantised in its products' launches
    if (st != LB_OK)
        return st;
    const size_t bytes = plan.table_bytes();
    if (bytes > (size_t)LB_STATIC_TABLE_BYTES) {
        char what[160];
        std::snprintf(what, sizeof(what), "the work list's tables need %zu bytes, above the static table's %d "
                                          "(use lowbit_batch_create)", bytes, (int)LB_STATIC_TABLE_BYTES);
        return fail(LB_ESHAPE, fn, what);
    }
    char *dev = nullptr;
    st = scratch_address(fn, plan.device, &dev);
    if (st != LB_OK)
        return st;
    std::vector<char> host(bytes);
    std::vector<lb_batch::Group> groups;
    std::vector<lb_batch::Quant> quants; // (none without pre-quantisation)
    plan.emit(host.data(), dev, groups, quants);
    // ordered on s after every earlier use of the table on s (a pageable source is staged by the runtime
    // before the call returns, so `host` may go away afterwards)
    hipError_t e = hipMemcpyAsync(dev, host.data(), bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
        return hip_fail(fn, e);
    return launch_groups(fn, quants, groups, s);
}

} // namespace

static lb_status batch_create(const lb_matvec_desc *list, int32_t n, lb_batch **out)
{
    const char *fn = "lowbit_batch_create";
    if (!out)
        return fail(LB_EINVAL, fn, "null output pointer");
    *out = nullptr;
    BatchPlan plan;
    lb_status st = batch_plan(fn, list, n, plan, true);
    if (st != LB_OK)
        return st;
    const size_t tbytes = std::max<size_t>(plan.table_bytes(), 256);
    std::vector<char> host(tbytes);
    std::unique_ptr<lb_batch> b(new lb_batch());
    b->device = plan.device;
    // nothing below allocates host memory once the device memory is held
    b->groups.reserve(plan.keys.size());
    b->quants.reserve(plan.preq.size());
    // the tables, then the q8_0 rows of the quantise launches at table_bytes() (written on the device by those
    // launches, not copied; there are none when the tables take fewer than 256 bytes)
    hipError_t e = hipMalloc(&b->dev, tbytes + plan.preq_bytes);
    if (e != hipSuccess)
        return hip_fail(fn, e);
    plan.emit(host.data(), static_cast<char *>(b->dev), b->groups, b->quants);
    e = hipMemcpy(b->dev, host.data(), tbytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(b->dev);
        return hip_fail(fn, e);
    }
    *out = b.release();
    return LB_OK;
}

lb_status lowbit_batch_create(const lb_matvec_desc *list, int32_t n, lb_batch **out)
{
    // the plan is built in host containers: an allocation failure is reported, not thrown through C
    try {
        return batch_create(list, n, out);
    } catch (const std::bad_alloc &) {
        return fail(LB_ENOMEM, "lowbit_batch_create", "host allocation failed while planning the batch");
    }
}

lb_status lowbit_matvec_batched(const lb_batch *b, hipStream_t s)
{
    const char *fn = "lowbit_matvec_batched";
    if (!b)
        return fail(LB_EINVAL, fn, "null batch");
    lb_status st = check_device(fn);
    if (st != LB_OK)
        return st;
    int dev = -1;
    (void)hipGetDevice(&dev); // succeeded in check_device
    if (dev != b->device)
        return fail(LB_EINVAL, fn, "the batch was created on another device");
    return launch_groups(fn, b->quants, b->groups, s);
}

lb_status lowbit_matvec_batched_static(const lb_matvec_desc *list, int32_t n, hipStream_t s)
{
    // the plan is built in host containers: an allocation failure is reported, not thrown through C
    try {
        return batched_static(list, n, s);
    } catch (const std::bad_alloc &) {
        return fail(LB_ENOMEM, "lowbit_matvec_batched_static", "host allocation failed while planning the batch");
    }
}

int32_t lowbit_batch_launches(const lb_batch *b)
{
    return b ? (int32_t)(b->quants.size() + b->groups.size()) : -1;
}

void lowbit_batch_destroy(lb_batch *b)
{
    if (!b)
        return;
    if (b->dev)
        (void)hipFree(b->dev);
    delete b;
}

} // extern "C"
