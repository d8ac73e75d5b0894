"""The C ABI on the host: the library loads, exports every entry point include/lowbit.h declares, and
rejects bad arguments with its status codes before touching a device."""
import ctypes
import os
import re

import pytest

import bit_quantized_matvec_q1_amd.lowbit as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lowbit.h")

A16 = 1 << 20  # a 16-byte-aligned stand-in address; never dereferenced (every call below fails validation)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*\b([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "lowbit_matvec" in names and "lowbit_gemm" in names and "dense_head_matvec" in names
    for n in names:
        assert hasattr(L.lib, n), n
        assert n in L.SIGNATURES, f"{n} declared in lowbit.h but not bound in lowbit.py"
    assert set(L.SIGNATURES) == set(names)


def test_status_strings():
    for st in range(7):
        assert L.lib.lowbit_status_str(st).startswith(b"LB_")
    assert L.lib.lowbit_status_str(0) == b"LB_OK"
    assert L.lib.lowbit_status_str(L.LB_ENOMEM).startswith(b"LB_ENOMEM")
    assert L.lib.lowbit_status_str(99) == b"unknown lb_status"


def test_last_error_is_bounded_and_names_the_call():
    # a failing call records "<function>: <reason>" in fixed per-thread storage
    assert L.lib.lowbit_gemm(L.Q2_0_G64, A16, 8, 64, 1.0, L.ACT_Q8_0, A16, A16, -1, A16, None) == L.LB_ESHAPE
    msg = L.lib.lowbit_last_error()
    assert msg.startswith(b"lowbit_gemm: ") and len(msg) < 512


def test_weight_bytes():
    assert L.lowbit_weight_bytes(L.Q1_0, 4096, 4096) == 2_359_296
    assert L.lowbit_weight_bytes(L.Q2_0_G64, 4096, 4096) == 4_718_592
    assert L.lowbit_weight_bytes(L.TERNARY_PLANAR, 6912, 2560) == 4_423_680
    assert L.lowbit_weight_bytes(L.Q8_0, 4096, 4096) == 17_825_792  # 34 bytes per 32 weights
    assert L.lowbit_weight_bytes(L.Q8_0, 4, 48) == -1
    assert L.lowbit_weight_bytes(L.TERNARY_B3, 2560, 6912) == 2560 * 87 * 16  # ceil(6912 / 80) beats per row
    assert L.lowbit_weight_bytes(L.TERNARY_B3, 2560, 2560) == 2560 * 512  # 1.6 bits per weight
    assert L.lowbit_weight_bytes(L.TERNARY_B3, 4, 80) == -1  # rows are whole planar widths
    assert L.lowbit_weight_bytes(L.Q1_0, 4, 64) == -1
    assert L.lowbit_weight_bytes(7, 4, 64) == -1
    assert L.lowbit_weight_bytes(L.Q2_0_G64, -1, 64) == -1


def mv(fmt=L.Q2_0_G64, W=A16, N=8, K=128, afmt=L.ACT_Q8_0, xq=A16, xs=A16, y=A16):
    return L.lib.lowbit_matvec(fmt, W, N, K, 1.0, afmt, xq, xs, y, None)


def test_matvec_validation_codes():
    assert mv(fmt=9) == L.LB_EINVAL
    assert mv(afmt=9) == L.LB_EINVAL
    assert mv(afmt=L.ACT_I8_ROW) == L.LB_EINVAL  # Q2_0 needs q8_0 activations
    assert mv(fmt=L.TERNARY_PLANAR, afmt=L.ACT_Q8_0) == L.LB_EINVAL
    assert mv(N=-1) == L.LB_ESHAPE
    assert mv(K=96) == L.LB_ESHAPE  # not a multiple of 64
    assert mv(fmt=L.Q1_0, K=192) == L.LB_ESHAPE  # not a multiple of 128
    assert mv(K=32768 + 64) == L.LB_ESHAPE
    assert mv(fmt=L.Q8_0, K=16384 + 32) == L.LB_ESHAPE  # Q8_0 rows are at most 16384 weights
    assert mv(fmt=L.Q8_0, K=48) == L.LB_ESHAPE  # not a multiple of 32
    assert mv(fmt=L.TERNARY_B3, afmt=L.ACT_I8_ROW, K=30720 + 64) == L.LB_ESHAPE  # base-3 rows <= 30720
    assert mv(fmt=L.TERNARY_B3, afmt=L.ACT_Q8_0) == L.LB_EINVAL  # base-3 takes per-token activations
    assert mv(W=None) == L.LB_EINVAL
    assert mv(y=None) == L.LB_EINVAL
    assert mv(W=A16 + 8) == L.LB_EALIGN
    assert mv(xq=A16 + 4) == L.LB_EALIGN
    assert mv(y=A16 + 2) == L.LB_EALIGN
    assert mv(N=0, W=None, y=None) == L.LB_OK  # empty product: nothing to do, nothing touched
    assert b"lowbit_matvec" in L.lib.lowbit_last_error()


def test_other_entry_points_validate():
    lib = L.lib
    assert lib.lowbit_batch_launches(None) == -1
    assert lib.lowbit_quantize_act(3, A16, 1, 64, A16, A16, None) == L.LB_EINVAL
    assert lib.lowbit_quantize_act(L.ACT_Q8_0, A16, 1, 48, A16, A16, None) == L.LB_ESHAPE
    assert lib.lowbit_quantize_act(L.ACT_Q8_0, A16 + 4, 1, 64, A16, A16, None) == L.LB_EALIGN
    assert lib.lowbit_quantize_act(L.ACT_Q8_0, A16, 0, 64, None, None, None) == L.LB_OK
    assert lib.lowbit_pack_weights(L.Q1_0, A16, 2, 64, A16, None) == L.LB_ESHAPE
    assert lib.lowbit_pack_weights(L.Q2_0_G64, A16, 2, 64, A16 + 8, None) == L.LB_EALIGN
    assert lib.lowbit_gemm(L.Q2_0_G64, A16, 8, 64, 1.0, L.ACT_Q8_0, A16, A16, -1, A16, None) == L.LB_ESHAPE
    assert lib.lowbit_gemm(L.Q2_0_G64, A16, 8, 64, 1.0, L.ACT_I8_ROW, A16, A16, 4, A16, None) == L.LB_EINVAL
    assert lib.lowbit_gemm(L.Q2_0_G64, A16, 1, 4096, 1.0, L.ACT_Q8_0, A16, A16, 1 << 20, A16, None) == L.LB_ESHAPE
    # Q8_0 prefill walks whole 128-column steps; decode of the same K is allowed (M = 1 goes to decode)
    assert lib.lowbit_gemm(L.Q8_0, A16, 8, 96, 1.0, L.ACT_Q8_0, A16, A16, 4, A16, None) == L.LB_ESHAPE
    assert lib.lowbit_block_sums(L.Q8_0, A16, 8, 160, L.ACT_Q8_0, A16, A16, 2, A16, None) == L.LB_ESHAPE
    assert lib.lowbit_block_sums(L.Q2_0_G64, A16, 8, 64, L.ACT_Q8_0, A16, A16, 1, None, None) == L.LB_EINVAL
    assert lib.dense_head_matvec(A16, 8, 12, A16, A16, None) == L.LB_ESHAPE
    assert lib.dense_head_matvec(A16, 8, 32768 + 8, A16, A16, None) == L.LB_ESHAPE
    assert lib.dense_head_matvec(A16, 1 << 20, 2048, A16, A16, None) == L.LB_ESHAPE  # 4 GiB of weights
    assert lib.dense_head_matvec(A16 + 2, 8, 64, A16, A16, None) == L.LB_EALIGN
    assert lib.lowbit_matvec_popcount(A16, 8, 8192 + 64, 1.0, A16, A16, A16, None, None) == L.LB_ESHAPE
    assert lib.lowbit_matvec_popcount(A16, 8, 96, 1.0, A16, A16, A16, None, None) == L.LB_ESHAPE  # K % 64
    assert lib.lowbit_matvec_popcount(A16, 8, 128, 1.0, A16, A16, None, None, None) == L.LB_EINVAL  # no output
    assert lib.lowbit_matvec_popcount(A16, 8, 128, 1.0, A16, A16, None, A16 + 2, None) == L.LB_EALIGN
    assert lib.dense_head_matvec_i8(A16, A16, 8, 24, A16, A16, None) == L.LB_ESHAPE  # K % 16
    assert lib.dense_head_matvec_i8(A16, A16, 8, 32768 + 16, A16, A16, None) == L.LB_ESHAPE
    assert lib.dense_head_matvec_i8(A16, A16, 1 << 20, 4096, A16, A16, None) == L.LB_ESHAPE  # 4 GiB of weights
    assert lib.dense_head_matvec_i8(A16 + 8, A16, 8, 64, A16, A16, None) == L.LB_EALIGN
    assert lib.dense_head_matvec_i8(A16, None, 8, 64, A16, A16, None) == L.LB_EINVAL
    assert lib.dense_head_matvec_i8(None, None, 0, 64, None, None, None) == L.LB_OK
    assert lib.lowbit_matvec_batched(None, None) == L.LB_EINVAL
    h = ctypes.c_void_p()
    assert lib.lowbit_batch_create(None, 0, ctypes.byref(h)) == L.LB_EINVAL
    bad = (L.lb_matvec_desc * 1)(L.lb_matvec_desc(L.Q2_0_G64, L.ACT_Q8_0, 8, 100, A16, 1.0, A16, A16, A16))
    assert lib.lowbit_batch_create(ctypes.cast(bad, ctypes.c_void_p), 1, ctypes.byref(h)) == L.LB_ESHAPE

    # fp32 activations quantised in the launch: Q1_0 / Q2_0_g64 only, x required and 16-byte aligned
    def fused(fmt, x, K=128):
        d = (L.lb_matvec_desc * 1)(L.lb_matvec_desc(fmt, L.ACT_F32_Q8_0, 8, K, A16, 1.0, None, None, A16, x))
        return lib.lowbit_batch_create(ctypes.cast(d, ctypes.c_void_p), 1, ctypes.byref(h))

    assert fused(L.TERNARY_PLANAR, A16) == L.LB_EUNSUPPORTED
    assert fused(L.Q8_0, A16) == L.LB_EUNSUPPORTED
    assert fused(L.Q2_0_G64, None) == L.LB_EINVAL
    assert fused(L.Q2_0_G64, A16 + 4) == L.LB_EALIGN
    assert fused(L.Q1_0, A16, K=192) == L.LB_ESHAPE  # K % 128


def _has_device():
    import torch

    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_has_device(), reason="checks the no-device refusal; would launch on a real device")
def test_no_device_is_refused_without_launch():
    assert mv() == L.LB_EUNSUPPORTED
    assert b"gfx950" in L.lib.lowbit_last_error()
    with pytest.raises(L.LowbitError):
        L.lowbit_matvec(L.Q2_0_G64, A16, 8, 128, 1.0, L.ACT_Q8_0, A16, A16, A16, stream=0)


def test_binding_refuses_host_tensors():
    # a host address handed to a kernel would be a memory fault: the binding refuses it before the call
    import torch

    host = torch.zeros(64, dtype=torch.int8)
    with pytest.raises(ValueError, match="device tensor required"):
        L.lowbit_matvec(L.Q2_0_G64, A16, 8, 64, 1.0, L.ACT_Q8_0, host, A16, A16)


def test_binding_checks_sizes_and_dtypes():
    # a buffer shorter than the sizes imply would be read or written past its end by the kernels: the
    # binding refuses it (ValueError) before the C call, as it does a wrong dtype; these checks come before
    # the device check, so host tensors exercise them without a GPU
    import torch

    N, K = 8, 128
    W = torch.zeros(L.lowbit_weight_bytes(L.Q2_0_G64, N, K), dtype=torch.uint8)
    xq = torch.zeros(K, dtype=torch.int8)
    xs = torch.zeros(K // 32, dtype=torch.uint16)
    y = torch.zeros(N, dtype=torch.float32)
    with pytest.raises(ValueError, match="W: needs at least"):
        L.lowbit_matvec(L.Q2_0_G64, W[:-1], N, K, 1.0, L.ACT_Q8_0, xq, xs, y)
    with pytest.raises(ValueError, match="xq: needs at least"):
        L.lowbit_matvec(L.Q2_0_G64, W, N, K, 1.0, L.ACT_Q8_0, xq[:64], xs, y)
    with pytest.raises(ValueError, match="xscale: needs at least"):
        L.lowbit_matvec(L.Q2_0_G64, W, N, K, 1.0, L.ACT_Q8_0, xq, xs[:3], y)
    with pytest.raises(ValueError, match="y: needs at least"):
        L.lowbit_matvec(L.Q2_0_G64, W, N, K, 1.0, L.ACT_Q8_0, xq, xs, y[:7])
    with pytest.raises(ValueError, match="y: dtype"):
        L.lowbit_matvec(L.Q2_0_G64, W, N, K, 1.0, L.ACT_Q8_0, xq, xs, y.double())
    with pytest.raises(ValueError, match="xscale: dtype"):  # per-row int8 activations take one fp32 scale
        L.lowbit_matvec(L.TERNARY_PLANAR, W, N, K, 1.0, L.ACT_I8_ROW, xq, xs, y)
    with pytest.raises(ValueError, match="Y: needs at least"):
        L.lowbit_gemm(L.Q2_0_G64, W, N, K, 1.0, L.ACT_Q8_0, xq.repeat(2), xs.repeat(2), 2, y)
    with pytest.raises(ValueError, match="sums: needs at least"):  # [M][N][K/32] for the ggml formats
        L.lowbit_block_sums(L.Q2_0_G64, W, N, K, L.ACT_Q8_0, xq, xs, 1, torch.zeros(N, dtype=torch.int32))
    with pytest.raises(ValueError, match="xq: needs at least"):
        L.lowbit_quantize_act(L.ACT_Q8_0, torch.zeros(2 * K), 2, K, xq, xs.repeat(2))
    with pytest.raises(ValueError, match="W: needs at least"):
        L.dense_head_matvec(torch.zeros(N * K - 1, dtype=torch.int16), N, K, torch.zeros(K), y)
    with pytest.raises(ValueError, match="row_scale: needs at least"):
        L.dense_head_matvec_i8(torch.zeros(N * K, dtype=torch.int8), torch.zeros(N - 1), N, K, torch.zeros(K), y)
    with pytest.raises(ValueError, match="packed: needs at least"):
        L.lowbit_pack_weights(L.Q1_0, W, N, K, W[:16])
    with pytest.raises(ValueError, match="x: needs at least"):
        L.desc(L.Q2_0_G64, W, N, K, None, None, y, x=torch.zeros(K - 32))
    # sizes that fit get as far as the device check: a host tensor is refused there
    with pytest.raises(ValueError, match="device tensor required"):
        L.lowbit_matvec(L.Q2_0_G64, W, N, K, 1.0, L.ACT_Q8_0, xq, xs, y)


def test_desc_keeps_its_tensors():
    # a batch holds the tensors of its entries, so none can be freed and reused while it can write them
    import torch

    N, K = 8, 128
    W = torch.zeros(L.lowbit_weight_bytes(L.Q2_0_G64, N, K), dtype=torch.uint8)
    y = torch.zeros(N)
    with pytest.raises(ValueError, match="device tensor required"):
        L.desc(L.Q2_0_G64, W, N, K, torch.zeros(K, dtype=torch.int8), torch.zeros(K // 32, dtype=torch.uint16), y)
    d = L.desc(L.Q2_0_G64, 1 << 12, N, K, 1 << 12, 1 << 12, 1 << 12)  # raw addresses pass through
    assert d._tensors == ()
