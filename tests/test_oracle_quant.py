"""Pins of the oracle's activation quantisers: closed-form ties, the absmax element, the zero block, the
round-to-nearest error bound, and agreement with numpy's IEEE fp32 arithmetic."""
import numpy as np
import pytest

import oracle
import synth


def test_q8_0_ties_round_half_to_even():
    """A block whose absmax is 127 has multiplier 127/127 = 1 exactly, so q = round_half_even(x)."""
    x = np.zeros(32, dtype=np.float32)
    x[:10] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -126.5]
    q, dh = oracle.quantize_q8_0(x)
    assert list(q[0, :10]) == [127, 2, 4, -2, -4, 0, 2, 0, 126, -126]
    assert dh[0, 0] == 0x3C00  # fp16(127/127) = 1.0


def test_q8_0_zero_block_and_absmax_maps_to_127():
    g = np.random.default_rng(1)
    x = g.standard_normal((4, 256)).astype(np.float32)
    x[1, 32:64] = 0.0
    q, dh = oracle.quantize_q8_0(x)
    assert np.all(q[1, 32:64] == 0) and dh[1, 1] == 0
    for m in range(4):
        for j in range(8):
            blk = x[m, 32 * j:32 * j + 32]
            if not np.any(blk):
                continue
            i = int(np.argmax(np.abs(blk)))
            assert q[m, 32 * j + i] == (127 if blk[i] > 0 else -127)
    assert np.abs(q.astype(np.int32)).max() <= 127


def test_q8_0_is_round_to_nearest_on_the_127_over_amax_grid():
    """|x - q*amax/127| <= amax/254 (+ fp32 slack): a wrong multiplier or truncation breaks it."""
    g = np.random.default_rng(2)
    x = (g.standard_normal((64, 1024)) * np.exp(g.uniform(-8, 8, (64, 1)))).astype(np.float32)
    q, dh = oracle.quantize_q8_0(x)
    xb = x.reshape(64, 32, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=2, keepdims=True)
    err = np.abs(xb - q.reshape(64, 32, 32) * amax / 127.0)
    assert np.all(err <= amax / 254.0 * (1 + 1e-5))
    # the stored scale is binary16(amax / 127), rounded to nearest even, from the fp32 quotient
    d32 = (amax[..., 0].astype(np.float32) / np.float32(127.0)).astype(np.float32)
    assert np.array_equal(dh, d32.astype(np.float16).view(np.uint16))


def test_q8_0_matches_numpy_fp32():
    g = np.random.default_rng(4)
    x = synth.activations(g, 8, 4096)
    q, _ = oracle.quantize_q8_0(x)
    xb = x.reshape(8, -1, 32)
    amax = np.abs(xb).max(axis=2, keepdims=True)
    with np.errstate(divide="ignore"):
        idv = np.where(amax > 0, np.float32(127.0) / amax, np.float32(0.0)).astype(np.float32)
    ref = np.rint((xb * idv).astype(np.float32)).astype(np.int8).reshape(8, -1)
    assert np.array_equal(q, ref)


def test_q8_0_rejects_ragged_k():
    with pytest.raises(ValueError):
        oracle.quantize_q8_0(np.zeros((1, 48), dtype=np.float32))


def test_i8_row_quantiser():
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 2560)).astype(np.float32)
    x[2] = 0.0
    q, s = oracle.quantize_i8_row(x)
    assert s[2] == 0 and np.all(q[2] == 0)
    for m in range(2):
        amax = np.abs(x[m]).max()
        assert s[m] == np.float32(amax) / np.float32(127)
        i = int(np.argmax(np.abs(x[m])))
        assert abs(int(q[m, i])) == 127
        err = np.abs(x[m].astype(np.float64) - q[m] * float(amax) / 127.0)
        assert np.all(err <= amax / 254.0 * (1 + 1e-5))
    # ties: absmax 127 gives multiplier 1
    t = np.array([[127.0, 0.5, 1.5, -2.5, 2.5]], dtype=np.float32)
    qt, st = oracle.quantize_i8_row(t)
    assert list(qt[0]) == [127, 0, 2, -2, 2] and st[0] == 1.0
