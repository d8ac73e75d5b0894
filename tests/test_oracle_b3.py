"""Pins of the oracle's base-3 ternary beats (five trits per byte): hand-decoded beats, the byte counts the
pages give (1.6 bits per trit, ~20 % less traffic than the planar body), round trips against the generator's
drawn weights, brute force against numpy, and the select-accumulate special cases."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
B3 = oracle.TERNARY_B3


def _golden():
    out = []
    with open(os.path.join(GOLDEN, "b3_beats.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            hexb, first, rest = [t.strip() for t in line.split("|")]
            out.append((bytes.fromhex(hexb.replace(" ", "")), [int(v) for v in first.split()], int(rest.split("=")[1])))
    return out


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c[0][:4].hex())
def test_hand_decoded_beats(case):
    raw, first, rest = case
    # one row of 64 columns takes one 80-column beat
    w = oracle.b3_decode(np.frombuffer(raw, dtype=np.uint8), 1, 64)
    assert list(w[0, :20]) == first
    assert np.all(w[0, 20:] == rest)


def _page_sizes():
    out = {}
    with open(os.path.join(GOLDEN, "page_sizes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value, _ = [t.strip() for t in line.split("|")]
                out[name] = float(value)
    return out


def test_sizes_against_the_pages():
    p = _page_sizes()
    assert 3 ** 5 == 243 <= 256
    assert 8 * oracle.block_bytes(B3) / oracle.block_weights(B3) == p["b3_bits_per_trit"]
    # the BitNet body in base-3 beats against the same body as planar beats
    planar = sum(oracle.weight_bytes(oracle.TERNARY_PLANAR, N, K) for _, N, K in synth.BITNET_2B_LAYER)
    b3 = sum(oracle.weight_bytes(B3, N, K) for _, N, K in synth.BITNET_2B_LAYER)
    assert round(1 - b3 / planar, 1) == p["b3_traffic_saving_on_ternary_body"]
    assert oracle.weight_bytes(B3, 6912, 2560) == 6912 * 512 and oracle.weight_bytes(B3, 2560, 6912) == 2560 * 87 * 16
    assert oracle.weight_bytes(B3, 4, 100) == -1  # rows are whole planar widths (K % 64 == 0)


@pytest.mark.parametrize("K", [64, 192, 2560, 6912])
def test_round_trip_and_generator_layout(K):
    g = np.random.default_rng(K)
    N = 5
    w = g.integers(-1, 2, (N, K)).astype(np.int8)
    raw = oracle.b3_encode(w, N, K)
    assert np.array_equal(oracle.b3_decode(raw, N, K), w)
    assert np.array_equal(raw, synth.lay_out_b3(w).ravel())  # the generator lays bytes out the same way
    assert raw.max() <= 242
    Wt = synth.make_weights(B3, N, K, seed=K + 1)
    assert np.array_equal(oracle.b3_decode(Wt.raw, N, K), Wt.w)


@pytest.mark.parametrize("K", [64, 2560, 6912])
def test_matvec_against_numpy(K):
    N = 24
    Wt = synth.make_weights(B3, N, K, seed=90 + K)
    x = synth.activations(np.random.default_rng(91), 1, K)
    q, s = oracle.quantize_i8_row(x)
    acc, y = oracle.matvec_b3(Wt.raw, N, K, q[0], s[0], Wt.s_w)
    ref = Wt.w.astype(np.int64) @ q[0].astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), ref)
    ref_y = (ref.astype(np.float32) * np.float32(s[0])).astype(np.float32) * np.float32(Wt.s_w)
    assert np.array_equal(y, ref_y.astype(np.float32))
    # the same weights as planar beats give the same sums (the two ternary layouts agree)
    acc_p, y_p = oracle.matvec_planar(synth.lay_out_planar(Wt.w), N, K, q[0], s[0], Wt.s_w)
    assert np.array_equal(acc, acc_p) and np.array_equal(y, y_p)


def test_special_cases():
    K = 2560
    q = np.random.default_rng(5).integers(-128, 128, K).astype(np.int8)
    for c, mult in ((0, 0), (1, 1), (-1, -1)):
        raw = oracle.b3_encode(np.full((1, K), c, np.int8), 1, K)
        acc, _ = oracle.matvec_b3(raw, 1, K, q, 1.0, 1.0)
        assert acc[0] == mult * int(q.astype(np.int64).sum())
    raw = oracle.b3_encode(np.full((1, K), -1, np.int8), 1, K)
    acc, y = oracle.matvec_b3(raw, 1, K, np.full(K, -128, np.int8), 1.0, 1.0)
    assert acc[0] == 128 * K and y[0] == 128.0 * K


def test_device_encoding_identity():
    """The kernels read each base-3 byte v as b = ceil(256 v / 243) (what lowbit_pack_weights writes): the
    leading m base-3 digits of v are floor(3^m b / 256), so digit 5-m is F_m - 3 F_(m-1), and v = floor(243 b / 256)
    returns the stored byte.  Checked for every v."""
    for v in range(243):
        b = -(-256 * v // 243)
        assert 0 <= b <= 255 and (243 * b) >> 8 == v
        digits = [(v // 3 ** t) % 3 for t in range(5)]
        F = [0] + [(3 ** m * b) >> 8 for m in range(1, 6)]
        assert [F[m] - 3 * F[m - 1] for m in range(1, 6)] == digits[::-1]
