"""Pins of the oracle's integer sums and outputs: the three exact forms of the select-accumulate identity,
brute force against numpy on the generator's drawn weights, the code-map special cases, the i8-negation
trap, exact rational arithmetic on small cases, and the planar and head outputs."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

Q_FMTS = [oracle.Q1_0, oracle.Q2_0_G64, oracle.Q8_0]


def _blocks_np(w, q):
    """numpy brute force: per-(row, 32-block) int64 sums of drawn weights times activations."""
    N, K = w.shape
    return np.einsum("njk,jk->nj", w.reshape(N, K // 32, 32).astype(np.int64),
                     q.reshape(K // 32, 32).astype(np.int64))


@pytest.mark.parametrize("fmt", Q_FMTS)
@pytest.mark.parametrize("K", [128, 384, 640])  # odd block counts per row ("tail blocks")
def test_three_forms_agree_and_match_brute_force(fmt, K):
    N = 6
    Wt = synth.make_weights(fmt, N, K, seed=100 + K, p=(0.25, 0.25, 0.25, 0.25))  # includes code 3 (+2)
    g = np.random.default_rng(K)
    q = g.integers(-128, 128, K).astype(np.int8)
    q[:5] = [-128, -128, 127, -127, 0]
    ref = _blocks_np(Wt.w, q)
    for form in ("multiply", "select", "offset"):
        s = oracle.block_sums(fmt, Wt.raw, N, K, q, form=form)
        assert np.array_equal(s.astype(np.int64), ref), form


def test_q2_code_map_special_cases():
    """All code 1 -> 0; all code 2 -> sum q; all code 0 -> -sum q; all code 3 -> 2 sum q."""
    K = 128
    g = np.random.default_rng(9)
    q = g.integers(-128, 128, K).astype(np.int8)
    sq = q.reshape(-1, 32).astype(np.int64).sum(axis=1)
    for code, mult in ((1, 0), (2, 1), (0, -1), (3, 2)):
        w = np.full((1, K), code - 1, dtype=np.int8)
        raw = oracle.encode(oracle.Q2_0_G64, w, np.full((1, 2), 0x3C00, np.uint16), 1, K)
        s = oracle.block_sums(oracle.Q2_0_G64, raw, 1, K, q)
        assert np.array_equal(s[0].astype(np.int64), mult * sq)


def test_q8_special_cases():
    """Q8_0 weights: a constant byte c gives c * sum q per block; the byte extremes -128 and +127 against
    activations -128 give 32 * 16384 and -32 * 16256 per block (no wrap anywhere); a one-hot activation
    reads one column of the dequantised weights."""
    K = 256
    q = np.random.default_rng(10).integers(-128, 128, K).astype(np.int8)
    sq = q.reshape(-1, 32).astype(np.int64).sum(axis=1)
    dh = np.full((1, K // 32), 0x3C00, np.uint16)
    for c in (-128, -1, 0, 1, 7, 127):
        raw = oracle.encode(oracle.Q8_0, np.full((1, K), c, np.int8), dh, 1, K)
        for form in ("multiply", "select", "offset"):
            assert np.array_equal(oracle.block_sums(oracle.Q8_0, raw, 1, K, q, form=form)[0].astype(np.int64),
                                  c * sq), (c, form)
    qm = np.full(K, -128, np.int8)
    for c, per in ((-128, 32 * 16384), (127, -32 * 16256)):
        raw = oracle.encode(oracle.Q8_0, np.full((1, K), c, np.int8), dh, 1, K)
        assert np.all(oracle.block_sums(oracle.Q8_0, raw, 1, K, qm) == per)
    Wt = synth.make_weights(oracle.Q8_0, 8, K, seed=52)
    k = 101
    q1 = np.zeros(K, np.int8)
    q1[k] = 1
    y, _ = oracle.matvec_q(oracle.Q8_0, Wt.raw, 8, K, q1, np.full(K // 32, 0x3C00, np.uint16))
    assert np.array_equal(y, Wt.w[:, k].astype(np.float64) * Wt.d[:, k // 32].astype(np.float64))


def test_q1_special_cases():
    K = 256
    q = np.random.default_rng(8).integers(-128, 128, K).astype(np.int8)
    sq = q.reshape(-1, 32).astype(np.int64).sum(axis=1)
    dh = np.full((1, 2), 0x3C00, np.uint16)
    for sign in (1, -1):
        raw = oracle.encode(oracle.Q1_0, np.full((1, K), sign, np.int8), dh, 1, K)
        assert np.array_equal(oracle.block_sums(oracle.Q1_0, raw, 1, K, q)[0].astype(np.int64), sign * sq)


@pytest.mark.parametrize("fmt", Q_FMTS + [oracle.TERNARY_PLANAR])
def test_minus_128_trap(fmt):
    """Activations all -128 against weights all -1: +4096 per 32-block, never a wrap in the i8 domain."""
    K = 256
    q = np.full(K, -128, np.int8)
    w = np.full((1, K), -1, np.int8)
    qk = oracle.block_weights(fmt)
    dh = None if fmt == oracle.TERNARY_PLANAR else np.full((1, K // qk), 0x3C00, np.uint16)
    raw = oracle.encode(fmt, w, dh, 1, K)
    if fmt == oracle.TERNARY_PLANAR:
        acc, y = oracle.matvec_planar(raw, 1, K, q, 1.0, 1.0)
        assert acc[0] == 128 * K and y[0] == 128.0 * K
    else:
        assert np.all(oracle.block_sums(fmt, raw, 1, K, q) == 4096)
        y, _ = oracle.matvec_q(fmt, raw, 1, K, q, np.full(K // 32, 0x3C00, np.uint16))
        assert y[0] == 128.0 * K


def _exact_y(w, d, q, dh):
    """Exact rational y for tiny cases: sum_b d_w * sum_j d_x * isum."""
    N, K = w.shape
    qk = K // d.shape[1]
    out = []
    for r in range(N):
        tot = Fraction(0)
        for j in range(K // 32):
            isum = int(np.dot(w[r, 32 * j:32 * j + 32].astype(np.int64), q[32 * j:32 * j + 32].astype(np.int64)))
            tot += Fraction(float(d[r, (32 * j) // qk])) * Fraction(float(dh.view(np.float16)[j])) * isum
        out.append(tot)
    return out


@pytest.mark.parametrize("fmt", Q_FMTS)
def test_matvec_q_against_exact_rationals(fmt):
    N, K = 5, 384
    Wt = synth.make_weights(fmt, N, K, seed=21)
    x = synth.activations(np.random.default_rng(22), 1, K)
    q, dh = oracle.quantize_q8_0(x)
    y, A = oracle.matvec_q(fmt, Wt.raw, N, K, q[0], dh[0])
    exact = _exact_y(Wt.w, Wt.d, q[0], dh[0])
    n = K // 32
    for r in range(N):
        # fp64 summation of n exact terms: |error| <= (n-1) * 2^-53 * A
        assert abs(Fraction(y[r]) - exact[r]) <= Fraction(n * 2.0 ** -53) * Fraction(A[r])


@pytest.mark.parametrize("fmt", Q_FMTS)
def test_matvec_q_brute_force_numpy(fmt):
    N, K = 64, 4096
    Wt = synth.make_weights(fmt, N, K, seed=31)
    x = synth.activations(np.random.default_rng(32), 1, K)
    q, dh = oracle.quantize_q8_0(x)
    y, A = oracle.matvec_q(fmt, Wt.raw, N, K, q[0], dh[0])
    isum = _blocks_np(Wt.w, q[0]).astype(np.float64)
    dw = np.repeat(Wt.d.astype(np.float64), K // 32 // Wt.d.shape[1], axis=1)
    dx = dh[0].view(np.float16).astype(np.float64)
    terms = dw * dx[None, :] * isum
    ref = np.array([np.float64(sum(sorted(t, key=abs))) for t in terms])
    assert np.allclose(A, np.abs(terms).sum(axis=1), rtol=1e-14)
    assert np.all(np.abs(y - ref) <= 2 * (K // 32) * 2.0 ** -53 * A)
    # row subsets give the same values as the full computation
    rows = np.array([63, 0, 17, 17])
    ys, As = oracle.matvec_q(fmt, Wt.raw, N, K, q[0], dh[0], rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(As, A[rows])


@pytest.mark.parametrize("fmt", Q_FMTS)
def test_unit_scales_give_integer_outputs(fmt):
    """With every binary16 scale 1.0 the output is the integer sum of the block sums, exactly."""
    N, K = 4, 512
    Wt = synth.make_weights(fmt, N, K, seed=41)
    qk = oracle.block_weights(fmt)
    raw = oracle.encode(fmt, Wt.w, np.full((N, K // qk), 0x3C00, np.uint16), N, K)
    q = np.random.default_rng(42).integers(-128, 128, K).astype(np.int8)
    y, _ = oracle.matvec_q(fmt, raw, N, K, q, np.full(K // 32, 0x3C00, np.uint16))
    assert np.array_equal(y, (Wt.w.astype(np.int64) @ q.astype(np.int64)).astype(np.float64))


def test_one_hot_activation_reads_one_dequantised_column():
    N, K = 8, 256
    Wt = synth.make_weights(oracle.Q2_0_G64, N, K, seed=51)
    k = 77
    q = np.zeros(K, np.int8)
    q[k] = 1
    dh = np.full(K // 32, 0x3C00, np.uint16)
    y, _ = oracle.matvec_q(oracle.Q2_0_G64, Wt.raw, N, K, q, dh)
    assert np.array_equal(y, Wt.w[:, k].astype(np.float64) * Wt.d[:, k // 64].astype(np.float64))


def test_planar_against_numpy():
    N, K = 32, 2560
    Wt = synth.make_weights(oracle.TERNARY_PLANAR, N, K, seed=61)
    x = synth.activations(np.random.default_rng(62), 1, K)
    q, s = oracle.quantize_i8_row(x)
    acc, y = oracle.matvec_planar(Wt.raw, N, K, q[0], s[0], Wt.s_w)
    ref_acc = Wt.w.astype(np.int64) @ q[0].astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), ref_acc)
    ref_y = (ref_acc.astype(np.float32) * np.float32(s[0])).astype(np.float32) * np.float32(Wt.s_w)
    assert np.array_equal(y, ref_y.astype(np.float32))


def test_planar_bit_serial_identity():
    """The bit-serial form the popcount kernel computes (two's-complement activation planes, sign plane weighing
    -128) gives the oracle's planar sums exactly, every activation byte included."""
    N, K = 16, 2560
    Wt = synth.make_weights(oracle.TERNARY_PLANAR, N, K, seed=63)
    q = np.random.default_rng(64).integers(-128, 128, K).astype(np.int8)
    q[:4] = [-128, 127, -1, 0]
    acc, _ = oracle.matvec_planar(Wt.raw, N, K, q, 1.0, 1.0)
    bits = np.unpackbits(q.view(np.uint8)[:, None], axis=1, bitorder="little")  # [K][8], plane p = bit p
    weight = np.array([1, 2, 4, 8, 16, 32, 64, -128], np.int64)
    pos, neg = (Wt.w == 1), (Wt.w == -1)
    serial = sum(weight[p] * ((pos & bits[:, p].astype(bool)).sum(axis=1) - (neg & bits[:, p].astype(bool)).sum(axis=1))
                 for p in range(8))
    assert np.array_equal(serial, acc.astype(np.int64))


def test_planar_both_planes_set_reads_zero():
    raw = np.zeros(16, np.uint8)
    raw[0] = 0xFF  # columns 0..7 in the +1 plane
    raw[8] = 0x0F  # columns 0..3 also in the -1 plane -> 0
    q = np.arange(1, 65, dtype=np.int8)
    acc, _ = oracle.matvec_planar(raw, 1, 64, q, 1.0, 1.0)
    assert acc[0] == sum(range(5, 9))


def test_head_against_numpy_fp64():
    N, K = 48, 2560
    W = synth.head_weights(N, K, seed=71)
    x = synth.activations(np.random.default_rng(72), 1, K)[0]
    y, A = oracle.head_matvec(W, N, K, x)
    Wf = torch.from_numpy(W.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    ref = Wf @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 2 * K * 2.0 ** -53 * A)
    assert np.allclose(A, np.abs(Wf * x.astype(np.float64)).sum(axis=1), rtol=1e-12)


def test_head_i8_against_numpy_and_rationals():
    """int8 head: fp64 numpy (exact products) on a full-width sample, exact rationals on a tiny case, and a
    per-row scale of 1 with integer x gives the integer dot product exactly."""
    N, K = 40, 2560
    W, s = synth.head_weights_i8(N, K, seed=73)
    x = synth.activations(np.random.default_rng(74), 1, K)[0]
    y, A = oracle.head_matvec_i8(W, s, N, K, x)
    dots = W.astype(np.float64) @ x.astype(np.float64)
    assert np.all(np.abs(y - s.astype(np.float64) * dots) <= 2 * K * 2.0 ** -53 * A)
    mags = np.abs(W.astype(np.float64) * x.astype(np.float64)).sum(axis=1)
    assert np.allclose(A, np.abs(s.astype(np.float64)) * mags, rtol=1e-12)
    Wt, st = W[:3, :16], s[:3]
    xt = x[:16]
    y3, _ = oracle.head_matvec_i8(Wt, st, 3, 16, xt)
    for r in range(3):
        exact = Fraction(float(st[r])) * sum(Fraction(int(Wt[r, k])) * Fraction(float(xt[k])) for k in range(16))
        assert abs(Fraction(y3[r]) - exact) <= Fraction(16 * 2.0 ** -52) * abs(exact) + Fraction(2.0 ** -1074)
    xi = np.random.default_rng(75).integers(-50, 50, K).astype(np.float32)
    yi, _ = oracle.head_matvec_i8(W, np.ones(N, np.float32), N, K, xi)
    assert np.array_equal(yi, (W.astype(np.int64) @ xi.astype(np.int64)).astype(np.float64))


def test_int8_head_speedup_the_pages_quote():
    """An int8 head (N*K bytes plus one fp32 scale per row) in place of the f32 one shrinks the tied-head
    2B token by the ~2.2x the pages give, with the ternary body that makes the f32 head 2.5:1."""
    import os
    p = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value, _ = [t.strip() for t in line.split("|")]
                p[name] = float(value)
    N, K = synth.BITNET_HEAD
    body = p["bitnet_gqa_ternary_body_bytes"]
    # the body the 2.5:1 figure implies: 4 x 2560^2 with k/v at 640 rows, 2 x 6912 x 2560, 2560 x 6912, 30 layers
    gqa = sum(oracle.weight_bytes(oracle.TERNARY_PLANAR, n, k) for n, k in
              ((2560, 2560), (640, 2560), (640, 2560), (2560, 2560), (6912, 2560), (6912, 2560), (2560, 6912))) * 30
    assert gqa == body and round(p["head_f32_bytes"] / body, 1) == 2.5
    # the generator's GQA block (used by the benchmark) is that body
    assert sum(oracle.weight_bytes(oracle.TERNARY_PLANAR, n, k) for _, n, k in synth.BITNET_2B_GQA_LAYER) * 30 == body
    int8_head = N * K + 4 * N
    assert round((p["head_f32_bytes"] + body) / (int8_head + body), 1) == p["head_int8_token_speedup"]


def test_gemm_rows_are_matvecs():
    N, K, M = 16, 512, 5
    Wt = synth.make_weights(oracle.Q1_0, N, K, seed=81)
    X = synth.activations(np.random.default_rng(82), M, K)
    Q, DH = oracle.quantize_q8_0(X)
    Y, A = oracle.gemm_q(oracle.Q1_0, Wt.raw, N, K, Q, DH)
    for m in range(M):
        isum = _blocks_np(Wt.w, Q[m]).astype(np.float64)
        dw = np.repeat(Wt.d.astype(np.float64), 4, axis=1)
        ref = (dw * DH[m].view(np.float16).astype(np.float64)[None, :] * isum).sum(axis=1)
        assert np.all(np.abs(Y[m] - ref) <= 2 * (K // 32) * 2.0 ** -53 * A[m])


def test_tolerance_rule():
    ok, worst, floored = oracle.tolerance_ok([1.0, 2.0], [1.0, 2.0 + 1e-6], [1.0, 2.0], 1)
    assert ok and floored == 0
    ok, *_ = oracle.tolerance_ok([1.0], [1.0 + 1e-4], [1.0], 1)
    assert not ok
    # a cancellation residue: |y| far below A/sqrt(n) is judged against the floor
    ok, worst, floored = oracle.tolerance_ok([1e-3 + 5e-7], [1e-3], [100.0], 100)
    assert ok and floored == 1
