"""GPU parity of the prefill product (int8 MFMA) against the CPU oracle: per-(row, column, block) integer
sums bit-exact, fp32 outputs within 1e-5 relative (cancellation floor), planar outputs bit-exact."""
import numpy as np
import pytest
import torch

import bit_quantized_matvec_q1_amd.lowbit as L
import oracle
import synth
from gpu_util import assert_close, dev, host, packed_weights, say

pytestmark = pytest.mark.gpu

NAMES = {synth.Q1_0: "Q1_0", synth.Q2_0_G64: "Q2_0_g64", synth.TERNARY_PLANAR: "planar", synth.Q8_0: "Q8_0"}
QK = {synth.Q1_0: 128, synth.Q2_0_G64: 64, synth.Q8_0: 32}


def acts(fmt, M, K, seed):
    X = synth.activations(synth.rng(seed), M, K)
    if fmt == synth.TERNARY_PLANAR:
        return oracle.quantize_i8_row(X)
    return oracle.quantize_q8_0(X)


def gpu_gemm(fmt, packed, N, K, Q, XS, M, w_scale=1.0):
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    afmt = L.ACT_I8_ROW if fmt == synth.TERNARY_PLANAR else L.ACT_Q8_0
    L.lowbit_gemm(fmt, packed, N, K, w_scale, afmt, dev(Q), dev(XS), M, Y)
    return host(Y)


def gpu_gemm_sums(fmt, packed, N, K, Q, XS, M):
    afmt = L.ACT_I8_ROW if fmt == synth.TERNARY_PLANAR else L.ACT_Q8_0
    shape = (M, N) if fmt == synth.TERNARY_PLANAR else (M, N, K // 32)
    S = torch.empty(shape, dtype=torch.int32, device="cuda")
    L.lowbit_block_sums(fmt, packed, N, K, afmt, dev(Q), dev(XS), M, S)
    return host(S)


def check(fmt, M, N, K, seed, p=synth.TERNARY_P, sums=True, m_rows=None, n_rows=None):
    say(f"case gemm {NAMES[fmt]} M={M} N={N} K={K} seed={seed}")
    Wt = synth.make_weights(fmt, N, K, seed, p=p)
    Q, XS = acts(fmt, M, K, seed + 1)
    packed = packed_weights(Wt)
    w_scale = Wt.s_w if Wt.s_w is not None else 1.0
    Y = gpu_gemm(fmt, packed, N, K, Q, XS, M, w_scale)
    ms = np.arange(M) if m_rows is None else np.asarray(m_rows)
    ns = np.arange(N) if n_rows is None else np.asarray(n_rows)
    if fmt == synth.TERNARY_PLANAR:
        for m in ms:
            acc, y_ref = oracle.matvec_planar(Wt.raw, N, K, Q[m], XS[m], Wt.s_w, rows=ns)
            assert np.array_equal(Y[m, ns], y_ref), f"planar prefill row {m} differs"
        if sums:
            S = gpu_gemm_sums(fmt, packed, N, K, Q, XS, M)
            for m in ms:
                acc, _ = oracle.matvec_planar(Wt.raw, N, K, Q[m], XS[m], Wt.s_w, rows=ns)
                assert np.array_equal(S[m, ns], acc)
        return Wt, packed, Q, XS
    Yr, A = oracle.gemm_q(fmt, Wt.raw, N, K, Q, XS, m_rows=ms, n_rows=ns)
    assert_close(Y[np.ix_(ms, ns)].ravel(), Yr.ravel(), A.ravel(), K // 32, f"{NAMES[fmt]} prefill {M}x{N}x{K}")
    if sums:
        S = gpu_gemm_sums(fmt, packed, N, K, Q, XS, M)
        for m in ms:
            ref = oracle.block_sums(fmt, Wt.raw, N, K, Q[m], rows=ns)
            assert np.array_equal(S[m, ns], ref), f"block sums of activation row {m} differ"
    return Wt, packed, Q, XS


@pytest.mark.parametrize("fmt", [synth.Q1_0, synth.Q2_0_G64, synth.TERNARY_PLANAR, synth.Q8_0], ids=NAMES.get)
@pytest.mark.parametrize("M,N,K", [(2, 1, 128), (64, 128, 128), (70, 130, 384), (33, 300, 640), (128, 256, 4096)])
def test_gemm_shapes(fmt, M, N, K):
    check(fmt, M, N, K, seed=6000 + M + N + K)


@pytest.mark.parametrize("fmt", [synth.Q1_0, synth.Q2_0_G64, synth.TERNARY_PLANAR, synth.Q8_0], ids=NAMES.get)
def test_gemm_largest_k(fmt):
    # the largest K the ABI takes (32768; 16384 for Q8_0), ragged in both M and N: every K-step rotation
    # of the walk and, for the 16-wave split workgroups, the longest per-half step count
    check(fmt, 70, 65, 16384 if fmt == synth.Q8_0 else 32768, seed=6050)


@pytest.mark.parametrize("fmt", [synth.Q2_0_G64, synth.TERNARY_PLANAR], ids=NAMES.get)
def test_gemm_odd_block_tail(fmt):
    # K = 7 blocks of 64: the last K-step of the kernel is half full
    check(fmt, 65, 129, 448, seed=6100)


@pytest.mark.parametrize("fmt", [synth.Q2_0_G64, synth.TERNARY_PLANAR], ids=NAMES.get)
@pytest.mark.parametrize("M,N,K", [(3, 70, 64), (130, 65, 192)])
def test_gemm_single_and_three_half_steps(fmt, M, N, K):
    # K = 64: one half step, so the second half of a split-K workgroup has no step at all; K = 192: one full
    # step and one half step, split one per half
    check(fmt, M, N, K, seed=6150 + K)


def test_gemm_code3_and_minus_128():
    say("case gemm code3/-128")
    fmt, M, N, K = synth.Q2_0_G64, 64, 128, 512
    Wt = synth.make_weights(fmt, N, K, 6200, p=(0.25, 0.25, 0.25, 0.25))
    Q, XS = acts(fmt, M, K, 6201)
    Q[::3, ::5] = -128
    packed = packed_weights(Wt)
    Y = gpu_gemm(fmt, packed, N, K, Q, XS, M)
    Yr, A = oracle.gemm_q(fmt, Wt.raw, N, K, Q, XS)
    assert_close(Y.ravel(), Yr.ravel(), A.ravel(), K // 32, "code3/-128")
    S = gpu_gemm_sums(fmt, packed, N, K, Q, XS, M)
    for m in range(M):
        assert np.array_equal(S[m], oracle.block_sums(fmt, Wt.raw, N, K, Q[m]))


def test_gemm_q8_0_extreme_bytes():
    """Q8_0 bytes -128 and +127 against activations -128 with unit scales: block sums of +2^19 and
    -32 * 16256, the largest the format allows, still exact through the biased accumulator."""
    say("case gemm Q8_0 extreme bytes")
    M, N, K = 70, 130, 512
    w = np.broadcast_to(np.where(np.arange(N)[:, None] % 2 == 0, -128, 127), (N, K)).astype(np.int8)
    ones = np.full((N, K // 32), 1.0, np.float16)
    Wt = synth.Weights(synth.Q8_0, N, K, synth.lay_out_q8_0(w, ones), w)
    Q = np.full((M, K), -128, np.int8)
    Q[1::2, ::7] = 127
    XS = np.full((M, K // 32), 0x3C00, np.uint16)
    packed = packed_weights(Wt)
    S = gpu_gemm_sums(synth.Q8_0, packed, N, K, Q, XS, M)
    for m in (0, 1, M - 1):
        assert np.array_equal(S[m], oracle.block_sums(synth.Q8_0, Wt.raw, N, K, Q[m]))
    assert S.max() == 32 * 16384 and S.min() == -32 * 16256
    Y = gpu_gemm(synth.Q8_0, packed, N, K, Q, XS, M)
    Yr, _ = oracle.gemm_q(synth.Q8_0, Wt.raw, N, K, Q, XS)
    assert np.array_equal(Y.astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", [synth.Q1_0, synth.Q2_0_G64, synth.Q8_0], ids=NAMES.get)
def test_gemm_unit_scales_bit_exact(fmt):
    say(f"case gemm unit scales {NAMES[fmt]}")
    M, N, K = 64, 256, 2048
    Wt = synth.make_weights(fmt, N, K, 6300)
    qk = QK[fmt]
    if fmt == synth.Q8_0:
        Wu = synth.Weights(fmt, N, K, synth.lay_out_q8_0(Wt.w, np.full((N, K // qk), 1.0, np.float16)), Wt.w)
        raw = Wu.raw
    else:
        raw = oracle.encode(fmt, Wt.w, np.full((N, K // qk), 0x3C00, np.uint16), N, K)
        Wu = synth.Weights(fmt, N, K, raw.reshape(N, K // qk, 18), Wt.w)
    Q, _ = acts(fmt, M, K, 6301)
    ones = np.full((M, K // 32), 0x3C00, np.uint16)
    Y = gpu_gemm(fmt, packed_weights(Wu), N, K, Q, ones, M)
    Yr, _ = oracle.gemm_q(fmt, raw, N, K, Q, ones)
    assert np.array_equal(Y.astype(np.float64), Yr)


@pytest.mark.parametrize("fmt", [synth.Q1_0, synth.Q2_0_G64, synth.Q8_0], ids=NAMES.get)
@pytest.mark.parametrize("N", [4096, 12288])
def test_gemm_full_size_sampled(fmt, N):
    """The prefill workload at full size (512 activation rows x N x 4096); the oracle checks a seeded
    sample of (row, column) pairs: every 64th activation row against 300 weight rows, outputs within the
    tolerance and the block sums of the same pairs bit-exact (taken from the device at full size, the
    sample gathered there)."""
    M, K = synth.PREFILL_M, 4096
    g = synth.rng(6400 + N)
    n_rows = np.unique(np.concatenate([g.integers(0, N, 300), [0, N - 1]]))
    m_rows = np.unique(np.concatenate([np.arange(0, M, 64), [M - 1]]))
    Wt, packed, Q, XS = check(fmt, M, N, K, seed=6401 + N, sums=False, m_rows=m_rows, n_rows=n_rows)
    S = torch.empty((M, N, K // 32), dtype=torch.int32, device="cuda")
    L.lowbit_block_sums(fmt, packed, N, K, L.ACT_Q8_0, dev(Q), dev(XS), M, S)
    mi, ni = torch.from_numpy(m_rows).cuda(), torch.from_numpy(n_rows).cuda()
    Ss = host(S[mi][:, ni])
    del S
    for a, m in enumerate(m_rows):
        ref = oracle.block_sums(fmt, Wt.raw, N, K, Q[m], rows=n_rows)
        assert np.array_equal(Ss[a], ref), f"full-size block sums of activation row {m} differ"


def test_gemm_rows_match_decode():
    """Row m of the prefill product equals the decode product on activation row m (same arithmetic,
    different kernels: both must sit within the tolerance of the oracle; here checked against each other
    through the oracle's tolerance rule)."""
    say("case gemm vs decode")
    fmt, M, N, K = synth.Q2_0_G64, 40, 256, 4096
    Wt = synth.make_weights(fmt, N, K, 6500)
    Q, XS = acts(fmt, M, K, 6501)
    packed = packed_weights(Wt)
    Y = gpu_gemm(fmt, packed, N, K, Q, XS, M)
    for m in (0, 17, 39):
        y = torch.empty(N, dtype=torch.float32, device="cuda")
        L.lowbit_matvec(fmt, packed, N, K, 1.0, L.ACT_Q8_0, dev(Q[m]), dev(XS[m]), y)
        yr, A = oracle.matvec_q(fmt, Wt.raw, N, K, Q[m], XS[m])
        assert_close(host(y), yr, A, K // 32, "decode row")
        assert_close(Y[m], yr, A, K // 32, "prefill row")


# --- seeded shape sweep: ragged M and N (partial tiles on both sides), K from one step to several, and grids
# on both sides of the split-K threshold ---------------------------------------------------------------------

def _sweep_cases(n=16, seed=9500):
    g = synth.rng(seed)
    fmts = [synth.Q1_0, synth.Q2_0_G64, synth.TERNARY_PLANAR, synth.Q8_0]
    cases = []
    for i in range(n):
        fmt = fmts[int(g.integers(0, len(fmts)))]
        blk = 128 if fmt in (synth.Q1_0, synth.Q8_0) else 64
        K = blk * int(g.integers(1, 2048 // blk + 1))
        cases.append((fmt, int(g.integers(1, 161)), int(g.integers(1, 201)), K, seed + 1 + i))
    return cases


@pytest.mark.parametrize("fmt,M,N,K,seed", _sweep_cases(), ids=lambda v: str(v))
def test_gemm_seeded_shape_sweep(fmt, M, N, K, seed):
    check(fmt, M, N, K, seed=seed)
