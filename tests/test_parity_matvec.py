"""GPU parity of the decode products (Q1_0, Q2_0_g64, planar, Q8_0) and the activation quantisers against the
CPU oracle, through the C ABI: per-block integer sums bit-exact, fp32 outputs within 1e-5 relative
(with the cancellation floor), planar outputs and quantised bytes bit-exact."""
import numpy as np
import pytest
import torch

import bit_quantized_matvec_q1_amd.lowbit as L
import oracle
import synth
from gpu_util import act_for, assert_close, dev, gpu_matvec, gpu_sums, host, packed_weights, say

pytestmark = pytest.mark.gpu

Q_FMTS = [synth.Q1_0, synth.Q2_0_G64, synth.Q8_0]
ALL_FMTS = Q_FMTS + [synth.TERNARY_PLANAR, synth.TERNARY_B3]
ROW_FMTS = (synth.TERNARY_PLANAR, synth.TERNARY_B3)  # per-token activations, per-tensor scale, row sums
NAMES = {synth.Q1_0: "Q1_0", synth.Q2_0_G64: "Q2_0_g64", synth.TERNARY_PLANAR: "planar", synth.Q8_0: "Q8_0",
         synth.TERNARY_B3: "base3"}
MAX_K = {synth.Q8_0: 16384, synth.TERNARY_B3: 30720}
QK = {synth.Q1_0: 128, synth.Q2_0_G64: 64, synth.Q8_0: 32}


def check_product(fmt, N, K, seed, p=synth.TERNARY_P, q_override=None, rows=None):
    say(f"case {NAMES[fmt]} N={N} K={K} seed={seed}")
    Wt = synth.make_weights(fmt, N, K, seed, p=p)
    q, xs, _ = act_for(fmt, K, seed + 1)
    if q_override is not None:
        q = q_override(q)
    packed = packed_weights(Wt)
    y = gpu_matvec(fmt, packed, N, K, q, xs, w_scale=Wt.s_w if Wt.s_w is not None else 1.0)
    sums = gpu_sums(fmt, packed, N, K, q[None, :], xs[None, :] if fmt not in ROW_FMTS else xs)[0]
    r = np.arange(N) if rows is None else np.asarray(rows)
    if fmt in ROW_FMTS:
        mv = oracle.matvec_planar if fmt == synth.TERNARY_PLANAR else oracle.matvec_b3
        acc, y_ref = mv(Wt.raw, N, K, q, xs[0], Wt.s_w, rows=r)
        assert np.array_equal(sums[r], acc), "row sums differ"
        assert np.array_equal(y[r], y_ref), "outputs differ"
    else:
        ref_sums = oracle.block_sums(fmt, Wt.raw, N, K, q, rows=r)
        assert np.array_equal(sums[r], ref_sums), "per-block integer sums differ"
        y_ref, A = oracle.matvec_q(fmt, Wt.raw, N, K, q, xs, rows=r)
        assert_close(y[r], y_ref, A, K // 32, f"{NAMES[fmt]} {N}x{K}")
    return y


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=NAMES.get)
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (300, 640), (1000, 1024), (517, 2560), (130, 4096),
                                 (70, 6912), (33, 12288)])
def test_matvec_shapes(fmt, N, K):
    if K > MAX_K.get(fmt, 32768):
        pytest.skip(f"{NAMES[fmt]} rows are limited to K <= {MAX_K[fmt]}")
    check_product(fmt, N, K, seed=1000 + N + K)


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=NAMES.get)
def test_matvec_odd_block_counts(fmt):
    # ragged tails: odd numbers of blocks per row, and row counts that leave partial tiles
    qk = QK.get(fmt, 64)
    for K in (qk * 3, qk * 5, qk * 9) if fmt == synth.Q1_0 else (qk * 3, qk * 7, qk * 33):
        check_product(fmt, 129, K, seed=2000 + K)


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=NAMES.get)
def test_matvec_largest_k(fmt):
    check_product(fmt, 20, MAX_K.get(fmt, 32768), seed=2100)


def test_q2_code3_and_minus_128():
    # every code including 3 (+2), and the activation extremes
    def extremes(q):
        q = q.copy()
        q[::7] = -128
        q[3::11] = 127
        return q

    check_product(synth.Q2_0_G64, 257, 4096, seed=2200, p=(0.25, 0.25, 0.25, 0.25), q_override=extremes)


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=NAMES.get)
def test_minus_128_against_all_minus_one(fmt):
    """The i8-negation trap: q = -128 everywhere, every weight -1 -> +4096 per block of 32."""
    N, K = 65, 1024
    say(f"case minus128 {NAMES[fmt]}")
    w = np.full((N, K), -1, np.int8)
    if fmt == synth.Q1_0:
        raw = synth.lay_out_q1_0(w, np.full((N, K // 128), 1.0, np.float16))
    elif fmt == synth.Q8_0:
        raw = synth.lay_out_q8_0(w, np.full((N, K // 32), 1.0, np.float16))
    elif fmt == synth.Q2_0_G64:
        raw = synth.lay_out_q2_0(w, np.full((N, K // 64), 1.0, np.float16))
    elif fmt == synth.TERNARY_B3:
        raw = synth.lay_out_b3(w)
    else:
        raw = synth.lay_out_planar(w)
    Wt = synth.Weights(fmt, N, K, raw, w, s_w=np.float32(1.0))
    q = np.full(K, -128, np.int8)
    xs = np.array([1.0], np.float32) if fmt in ROW_FMTS else np.full(K // 32, 0x3C00, np.uint16)
    packed = packed_weights(Wt)
    sums = gpu_sums(fmt, packed, N, K, q[None, :], xs[None, :] if fmt not in ROW_FMTS else xs)[0]
    y = gpu_matvec(fmt, packed, N, K, q, xs)
    if fmt in ROW_FMTS:
        assert np.all(sums == 128 * K)
    else:
        assert np.all(sums == 4096)
    assert np.all(y == 128.0 * K)


def test_q8_byte_extremes():
    """Q8_0 bytes -128 and +127 against activations -128: 32 * 16384 and -32 * 16256 per block, and with
    unit scales the row totals 2^24 and -16256 * 1024 exactly (no wrap in any 8- or 16-bit step)."""
    N, K = 40, 1024
    q = np.full(K, -128, np.int8)
    ones = np.full(K // 32, 0x3C00, np.uint16)
    for c, per in ((-128, 32 * 16384), (127, -32 * 16256)):
        say(f"case q8 extremes c={c}")
        w = np.full((N, K), c, np.int8)
        Wt = synth.Weights(synth.Q8_0, N, K, synth.lay_out_q8_0(w, np.full((N, K // 32), 1.0, np.float16)), w)
        packed = packed_weights(Wt)
        assert np.all(gpu_sums(synth.Q8_0, packed, N, K, q[None, :], ones[None, :])[0] == per)
        assert np.all(gpu_matvec(synth.Q8_0, packed, N, K, q, ones) == float(per * (K // 32)))


@pytest.mark.parametrize("fmt", Q_FMTS, ids=NAMES.get)
def test_unit_scales_bit_exact(fmt):
    """With every binary16 scale 1.0 each term is an integer below 2^24: y must equal the oracle exactly."""
    N, K = 300, 4096
    say(f"case unit-scales {NAMES[fmt]}")
    Wt = synth.make_weights(fmt, N, K, seed=2300)
    qk = QK[fmt]
    # Q8_0 bytes are brought down to [-15, 15] so that every partial sum of a row stays below 2^24
    w = (Wt.w // 8).astype(np.int8) if fmt == synth.Q8_0 else Wt.w
    raw = oracle.encode(fmt, w, np.full((N, K // qk), 0x3C00, np.uint16), N, K)
    Wu = synth.Weights(fmt, N, K, raw.reshape(N, K // qk, synth.BLOCK_BYTES[fmt]), w)
    q, _, _ = act_for(fmt, K, 2301)
    ones = np.full(K // 32, 0x3C00, np.uint16)
    y = gpu_matvec(fmt, packed_weights(Wu), N, K, q, ones)
    y_ref, _ = oracle.matvec_q(fmt, raw, N, K, q, ones)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("fmt", Q_FMTS, ids=NAMES.get)
def test_zero_activation_blocks(fmt):
    """amax = 0 blocks: scale 0, every q 0."""
    K = 4096
    x = synth.activations(synth.rng(2400), 1, K)
    x[0, 64:160] = 0.0
    q, dh, _ = act_for(fmt, K, 0, x=x)
    assert np.all(q[64:160] == 0)
    N = 128
    Wt = synth.make_weights(fmt, N, K, 2401)
    packed = packed_weights(Wt)
    y = gpu_matvec(fmt, packed, N, K, q, dh)
    y_ref, A = oracle.matvec_q(fmt, Wt.raw, N, K, q, dh)
    assert_close(y, y_ref, A, K // 32, "zero blocks")


def test_empty_and_k0():
    say("case empty")
    y = torch.full((5,), 7.0, device="cuda")
    q = torch.zeros(16, dtype=torch.int8, device="cuda")
    xs = torch.zeros(8, dtype=torch.uint16, device="cuda")
    W = torch.zeros(16, dtype=torch.uint8, device="cuda")
    L.lowbit_matvec(synth.Q2_0_G64, W, 0, 64, 1.0, L.ACT_Q8_0, q, xs, y)  # N = 0: untouched
    assert np.all(host(y) == 7.0)
    L.lowbit_matvec(synth.Q2_0_G64, W, 5, 0, 1.0, L.ACT_Q8_0, q, xs, y)  # K = 0: empty sums
    assert np.all(host(y) == 0.0)


@pytest.mark.parametrize("N,K", [(1, 64), (37, 384), (300, 640), (517, 2560), (70, 6912), (9, 8192)])
def test_popcount_agrees_with_select_accumulate_and_oracle(N, K):
    """Three implementations of the planar product (tritium "Architecture", section 5): the bit-serial popcount
    kernel, the select-accumulate kernel and the oracle give the same row sums and the same fp32 outputs, bit
    for bit, with the activation extremes included."""
    fmt = synth.TERNARY_PLANAR
    say(f"case popcount N={N} K={K}")
    Wt = synth.make_weights(fmt, N, K, 2700 + K)
    q, xs, _ = act_for(fmt, K, 2701 + K)
    q = q.copy()
    q[::13] = -128
    q[5::17] = 127
    packed = packed_weights(Wt)
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    sums = torch.empty(N, dtype=torch.int32, device="cuda")
    L.lowbit_matvec_popcount(packed, N, K, float(Wt.s_w), dev(q), dev(xs), y, sums)
    acc, y_ref = oracle.matvec_planar(Wt.raw, N, K, q, xs[0], Wt.s_w)
    assert np.array_equal(host(sums), acc)
    assert np.array_equal(host(y), y_ref)
    assert np.array_equal(host(y), gpu_matvec(fmt, packed, N, K, q, xs, w_scale=Wt.s_w))
    y_only = torch.empty(N, dtype=torch.float32, device="cuda")
    L.lowbit_matvec_popcount(packed, N, K, float(Wt.s_w), dev(q), dev(xs), y_only)
    assert np.array_equal(host(y_only), y_ref)


def test_b3_pack_round_trip():
    """Base-3 beats: pack writes ceil(256 v / 243) per byte and unpack restores every byte exactly."""
    say("case pack base3")
    Wt = synth.make_weights(synth.TERNARY_B3, 77, 2560, 2510)
    packed = packed_weights(Wt)
    v = Wt.raw.reshape(-1).astype(np.int64)
    assert np.array_equal(host(packed).astype(np.int64), -(-256 * v // 243))
    back = torch.empty(Wt.raw.size, dtype=torch.uint8, device="cuda")
    L.lowbit_unpack_weights(synth.TERNARY_B3, packed, 77, 2560, back)
    assert np.array_equal(host(back), Wt.raw.reshape(-1))


@pytest.mark.parametrize("K", [320, 2560, 6912])
def test_b3_every_byte_value_at_every_position(K):
    """Base-3 decode covers all 243 byte values at every byte position of a beat: row r holds value
    (r + 7 j) mod 243 at byte j, so each of the 16 positions (three of every four record dwords decoded by
    table, the fourth by digit arithmetic) meets every value across the 243 rows.  Row sums and outputs
    bit for bit against the oracle, with random activations including -128 and +127."""
    N = 243
    nbt = -(-K // 80)
    say(f"case base3 all bytes K={K}")
    j = np.arange(nbt * 16)
    v = ((np.arange(N)[:, None] + 7 * j[None, :]) % 243).astype(np.int64)
    digits = np.stack([(v // 3 ** t) % 3 for t in range(5)], axis=-1).reshape(N, nbt * 80)
    w = (digits[:, :K] - 1).astype(np.int8)
    raw = synth.lay_out_b3(w)  # columns past K are coded 0, so the last beat's tail bytes differ from v
    assert np.array_equal(raw.reshape(N, -1)[:, : K // 5], v[:, : K // 5].astype(np.uint8))
    Wt = synth.Weights(synth.TERNARY_B3, N, K, raw, w, s_w=np.float32(0.75))
    g = synth.rng(2600 + K)
    q = g.integers(-128, 128, size=K).astype(np.int8)
    q[:: 97] = -128
    q[1:: 89] = 127
    xs = np.array([0.03125], np.float32)
    packed = packed_weights(Wt)
    y = gpu_matvec(synth.TERNARY_B3, packed, N, K, q, xs, w_scale=0.75)
    sums = gpu_sums(synth.TERNARY_B3, packed, N, K, q[None, :], xs)[0]
    acc, y_ref = oracle.matvec_b3(raw, N, K, q, xs[0], np.float32(0.75))
    assert np.array_equal(sums, acc), "row sums differ"
    assert np.array_equal(y, y_ref), "outputs differ"


@pytest.mark.parametrize("fmt", Q_FMTS, ids=NAMES.get)
def test_pack_round_trip(fmt):
    say(f"case pack {NAMES[fmt]}")
    Wt = synth.make_weights(fmt, 77, 1024, 2500)
    packed = packed_weights(Wt)
    back = torch.empty(Wt.raw.size, dtype=torch.uint8, device="cuda")
    L.lowbit_unpack_weights(fmt, packed, 77, 1024, back)
    assert np.array_equal(host(back), Wt.raw.reshape(-1))
    # the device layout is all code records (32 bytes for Q8_0, 16 otherwise), then all scales
    p = host(packed)
    nb = Wt.raw.shape[1]
    rb = synth.BLOCK_BYTES[fmt] - 2
    assert np.array_equal(p[: 77 * nb * rb].reshape(77, nb, rb), device_records(fmt, Wt.raw))
    assert np.array_equal(p[77 * nb * rb:].reshape(77, nb, 2), Wt.raw[:, :, :2])


def device_records(fmt, raw):
    """The documented device records of ggml blocks: Q2_0_g64 code bytes and Q8_0 weight bytes as they are;
    Q1_0 with the sign of weight 32r + 8m + k moved to bit 4k + r of little-endian dword m."""
    codes = raw[:, :, 2:]
    if fmt != synth.Q1_0:
        return codes
    bits = np.unpackbits(codes, axis=-1, bitorder="little")  # [..., 128], natural weight order
    r, m, k = np.meshgrid(np.arange(4), np.arange(4), np.arange(8), indexing="ij")
    dev = np.empty_like(bits)
    dev[..., (32 * m + 4 * k + r).ravel()] = bits[..., (32 * r + 8 * m + k).ravel()]
    return np.packbits(dev, axis=-1, bitorder="little")


def test_launch_geometry_invariance():
    """A row's result does not depend on which tile or how many rows the launch covers."""
    say("case geometry")
    fmt, N, K = synth.Q2_0_G64, 4096, 4096
    Wt = synth.make_weights(fmt, N, K, 2600)
    q, dh, _ = act_for(fmt, K, 2601)
    packed = packed_weights(Wt)
    y_full = gpu_matvec(fmt, packed, N, K, q, dh)
    y_again = gpu_matvec(fmt, packed, N, K, q, dh)
    assert np.array_equal(y_full, y_again)
    row_bytes = (K // 64) * 16
    # rows 512.. as their own tensor: a different tile layout over the same rows
    sub = Wt.raw[512:1536]
    Wsub = synth.Weights(fmt, 1024, K, sub, Wt.w[512:1536])
    y_sub = gpu_matvec(fmt, packed_weights(Wsub), 1024, K, q, dh)
    assert np.array_equal(y_sub, y_full[512:1536])
    assert row_bytes > 0


# --- quantisers -----------------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (2, 4128), (1, 4096), (7, 12288), (512, 4096)])
def test_quantize_q8_0_bytes(M, K):
    say(f"case quantize q8_0 M={M} K={K}")
    g = synth.rng(3000 + M + K)
    x = (g.standard_normal((M, K)) * np.exp(g.uniform(-6, 6, (M, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    if K >= 64:
        x[0, 32:64] = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5] * 4, np.float32)
    q_ref, d_ref = oracle.quantize_q8_0(x)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M, K // 32), dtype=torch.uint16, device="cuda")
    L.lowbit_quantize_act(L.ACT_Q8_0, dev(x), M, K, xq, xs)
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(host(xs), d_ref)


# K spans each kernel variant: rows held in registers as 1, 2, 4 or 8 float4 chunks per thread (K % 4 == 0,
# K <= 8192), and the two-pass loop (K % 4 != 0, so rows after the first are not 16-byte aligned; K > 8192)
@pytest.mark.parametrize("M,K", [(1, 2560), (3, 6912), (2, 100), (4, 4), (2, 1028), (3, 4100), (2, 8192),
                                 (2, 8196), (3, 30), (2, 12288)])
def test_quantize_i8_row_bytes(M, K):
    say(f"case quantize i8_row M={M} K={K}")
    x = synth.activations(synth.rng(3100 + K), M, K)
    x[-1] = 0.0
    q_ref, s_ref = oracle.quantize_i8_row(x)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    L.lowbit_quantize_act(L.ACT_I8_ROW, dev(x), M, K, xq, xs)
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(host(xs), s_ref)


# --- seeded shape sweep: every K the decode kernels take is a configuration choice (lanes per row, records
# per lane, a full or clamped last lane); a seeded draw of formats, row counts and K covers the choices the
# hand-picked shapes above do not ---------------------------------------------------------------------------

def _sweep_cases(n=24, seed=9000):
    g = synth.rng(seed)
    cases = []
    for i in range(n):
        fmt = ALL_FMTS[int(g.integers(0, len(ALL_FMTS)))]
        blk = {synth.Q1_0: 128, synth.Q8_0: 32}.get(fmt, 64)
        kmax = min(MAX_K.get(fmt, 32768), 8192)
        K = blk * int(g.integers(1, kmax // blk + 1))
        N = int(g.integers(1, 400))
        cases.append((fmt, N, K, seed + 1 + i))
    return cases


@pytest.mark.parametrize("fmt,N,K,seed", _sweep_cases(), ids=lambda v: str(v))
def test_matvec_seeded_shape_sweep(fmt, N, K, seed):
    check_product(fmt, N, K, seed=seed)
