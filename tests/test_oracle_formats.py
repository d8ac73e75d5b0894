"""Pins of the oracle's format handling: binary16/bfloat16 conversions, block layouts, decode/encode and
the size accounting, each against something other than the oracle itself (hand-decoded blocks, numpy
and torch conversion routines, the byte counts the pages print, the generator's drawn values)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- binary16 / bfloat16 ------------------------------------------------------------------------

def test_half_to_float_exhaustive_against_numpy():
    """All 65,536 binary16 patterns decode as numpy's float16 -> float32 conversion does (the practice of
    checking a half-precision converter over every pattern)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle.halves_to_float(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_rne_sweep_against_numpy():
    g = np.random.default_rng(7)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 5.960464477539063e-08,
            2.9802322387695312e-08, 2.98023224e-08, 2.9802326e-08, 6.103515625e-05, 6.1e-05, 1e-10]
    # exact ties between neighbouring halves (both parities) in the normal and subnormal ranges
    for e in (-24, -20, -15, -14, -3, 0, 5, 14):
        ulp = 2.0 ** (e - 10) if e >= -14 else 2.0 ** -24
        base = 2.0 ** e
        for k in range(4):
            vals.append(base + (k + 0.5) * ulp)
    vals += list(g.standard_normal(3000) * 0.02) + list(g.standard_normal(3000) * 100.0)
    vals += list(np.exp(g.uniform(-20, 11.1, 3000)) * g.choice([-1, 1], 3000))
    x = np.array(vals, dtype=np.float32)
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_to_float_against_torch():
    bits = np.arange(0, 65536, 37, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --- hand-decoded blocks --------------------------------------------------------------------------

def _golden_blocks():
    rows = []
    with open(os.path.join(GOLDEN, "format_blocks.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fmt, hexb, d, first, rest = [s.strip() for s in line.split("|")]
            rows.append((fmt, bytes.fromhex(hexb.replace(" ", "")), d, [int(v) for v in first.split()],
                         int(rest.split("=")[1])))
    return rows


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c[0] + c[1][:4].hex())
def test_decode_hand_decoded_blocks(case):
    name, raw, d, first, rest = case
    fmt = {"q1": oracle.Q1_0, "q2": oracle.Q2_0_G64, "planar": oracle.TERNARY_PLANAR, "q8": oracle.Q8_0}[name]
    K = oracle.block_weights(fmt)
    w, dd = oracle.decode(fmt, np.frombuffer(raw, dtype=np.uint8), 1, K)
    assert list(w[0, :16]) == first
    assert np.all(w[0, 16:] == rest)
    if d != "d=none":
        assert dd[0, 0] == float(d.split("=")[1])


# --- sizes against the pages' numbers ---------------------------------------------------------------

def _page_sizes():
    out = {}
    with open(os.path.join(GOLDEN, "page_sizes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, value, _src = [s.strip() for s in line.split("|")]
            out[name] = float(value)
    return out


def test_block_sizes_and_bits_per_weight():
    p = _page_sizes()
    for fmt in (oracle.Q1_0, oracle.Q2_0_G64):
        assert oracle.block_bytes(fmt) == p["ggml_block_bytes"]
    assert oracle.block_bytes(oracle.TERNARY_PLANAR) == p["planar_beat_bytes"]
    assert oracle.block_weights(oracle.TERNARY_PLANAR) == 64
    assert 8 * oracle.block_bytes(oracle.Q1_0) / oracle.block_weights(oracle.Q1_0) == p["q1_bits_per_weight"]
    assert 8 * oracle.block_bytes(oracle.Q2_0_G64) / oracle.block_weights(oracle.Q2_0_G64) == p["q2_bits_per_weight"]
    assert oracle.weight_bytes(oracle.Q1_0, 4, 100) == -1  # K not a whole number of blocks


def test_q8_0_block_size_against_the_cache_fraction():
    """A q8_0 block is a binary16 scale and 32 bytes: 34 bytes where f16 takes 64, the "53 %" the pages give
    for the q8_0 KV cache, and 8.5 bits per weight."""
    p = _page_sizes()
    assert oracle.block_weights(oracle.Q8_0) == 32 and oracle.block_bytes(oracle.Q8_0) == 34
    assert round(100 * oracle.block_bytes(oracle.Q8_0) / (2 * oracle.block_weights(oracle.Q8_0))) == p[
        "q8_0_cache_percent_of_f16"]
    assert oracle.weight_bytes(oracle.Q8_0, 4096, 4096) == 4096 * 4096 * 17 // 16
    assert oracle.weight_bytes(oracle.Q8_0, 4, 48) == -1


def test_qwen3_8b_shapes_reproduce_the_pages_counts():
    p = _page_sizes()
    layer = sum(N * K for _, N, K in synth.QWEN3_8B_LAYER)
    _, vocab, dim = synth.QWEN3_8B_OUTPUT
    # 36 layers of 7 projections, plus the token embedding and the output matrix
    assert synth.QWEN3_8B_LAYERS * layer + 2 * vocab * dim == p["qwen3_8b_weights"]
    # one ternary token: the 252 layer products plus the output matrix
    tok = sum(oracle.weight_bytes(oracle.Q2_0_G64, N, K) for _, N, K in synth.QWEN3_8B_LAYER) * synth.QWEN3_8B_LAYERS
    tok += oracle.weight_bytes(oracle.Q2_0_G64, vocab, dim)
    assert tok == 2_128_219_776
    assert round(tok / 1e9, 2) == p["ternary_token_bytes_gb"]


def test_bitnet_shapes_reproduce_the_pages_counts():
    p = _page_sizes()
    largest = max(oracle.weight_bytes(oracle.TERNARY_PLANAR, N, K) for _, N, K in synth.BITNET_2B_LAYER)
    assert largest == 4_423_680 and round(largest / 1e6, 1) == p["largest_planar_product_mb"]
    N, K = synth.BITNET_HEAD
    assert N * K * 2 == p["head_bf16_bytes"] and N * K * 4 == p["head_f32_bytes"]
    assert len(synth.BITNET_2B_LAYER) * synth.BITNET_2B_LAYERS == 210  # "210 ternary matvecs" per step


def test_generator_format_bytes_agree_with_oracle():
    for fmt in (oracle.Q1_0, oracle.Q2_0_G64, oracle.TERNARY_PLANAR, oracle.Q8_0):
        for N, K in ((3, 128), (1024, 4096), (7, 12288)):
            assert synth.format_bytes(fmt, N, K) == oracle.weight_bytes(fmt, N, K)


# --- decode / encode against the generator's drawn values ----------------------------------------------

@pytest.mark.parametrize("fmt", [oracle.Q1_0, oracle.Q2_0_G64, oracle.TERNARY_PLANAR, oracle.Q8_0])
def test_decode_recovers_drawn_weights(fmt):
    Wt = synth.make_weights(fmt, 9, 384, seed=11)
    w, d = oracle.decode(fmt, Wt.raw, 9, 384)
    assert np.array_equal(w, Wt.w)
    if fmt != oracle.TERNARY_PLANAR:
        assert np.array_equal(d, Wt.d.astype(np.float32))


@pytest.mark.parametrize("fmt", [oracle.Q1_0, oracle.Q2_0_G64, oracle.TERNARY_PLANAR, oracle.Q8_0])
def test_encode_decode_round_trip(fmt):
    g = np.random.default_rng(3)
    N, K = 5, 640
    if fmt == oracle.Q1_0:
        w = np.where(g.integers(0, 2, (N, K)) == 1, 1, -1).astype(np.int8)
    elif fmt == oracle.Q8_0:
        w = g.integers(-128, 128, (N, K)).astype(np.int8)  # every byte, -128 included
    elif fmt == oracle.Q2_0_G64:
        w = g.integers(-1, 3, (N, K)).astype(np.int8)  # includes code 3 (+2)
    else:
        w = g.integers(-1, 2, (N, K)).astype(np.int8)
    qk = oracle.block_weights(fmt)
    dh = g.integers(0, 0x7c00, (N, K // qk)).astype(np.uint16) if fmt != oracle.TERNARY_PLANAR else None
    raw = oracle.encode(fmt, w, dh, N, K)
    w2, d2 = oracle.decode(fmt, raw, N, K)
    assert np.array_equal(w2, w)
    if dh is not None:
        assert np.array_equal(d2, dh.view(np.float16).astype(np.float32))
        # the oracle's encoder lays bytes out exactly as the generator does
        lay = {oracle.Q1_0: synth.lay_out_q1_0, oracle.Q2_0_G64: synth.lay_out_q2_0, oracle.Q8_0: synth.lay_out_q8_0}
        gen = lay[fmt](w, dh.view(np.float16))
        assert np.array_equal(raw, gen.ravel())
    else:
        assert np.array_equal(raw, synth.lay_out_planar(w).ravel())


def test_generator_distribution():
    """Codes -1/0/+1/+2 at 31/38/31/0 % within 5 sigma; sign bits fair (generator check)."""
    n = 1 << 20
    Wt = synth.make_weights(oracle.Q2_0_G64, 256, n // 256, seed=5)
    w, _ = oracle.decode(oracle.Q2_0_G64, Wt.raw, 256, n // 256)
    for v, p in zip((-1, 0, 1, 2), synth.TERNARY_P):
        f = np.mean(w == v)
        assert abs(f - p) <= 5 * np.sqrt(max(p * (1 - p), 1e-12) / n) + (0 if p else 0.0)
    W1 = synth.make_weights(oracle.Q1_0, 256, n // 256, seed=6)
    w1, _ = oracle.decode(oracle.Q1_0, W1.raw, 256, n // 256)
    assert abs(np.mean(w1 == 1) - 0.5) <= 5 * np.sqrt(0.25 / n)
    Wp = synth.make_weights(oracle.TERNARY_PLANAR, 256, n // 256, seed=7)
    wp, _ = oracle.decode(oracle.TERNARY_PLANAR, Wp.raw, 256, n // 256)
    assert not np.any(wp == 2)
    for v, p in zip((-1, 0, 1), synth.TERNARY_P):
        assert abs(np.mean(wp == v) - p) <= 5 * np.sqrt(p * (1 - p) / n)
