"""Seeded synthetic inputs for the packed low-bit x int8 product.

This module only *draws* inputs and lays them out in the weight formats' byte layouts; it holds none
of the product's arithmetic (no decode, no quantiser, no dot products, no scaling). Both sides of every
parity check consume the bytes it returns: the CPU oracle under ``oracle/`` and the HIP library.

Formats (byte layouts as the pages define them):

* ggml ``Q1_0`` -- bankml technical report, section III.2 "The Q1_0 format and its arithmetic":
  18-byte blocks of 128 weights, a little-endian binary16 scale ``d`` first, then 16 bytes of sign
  bits, least-significant bit first (weight i sits at byte i//8, bit i%8).
* ggml ``Q2_0_g64`` -- same report, section III.5 "The Q2_0_g64 (ternary) kernel": 18-byte blocks of
  64 weights, binary16 ``d`` first, then 16 bytes of 2-bit codes, lowest bits first (weight i at byte
  i//4, bits 2*(i%4)); code c stands for weight c-1.
* planar ternary ``.trit v1`` beat -- tritium "Architecture", section 2 "The one design commitment: bit
  planes": 16 bytes per 64 consecutive columns of one row, ``{u64 pos, u64 neg}``, column c at bit c.
* base-3 ternary beats -- the bankml report, section III.8 "Information" (five trits fit in one byte,
  3^5 = 243 <= 256) and tritium "Architecture", section 10 (base-3 packing at 1.6 b/w for the ternary
  body): 16 bytes per 80 consecutive columns of one row, byte j holding columns 5j..5j+4 as the base-3
  integer sum_t (w + 1) * 3^t, lowest digit first; a row takes ceil(K/80) beats, columns past K coded 0.
* ggml ``Q8_0`` weights -- the q8_0 block of the bankml report, section III.2 (a binary16 scale, then 32
  signed bytes), used for weights as the build history's 0.3.9 entry and its "Q8_0 weights" item do:
  34-byte blocks of 32 weights.

Workload shapes and value distributions follow the five workloads this library is measured on: block
scales fp16(|N(0,1)|*0.02), ternary codes -1/0/+1 at 31/38/31 % (the split the bankml report observed
in Ternary-Bonsai-8B), 1-bit signs Bernoulli(0.5), activations fp32 N(0,1), head weights N(0,0.02)
rounded to bfloat16.  Q8_0 weights (no workload on the pages fixes their values) take signed bytes
rint(36 * N(0,1)) clipped to [-127, 127] -- about 3.5 standard deviations to the byte's end, as a block
scaled to its largest value would hold -- with scales fp16(|N(0,1)| * 0.02 / 36).  Random numbers come from numpy's PCG64 stream seeded per input.
"""
from __future__ import annotations

import numpy as np

Q1_0 = 1
Q2_0_G64 = 2
TERNARY_PLANAR = 3
Q8_0 = 4
TERNARY_B3 = 5

QK1 = 128  # weights per Q1_0 block
QK2 = 64  # weights per Q2_0_g64 block
QKP = 64  # columns per planar beat
QKB3 = 80  # columns per base-3 beat (16 bytes of five trits)
QK8 = 32  # activations per q8_0 block (and weights per Q8_0 weight block)

BLOCK_BYTES = {Q1_0: 18, Q2_0_G64: 18, TERNARY_PLANAR: 16, Q8_0: 34}
BLOCK_WEIGHTS = {Q1_0: QK1, Q2_0_G64: QK2, TERNARY_PLANAR: QKP, Q8_0: QK8}

# ternary weight distribution of the ggml file the pages measured: P(-1), P(0), P(+1), P(+2)
TERNARY_P = (0.31, 0.38, 0.31, 0.0)


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.PCG64(seed))


def fp16_scales(g: np.random.Generator, n: int) -> np.ndarray:
    """fp16(|z| * 0.02), z ~ N(0,1): the block-scale recipe of every ggml-format workload."""
    return (np.abs(g.standard_normal(n)) * 0.02).astype(np.float16)


def ternary_weights(g: np.random.Generator, N: int, K: int, p=TERNARY_P) -> np.ndarray:
    """Dense int8 matrix of weights in {-1, 0, +1, +2} drawn i.i.d. with probabilities ``p``."""
    return (g.choice(4, size=(N, K), p=np.asarray(p, dtype=np.float64)) - 1).astype(np.int8)


def sign_weights(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Dense int8 matrix of weights in {-1, +1}, each sign a fair coin."""
    return np.where(g.integers(0, 2, size=(N, K), dtype=np.int8) == 1, 1, -1).astype(np.int8)


def byte_weights(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Dense int8 matrix of signed-byte weights: rint(36 * N(0,1)) clipped to [-127, 127]."""
    return np.clip(np.rint(g.standard_normal((N, K)) * 36.0), -127, 127).astype(np.int8)


def q8_scales(g: np.random.Generator, n: int) -> np.ndarray:
    """fp16(|z| * 0.02 / 36): Q8_0 block scales that give the byte weights a spread of about 0.02."""
    return (np.abs(g.standard_normal(n)) * (0.02 / 36.0)).astype(np.float16)


def _bits_lsb_first(bits: np.ndarray) -> np.ndarray:
    """Pack 0/1 values along the last axis, 8 per byte, least-significant bit first."""
    return np.packbits(bits.astype(np.uint8), axis=-1, bitorder="little")


def lay_out_q1_0(w: np.ndarray, d: np.ndarray) -> np.ndarray:
    """ggml Q1_0 bytes for sign weights ``w`` [N][K] (+1 -> bit 1, -1 -> bit 0) and fp16 scales ``d``
    [N][K/128].  Returns uint8 [N][K/128][18]."""
    N, K = w.shape
    nb = K // QK1
    assert K % QK1 == 0 and d.shape == (N, nb)
    out = np.empty((N, nb, 18), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:18] = _bits_lsb_first((w > 0).reshape(N, nb, QK1))
    return out


def lay_out_q2_0(w: np.ndarray, d: np.ndarray) -> np.ndarray:
    """ggml Q2_0_g64 bytes for weights ``w`` [N][K] in {-1,0,1,2} (code = w + 1, lowest bits first)
    and fp16 scales ``d`` [N][K/64].  Returns uint8 [N][K/64][18]."""
    N, K = w.shape
    nb = K // QK2
    assert K % QK2 == 0 and d.shape == (N, nb)
    codes = (w.astype(np.int16) + 1).astype(np.uint8).reshape(N, nb, 16, 4)
    packed = codes[..., 0] | (codes[..., 1] << 2) | (codes[..., 2] << 4) | (codes[..., 3] << 6)
    out = np.empty((N, nb, 18), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:18] = packed
    return out


def lay_out_q8_0(w: np.ndarray, d: np.ndarray) -> np.ndarray:
    """ggml Q8_0 bytes for signed-byte weights ``w`` [N][K] and fp16 scales ``d`` [N][K/32]: per block the
    little-endian binary16 scale, then the 32 weights as two's-complement bytes.  Returns uint8 [N][K/32][34]."""
    N, K = w.shape
    nb = K // QK8
    assert K % QK8 == 0 and d.shape == (N, nb)
    out = np.empty((N, nb, 34), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:34] = w.reshape(N, nb, QK8).view(np.uint8)
    return out


def lay_out_b3(w: np.ndarray) -> np.ndarray:
    """Base-3 beats for ternary ``w`` [N][K] in {-1,0,+1}: columns padded with 0 to a whole number of 80-column
    beats, then byte j of a row = sum_t (w[5j+t] + 1) * 3^t.  Returns uint8 [N][ceil(K/80)][16]."""
    N, K = w.shape
    nbt = -(-K // QKB3)
    c = np.ones((N, nbt * QKB3), dtype=np.int64)  # code 1 = weight 0 for the padding columns
    c[:, :K] = w.astype(np.int64) + 1
    digits = c.reshape(N, nbt * 16, 5)
    v = digits[..., 0] + 3 * digits[..., 1] + 9 * digits[..., 2] + 27 * digits[..., 3] + 81 * digits[..., 4]
    return v.astype(np.uint8).reshape(N, nbt, 16)


def lay_out_planar(w: np.ndarray) -> np.ndarray:
    """Planar beats for ternary ``w`` [N][K] in {-1,0,+1}: per 64 columns 8 bytes of the "+1" plane
    then 8 bytes of the "-1" plane, column c at bit c (little-endian u64).  Returns uint8 [N][K/64][16]."""
    N, K = w.shape
    nb = K // QKP
    assert K % QKP == 0
    out = np.empty((N, nb, 16), dtype=np.uint8)
    out[:, :, 0:8] = _bits_lsb_first((w == 1).reshape(N, nb, QKP))
    out[:, :, 8:16] = _bits_lsb_first((w == -1).reshape(N, nb, QKP))
    return out


def activations(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """fp32 N(0,1) activation rows [M][K]."""
    return g.standard_normal((M, K)).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even, via torch) and return the raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


class Weights:
    """One synthetic weight tensor: the format bytes plus the values drawn to make them."""

    def __init__(self, fmt, N, K, raw, w, d=None, s_w=None):
        self.fmt, self.N, self.K = fmt, N, K
        self.raw = raw  # uint8, ggml blocks [N][K/QK][18 or 34] or planar beats [N][K/64][16]
        self.w = w  # int8 [N][K], the drawn weight values (before scaling)
        self.d = d  # fp16 [N][K/QK] block scales (ggml formats)
        self.s_w = s_w  # fp32 per-tensor scale (planar)

    @property
    def nbytes(self) -> int:
        return int(self.raw.size)


def make_weights(fmt: int, N: int, K: int, seed: int, p=TERNARY_P) -> Weights:
    g = rng(seed)
    if fmt == Q1_0:
        w = sign_weights(g, N, K)
        d = fp16_scales(g, N * (K // QK1)).reshape(N, K // QK1)
        return Weights(fmt, N, K, lay_out_q1_0(w, d), w, d=d)
    if fmt == Q2_0_G64:
        w = ternary_weights(g, N, K, p)
        d = fp16_scales(g, N * (K // QK2)).reshape(N, K // QK2)
        return Weights(fmt, N, K, lay_out_q2_0(w, d), w, d=d)
    if fmt == Q8_0:
        w = byte_weights(g, N, K)
        d = q8_scales(g, N * (K // QK8)).reshape(N, K // QK8)
        return Weights(fmt, N, K, lay_out_q8_0(w, d), w, d=d)
    if fmt == TERNARY_B3:
        p3 = np.asarray(p[:3], dtype=np.float64)
        w = ternary_weights(g, N, K, tuple(p3 / p3.sum()) + (0.0,))
        s_w = np.float32(abs(g.standard_normal()) * 0.02)
        return Weights(fmt, N, K, lay_out_b3(w), w, s_w=s_w)
    if fmt == TERNARY_PLANAR:
        p3 = np.asarray(p[:3], dtype=np.float64)
        w = ternary_weights(g, N, K, tuple(p3 / p3.sum()) + (0.0,))
        s_w = np.float32(abs(g.standard_normal()) * 0.02)
        return Weights(fmt, N, K, lay_out_planar(w), w, s_w=s_w)
    raise ValueError(f"unknown weight format {fmt}")


def head_weights(N: int, K: int, seed: int) -> np.ndarray:
    """Dense head: N(0, 0.02) rounded to bfloat16, raw uint16 bits [N][K]."""
    g = rng(seed)
    return bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))


def head_weights_i8(N: int, K: int, seed: int):
    """int8 head: signed bytes rint(36 * N(0,1)) clipped to [-127, 127] [N][K] and one fp32 scale per row,
    |N(0,1)| * 0.02 / 36 (so the weights spread like the bf16 head's N(0, 0.02))."""
    g = rng(seed)
    W = byte_weights(g, N, K)
    s = (np.abs(g.standard_normal(N)) * (0.02 / 36.0)).astype(np.float32)
    return W, s


# --- the measured workloads' shapes -------------------------------------------------------------

# Qwen3-8B-like projections (rows x K) of one transformer block, in file order.
QWEN3_8B_LAYER = (
    ("attn_q", 4096, 4096),
    ("attn_k", 1024, 4096),
    ("attn_v", 1024, 4096),
    ("attn_output", 4096, 4096),
    ("ffn_gate", 12288, 4096),
    ("ffn_up", 12288, 4096),
    ("ffn_down", 4096, 12288),
)
QWEN3_8B_LAYERS = 36
QWEN3_8B_OUTPUT = ("output", 151669, 4096)

# BitNet-b1.58-2B-like block with the attention projections as 2560x2560 (the workload as stated).
BITNET_2B_LAYER = (
    ("attn_q", 2560, 2560),
    ("attn_k", 2560, 2560),
    ("attn_v", 2560, 2560),
    ("attn_output", 2560, 2560),
    ("ffn_gate", 6912, 2560),
    ("ffn_up", 6912, 2560),
    ("ffn_down", 2560, 6912),
)
BITNET_2B_LAYERS = 30
# The same block with grouped-query attention (k/v at 640 rows): the body the pages' 2.5:1 head-to-body
# ratio implies.
BITNET_2B_GQA_LAYER = tuple((n, 640 if n in ("attn_k", "attn_v") else N, K) for n, N, K in BITNET_2B_LAYER)
BITNET_HEAD = (128256, 2560)

PREFILL_M = 512
PREFILL_SHAPES = ((4096, 4096), (12288, 4096))


def format_bytes(fmt: int, N: int, K: int) -> int:
    """Bytes of a packed weight tensor in its on-disk format (18 or 34 B per ggml block, 16 B per beat)."""
    if fmt == TERNARY_B3:
        return N * (-(-K // QKB3)) * 16
    return N * (K // BLOCK_WEIGHTS[fmt]) * BLOCK_BYTES[fmt]


# --- device-side drawing for the bandwidth workloads --------------------------------------------------
# The same recipes drawn with torch's seeded generator directly in device memory, for tensors too large
# to draw on the host in reasonable time (a whole 8B-shape token is 1-2 GB of packed weights).  Parity
# tests use the host generators above; the bench uses these.

def device_ggml_blocks(fmt: int, N: int, K: int, seed: int, device="cuda"):
    """ggml Q1_0 / Q2_0_g64 blocks [N][K/QK][18] or Q8_0 blocks [N][K/32][34] (uint8) drawn on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    qk = BLOCK_WEIGHTS[fmt]
    nb = K // qk
    if fmt == Q8_0:
        d = (torch.randn((N, nb), generator=g, device=device).abs() * (0.02 / 36.0)).to(torch.float16)
        out = torch.empty((N, nb, 34), dtype=torch.uint8, device=device)
        out[:, :, 0:2] = d.view(torch.uint8).view(N, nb, 2)
        w = (torch.randn((N, nb, 32), generator=g, device=device) * 36.0).round().clamp(-127, 127).to(torch.int8)
        out[:, :, 2:34] = w.view(torch.uint8)
        return out
    d = (torch.randn((N, nb), generator=g, device=device).abs() * 0.02).to(torch.float16)
    out = torch.empty((N, nb, 18), dtype=torch.uint8, device=device)
    out[:, :, 0:2] = d.view(torch.uint8).view(N, nb, 2)
    if fmt == Q1_0:
        out[:, :, 2:18] = torch.randint(0, 256, (N, nb, 16), generator=g, device=device, dtype=torch.uint8)
    else:
        u = torch.rand((N, nb, 16, 4), generator=g, device=device)
        lo, hi = TERNARY_P[0], TERNARY_P[0] + TERNARY_P[1]
        c = (u >= lo).to(torch.uint8) + (u >= hi).to(torch.uint8)  # code 0, 1, 2 = weight -1, 0, +1
        out[:, :, 2:18] = c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)
    return out


def device_planar_beats(N: int, K: int, seed: int, device="cuda"):
    """Planar beats [N][K/64][16] (uint8) with weights -1/0/+1 at 31/38/31 %, drawn on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nb = K // QKP
    u = torch.rand((N, nb, 2, 8, 8), generator=g, device=device)
    lo, hi = TERNARY_P[0], TERNARY_P[0] + TERNARY_P[1]
    pos = (u >= hi).to(torch.uint8)
    neg = (u < lo).to(torch.uint8)
    shifts = torch.arange(8, device=device, dtype=torch.uint8)
    out = torch.empty((N, nb, 16), dtype=torch.uint8, device=device)
    out[:, :, 0:8] = (pos[:, :, 0] << shifts).sum(dim=-1, dtype=torch.uint8)
    out[:, :, 8:16] = (neg[:, :, 0] << shifts).sum(dim=-1, dtype=torch.uint8)
    return out


def device_b3_beats(N: int, K: int, seed: int, device="cuda"):
    """Base-3 beats [N][ceil(K/80)][16] (uint8) with weights -1/0/+1 at 31/38/31 %, drawn on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nbt = -(-K // QKB3)
    u = torch.rand((N, nbt * QKB3), generator=g, device=device)
    lo, hi = TERNARY_P[0], TERNARY_P[0] + TERNARY_P[1]
    c = (u >= lo).to(torch.int32) + (u >= hi).to(torch.int32)  # code 0, 1, 2 = weight -1, 0, +1
    c[:, K:] = 1
    d = c.view(N, nbt * 16, 5)
    v = d[..., 0] + 3 * d[..., 1] + 9 * d[..., 2] + 27 * d[..., 3] + 81 * d[..., 4]
    return v.to(torch.uint8).view(N, nbt, 16)


def device_head_weights_i8(N: int, K: int, seed: int, device="cuda"):
    """int8 head weights [N][K] and fp32 row scales [N] with the recipe of head_weights_i8, on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    W = (torch.randn((N, K), generator=g, device=device) * 36.0).round().clamp(-127, 127).to(torch.int8)
    s = torch.randn(N, generator=g, device=device).abs() * (0.02 / 36.0)
    return W, s


def device_head_weights(N: int, K: int, seed: int, device="cuda"):
    """Head weights N(0, 0.02) in bfloat16, returned as int16 bits [N][K], drawn on the device."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn((N, K), generator=g, device=device) * 0.02).to(torch.bfloat16).view(torch.int16)
