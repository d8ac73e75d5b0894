"""Helpers for the GPU parity tests: move seeded host inputs to the device and run the HIP library
through its C ABI.  Expected values always come from the CPU oracle on the same host bytes."""
from __future__ import annotations

import numpy as np
import torch

import bit_quantized_matvec_q1_amd.lowbit as L
import oracle
import synth


def say(*a):
    print(*a, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed_weights(Wt: synth.Weights) -> torch.Tensor:
    """ggml/planar bytes -> device layout through lowbit_pack_weights."""
    blocks = dev(Wt.raw.reshape(-1))
    packed = torch.empty(L.lowbit_weight_bytes(Wt.fmt, Wt.N, Wt.K), dtype=torch.uint8, device="cuda")
    L.lowbit_pack_weights(Wt.fmt, blocks, Wt.N, Wt.K, packed)
    return packed


def act_for(fmt: int, K: int, seed: int, x: np.ndarray | None = None):
    """Oracle-quantised activation for one token: (q int8 [K], scale array, host x)."""
    if x is None:
        x = synth.activations(synth.rng(seed), 1, K)
    if fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3):
        q, s = oracle.quantize_i8_row(x)
        return q[0], s, x
    q, dh = oracle.quantize_q8_0(x)
    return q[0], dh[0], x


def gpu_matvec(fmt, packed, N, K, q, xs, w_scale=1.0):
    y = torch.empty(max(N, 1), dtype=torch.float32, device="cuda")
    afmt = L.ACT_I8_ROW if fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3) else L.ACT_Q8_0
    L.lowbit_matvec(fmt, packed, N, K, w_scale, afmt, dev(q), dev(xs), y)
    return host(y)[:N]


def gpu_sums(fmt, packed, N, K, Q, XS, M=1):
    row_sums = fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3)
    afmt = L.ACT_I8_ROW if row_sums else L.ACT_Q8_0
    shape = (M, N) if row_sums else (M, N, K // 32)
    sums = torch.empty(shape, dtype=torch.int32, device="cuda")
    L.lowbit_block_sums(fmt, packed, N, K, afmt, dev(Q), dev(XS), M, sums)
    return host(sums)


def assert_close(y, y_ref, A, n_terms, what=""):
    ok, worst, floored = oracle.tolerance_ok(y, y_ref, A, n_terms)
    rel = np.max(np.abs(y - y_ref) / np.maximum(np.abs(y_ref), 1e-300)) if len(y) else 0.0
    say(f"  {what}: worst err/allowance {worst:.3g}, rows on the floor {floored}, plain max rel {rel:.3g}")
    assert ok, f"{what}: fp32 output outside 1e-5 relative (worst ratio {worst})"
