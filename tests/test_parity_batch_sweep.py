"""Seeded random work lists through the batched entry points: mixed formats, row counts from 1 to 400, K from
one block to 4096 (12288 for some fp32-input products, which the batch quantises with a launch of its own),
q8_0 / per-token int8 inputs and fp32 inputs quantised by the batch, and empty products.  Each product run as
part of a batch must equal its own single launch bit for bit (an fp32-input product: quantising first, then
the single launch), the allocation-free entry point must equal the batch bit for bit, and every product must
meet the oracle (within the tolerance; planar and base-3 bit for bit)."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_matvec_q1_amd.lowbit as L
import oracle
import synth
from gpu_util import act_for, assert_close, dev, host, packed_weights, say

pytestmark = pytest.mark.gpu

FMTS = [synth.Q1_0, synth.Q2_0_G64, synth.TERNARY_PLANAR, synth.Q8_0, synth.TERNARY_B3]
BLK = {synth.Q1_0: 128, synth.Q2_0_G64: 64, synth.TERNARY_PLANAR: 64, synth.Q8_0: 32, synth.TERNARY_B3: 64}


def _lists(n=8, seed=9900):
    g = synth.rng(seed)
    out = []
    for i in range(n):
        items = []
        for _ in range(int(g.integers(2, 13))):
            fmt = FMTS[int(g.integers(0, len(FMTS)))]
            f32 = fmt in (synth.Q1_0, synth.Q2_0_G64) and g.random() < 0.5
            K = 12288 if f32 and g.random() < 0.2 else BLK[fmt] * int(g.integers(1, 4096 // BLK[fmt] + 1))
            N = 0 if g.random() < 0.08 else int(g.integers(1, 401))
            items.append((fmt, N, K, f32))
        out.append((seed + 1 + i, items))
    return out


def _static(descs):
    arr = (L.lb_matvec_desc * len(descs))(*descs)
    return L.lib.lowbit_matvec_batched_static(ctypes.cast(arr, ctypes.c_void_p), len(descs),
                                              torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("seed,items", _lists(), ids=lambda v: str(v) if isinstance(v, int) else f"{len(v)}prods")
def test_batched_seeded_work_lists(seed, items):
    say(f"case batch sweep seed={seed} items={items}")
    prods, descs_b, descs_s = [], [], []
    for i, (fmt, N, K, f32) in enumerate(items):
        s = seed * 100 + i
        yb = torch.full((max(N, 1),), float("nan"), dtype=torch.float32, device="cuda")
        ys = torch.full((max(N, 1),), float("nan"), dtype=torch.float32, device="cuda")
        if N == 0:  # an empty product: nothing to do, nothing written
            Wd = torch.empty(16, dtype=torch.uint8, device="cuda")
            qd = torch.empty(max(K, 16), dtype=torch.int8, device="cuda")
            xsd = torch.empty(max(K // 32, 4), dtype=torch.float32 if fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3)
                              else torch.uint16, device="cuda")
            descs_b.append(L.desc(fmt, Wd, 0, K, qd, xsd, yb))
            descs_s.append(L.desc(fmt, Wd, 0, K, qd, xsd, ys))
            prods.append(None)
            continue
        Wt = synth.make_weights(fmt, N, K, s)
        packed = packed_weights(Wt)
        w_scale = Wt.s_w if Wt.s_w is not None else 1.0
        if f32:
            x = synth.activations(synth.rng(s + 1), 1, K)[0]
            xd = dev(x)
            descs_b.append(L.desc(fmt, packed, N, K, None, None, yb, x=xd))
            descs_s.append(L.desc(fmt, packed, N, K, None, None, ys, x=xd))
            q, xs = oracle.quantize_q8_0(x)
            q, xs = q[0], xs[0]
        else:
            q, xs, _ = act_for(fmt, K, s + 1)
            qd, xsd = dev(q), dev(xs)
            descs_b.append(L.desc(fmt, packed, N, K, qd, xsd, yb, w_tensor_scale=w_scale))
            descs_s.append(L.desc(fmt, packed, N, K, qd, xsd, ys, w_tensor_scale=w_scale))
            xd = None
        prods.append((fmt, N, K, Wt, packed, w_scale, q, xs, xd, yb, ys))
    b = L.Batch(descs_b)
    b.run()
    st = _static(descs_s)
    assert st == L.LB_OK, L.lib.lowbit_last_error().decode()
    torch.cuda.synchronize()
    for p in prods:
        if p is None:
            continue
        fmt, N, K, Wt, packed, w_scale, q, xs, xd, yb, ys = p
        what = f"format {fmt} {N}x{K}{' fp32 input' if xd is not None else ''}"
        # the single launch on the same (device-quantised, for fp32 inputs) activations
        planar = fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3)
        afmt = L.ACT_I8_ROW if planar else L.ACT_Q8_0
        if xd is not None:
            xq1 = torch.empty(K, dtype=torch.int8, device="cuda")
            xs1 = torch.empty(K // 32, dtype=torch.uint16, device="cuda")
            L.lowbit_quantize_act(L.ACT_Q8_0, xd, 1, K, xq1, xs1)
            assert np.array_equal(host(xq1), q) and np.array_equal(host(xs1), xs), "device quantisation != oracle"
        else:
            xq1, xs1 = dev(q), dev(xs)
        y1 = torch.empty(N, dtype=torch.float32, device="cuda")
        L.lowbit_matvec(fmt, packed, N, K, w_scale, afmt, xq1, xs1, y1)
        a, s_, one = host(yb)[:N], host(ys)[:N], host(y1)
        assert np.array_equal(a, one), f"{what}: batch != single launch"
        assert np.array_equal(s_, a), f"{what}: allocation-free entry point != batch"
        if planar:
            mv = oracle.matvec_planar if fmt == synth.TERNARY_PLANAR else oracle.matvec_b3
            _, y_ref = mv(Wt.raw, N, K, q, xs[0], Wt.s_w)
            assert np.array_equal(a, y_ref), f"{what}: differs from the oracle"
        else:
            y_ref, A = oracle.matvec_q(fmt, Wt.raw, N, K, q, xs)
            assert_close(a, y_ref, A, K // 32, what)
    b.close()
