"""lowbit_matvec_batched_static (the entry point for callers that cannot allocate): called through the C ABI,
its outputs must equal those of the same work list run as a batch (lowbit_batch_create /
lowbit_matvec_batched) bit for bit, on two calls in a row -- the second with a smaller list -- and a list
whose tables exceed the static array is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_matvec_q1_amd.lowbit as L
import oracle
import synth
from gpu_util import act_for, assert_close, dev, host, packed_weights, say

pytestmark = pytest.mark.gpu


def _call_static(descs):
    arr = (L.lb_matvec_desc * len(descs))(*descs)
    s = torch.cuda.current_stream().cuda_stream
    return L.lib.lowbit_matvec_batched_static(ctypes.cast(arr, ctypes.c_void_p), len(descs), s)


def _work_list(items, seed):
    prods, descs_a, descs_b = [], [], []
    for i, (fmt, N, K) in enumerate(items):
        Wt = synth.make_weights(fmt, N, K, seed + 10 * i)
        packed = packed_weights(Wt)
        q, xs, _ = act_for(fmt, K, seed + 10 * i + 1)
        qd, xsd = dev(q), dev(xs)
        w_scale = Wt.s_w if Wt.s_w is not None else 1.0
        ya = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        yb = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        prods.append((fmt, N, K, Wt, q, xs, ya, yb))
        descs_a.append(L.desc(fmt, packed, N, K, qd, xsd, ya, w_tensor_scale=w_scale))
        descs_b.append(L.desc(fmt, packed, N, K, qd, xsd, yb, w_tensor_scale=w_scale))
    return prods, descs_a, descs_b


def _check(prods, descs_a, descs_b):
    st = _call_static(descs_a)
    assert st == L.LB_OK, L.lib.lowbit_last_error().decode()
    b = L.Batch(descs_b)
    b.run()
    torch.cuda.synchronize()
    for fmt, N, K, Wt, q, xs, ya, yb in prods:
        a_, b_ = host(ya), host(yb)
        assert np.array_equal(a_, b_), f"static table != batch for format {fmt} {N}x{K}"
        if fmt in (synth.Q1_0, synth.Q2_0_G64, synth.Q8_0):
            y_ref, A = oracle.matvec_q(fmt, Wt.raw, N, K, q, xs)
            assert_close(a_, y_ref, A, K // 32, f"static {fmt} {N}x{K}")
        else:
            mv = oracle.matvec_planar if fmt == synth.TERNARY_PLANAR else oracle.matvec_b3
            _, y_ref = mv(Wt.raw, N, K, q, xs[0], Wt.s_w)
            assert np.array_equal(a_, y_ref)
    b.close()


def test_static_table_matches_batch_twice():
    say("case static table: first list (all formats, two configurations of Q2_0)")
    first = [(synth.Q2_0_G64, 1024, 4096), (synth.Q2_0_G64, 300, 12288), (synth.Q1_0, 512, 4096),
             (synth.TERNARY_PLANAR, 640, 2560), (synth.Q8_0, 200, 4096), (synth.TERNARY_B3, 130, 2560),
             (synth.Q1_0, 129, 12288)]
    _check(*_work_list(first, 7100))
    say("case static table: second, smaller list")
    second = [(synth.Q2_0_G64, 96, 1024), (synth.Q1_0, 33, 4096)]
    _check(*_work_list(second, 7200))


def test_static_table_refuses_oversized_list():
    # 20,000 one-row products need more descriptor bytes than the static table holds: refused on the host,
    # nothing enqueued (the addresses below are never dereferenced)
    say("case static table: oversized list refused")
    base = 1 << 24
    descs = [L.lb_matvec_desc(L.Q2_0_G64, L.ACT_Q8_0, 1, 64, base, 1.0, base, base, base, None)
             for _ in range(20000)]
    assert _call_static(descs) == L.LB_ESHAPE
    assert b"static table" in L.lib.lowbit_last_error()
