"""GPU parity at full size, in the launch configuration bench.py times: one whole decode token (the
batched plan over every product of every layer, plus the token's activation quantisation), checked
against the CPU oracle on the same bytes -- every quantised activation byte, and a seeded sample of
output rows of every product."""
import numpy as np
import pytest
import torch

import oracle
import synth
from bench import DecodeToken, LayeredGraph
from gpu_util import say

pytestmark = pytest.mark.gpu


def _run_token(fmt, layer, layers, seed):
    tok = DecodeToken(fmt, layer, layers, seed=seed, keep_blocks_layers=layers)
    tok.quantize()
    tok.products_launch()
    torch.cuda.synchronize()
    return tok


def _check_token(tok, rows_per_product=64, seed=0):
    g = synth.rng(seed)
    planar = tok.fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3)
    # every activation row of the token, byte for byte
    refs = {}
    for K, x in tok.x.items():
        xh = x.cpu().numpy()
        q_ref, s_ref = oracle.quantize_i8_row(xh) if planar else oracle.quantize_q8_0(xh)
        assert np.array_equal(tok.xq[K].cpu().numpy(), q_ref), f"quantised activations (K={K}) differ"
        assert np.array_equal(tok.xs[K].cpu().numpy(), s_ref), f"activation scales (K={K}) differ"
        refs[K] = (q_ref, s_ref)
    worst = 0.0
    for j, p in enumerate(tok.products):
        N, K = p["N"], p["K"]
        rows = np.unique(np.concatenate([g.integers(0, N, rows_per_product), [0, N - 1]]))
        raw = tok.blocks[(p["layer"], p["j"])]
        raw_rows = raw[torch.from_numpy(rows).to(raw.device)].cpu().numpy()  # only the sampled rows
        Kx, r = p["feed"]
        q_ref, s_ref = refs[Kx]
        y = p["y"][torch.from_numpy(rows).to(p["y"].device)].cpu().numpy()
        n = len(rows)
        if planar:
            mv = oracle.matvec_planar if tok.fmt == synth.TERNARY_PLANAR else oracle.matvec_b3
            _, y_ref = mv(raw_rows, n, K, q_ref[r], s_ref[r], p["w_scale"])
            assert np.array_equal(y, y_ref), f"planar product {j} differs"
        else:
            y_ref, A = oracle.matvec_q(tok.fmt, raw_rows, n, K, q_ref[r], s_ref[r])
            ok, ratio, _ = oracle.tolerance_ok(y, y_ref, A, K // 32)
            worst = max(worst, ratio)
            assert ok, f"product {j} ({p['name']} layer {p['layer']}) outside tolerance (ratio {ratio})"
    say(f"  {len(tok.products)} products checked, worst err/allowance {worst:.3g}")
    assert len(tok.products) == 7 * tok.layers


@pytest.mark.parametrize("fmt", [synth.Q2_0_G64, synth.Q1_0, synth.Q8_0], ids=["Q2_0_g64", "Q1_0", "Q8_0"])
def test_qwen3_8b_token_full_size(fmt):
    say(f"case full token fmt={fmt}")
    tok = _run_token(fmt, synth.QWEN3_8B_LAYER, synth.QWEN3_8B_LAYERS, seed=7000 + fmt)
    _check_token(tok, seed=7100 + fmt)
    tok.batch.close()


@pytest.mark.parametrize("fmt", [synth.TERNARY_PLANAR, synth.TERNARY_B3], ids=["planar", "base3"])
def test_bitnet_token_full_size(fmt):
    say(f"case full 2B token fmt={fmt}")
    tok = _run_token(fmt, synth.BITNET_2B_LAYER, synth.BITNET_2B_LAYERS, seed=7300 + fmt)
    _check_token(tok, seed=7301)
    tok.batch.close()


def test_bitnet_gqa_token_full_size():
    """The grouped-query BitNet token bench.py times (k/v 640x2560 in every layer), planar, at full size."""
    say("case full 2B GQA token")
    tok = _run_token(synth.TERNARY_PLANAR, synth.BITNET_2B_GQA_LAYER, synth.BITNET_2B_LAYERS, seed=7400)
    _check_token(tok, seed=7401)
    tok.batch.close()


@pytest.mark.parametrize("fmt", [synth.Q2_0_G64, synth.TERNARY_PLANAR], ids=["Q2_0_g64", "planar"])
def test_layered_graph_replays_match_eager_and_oracle(fmt):
    """The dependency-ordered token captured as one HIP graph: every replay (with eager work and a clobber of
    every output between replays) gives the eager outputs bit for bit, and those match the oracle."""
    layer = synth.QWEN3_8B_LAYER if fmt != synth.TERNARY_PLANAR else synth.BITNET_2B_LAYER
    say(f"case layered graph fmt={fmt}")
    tok = DecodeToken(fmt, layer, 3, seed=7400 + fmt, keep_blocks_layers=3)
    lg = LayeredGraph(tok)
    lg.eager()
    torch.cuda.synchronize()
    ref = [p["y"].clone() for p in tok.products]
    _check_token(tok, seed=7401)
    for rep in range(3):
        for p in tok.products:
            p["y"].fill_(float("nan"))
        tok.xqbuf.zero_()
        torch.cuda.synchronize()
        lg.graph.replay()
        torch.cuda.synchronize()
        for p, y0 in zip(tok.products, ref):
            assert torch.equal(p["y"], y0), f"replay {rep}: {p['name']} layer {p['layer']} differs from eager"
        tok.step()  # eager work between replays
        torch.cuda.synchronize()
    lg.close()
    tok.batch.close()


def test_layered_graph_fused_quantisation_matches_separate():
    """The dependency-ordered token with every phase quantising its own fp32 input inside its batched launch
    (LB_ACT_F32_Q8_0: one launch per phase, two for the long-row down projection, whose row the batch
    quantises ahead of it): every replay gives the outputs of the separate-quantise graph bit for bit, with
    the int8 activation buffers clobbered (the fused path does not read them)."""
    fmt = synth.Q2_0_G64
    say("case layered graph fused quantisation")
    tok = DecodeToken(fmt, synth.QWEN3_8B_LAYER, 3, seed=7500, keep_blocks_layers=0)
    sep = LayeredGraph(tok)
    sep.eager()
    torch.cuda.synchronize()
    ref = [p["y"].clone() for p in tok.products]
    fused = LayeredGraph(tok, fused=True)
    # one launch per phase; the down projection's 12288-column input gets a quantise launch of its own
    long_rows = sum(1 for K, _, _ in fused.phases if K > 8192)
    assert sep.launches() == 2 * len(sep.phases)
    assert fused.launches() == len(fused.phases) + long_rows and long_rows == tok.layers
    for rep in range(3):
        for p in tok.products:
            p["y"].fill_(float("nan"))
        tok.xqbuf.zero_()
        tok.xsbuf.zero_()
        torch.cuda.synchronize()
        fused.graph.replay()
        torch.cuda.synchronize()
        for p, y0 in zip(tok.products, ref):
            assert torch.equal(p["y"], y0), f"replay {rep}: {p['name']} layer {p['layer']} differs"
        tok.step()  # eager work between replays
        torch.cuda.synchronize()
    fused.close()
    sep.close()
    tok.batch.close()
