#!/usr/bin/env python3
"""Benchmark: one batch-1 decode token of a Qwen3-8B-shape Q2_0_g64 (ternary) model on one MI355X.

A step is one pass of the decode hot path over one token: quantise the token's activations to q8_0
(the 108 K=4096 rows and 36 K=12288 rows feeding the 252 products, kept in one buffer, so one launch)
and run all 252 products -- 36 layers x {q, k, v, o, gate, up, down} with distinct weights per layer,
1,953,497,088 bytes of packed weights -- as one batched launch (two kernels, one per configuration).
Inputs are synthetic (seeded), with the shapes and value distributions of the workload, and resident in
HBM before timing starts.

Prints ONE JSON line: the effective weight GB/s of the step (weight bytes / step time), the roofline of
the dominant kernel (the batched decode launch) measured with HIP events on the stream it runs on, the
same token in dependency order (layer by layer, as one HIP graph), a streaming-read probe run in the same
process (the bound the decode kernels are reported against beside the HBM peak), the shader clock while
the step runs, and the CPU oracle timed on the host's cores (rows split over threads, never a reduction)
on a bounded sample of the same bytes.  ``--gpus`` above 1 exits: this library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8, published
METRIC = "effective weight GB/s & % HBM peak, 8B-shape batch-1 ternary matvec; prefill TOPS"
PROFILE_PMC = os.path.join(ROOT, "profiles", "matvec_batched_q2_8b_token.pmc.txt")
# the decode kernel and the batch tile planner: both decide the batched launch's traffic
KERNEL_SRCS = [os.path.join(ROOT, "bit_quantized_matvec_q1_amd", "csrc", f) for f in ("matvec.hip", "abi.cpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class DecodeToken:
    """All products of one decode token of a layered model, batched into one launch plan."""

    def __init__(self, fmt, layer_shapes, layers, seed, keep_blocks_layers=0, head=None):
        import torch

        import bit_quantized_matvec_q1_amd.lowbit as L
        import synth

        self.fmt, self.layers, self.L = fmt, layers, L
        planar = fmt in (synth.TERNARY_PLANAR, synth.TERNARY_B3)  # per-token activations, per-tensor scale
        # distinct activation vectors per layer: attention input (q, k, v), o input, ffn input (gate, up),
        # down input -- grouped by K so each group is quantised by one launch
        names = [n for n, _, _ in layer_shapes]
        feeds = {"attn_q": 0, "attn_k": 0, "attn_v": 0, "attn_output": 1, "ffn_gate": 2, "ffn_up": 2, "ffn_down": 3}
        feed_k = {}
        for n, N, K in layer_shapes:
            feed_k[feeds[n]] = K
        self.groups = {}  # K -> list of (layer, feed)
        for l in range(layers):
            for f in sorted(feed_k):
                self.groups.setdefault(feed_k[f], []).append((l, f))
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        # every activation row of the token in one fp32 buffer (and one int8 / one scale buffer), grouped by K
        self.total = sum(len(rows) * K for K, rows in self.groups.items())
        self.xbuf = torch.randn(self.total, generator=g, device="cuda")
        self.xqbuf = torch.empty(self.total, dtype=torch.int8, device="cuda")
        nrows = sum(len(rows) for rows in self.groups.values())
        self.xsbuf = torch.empty(nrows if planar else self.total // 32, dtype=torch.float32 if planar else torch.uint16,
                                 device="cuda")
        self.x, self.xq, self.xs, self.row_of = {}, {}, {}, {}
        off = roff = 0
        for K, rows in self.groups.items():
            M = len(rows)
            self.x[K] = self.xbuf[off:off + M * K].view(M, K)
            self.xq[K] = self.xqbuf[off:off + M * K].view(M, K)
            self.xs[K] = self.xsbuf[roff:roff + M] if planar else self.xsbuf[off // 32:(off + M * K) // 32].view(M, K // 32)
            off += M * K
            roff += M
            for i, key in enumerate(rows):
                self.row_of[key] = (K, i)
        self.products, descs = [], []
        self.weight_bytes = self.act_bytes = self.out_bytes = 0
        self.blocks = {}
        for l in range(layers):
            for j, (n, N, K) in enumerate(layer_shapes):
                s = seed + 1000 * (l + 1) + j
                if fmt == synth.TERNARY_PLANAR:
                    raw = synth.device_planar_beats(N, K, s)
                    packed = raw.reshape(-1)
                    w_scale = float(abs(torch.randn((), generator=g, device="cuda").item()) * 0.02)
                elif fmt == synth.TERNARY_B3:
                    raw = synth.device_b3_beats(N, K, s)
                    packed = torch.empty(L.lowbit_weight_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
                    L.lowbit_pack_weights(fmt, raw.reshape(-1), N, K, packed)
                    w_scale = float(abs(torch.randn((), generator=g, device="cuda").item()) * 0.02)
                else:
                    raw = synth.device_ggml_blocks(fmt, N, K, s)
                    packed = torch.empty(L.lowbit_weight_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
                    L.lowbit_pack_weights(fmt, raw.reshape(-1), N, K, packed)
                    w_scale = 1.0
                if l < keep_blocks_layers:
                    self.blocks[(l, j)] = raw
                Kx, r = self.row_of[(l, feeds[n])]
                y = torch.empty(N, dtype=torch.float32, device="cuda")
                xq = self.xq[Kx][r]
                xs = self.xs[Kx][r] if not planar else self.xs[Kx][r:r + 1]
                self.products.append(dict(layer=l, j=j, name=n, N=N, K=K, W=packed, y=y, xq=xq, xs=xs, w_scale=w_scale,
                                          feed=(Kx, r)))
                descs.append(L.desc(fmt, packed, N, K, xq, xs, y, w_tensor_scale=w_scale))
                self.weight_bytes += L.lowbit_weight_bytes(fmt, N, K)
                self.act_bytes += K + (4 if planar else K // 16)
                self.out_bytes += 4 * N
        self.batch = L.Batch(descs)
        self.afmt = L.ACT_I8_ROW if planar else L.ACT_Q8_0
        # the dense bf16 output head of the token (its input is the final hidden state, fp32)
        self.head, self.head_bytes = None, 0
        if head is not None:
            hn, hk = head
            self.head = dict(N=hn, K=hk, W=synth.device_head_weights(hn, hk, seed + 7),
                             x=torch.randn(hk, generator=g, device="cuda"),
                             y=torch.empty(hn, dtype=torch.float32, device="cuda"))
            self.head_bytes = 2 * hn * hk
            self.weight_bytes += self.head_bytes
        torch.cuda.synchronize()

    def quantize(self):
        if self.afmt == self.L.ACT_Q8_0:
            # q8_0 blocks do not depend on the row length: one launch quantises every row of the token
            self.L.lowbit_quantize_act(self.afmt, self.xbuf, 1, self.total, self.xqbuf, self.xsbuf)
        else:
            for K, x in self.x.items():  # per-token scales: one launch per row length
                self.L.lowbit_quantize_act(self.afmt, x, x.shape[0], K, self.xq[K], self.xs[K])

    def products_launch(self):
        self.batch.run()

    def head_launch(self):
        if self.head is not None:
            h = self.head
            self.L.dense_head_matvec(h["W"], h["N"], h["K"], h["x"], h["y"])

    def step(self):
        self.quantize()
        self.products_launch()
        self.head_launch()

    @property
    def algorithmic_bytes(self):
        """Bytes of the batched products launch (the head, if any, is a launch of its own)."""
        return self.weight_bytes - self.head_bytes + self.act_bytes + self.out_bytes


FEEDS = {"attn_q": 0, "attn_k": 0, "attn_v": 0, "attn_output": 1, "ffn_gate": 2, "ffn_up": 2, "ffn_down": 3}


class LayeredGraph:
    """A token in dependency order: per layer, the q/k/v products, then o, then gate/up, then down, captured
    once as a HIP graph and replayed.  Each phase is one batched launch after the quantisation of its own
    input row (288 launches for 36 layers), or, fused (ggml formats), one batched launch whose fp32 input
    the batch quantises itself (inside the launch; the long down-projection row by a quantise launch the
    batch makes ahead of it: 180 launches)."""

    def __init__(self, tok, fused=False):
        import torch

        L = tok.L
        self.tok, self.phases, self.fused = tok, [], fused
        for l in range(tok.layers):
            for f in range(4):
                prods = [p for p in tok.products if p["layer"] == l and FEEDS[p["name"]] == f]
                if not prods:
                    continue
                K, r = prods[0]["feed"]
                if fused:
                    descs = [L.desc(tok.fmt, p["W"], p["N"], p["K"], None, None, p["y"], x=tok.x[K][r]) for p in prods]
                else:
                    descs = [L.desc(tok.fmt, p["W"], p["N"], p["K"], p["xq"], p["xs"], p["y"],
                                    w_tensor_scale=p["w_scale"]) for p in prods]
                self.phases.append((K, r, L.Batch(descs)))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.eager()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.eager()
        torch.cuda.synchronize()

    def eager(self):
        t, L = self.tok, self.tok.L
        for K, r, b in self.phases:
            if not self.fused:
                L.lowbit_quantize_act(t.afmt, t.x[K][r:r + 1], 1, K, t.xq[K][r:r + 1], t.xs[K][r:r + 1])
            b.run()

    def launches(self):
        return sum(b.launches() for _, _, b in self.phases) + (0 if self.fused else len(self.phases))

    def close(self):
        for _, _, b in self.phases:
            b.close()


def graph_launch_floor(n, steps=50, warmup=10):
    """ms per replay of a HIP graph of n dependent launches that do (almost) nothing: a one-element fill each.
    It prices the graph's own launch chain, which any n-phase dependency-ordered token pays."""
    import torch

    t = torch.zeros(1, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            t.fill_(float(i))
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            t.fill_(float(i))
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) / steps)
    del g
    return best


def time_graph(lg, steps, warmup):
    """ms per replay of the layered token graph, by HIP events on the replay stream."""
    import torch

    for _ in range(warmup):
        lg.graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        lg.graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def warm_steps(tok, ms=100.0):
    """Warm-up steps worth about `ms` of GPU time (at 6 TB/s): a freshly generated token's first ~15 ms of
    steps run up to 15 % slower than the steady state, so a fixed small count is not enough."""
    return max(20, int(ms * 1e-3 / (tok.weight_bytes / 6e12)))


def time_token(tok, steps, warmup):
    """Time `steps` whole steps (quantise + batched products [+ head]) with nothing else in the stream, then
    `steps` batched launches alone, each bracketed by HIP events on the stream the kernels run on (torch's
    current stream).  The events sit in a pass of their own: an event recorded between two kernels of a
    step holds the stream for a few microseconds, which would be counted in the step time."""
    import torch

    for _ in range(warmup):
        tok.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        tok.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        tok.products_launch()
        b.record()
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    return wall / steps * 1e3, sum(launch_ms) / len(launch_ms)


def stored_traffic(kernel_name, algorithmic_bytes):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken on the current
    kernel and tile-planner sources (sha256 over matvec.hip then abi.cpp); otherwise None."""
    if not os.path.exists(PROFILE_PMC):
        return None
    text = open(PROFILE_PMC).read()
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    src_hash = h.hexdigest()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def host_info():
    """The host the oracle runs on: CPU model (/proc/cpuinfo), logical CPUs, the CPUs this process may use,
    and the worker threads the oracle legs use (the machine's CPU share per GPU is 16)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable, "threads": max(1, min(usable, 16))}


def oracle_rows(fn, n_rows, threads):
    """Run fn(r0, r1) -> array over contiguous row chunks on `threads` host threads (the oracle's C calls
    release the GIL) and concatenate: rows are split, never a reduction, so the result does not depend on
    the thread count."""
    import concurrent.futures as cf

    import numpy as np

    chunks = [(n_rows * t // threads, n_rows * (t + 1) // threads) for t in range(threads)]
    chunks = [(a, b) for a, b in chunks if b > a]
    if len(chunks) == 1:
        return fn(*chunks[0])
    with cf.ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        parts = list(ex.map(lambda c: fn(*c), chunks))
    return np.concatenate(parts)


def oracle_matvec_rows(fmt, raw, N, K, q, xs, s_w, threads):
    """The oracle's product of one weight tensor, rows split over threads -> y."""
    import numpy as np

    import oracle

    if fmt == 3:  # planar: per-token activations, ((float)acc * s_x) * s_w
        return oracle_rows(lambda a, b: oracle.matvec_planar(raw, N, K, q, xs[0], s_w, rows=np.arange(a, b))[1],
                           N, threads)
    return oracle_rows(lambda a, b: oracle.matvec_q(fmt, raw, N, K, q, xs, rows=np.arange(a, b))[0], N, threads)


def oracle_thread_identity(threads):
    """The 1024 x 1024 Q2_0_g64 product (the small parity workload) by the oracle on one thread and on
    `threads` threads: True when the outputs are bit-identical."""
    import numpy as np

    import oracle
    import synth

    Wt = synth.make_weights(synth.Q2_0_G64, 1024, 1024, seed=1001)
    q, dh = oracle.quantize_q8_0(synth.activations(synth.rng(1002), 1, 1024))
    y1 = oracle_matvec_rows(synth.Q2_0_G64, Wt.raw, 1024, 1024, q[0], dh[0], 1.0, 1)
    yt = oracle_matvec_rows(synth.Q2_0_G64, Wt.raw, 1024, 1024, q[0], dh[0], 1.0, threads)
    return bool(np.array_equal(y1.view(np.uint64), yt.view(np.uint64)))


def cpu_baseline(tok, threads, budget_s=12.0):
    """The oracle, as it stands, on the same bytes as the GPU step: layers in order (quantise the layer's
    activations, then all of its products, each product's rows split over `threads` host threads) until
    the time budget is spent or the token is done.  Returns (seconds, weight bytes, layers)."""
    import oracle

    planar = tok.fmt == 3
    t_total, wbytes, layers_done = 0.0, 0, 0
    xs_host = {K: x.cpu().numpy() for K, x in tok.x.items()}
    for l in range(tok.layers):
        if (l, 0) not in tok.blocks:
            break
        raws = [(p, tok.blocks[(l, j)].cpu().numpy().reshape(-1))
                for j, p in enumerate([p for p in tok.products if p["layer"] == l])]
        head = None
        if tok.head is not None and l == tok.layers - 1:  # the token's dense head follows its last layer
            import numpy as np

            h = tok.head
            head = (h["W"].cpu().numpy().view(np.uint16), h["N"], h["K"], h["x"].cpu().numpy())
        t0 = time.perf_counter()
        qcache = {}
        for p, raw in raws:
            K, r = p["feed"]
            if (K, r) not in qcache:
                x = xs_host[K][r:r + 1]
                qcache[(K, r)] = oracle.quantize_i8_row(x) if planar else oracle.quantize_q8_0(x)
            q, sc = qcache[(K, r)]
            oracle_matvec_rows(tok.fmt, raw, p["N"], p["K"], q[0], sc if planar else sc[0], p["w_scale"], threads)
            wbytes += raw.size
        if head is not None:
            W, hn, hk, xh = head
            oracle_rows(lambda a, b: oracle.head_matvec(W, hn, hk, xh, rows=range(a, b))[0], hn, threads)
            wbytes += W.nbytes
        t_total += time.perf_counter() - t0
        layers_done += 1
        if t_total >= budget_s:
            break
    return t_total, wbytes, layers_done


def cpu_prefill(fmt, N, K, M, threads, seed=1004):
    """The oracle's prefill product on a bounded sample: the first activation rows of the M-row workload,
    all N weight rows each, rows of W split over threads, until ~4 s are spent.  -> (TOPS, rows done)."""
    import numpy as np

    import oracle
    import synth

    Wt = synth.make_weights(fmt, N, K, seed)
    X = synth.activations(synth.rng(seed + 1), M, K)
    Q, DH = oracle.quantize_q8_0(X)
    t0, m = time.perf_counter(), 0
    while m < M and time.perf_counter() - t0 < 4.0:
        oracle_rows(lambda a, b: oracle.matvec_q(fmt, Wt.raw, N, K, Q[m], DH[m], rows=np.arange(a, b))[0], N,
                    threads)
        m += 1
    dt = time.perf_counter() - t0
    return 2.0 * m * N * K / dt / 1e12, m


def warm_up(fn, ms=100.0):
    """Call fn (at least 3 times) until about `ms` of wall time has passed, synchronising every 8 calls so
    the wall time is GPU time: short kernels on a GPU that was idle run slow for their first ~15 ms."""
    import torch

    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < 3 or (time.perf_counter() - t0) * 1e3 < ms:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def head_gbs(N, K, reps=100, seed=1006):
    """The dense bf16 head matvec alone on weights resident in HBM: (ms, GB/s of its bytes)."""
    import torch

    import bit_quantized_matvec_q1_amd.lowbit as L
    import synth

    W = synth.device_head_weights(N, K, seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    x = torch.randn(K, generator=g, device="cuda")
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    warm_up(lambda: L.dense_head_matvec(W, N, K, x, y))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.dense_head_matvec(W, N, K, x, y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return ms, (2 * N * K + 4 * K + 4 * N) / (ms * 1e-3) / 1e9


def head_i8_gbs(N, K, reps=100, seed=1008):
    """The int8 head with one fp32 scale per row: (ms per launch, GB/s of its N*K + 4N weight bytes)."""
    import torch

    import bit_quantized_matvec_q1_amd.lowbit as L
    import synth

    W, s = synth.device_head_weights_i8(N, K, seed)
    x = torch.randn(K, device="cuda")
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    warm_up(lambda: L.dense_head_matvec_i8(W, s, N, K, x, y))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        L.dense_head_matvec_i8(W, s, N, K, x, y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return ms, (N * K + 4 * N) / (ms * 1e-3) / 1e9


def popcount_gbs(reps=100, seed=1010):
    """The bit-serial popcount kernel over one BitNet-2B layer's seven planar products: (ms per layer, GB/s)."""
    import torch

    import bit_quantized_matvec_q1_amd.lowbit as L
    import synth

    prods = []
    for j, (_, N, K) in enumerate(synth.BITNET_2B_LAYER):
        W = synth.device_planar_beats(N, K, seed + j).reshape(-1)
        xq = torch.randint(-128, 128, (K,), dtype=torch.int8, device="cuda")
        xs = torch.ones(1, dtype=torch.float32, device="cuda")
        prods.append((W, N, K, xq, xs, torch.empty(N, dtype=torch.float32, device="cuda")))
    nbytes = sum(W.numel() for W, *_ in prods)

    def layer():
        for W, N, K, xq, xs, y in prods:
            L.lowbit_matvec_popcount(W, N, K, 1.0, xq, xs, y)

    warm_up(layer)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        layer()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return ms, nbytes / (ms * 1e-3) / 1e9


def prefill_tops(fmt, N, K, M, reps=100, seed=1004):
    """Time the prefill product (M activation rows x N weight rows x K) on inputs resident in HBM."""
    import torch

    import bit_quantized_matvec_q1_amd.lowbit as L
    import synth

    raw = synth.device_ggml_blocks(fmt, N, K, seed)
    W = torch.empty(L.lowbit_weight_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
    L.lowbit_pack_weights(fmt, raw.reshape(-1), N, K, W)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    X = torch.randn((M, K), generator=g, device="cuda")
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    Xs = torch.empty((M, K // 32), dtype=torch.uint16, device="cuda")
    L.lowbit_quantize_act(L.ACT_Q8_0, X, M, K, Xq, Xs)
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    warm_up(lambda: L.lowbit_gemm(fmt, W, N, K, 1.0, L.ACT_Q8_0, Xq, Xs, M, Y))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.lowbit_gemm(fmt, W, N, K, 1.0, L.ACT_Q8_0, Xq, Xs, M, Y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return ms, 2.0 * M * N * K / (ms * 1e-3) / 1e12


def single_launch(fmt, shapes, reps=30, seed=1011):
    """One lowbit_matvec launch per shape (one product, batch 1): the median of `reps` launches timed with
    HIP events, warm (the same weights launch after launch, resident in the 256 MB last-level cache when
    they fit) and cold (a 512 MB buffer is rewritten before each launch, evicting every cache level).
    Returns {shape: {...}}."""
    import statistics

    import torch

    import bit_quantized_matvec_q1_amd.lowbit as L
    import synth

    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for i, (N, K) in enumerate(shapes):
        raw = synth.device_ggml_blocks(fmt, N, K, seed + i)
        W = torch.empty(L.lowbit_weight_bytes(fmt, N, K), dtype=torch.uint8, device="cuda")
        L.lowbit_pack_weights(fmt, raw.reshape(-1), N, K, W)
        del raw
        g = torch.Generator(device="cuda")
        g.manual_seed(seed + 100 + i)
        x = torch.randn(K, generator=g, device="cuda")
        xq = torch.empty(K, dtype=torch.int8, device="cuda")
        xs = torch.empty(K // 32, dtype=torch.uint16, device="cuda")
        L.lowbit_quantize_act(L.ACT_Q8_0, x, 1, K, xq, xs)
        y = torch.empty(N, dtype=torch.float32, device="cuda")

        def launch():
            L.lowbit_matvec(fmt, W, N, K, 1.0, L.ACT_Q8_0, xq, xs, y)

        warm_up(launch)
        times = {}
        for mode in ("warm", "cold"):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            # hold the GPU (a bounded spin) while the host queues every launch, so that warm launches run back
            # to back instead of each waiting for the host's next call
            torch.cuda._sleep(20_000_000)
            for a, b in ev:
                if mode == "cold":
                    flush.fill_(1)
                a.record()
                launch()
                b.record()
            torch.cuda.synchronize()
            el = [a.elapsed_time(b) for a, b in ev]
            times[mode] = statistics.median(el)
            times[mode + "_min"] = min(el)
        nbytes = L.lowbit_weight_bytes(fmt, N, K)
        out[f"{N}x{K}"] = {"weight_bytes": nbytes, "warm_us": round(times["warm"] * 1e3, 2),
                           "warm_min_us": round(times["warm_min"] * 1e3, 2),
                           "cold_us": round(times["cold"] * 1e3, 2),
                           "cold_min_us": round(times["cold_min"] * 1e3, 2),
                           "cold_gbs": round(nbytes / (times["cold"] * 1e-3) / 1e9, 1)}
    del flush
    torch.cuda.empty_cache()
    return out


def read_probe_gbs(nbytes=1 << 31, reps=5):
    """A stream read of a buffer far larger than the 256 MB last-level cache: torch's fp32 sum, read GB/s."""
    import torch

    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    a.sum()
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a.sum()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a
    torch.cuda.empty_cache()
    return best


def device_clocks(props):
    """The current shader, memory and fabric clock levels of this GPU, read from sysfs (the DPM table line
    marked current), with no child process.  The card is matched on the PCI bus number torch reports; None
    when nothing matches or the files are not readable."""
    import glob

    bus = getattr(props, "pci_bus_id", None)
    for dev_dir in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev_dir, "uevent")) as f:
                slot = next((l.split("=", 1)[1].strip() for l in f if l.startswith("PCI_SLOT_NAME=")), "")
        except OSError:
            continue
        if bus is None or not slot or int(slot.split(":")[1], 16) != bus:
            continue
        out = {"pci": slot}
        for name in ("sclk", "mclk", "fclk"):
            try:
                with open(os.path.join(dev_dir, f"pp_dpm_{name}")) as f:
                    cur = [l.split(":", 1)[1].replace("*", "").strip() for l in f if l.rstrip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[name] = cur[0]
        return out
    return None


def copy_probe_gbs(nbytes=1 << 31, reps=5):
    """Device-to-device copy of a buffer far larger than the 256 MB last-level cache: read+write GB/s."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a, b
    torch.cuda.empty_cache()
    return best


def hip_read_probe_gbs(nbytes=4 << 30, reps=5):
    """The library's streaming-read probe (16-byte non-temporal loads, the decode kernels' weight access
    pattern) over a buffer 16x the 256 MB last-level cache: best of `reps` by HIP events, GB/s."""
    import torch

    import bit_quantized_matvec_q1_amd.lowbit as L

    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    warm_up(lambda: L.lowbit_read_probe(a, nbytes, sink), ms=50.0)
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.lowbit_read_probe(a, nbytes, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a, sink
    torch.cuda.empty_cache()
    return best


def _sysfs_card(props):
    """The sysfs device directory of this GPU (matched on the PCI bus number torch reports), or None."""
    import glob

    bus = getattr(props, "pci_bus_id", None)
    for dev_dir in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev_dir, "uevent")) as f:
                slot = next((l.split("=", 1)[1].strip() for l in f if l.startswith("PCI_SLOT_NAME=")), "")
        except OSError:
            continue
        if bus is not None and slot and int(slot.split(":")[1], 16) == bus:
            return dev_dir
    return None


def _read_sclk_mhz(dev_dir):
    """The shader clock now, in MHz: the hwmon frequency input if there is one, else the DPM level sysfs
    marks as current."""
    import glob

    for f in sorted(glob.glob(os.path.join(dev_dir, "hwmon", "hwmon*", "freq1_input"))):
        try:
            with open(f) as fh:
                return int(fh.read().strip()) / 1e6
        except (OSError, ValueError):
            pass
    try:
        with open(os.path.join(dev_dir, "pp_dpm_sclk")) as fh:
            for line in fh:
                if line.rstrip().endswith("*"):
                    v = line.split(":", 1)[1].replace("*", "").strip().lower().replace("mhz", "")
                    return float(v)
    except (OSError, ValueError):
        pass
    return None


def clocks_under_load(props, fn, n):
    """The shader clock while this leg's work runs: enqueue fn() n times (tens of milliseconds of GPU
    work), then sample the clock every ~2 ms until the stream drains.  A pass of its own, outside every
    timed region.  -> {"sclk_mhz_median", "sclk_mhz_max", "samples"} or None."""
    import statistics

    import torch

    dev_dir = _sysfs_card(props)
    if dev_dir is None:
        return None
    torch.cuda.synchronize()
    for _ in range(n):
        fn()
    stream = torch.cuda.current_stream()
    samples = []
    while not stream.query():
        v = _read_sclk_mhz(dev_dir)
        if v is not None:
            samples.append(v)
        time.sleep(0.002)
    torch.cuda.synchronize()
    if not samples:
        return None
    return {"sclk_mhz_median": statistics.median(samples), "sclk_mhz_max": max(samples), "samples": len(samples)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--secondary", default="layered,q1,planar,b3,q8,prefill,single",
                    help="comma list of extra workloads: layered, q1, planar, b3, q8, prefill, single, none")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Each product would shard by rows: N / G rows per GPU, the activation replicated, one all-gather "
              "of y.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.cuda.get_device_properties(0)
    log(f"device: {dev.name} ({getattr(dev, 'gcnArchName', '?')}), {dev.multi_processor_count} CUs")
    host = host_info()
    log(f"host: {host}")

    hprobe = hip_read_probe_gbs()
    log(f"streaming-read probe (16-byte non-temporal loads, 4 GiB, best of 5): {hprobe:.0f} GB/s")
    probe = copy_probe_gbs()
    log(f"copy probe: {probe:.0f} GB/s (read+write)")
    rprobe = read_probe_gbs()
    log(f"read probe: {rprobe:.0f} GB/s (torch fp32 sum)")
    clocks = device_clocks(dev)
    log(f"clocks (idle, between legs): {clocks}")

    tok = DecodeToken(synth.Q2_0_G64, synth.QWEN3_8B_LAYER, synth.QWEN3_8B_LAYERS, seed=1003,
                      keep_blocks_layers=0 if args.no_cpu_baseline else synth.QWEN3_8B_LAYERS)
    log(f"Q2_0_g64 token: {len(tok.products)} products, {tok.weight_bytes} weight bytes")
    warm = max(args.warmup, warm_steps(tok))
    ms_step, ms_launch = time_token(tok, args.steps, warm)
    value = tok.weight_bytes / (ms_step * 1e-3) / 1e9
    achieved = tok.algorithmic_bytes / (ms_launch * 1e-3) / 1e9
    traffic = stored_traffic("matvec_batched_kernel", tok.algorithmic_bytes)
    log(f"step {ms_step:.4f} ms, batched launch {ms_launch:.4f} ms -> {value:.0f} GB/s weights, "
        f"launch {achieved:.0f} GB/s algorithmic")
    clk = clocks_under_load(dev, tok.step, max(50, int(100.0 / ms_step)))
    log(f"shader clock while the step runs: {clk}")

    # the same token in dependency order (per layer q/k/v, o, gate/up, down), replayed as one HIP graph
    layered = {}
    for fused, key, what in ((True, "fused", "each phase one batched launch whose fp32 input the batch "
                                             "quantises to q8_0 (inside the launch; the 12288-column down "
                                             "input by a quantise launch of the batch's own ahead of it)"),
                             (False, "separate_quantise", "each phase a q8_0 quantise launch plus one batched "
                                                          "launch")):
        # both legs replay a HIP graph: left out unless asked for ("layered"), e.g. under counter collection
        if "layered" not in args.secondary.split(","):
            continue
        lg = LayeredGraph(tok, fused=fused)
        msg = time_graph(lg, args.steps, warm)
        floor = graph_launch_floor(lg.launches())
        layered[key] = {
            "workload": "the headline token in dependency order: per layer q/k/v, o, gate/up, down, " + what +
                        ", captured as one HIP graph",
            "launches": lg.launches(), "ms_per_token": round(msg, 5),
            # the same number of dependent launches of a one-element fill in one graph: the chain's own cost
            "launch_floor_ms": round(floor, 5),
            "tokens_per_s": round(1e3 / msg, 1),
            "gbs": round(tok.weight_bytes / (msg * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * tok.weight_bytes / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        }
        lg.close()
        log(f"dependency-ordered token ({key}): {msg:.4f} ms")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "Q2_0_g64 decode token, Qwen3-8B shapes: 36 layers x {q 4096x4096, k/v 1024x4096, "
                        "o 4096x4096, gate/up 12288x4096, down 4096x12288}, batch 1, q8_0 activations; a step "
                        "quantises the token's 144 activation rows and runs all 252 products as independent "
                        "work in one batched launch (layer order not enforced: the dependency-ordered figures "
                        "are under dependency_ordered_token)",
            "products": len(tok.products),
            "weight_bytes": tok.weight_bytes,
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "pct_of_read_probe": round(100.0 * value / hprobe, 2),
        "token_products_per_s_equiv": round(1e3 / ms_step, 1),
        "dependency_ordered_token": layered.get("fused"),
        "read_probe_hip_gbs": round(hprobe, 1),
        "copy_probe_gbs": round(probe, 1),
        "read_probe_torch_sum_gbs": round(rprobe, 1),
        "device": {"name": dev.name, "arch": getattr(dev, "gcnArchName", None), "cus": dev.multi_processor_count,
                   "clocks_idle": clocks, "clock_during_step": clk},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "matvec_batched_kernel<Q2_0_g64>",
            "algorithmic_bytes_per_launch": tok.algorithmic_bytes,
            "launch_ms": round(ms_launch, 5),
            "frac_of_read_probe": round(achieved / hprobe, 4),
        },
    }

    threads = host["threads"]
    if not args.no_cpu_baseline:
        same = oracle_thread_identity(threads)
        t_cpu, wb, layers = cpu_baseline(tok, threads)
        out["cpu_baseline"] = {
            "value": round(wb / t_cpu / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"first {layers} of 36 layers (all 7 products each, q8_0 quantise included), the same "
                      f"bytes as the GPU run: {wb} weight bytes in {t_cpu:.2f} s, rows split over {threads} "
                      f"host threads",
            "tokens_per_s": round((wb / tok.weight_bytes) / t_cpu, 3),
            "host": host,
            "bit_identical_to_one_thread": same,
        }
        log(f"cpu baseline: {out['cpu_baseline']}")
    secondary = {}
    if "layered" in args.secondary.split(","):
        for key, v in layered.items():
            secondary["q2_0_8b_token_layered_graph" + ("" if key == "fused" else "_" + key)] = v
    tok.batch.close()
    del tok
    torch.cuda.empty_cache()

    for name in [s for s in args.secondary.split(",") if s and s != "none"]:
        if name == "q1":
            t1 = DecodeToken(synth.Q1_0, synth.QWEN3_8B_LAYER, synth.QWEN3_8B_LAYERS, seed=1002,
                             keep_blocks_layers=0 if args.no_cpu_baseline else synth.QWEN3_8B_LAYERS)
            ms1, ml1 = time_token(t1, max(50, args.steps // 2), warm_steps(t1))
            secondary["q1_0_8b_token"] = {
                "weight_bytes": t1.weight_bytes, "ms_per_step": round(ms1, 5),
                "gbs": round(t1.weight_bytes / (ms1 * 1e-3) / 1e9, 1),
                "launch_gbs": round(t1.algorithmic_bytes / (ml1 * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * t1.weight_bytes / (ms1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "pct_of_read_probe": round(100 * t1.weight_bytes / (ms1 * 1e-3) / 1e9 / hprobe, 2),
                "token_products_per_s_equiv": round(1e3 / ms1, 1),
            }
            if not args.no_cpu_baseline:
                tc, wb, nl = cpu_baseline(t1, threads, budget_s=4.0)
                secondary["q1_0_8b_token"]["cpu_baseline"] = {
                    "value": round(wb / tc / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
                    "sample": f"first {nl} of 36 layers, {wb} weight bytes in {tc:.2f} s",
                    "tokens_per_s": round((wb / t1.weight_bytes) / tc, 3)}
            t1.batch.close()
            del t1
        elif name == "single":
            # one product per launch (no batching), warm and cold: the 1024x1024 parity case and the four
            # distinct Qwen3-8B shapes
            shapes = [(1024, 1024)] + sorted({(N, K) for _, N, K in synth.QWEN3_8B_LAYER})
            secondary["q2_0_single_launch"] = {
                "workload": "one Q2_0_g64 product per lowbit_matvec launch, batch 1: median of 30 launches, warm "
                            "(weights resident in cache when they fit) and cold (every cache evicted first)",
                **single_launch(synth.Q2_0_G64, shapes)}
        elif name == "planar":
            tp = DecodeToken(synth.TERNARY_PLANAR, synth.BITNET_2B_LAYER, synth.BITNET_2B_LAYERS, seed=1005,
                             head=synth.BITNET_HEAD,
                             keep_blocks_layers=0 if args.no_cpu_baseline else synth.BITNET_2B_LAYERS)
            msp, mlp = time_token(tp, max(50, args.steps // 2), warm_steps(tp))
            secondary["planar_2b_token"] = {
                "workload": "BitNet-b1.58-2B shapes, 30 layers x 7 planar products + the dense bf16 head "
                            "128256x2560; per-token int8 activations",
                "weight_bytes": tp.weight_bytes, "ms_per_step": round(msp, 5),
                "gbs": round(tp.weight_bytes / (msp * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * tp.weight_bytes / (msp * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "pct_of_read_probe": round(100 * tp.weight_bytes / (msp * 1e-3) / 1e9 / hprobe, 2),
                "tokens_per_s_equiv": round(1e3 / msp, 1),
                "products_launch_ms": round(mlp, 5),
                "products_launch_gbs": round(tp.algorithmic_bytes / (mlp * 1e-3) / 1e9, 1),
            }
            if not args.no_cpu_baseline:
                tc, wb, nl = cpu_baseline(tp, threads, budget_s=4.0)
                secondary["planar_2b_token"]["cpu_baseline"] = {
                    "value": round(wb / tc / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
                    "sample": f"first {nl} of 30 layers (the head after the last), {wb} weight bytes in "
                              f"{tc:.2f} s",
                    "tokens_per_s": round((wb / tp.weight_bytes) / tc, 3)}
            hms, hg = head_gbs(*synth.BITNET_HEAD)
            secondary["head_bf16_128256x2560"] = {"ms": round(hms, 4), "gbs": round(hg, 1),
                                                  "pct_hbm_peak": round(100 * hg / HBM_PEAK_GBS, 2)}
            ims, ig = head_i8_gbs(*synth.BITNET_HEAD)
            secondary["head_int8_128256x2560"] = {"ms": round(ims, 4), "gbs": round(ig, 1),
                                                  "pct_hbm_peak": round(100 * ig / HBM_PEAK_GBS, 2),
                                                  "speedup_vs_bf16_head": round(hms / ims, 3)}
            pms, pg = popcount_gbs()
            secondary["planar_popcount_2b_layer"] = {
                "workload": "the bit-serial popcount kernel (the third implementation of the planar product) over "
                            "one BitNet-2B layer's seven products, one launch each",
                "ms": round(pms, 4), "gbs": round(pg, 1)}
            tp.batch.close()
            del tp
            torch.cuda.empty_cache()
            # the same model with grouped-query attention (k/v 640 x 2560): the body behind the pages' 2.5:1
            tg = DecodeToken(synth.TERNARY_PLANAR, synth.BITNET_2B_GQA_LAYER, synth.BITNET_2B_LAYERS, seed=1012,
                             head=synth.BITNET_HEAD)
            msg, mlg = time_token(tg, max(50, args.steps // 2), warm_steps(tg))
            secondary["planar_2b_gqa_token"] = {
                "workload": "BitNet-b1.58-2B with grouped-query attention (k/v 640x2560), 30 layers x 7 planar "
                            "products + the dense bf16 head 128256x2560; per-token int8 activations",
                "weight_bytes": tg.weight_bytes, "ms_per_step": round(msg, 5),
                "gbs": round(tg.weight_bytes / (msg * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * tg.weight_bytes / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "tokens_per_s_equiv": round(1e3 / msg, 1),
                "products_launch_ms": round(mlg, 5),
                "products_launch_gbs": round(tg.algorithmic_bytes / (mlg * 1e-3) / 1e9, 1),
            }
            tg.batch.close()
            del tg
        elif name == "b3":
            tb = DecodeToken(synth.TERNARY_B3, synth.BITNET_2B_LAYER, synth.BITNET_2B_LAYERS, seed=1009,
                             head=synth.BITNET_HEAD)
            msb, mlb = time_token(tb, max(50, args.steps // 2), warm_steps(tb))
            secondary["base3_2b_token"] = {
                "workload": "the BitNet-b1.58-2B token with base-3 ternary beats (five trits per byte, 1.6 b/w) "
                            "in place of planar beats, 30 layers x 7 products + the dense bf16 head",
                "weight_bytes": tb.weight_bytes, "ms_per_step": round(msb, 5),
                "gbs": round(tb.weight_bytes / (msb * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * tb.weight_bytes / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "products_launch_ms": round(mlb, 5),
                "products_launch_gbs": round(tb.algorithmic_bytes / (mlb * 1e-3) / 1e9, 1),
            }
            tb.batch.close()
            del tb
        elif name == "q8":
            t8 = DecodeToken(synth.Q8_0, synth.QWEN3_8B_LAYER, synth.QWEN3_8B_LAYERS, seed=1007)
            ms8, ml8 = time_token(t8, max(20, args.steps // 5), warm_steps(t8))
            secondary["q8_0_8b_token"] = {
                "workload": "Q8_0 weights x q8_0 activations (vec_dot_q8_0_q8_0), Qwen3-8B shapes, 36 layers x 7 "
                            "products, batch 1",
                "weight_bytes": t8.weight_bytes, "ms_per_step": round(ms8, 5),
                "gbs": round(t8.weight_bytes / (ms8 * 1e-3) / 1e9, 1),
                "launch_gbs": round(t8.algorithmic_bytes / (ml8 * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * t8.weight_bytes / (ms8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            }
            t8.batch.close()
            del t8
        elif name == "prefill":
            pre = {}
            for fmt, fname in ((synth.Q2_0_G64, "q2_0_g64"), (synth.Q1_0, "q1_0"), (synth.Q8_0, "q8_0")):
                for N, K in synth.PREFILL_SHAPES:
                    ms, tops = prefill_tops(fmt, N, K, synth.PREFILL_M)
                    pre[f"{fname}_{synth.PREFILL_M}x{N}x{K}"] = {
                        "ms": round(ms, 4), "tops": round(tops, 1),
                        "frac_int8_mfma_peak": round(tops / MFMA_I8_PEAK_TOPS, 4)}
            if not args.no_cpu_baseline:
                N, K = synth.PREFILL_SHAPES[0]
                ctops, rows = cpu_prefill(synth.Q2_0_G64, N, K, synth.PREFILL_M, threads)
                pre["cpu_baseline"] = {
                    "value": round(ctops, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
                    "sample": f"Q2_0_g64 {N}x{K}: the first {rows} of the {synth.PREFILL_M} activation rows (one "
                              "oracle product of all N weight rows per activation row)"}
            secondary["prefill"] = pre
        torch.cuda.empty_cache()
    if secondary:
        out["secondary"] = secondary
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
