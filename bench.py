"""Benchmark of the AWQ W4A16 hot path on one MI355X.

Timed step: one decode pass (M = 1) through the 7 linear layers of a
Llama-2-7B block -- (K, N) = (4096, 4096) x 4, (4096, 11008) x 2, (11008, 4096)
-- with int4 group-128 weights, fp16 activations.  Each step is one replay of a
HIP graph holding the 7 GEMV launches; successive steps rotate through copies of
the weights totalling more than 1 GiB so that the 256 MB Infinity Cache cannot
serve them.  `value` is algorithmic bytes moved per second (packed codes, fp16
scales, 4-bit zeros, x and y).

Also reported in the same JSON line:
  roofline       the GEMV kernel's achieved algorithmic GB/s (per-launch HIP event
                 timing of the same launches) against the 8 TB/s HBM peak, and the
                 HBM traffic measured with rocprofv3 counters when a summary for the
                 current kernel source exists under profiles/;
  cpu_baseline   the CPU oracle's W4A16 product on the same layers, timed on the
                 host cores (bounded sample);
  legs           the same decode step with q/k/v and gate/up stored as one packed
                 matrix each (4 launches instead of 7; same weight bytes), the M = 256
                 GEMM on the (4096, 11008) layer (TFLOP/s against the
                 2.5 PFLOP/s dense fp16 peak), the batch sweep M = 1..1024 on that
                 layer, awq_quantize over the 7 layers of a 7B block with 65,536
                 calibration rows (seconds per layer), and the same block searched
                 with one shared s per input (q/k/v and gate/up jointly).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--no-search] [--no-sweep] [--no-decode-legs] [--profile-mode gemv|copy|gemm|ring]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV GB/s & % HBM peak (M=1); GEMM TFLOP/s (M=256); search s/layer"
HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
LAYERS_7B = [("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096), ("o_proj", 4096, 4096),
             ("gate_proj", 4096, 11008), ("up_proj", 4096, 11008), ("down_proj", 11008, 4096)]
GEMV_SOURCES = ["weight_only_quantization_gemm_amd/csrc/gemv.hip", "weight_only_quantization_gemm_amd/csrc/awq_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_llama2_7b_decode_m1_counters.txt")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def gemv_bytes(M: int, K: int, N: int, bits: int = 4) -> int:
    """Algorithmic bytes of one product: codes (bits per weight), fp16 scales and 4-bit
    zero points per 128-channel group, x and y once."""
    G = K // 128
    return N * K * bits // 8 + 2 * N * G + N * ((G + 1) // 2) + 2 * M * K + 2 * M * N


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(per_launch_alg_bytes: float):
    """HBM bytes per GEMV launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"^source_hash:\s*(\S+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not (m_hash and m_bytes) or m_hash.group(1) != source_hash(GEMV_SOURCES):
        return None
    return float(m_bytes.group(1))


class Layer:
    def __init__(self, name, K, N, torch, awq, copies, dev, bits=4):
        from gen import activations_fp16, normal_fp16
        self.name, self.K, self.N = name, K, N
        W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=2000 + K + N)).to(dev)
        p, s, z = awq.awq_pack(W, bits=bits)  # plain round-to-nearest; values do not change the speed
        del W
        self.copies = [(p, s, z)] + [(p.clone(), s.clone(), z.clone()) for _ in range(copies - 1)]
        self.x = torch.from_numpy(activations_fp16(1, K, seed=2100 + K)).to(dev)
        self.y = torch.empty((1, N), dtype=torch.float16, device=dev)
        self.bytes = gemv_bytes(1, K, N, bits)


def graph_of(torch, fn):
    """Captures fn() (a sequence of libawq launches on the current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(torch, graphs, steps, warmup):
    """Mean ms per replay over `steps` replays (cycling through `graphs`), HIP events
    on the replay stream bracketing the whole timed region."""
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def step_graphs(torch, step, copies, n):
    """HIP graphs whose replays, in order, run exactly n steps, cycling through the weight
    copies: each graph holds up to `copies` consecutive steps on distinct weights, as a
    model's decode graph holds its consecutive transformer blocks."""
    seq = []
    if n >= copies:
        seq += [graph_of(torch, lambda: [step(c) for c in range(copies)])] * (n // copies)
    if n % copies:
        seq.append(graph_of(torch, lambda r=n % copies: [step(c) for c in range(r)]))
    return seq


def time_steps(torch, step, copies, steps, warmup):
    """Mean ms per step over exactly `steps` steps replayed from multi-step graphs, HIP
    events on the replay stream bracketing the whole timed region."""
    warm, timed = step_graphs(torch, step, copies, warmup), step_graphs(torch, step, copies, steps)
    for g in warm:
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for g in timed:
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def run_decode(args, torch, awq, dev, per_layer=True):
    step_bytes = sum(gemv_bytes(1, K, N) for _, K, N in LAYERS_7B)
    copies = max(2, int(np.ceil((1 << 30) / step_bytes)) + 1)
    layers = [Layer(n, K, N, torch, awq, copies, dev) for n, K, N in LAYERS_7B]
    torch.cuda.synchronize()

    def step(c):
        for L in layers:
            p, s, z = L.copies[c]
            awq.awq_gemm(L.x, p, s, z, out=L.y)

    t0 = time.perf_counter()
    ms_per_step = time_steps(torch, step, copies, args.steps, args.warmup)
    wall = time.perf_counter() - t0
    launches = len(layers)
    kern_ms = ms_per_step / launches  # the timed region holds nothing but these launches
    bytes_per_launch = step_bytes / launches
    achieved = bytes_per_launch / (kern_ms * 1e-3) / 1e9

    # per layer: a graph of that layer alone over its own rotating copies, more than 1 GiB of
    # that layer's bytes (so the 256 MB Infinity Cache cannot serve them)
    detail = {}
    for L in (layers if per_layer else []):
        own = max(3, -(-(1 << 30) // L.bytes) + 1)
        extra = [tuple(t.clone() for t in L.copies[0]) for _ in range(max(0, own - copies))]
        pool = (L.copies + extra)[:own]

        def one(L=L, pool=pool):
            for p, s, z in pool:
                awq.awq_gemm(L.x, p, s, z, out=L.y)
        g = graph_of(torch, one)
        ms = time_replays(torch, [g], max(5, args.steps // len(pool)), 2) / len(pool)
        detail[L.name] = dict(K=L.K, N=L.N, bytes=L.bytes, us=round(ms * 1e3, 3), copies=len(pool),
                              GBs=round(L.bytes / (ms * 1e-3) / 1e9, 1))
        del g, pool, extra
        torch.cuda.empty_cache()
    return dict(step_bytes=step_bytes, copies=copies, ms_per_step=ms_per_step, wall_s=wall,
                kern_ms=kern_ms, achieved=achieved, bytes_per_launch=bytes_per_launch, per_layer=detail,
                layers=layers)


LAYERS_7B_FUSED = [("qkv_proj", 4096, 3 * 4096), ("o_proj", 4096, 4096), ("gate_up_proj", 4096, 2 * 11008),
                   ("down_proj", 11008, 4096)]


def run_decode_fused(args, torch, awq, dev):
    """The same 7 weight matrices with q/k/v and gate/up stored as one packed matrix each
    (rows concatenated), so a decode step is 4 launches; same weight bytes, x read once
    per fused launch."""
    step_bytes = sum(gemv_bytes(1, K, N) for _, K, N in LAYERS_7B_FUSED)
    copies = max(2, int(np.ceil((1 << 30) / step_bytes)) + 1)
    layers = [Layer(n, K, N, torch, awq, copies, dev) for n, K, N in LAYERS_7B_FUSED]
    torch.cuda.synchronize()

    def step(c):
        for L in layers:
            p, s, z = L.copies[c]
            awq.awq_gemm(L.x, p, s, z, out=L.y)

    ms = time_steps(torch, step, copies, args.steps, args.warmup)
    del layers
    return dict(us_per_step=round(ms * 1e3, 3), GBs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                hbm_frac=round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), bytes_per_step=step_bytes,
                launches=len(LAYERS_7B_FUSED), layers_KN=[[K, N] for _, K, N in LAYERS_7B_FUSED])


def run_decode_3bit(args, torch, awq, dev):
    """The 7-launch decode step of run_decode with the weights packed at 3 bits (the same
    layers and inputs; 3.156 instead of 4.156 bits per weight)."""
    step_bytes = sum(gemv_bytes(1, K, N, 3) for _, K, N in LAYERS_7B)
    copies = max(2, int(np.ceil((1 << 30) / step_bytes)) + 1)
    layers = [Layer(n, K, N, torch, awq, copies, dev, bits=3) for n, K, N in LAYERS_7B]
    torch.cuda.synchronize()

    def step(c):
        for L in layers:
            p, s, z = L.copies[c]
            awq.awq_gemm(L.x, p, s, z, out=L.y)

    ms = time_steps(torch, step, copies, args.steps, args.warmup)
    del layers
    return dict(us_per_step=round(ms * 1e3, 3), GBs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                hbm_frac=round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), bytes_per_step=step_bytes,
                launches=len(LAYERS_7B), bits=3)


def run_decode_scaled(args, torch, awq, dev):
    """The decode step of run_decode with x not yet divided by s: awq_gemm_scaled divides it
    exactly (one scaling launch into a workspace, then the product) on every layer.  Bytes per
    step add s (4 K per layer).  s is a^0.5 of a lognormal channel profile."""
    from gen import activations_fp16
    step_bytes = sum(gemv_bytes(1, K, N) + 4 * K for _, K, N in LAYERS_7B)
    copies = max(2, int(np.ceil((1 << 30) / step_bytes)) + 1)
    layers = [Layer(n, K, N, torch, awq, copies, dev) for n, K, N in LAYERS_7B]
    for L in layers:
        g = np.random.default_rng(2200 + L.K)
        sv = np.sqrt(np.exp(g.normal(0.0, 0.8, L.K))).astype(np.float32)
        L.s = torch.from_numpy(sv).to(dev)
        L.ws = torch.empty(awq.awq_gemm_scaled_workspace_bytes(1, L.N, L.K), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(c):
        for L in layers:
            p, s, z = L.copies[c]
            awq.awq_gemm_scaled(L.x, L.s, p, s, z, out=L.y, workspace=L.ws)

    ms = time_steps(torch, step, copies, args.steps, args.warmup)
    del layers
    return dict(us_per_step=round(ms * 1e3, 3), GBs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                hbm_frac=round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), bytes_per_step=step_bytes,
                launches=2 * len(LAYERS_7B))


def run_sweep(args, torch, awq, dev):
    """awq_gemm on the (K=4096, N=11008) layer at M = 1..1024, rotating weight copies."""
    from gen import activations_fp16, normal_fp16
    K, N = 4096, 11008
    W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=3001)).to(dev)
    base = awq.awq_pack(W)
    del W
    copies = 48  # 48 x 23.4 MB > 1 GiB
    packs = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    out = {}
    for M in (1, 2, 4, 8, 16, 64, 256, 1024):
        x = torch.from_numpy(activations_fp16(M, K, seed=3100 + M)).to(dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)

        def run(x=x, y=y):
            for c in range(copies):
                awq.awq_gemm(x, *packs[c], out=y)
        g = graph_of(torch, run)
        ms = time_replays(torch, [g], max(3, args.steps // copies), 1) / copies
        del g
        us = ms * 1e3
        nbytes = gemv_bytes(M, K, N)
        flops = 2.0 * M * N * K
        out[str(M)] = dict(us=round(us, 3), GBs=round(nbytes / us / 1e3, 1),
                           hbm_frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                           TFLOPs=round(flops / us / 1e6, 2), mfma_frac=round(flops / us / 1e6 / FP16_PEAK_TFLOPS, 4),
                           kernel=awq.awq_gemm_kernel(M, N, K))
    return out


def run_sweep3(args, torch, awq, dev):
    """The same (K=4096, N=11008) layer with 3-bit codes at M = 1..1024 (`kernel` names what the
    library's dispatch launched)."""
    from gen import activations_fp16, normal_fp16
    K, N = 4096, 11008
    W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=3001)).to(dev)
    base = awq.awq_pack(W, bits=3)
    del W
    copies = 64  # 64 x 17.6 MB > 1 GiB
    packs = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    out = {}
    for M in (1, 2, 4, 8, 16, 64, 256, 1024):
        x = torch.from_numpy(activations_fp16(M, K, seed=3100 + M)).to(dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)

        def run(x=x, y=y):
            for c in range(copies):
                awq.awq_gemm(x, *packs[c], out=y)
        g = graph_of(torch, run)
        us = time_replays(torch, [g], max(3, args.steps // copies), 1) / copies * 1e3
        del g
        nbytes = gemv_bytes(M, K, N, bits=3)
        out[str(M)] = dict(us=round(us, 3), GBs=round(nbytes / us / 1e3, 1),
                           hbm_frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                           TFLOPs=round(2.0 * M * N * K / us / 1e6, 2),
                           kernel=awq.awq_gemm_kernel(M, N, K, bits=3))
    del packs
    return out


LAYERS_70B = [("qkv", 8192, 10240), ("o", 8192, 8192), ("gate", 8192, 28672), ("up", 8192, 28672),
              ("down", 28672, 8192)]


def run_70b(args, torch, awq, dev):
    """awq_gemm on the Llama-2 70B linears (fused q/k/v with grouped K/V heads, o, gate, up,
    down) at M = 1, 8, 16, each layer on rotating weight copies (> 1 GiB per layer shape), and
    the five launches of one block's decode step summed."""
    from gen import activations_fp16, normal_fp16
    out = {}
    packs = {}
    for _, K, N in LAYERS_70B:
        if (K, N) in packs:
            continue
        W = torch.from_numpy(normal_fp16((N, K), 0.015, seed=7000 + K + N)).to(dev)
        base = awq.awq_pack(W)
        del W
        copies = max(3, -(-int(1.2e9) // gemv_bytes(1, K, N)))
        packs[(K, N)] = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    for M in (1, 8, 16):
        per, step_us, step_bytes = {}, 0.0, 0
        for name, K, N in LAYERS_70B:
            cp = packs[(K, N)]
            x = torch.from_numpy(activations_fp16(M, K, seed=7100 + M + K)).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)

            def run(x=x, y=y, cp=cp):
                for c in cp:
                    awq.awq_gemm(x, *c, out=y)
            g = graph_of(torch, run)
            us = time_replays(torch, [g], max(3, args.steps // len(cp)), 1) / len(cp) * 1e3
            del g
            nbytes = gemv_bytes(M, K, N)
            per[name] = dict(K=K, N=N, us=round(us, 3), GBs=round(nbytes / us / 1e3, 1),
                             hbm_frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), kernel=awq.awq_gemm_kernel(M, N, K))
            step_us += us
            step_bytes += nbytes
        out[str(M)] = dict(step_us=round(step_us, 3), GBs=round(step_bytes / step_us / 1e3, 1),
                           hbm_frac=round(step_bytes / step_us / 1e3 / HBM_PEAK_GBS, 4), layers=per)
    del packs
    return out


def run_ablation(torch, awq, dev, W, X, search_loss):
    """Keep 1% of the input channels in fp16 and round the rest (s = 1): output MSE on the
    calibration rows, relative to plain rounding, for channels chosen by activation, by weight
    magnitude and at random, next to the searched scales' loss."""
    N, K = W.shape
    n_keep = round(0.01 * K)
    rnd = torch.from_numpy(np.random.default_rng(5150).permutation(K)[:n_keep].astype(np.int32)).to(dev)
    awq.awq_keep_fp16_ablation(W, X, n_keep, rnd)  # warm-up
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    r = awq.awq_keep_fp16_ablation(W, X, n_keep, rnd)
    b.record()
    torch.cuda.synchronize()
    L = r["loss"].cpu().numpy()
    assert L[0] == search_loss[0], "plain rounding must give the search's alpha = 0 loss"
    return dict(n_keep=n_keep, ms=round(a.elapsed_time(b), 2),
                mse_ratio_vs_rtn={k: float(L[i] / L[0]) for i, k in enumerate(r["order"]) if i > 0},
                awq_search_ratio_vs_rtn=float(search_loss.min() / search_loss[0]))


def search_roofline_ms(M, K, N, n_alpha=20, statistics=True, accounting="method"):
    """Composite roofline of one awq_quantize call: the sum over its phases of
    max(bytes / 8 TB/s, flops / 2.5 PFLOP/s), in milliseconds.

    accounting="method" counts what the method needs: the statistics read X once
    (2 M K bytes) and, where the Gram form applies (M >= K), form G as a symmetric product
    (M K (K + 1) flops); each alpha reads W once (2 N K bytes) and evaluates the output MSE
    as a quadratic form (2 N K min(M, K) flops); the pack reads W and writes the packed
    layer.  accounting="split" counts the work of this implementation's loss instead: per
    alpha the error written and read back as an fp16 hi/lo pair (6 N K bytes) and the
    quadratic form as the three-term split (3 x 2 N K^2 flops)."""
    bw, pk = HBM_PEAK_GBS * 1e9, FP16_PEAK_TFLOPS * 1e12
    t = 0.0
    if statistics:  # without: taken from an earlier call on the same input
        t += 2.0 * M * K / bw
        if M >= K:
            t += M * K * (K + 1) / pk
    if accounting == "method":
        t += n_alpha * max(2.0 * N * K / bw, 2.0 * N * K * min(M, K) / pk)
    else:
        t += n_alpha * max(6.0 * N * K / bw, 6.0 * N * K * K / pk)
    t += (2.0 * N * K + gemv_bytes(1, K, N)) / bw
    return t * 1e3


def run_search(args, torch, awq, dev):
    """awq_quantize on the 7 linears of a 7B block, 65,536 calibration rows per input."""
    from gen import activations_fp16, normal_fp16, seed_for
    from gen.workloads import layer_inputs_7b_block
    M = 65536
    inputs = {}
    sizes = {"attn_in": 4096, "o_in": 4096, "mlp_in": 4096, "down_in": 11008}
    for i, (name, K) in enumerate(sizes.items()):
        inputs[name] = torch.from_numpy(activations_fp16(M, K, seed=seed_for(5, 10 + i), lognormal=True)).to(dev)
    Ks = {n: (K, N) for n, K, N in LAYERS_7B}
    res = {}
    total_ms = 0.0
    for li, (lname, src) in enumerate(layer_inputs_7b_block()):
        K, N = Ks[lname]
        W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=seed_for(5, 100 + li))).to(dev)
        ws = torch.empty((awq.awq_quantize_workspace_bytes(N, K, M, 128, 20),), dtype=torch.uint8, device=dev)
        awq.awq_quantize(W, inputs[src], None, workspace=ws)  # warm-up (first-touch of the workspace)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = awq.awq_quantize(W, inputs[src], None, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        total_ms += ms
        loss = r["loss"].cpu().numpy()
        best = int(r["best_alpha"].item())
        res[lname] = dict(K=K, N=N, ms=round(ms, 2), alpha_index=best, alpha=float(r["alphas"][best]),
                          mse_ratio_vs_rtn=float(loss[best] / loss[0]))
        if lname == "q_proj":
            res[lname]["keep_fp16_ablation"] = run_ablation(torch, awq, dev, W, inputs[src], loss)
        del W, ws, r
        torch.cuda.empty_cache()
    # The same 7 searches with the statistics of each input computed once: layers that read
    # one input run on one workspace, and the later ones reuse its statistics
    # (awq_quantize_shared; q/k/v share the attention input, gate/up the MLP input).
    shared_ms, by_src = 0.0, {}
    for li, (lname, src) in enumerate(layer_inputs_7b_block()):
        by_src.setdefault(src, []).append((li, lname))
    for src, group in by_src.items():
        K = Ks[group[0][1]][0]
        nmax = max(Ks[l][1] for _, l in group)
        ws = torch.empty((awq.awq_quantize_workspace_bytes(nmax, K, M, 128, 20),), dtype=torch.uint8, device=dev)
        Ws = {l: torch.from_numpy(normal_fp16((Ks[l][1], K), 0.02, seed=seed_for(5, 100 + li))).to(dev)
              for li, l in group}
        awq.awq_quantize(Ws[group[0][1]], inputs[src], None, workspace=ws)  # warm-up
        torch.cuda.synchronize()
        for j, (li, l) in enumerate(group):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            r = awq.awq_quantize(Ws[l], inputs[src], None, workspace=ws, reuse_statistics=j > 0)
            b.record()
            torch.cuda.synchronize()
            res[l]["ms_shared_statistics"] = round(a.elapsed_time(b), 2)
            shared_ms += a.elapsed_time(b)
            assert int(r["best_alpha"].item()) == res[l]["alpha_index"]
            del r
        del ws, Ws
        torch.cuda.empty_cache()
    roof = sum(search_roofline_ms(M, K, N) for _, K, N in LAYERS_7B)
    roof_split = sum(search_roofline_ms(M, K, N, accounting="split") for _, K, N in LAYERS_7B)
    roof_shared = sum(search_roofline_ms(M, Ks[l][0], Ks[l][1], statistics=j == 0)
                      for group in by_src.values() for j, (_, l) in enumerate(group))
    for lname, r_ in res.items():
        r_["roofline_ms"] = round(search_roofline_ms(M, r_["K"], r_["N"]), 3)
        r_["roofline_ms_split_accounting"] = round(search_roofline_ms(M, r_["K"], r_["N"], accounting="split"), 3)
    return dict(layers=res, s_per_layer=round(total_ms / 7 / 1e3, 4), total_s=round(total_ms / 1e3, 3),
                calib_rows=M, n_alpha=20, composite_roofline_s=round(roof / 1e3, 4),
                composite_roofline_frac=round(roof / total_ms, 4),
                composite_roofline_accounting="method: X read once, symmetric Gram, per alpha W read once "
                                              "and 2 N K min(M, K) loss flops at the fp16 peak, pack",
                composite_roofline_s_split_accounting=round(roof_split / 1e3, 4),
                composite_roofline_frac_split_accounting=round(roof_split / total_ms, 4),
                total_s_shared_statistics=round(shared_ms / 1e3, 3),
                s_per_layer_shared_statistics=round(shared_ms / 7 / 1e3, 4),
                composite_roofline_s_shared_statistics=round(roof_shared / 1e3, 4),
                composite_roofline_frac_shared_statistics=round(roof_shared / shared_ms, 4))


def run_search_joint(args, torch, awq, dev):
    """The same block with one shared s per input: q/k/v and gate/up searched jointly as
    row-concatenated weights (4 searches instead of 7; statistics and Gram matrix formed once
    per input).  The packed outputs are the fused matrices of the 4-launch decode step."""
    from gen import activations_fp16, normal_fp16, seed_for
    M = 65536
    specs = [("qkv_proj", "attn_in", 4096, 3 * 4096), ("o_proj", "o_in", 4096, 4096),
             ("gate_up_proj", "mlp_in", 4096, 2 * 11008), ("down_proj", "down_in", 11008, 4096)]
    res = {}
    total_ms = 0.0
    for li, (lname, src, K, N) in enumerate(specs):
        X = torch.from_numpy(activations_fp16(M, K, seed=seed_for(5, 10 + li), lognormal=True)).to(dev)
        W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=seed_for(5, 200 + li))).to(dev)
        ws = torch.empty((awq.awq_quantize_workspace_bytes(N, K, M, 128, 20),), dtype=torch.uint8, device=dev)
        awq.awq_quantize(W, X, None, workspace=ws)  # warm-up
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = awq.awq_quantize(W, X, None, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        total_ms += ms
        best = int(r["best_alpha"].item())
        res[lname] = dict(K=K, N=N, ms=round(ms, 2), alpha_index=best)
        del W, X, ws, r
        torch.cuda.empty_cache()
    return dict(layers=res, total_s=round(total_ms / 1e3, 3), s_per_linear=round(total_ms / 7 / 1e3, 4),
                calib_rows=M, n_alpha=20)


def host_cpu():
    """The host's CPU model and the threads the oracle's OpenMP loops use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", 0) or os.cpu_count() or 1)
    return model, threads, os.cpu_count()


def run_cpu_baseline(layers_spec, budget_s: float):
    """The C++ oracle's fp64 W4A16 product over the 7 decode layers, on the host cores."""
    import oracle
    from gen import activations_fp16, normal_fp16
    model, threads, ncpu = host_cpu()
    prepared = []
    for name, K, N in layers_spec:
        W = normal_fp16((N, K), 0.02, seed=2000 + K + N)
        q, z, sc = oracle.quantize_groups(oracle.scale_weights(W, np.ones(K, np.float32)))
        x = activations_fp16(1, K, seed=2100 + K)
        prepared.append((x, q, z, sc, gemv_bytes(1, K, N)))
    nbytes = 0
    t0 = time.perf_counter()
    steps = 0
    while True:
        for x, q, z, sc, b in prepared:
            oracle.gemm(x, q, z, sc)
            nbytes += b
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(nbytes / dt / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                cpu_model=model, host_cpus=ncpu,
                sample=f"{steps} full decode steps (7 layers of the 7B block, M=1) through the C++ oracle's gemm "
                       f"(fp64 dequantize + product, OpenMP over output rows), {dt:.1f} s")


def run_oracle_timings(args):
    """The C++ oracle timed on the host cores for the other timed workloads: the (4096, 11008)
    product at every M of the batch sweep, the Llama-2 70B linears at M = 1, 8, 16, and per
    7B-block search shape class the statistics, the Gram matrix (65,536 rows) and one alpha
    (quantize, error, loss); a full search is the statistics plus 20 alphas.  Seconds, with the
    thread count and CPU model."""
    import oracle
    from gen import activations_fp16, normal_fp16, seed_for
    model, threads, ncpu = host_cpu()
    out = dict(cpu_model=model, threads=threads, host_cpus=ncpu)
    K, N, M = 4096, 11008, 256
    W = normal_fp16((N, K), 0.02, seed=3001)
    q, z, sc = oracle.quantize_groups(oracle.scale_weights(W, np.ones(K, np.float32)))
    x = activations_fp16(M, K, seed=3100 + M)
    t0 = time.perf_counter()
    oracle.gemm(x, q, z, sc)
    dt = time.perf_counter() - t0
    out["gemm_m256_4096x11008"] = dict(s=round(dt, 3), GFLOPs=round(2.0 * M * N * K / dt / 1e9, 2))
    # the batch sweep on the same layer, and the Llama-2 70B linears at M = 1, 8, 16: one product each
    sweep = {}
    for Ms in (1, 2, 4, 8, 16, 64, 256, 1024):
        xs = activations_fp16(Ms, K, seed=3100 + Ms)
        t0 = time.perf_counter()
        oracle.gemm(xs, q, z, sc)
        dt = time.perf_counter() - t0
        sweep[str(Ms)] = dict(s=round(dt, 4), GFLOPs=round(2.0 * Ms * N * K / dt / 1e9, 2))
    out["sweep_4096x11008"] = sweep
    l70 = {}
    for name, K7, N7 in LAYERS_70B:
        W7 = normal_fp16((N7, K7), 0.015, seed=7000 + K7 + N7)
        q7, z7, sc7 = oracle.quantize_groups(oracle.scale_weights(W7, np.ones(K7, np.float32)))
        del W7
        for M7 in (1, 8, 16):
            x7 = activations_fp16(M7, K7, seed=7100 + M7 + K7)
            t0 = time.perf_counter()
            oracle.gemm(x7, q7, z7, sc7)
            dt = time.perf_counter() - t0
            l70[f"{name}_m{M7}"] = dict(K=K7, N=N7, M=M7, s=round(dt, 4),
                                         GBs=round(gemv_bytes(M7, K7, N7) / dt / 1e9, 3))
        del q7, z7, sc7
    out["llama2_70b_layers"] = l70
    log(f"oracle sweep and 70B layers: {sweep['1024']['s']} s at M = 1024")
    Mc = 65536
    for li, (name, K, N) in enumerate([("q_proj", 4096, 4096), ("gate_proj", 4096, 11008), ("down_proj", 11008, 4096)]):
        X = activations_fp16(Mc, K, seed=seed_for(5, 10 + li), lognormal=True)
        W = normal_fp16((N, K), 0.02, seed=seed_for(5, 100 + li))
        t0 = time.perf_counter()
        a = oracle.channel_mean_abs(X)
        t1 = time.perf_counter()
        G = oracle.gram(X)
        t2 = time.perf_counter()
        qa, za, sca, s = oracle.quantize_at(W, a, 0.35)
        E = oracle.weight_error(W, qa, za, sca, s)
        oracle.output_mse_gram(G, E, Mc)
        t3 = time.perf_counter()
        out[f"search_{name}_{K}x{N}"] = dict(stats_s=round(t1 - t0, 2), gram_s=round(t2 - t1, 2),
                                             one_alpha_s=round(t3 - t2, 2),
                                             full_search_s=round((t2 - t0) + 20 * (t3 - t2), 1))
        log(f"oracle {name}: {out[f'search_{name}_{K}x{N}']}")
        del X, W, G, E
    return out


def load_ceilings():
    """ctypes view of libawq_ceilings.so (include/awq_ceilings.h)."""
    import ctypes
    path = os.path.join(ROOT, "weight_only_quantization_gemm_amd", "libawq_ceilings.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    lib.awq_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p]
    lib.awq_ceiling_stream_read_store.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_int32, ctypes.c_void_p]
    lib.awq_ceiling_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p]
    return lib


CEILING_READ_SIZES = [("7B 4096x4096 layer", 8732672), ("7B 4096x11008 layer", 23455232),
                      ("70B 8192x10240 layer", 43618304), ("70B 8192x28672 layer", 122101760), ("1 GiB", 1 << 30)]


def run_ceilings(args, torch, dev):
    """What one device reaches with nothing but the product kernels' own access pattern:
    a streaming read of each decode layer's size with 16-byte non-temporal loads, one round
    trip per thread (rotating copies over more than 1 GiB, graph-timed; the faster of one and
    two loads per thread), the same read with each block ending in one dependent store (as a
    decode GEMV block ends with its y values), and dense fp16 matrix-core throughput (v_mfma_f32_32x32x16_f16, 8
    independent chains per wave, one or two waves per SIMD)."""
    lib = load_ceilings()
    out = {"stream_read": {}, "stream_read_store": {}, "mfma_f16_32x32x16": {}}
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    for label, nbytes in CEILING_READ_SIZES:
        nb = nbytes // 16 * 16
        copies = max(2, -(-int(1.1 * (1 << 30)) // nb) + 1)
        bufs = [torch.zeros(nb, dtype=torch.uint8, device=dev) for _ in range(copies)]
        words = -(-nb // 4096)  # blocks at one load per thread
        outs = torch.zeros(words, dtype=torch.int32, device=dev)
        for kind in ("stream_read", "stream_read_store"):
            best = None
            for L in (1, 2):
                def run(bufs=bufs, nb=nb, L=L, kind=kind):
                    st = torch.cuda.current_stream().cuda_stream
                    for b in bufs:
                        if kind == "stream_read":
                            assert lib.awq_ceiling_stream_read(b.data_ptr(), nb, sink.data_ptr(), L, st) == 0
                        else:
                            assert lib.awq_ceiling_stream_read_store(b.data_ptr(), nb, outs.data_ptr(), words, L, st) == 0
                g = graph_of(torch, run)
                ms = time_replays(torch, [g], max(3, 40 // copies), 1) / copies
                del g
                if best is None or ms < best[0]:
                    best = (ms, L)
            ms, L = best
            out[kind][label] = dict(bytes=nb, us=round(ms * 1e3, 3), GBs=round(nb / (ms * 1e-3) / 1e9, 1),
                                    hbm_frac=round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), copies=copies,
                                    loads_per_thread=L)
        del bufs, outs
        torch.cuda.empty_cache()
    for wps in (1, 2):
        blocks, iters = 256, 8192
        sink = torch.empty(blocks * 4 * wps, dtype=torch.float32, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        assert lib.awq_ceiling_mfma_f16(sink.data_ptr(), blocks, 16, wps, st) == 0  # warm-up
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        assert lib.awq_ceiling_mfma_f16(sink.data_ptr(), blocks, iters, wps, st) == 0
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        flops = blocks * 4 * wps * iters * 8 * 32768.0
        out["mfma_f16_32x32x16"][f"{wps}_wave_per_simd"] = dict(
            us=round(ms * 1e3, 1), TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1),
            frac=round(flops / (ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4))
    return out


TRACE_FILE = os.path.join(ROOT, "profiles", "gemv_llama2_7b_decode_m1_trace.md")


def trace_summary_for_roofline():
    """The headline kernel's figures from the committed rocprofv3 trace summary of the decode
    profile mode (the same step graphs as the timed region), when it was taken on the current
    GEMV source; else None."""
    if not os.path.exists(TRACE_FILE):
        return None
    text = open(TRACE_FILE).read()
    fields = dict(re.findall(r"^(source_hash|mean_launch_us|span_per_launch_us|dispatches):\s*(\S+)", text, re.M))
    if fields.get("source_hash") != source_hash(GEMV_SOURCES):
        return None
    return dict(file=os.path.relpath(TRACE_FILE, ROOT), mean_launch_us=float(fields["mean_launch_us"]),
                span_per_launch_us=float(fields["span_per_launch_us"]), dispatches=int(fields["dispatches"]))


def summarize_trace(csv_path, pattern, out_lines, last=0):
    """Dispatch statistics from a rocprofv3 kernel_trace.csv of the kernels whose name contains
    `pattern` (only the last `last` such dispatches when last > 0: the timed region of a
    profile-mode run): count, mean / median duration, per grid size, and the span from the
    first dispatch's start to the last one's end divided by their count (the trace's analogue
    of a timed region divided by its launches)."""
    import csv
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if pattern in r.get("Kernel_Name", ""):
                grid = r.get("Grid_Size_X", r.get("Grid_Size", "?"))
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), grid))
    if not rows:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r} in {csv_path}")
    rows.sort()
    if last > 0:
        rows = rows[-last:]
    d = np.array([e - b for b, e, _ in rows], dtype=np.float64) / 1e3
    span = (max(e for _, e, _ in rows) - rows[0][0]) / 1e3
    out_lines += [f"dispatches: {len(rows)}", f"mean_launch_us: {d.mean():.3f}",
                  f"median_launch_us: {np.median(d):.3f}", f"min_launch_us: {d.min():.3f}",
                  f"max_launch_us: {d.max():.3f}", f"span_per_launch_us: {span / len(rows):.3f}",
                  f"source_hash: {source_hash(GEMV_SOURCES)}"]
    grids = {}
    for (b, e, g) in rows:
        grids.setdefault(g, []).append((e - b) / 1e3)
    for g, v in sorted(grids.items(), key=lambda kv: int(kv[0]) if kv[0].isdigit() else 0):
        out_lines.append(f"grid {g}: dispatches {len(v)}, mean_us {np.mean(v):.3f}, median_us {np.median(v):.3f}")
    return out_lines


SEARCH_SOURCES = [f"weight_only_quantization_gemm_amd/csrc/{f}" for f in ("quant.hip", "loss.hip", "gram.hip", "stats.hip")]
SEARCH_PROFILE_LAYERS = [("q_proj", 4096, 4096), ("gate_proj", 4096, 11008), ("down_proj", 11008, 4096)]


def summarize_decode_counters(dec_fetch, dec_write, copy_fetch, copy_write, steps=40):
    """The body of profiles/gemv_llama2_7b_decode_m1_counters.txt from four rocprofv3 --pmc
    output directories: FETCH_SIZE and WRITE_SIZE over `--profile-mode decode` and over
    `--profile-mode copy` (a 256 MiB device copy, which calibrates each counter)."""
    import csv
    import glob

    def rows(d):
        out = []
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r.get("Grid_Size", "0")),
                            float(r["Counter_Value"])))
        return sorted(out)

    def calib(d, copied_kib):
        v = [c for _, name, _, c in rows(d) if "copyBuffer" in name or "copy" in name.lower()]
        return float(np.median(v)) / copied_kib, float(np.median(v))

    copied = (256 << 20) / 1024
    f_fac, f_raw = calib(copy_fetch, copied)
    w_fac, w_raw = calib(copy_write, copied)
    per_shape = {}
    for d, key in ((dec_fetch, "f"), (dec_write, "w")):
        g = [x for x in rows(d) if "gemv_kernel" in x[1]][-7 * steps:]
        for _, _, grid, c in g:
            per_shape.setdefault(grid, {"f": [], "w": []})[key].append(c)
    # grid threads = (N / 4) blocks of 4 rows x one wave per 2048 channels x 64 lanes
    shapes = {(N // 4) * (-(-K // 2048)) * 64: (K, N) for _, K, N in LAYERS_7B}
    out = [f"source_hash: {source_hash(GEMV_SOURCES)}   (sha256[:16] of csrc/gemv.hip + csrc/awq_common.h when "
           "the counters were taken)",
           "Commands (one counter per pass; `cd /tmp && export TMPDIR=/tmp` first; `$REPO` is the repository root):",
           f"  rocprofv3 --pmc FETCH_SIZE -d $REPO/gpurun_out/pmc_decode_FETCH_SIZE -o pmc --output-format csv -- "
           f"python $REPO/bench.py --profile-mode decode --steps {steps} --warmup 5",
           f"  rocprofv3 --pmc WRITE_SIZE -d $REPO/gpurun_out/pmc_decode_WRITE_SIZE -o pmc --output-format csv -- "
           f"python $REPO/bench.py --profile-mode decode --steps {steps} --warmup 5",
           "  (the same two with --profile-mode copy: a 256 MiB device-to-device copy, for calibration)",
           "  python bench.py --summarize-decode-counters gpurun_out/pmc_decode_FETCH_SIZE "
           "gpurun_out/pmc_decode_WRITE_SIZE gpurun_out/pmc_copy_FETCH_SIZE gpurun_out/pmc_copy_WRITE_SIZE",
           "",
           f"Calibration (256 MiB copy = {copied:.0f} KiB read and written): FETCH_SIZE reads {f_raw:.1f} KiB -> "
           f"factor {f_fac:.5f}; WRITE_SIZE reads {w_raw:.1f} KiB -> factor {w_fac:.5f}.  HBM bytes = FETCH_SIZE / "
           "fetch factor + WRITE_SIZE / write factor.",
           f"Figures: medians over the {7 * steps} GEMV dispatches of the {steps} timed steps.",
           "",
           "| shape (K, N) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes | algorithmic bytes | ratio |",
           "|---|---|---|---|---|---|---|"]
    hbm_step, alg_step = 0.0, 0.0
    for grid in sorted(per_shape):
        K, N = shapes.get(grid, (None, None))
        if K is None:
            continue
        fk = float(np.median(per_shape[grid]["f"]))
        wk = float(np.median(per_shape[grid]["w"]))
        hbm = fk * 1024 / f_fac + wk * 1024 / w_fac
        alg = gemv_bytes(1, K, N)
        n_in_step = sum(1 for _, k, nn in LAYERS_7B if (k, nn) == (K, N))
        hbm_step += n_in_step * hbm
        alg_step += n_in_step * alg
        out.append(f"| ({K}, {N}) | {len(per_shape[grid]['f'])} | {fk:.1f} | {wk:.1f} | {hbm:.0f} | {alg} | "
                   f"{hbm / alg:.4f} |")
    n = len(LAYERS_7B)
    out += ["", f"hbm_bytes_per_launch: {hbm_step / n:.1f}", f"alg_bytes_per_launch: {alg_step / n:.1f}",
            f"ratio: {hbm_step / alg_step:.4f}   (step-weighted over the {n} launches of a decode step)"]
    return out


def search_call_layers(names):
    """Layer (an entry of SEARCH_PROFILE_LAYERS) of each dispatch of `--profile-mode search`, from
    the kernel names in dispatch order: every awq_quantize call starts with its statistics pass,
    and call c searches layer c // 2."""
    starts = [i for i, n in enumerate(names) if "stats_accumulate" in n]
    layer_of = [None] * len(names)
    for c, i0 in enumerate(starts):
        i1 = starts[c + 1] if c + 1 < len(starts) else len(names)
        for i in range(i0, i1):
            layer_of[i] = SEARCH_PROFILE_LAYERS[min(c // 2, len(SEARCH_PROFILE_LAYERS) - 1)]
    return layer_of


def is_gram_kernel(name):
    """The Gram's own dispatches: gram_kernel and, where tiles are split, gram_fixup_kernel."""
    return "gram_kernel" in name or "gram_fixup_kernel" in name


def summarize_search_trace(csv_path, calib_rows=65536, n_alpha=20):
    """Markdown tables from the rocprofv3 kernel_trace.csv of `--profile-mode search` (each
    layer searched twice on one workspace, in SEARCH_PROFILE_LAYERS order): the top kernels,
    the loss per alpha of each layer's timed call, the HBM-bound phases against their
    algorithmic bytes, and the Gram per K."""
    import csv
    from collections import defaultdict
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                         int(r.get("Grid_Size_X", r.get("Grid_Size", "0")))))
    rows.sort()
    us = lambda r: (r[1] - r[0]) / 1e3
    out = []
    tot = defaultdict(float)
    cnt = defaultdict(int)
    for r in rows:
        tot[r[2]] += us(r)
        cnt[r[2]] += 1
    allt = sum(tot.values())
    out += ["## top kernels", "", "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for k in sorted(tot, key=lambda k: -tot[k])[:10]:
        out.append(f"| `{k[:90]}` | {cnt[k]} | {tot[k]:.1f} | {tot[k] / cnt[k]:.1f} | {100 * tot[k] / allt:.1f} |")
    # loss: 2 calls x n_alpha dispatches per layer, in layer order; the second call is the timed one
    loss = [r for r in rows if "loss_full" in r[2]]
    out += ["", "## loss per alpha (median over each layer's timed call)", "",
            "Rates by the flops the kernel performs (three terms over the block-upper triangle of 256-blocks)",
            "and by the method's own count (2 N K^2 per alpha: one full quadratic form).", "",
            "| layer (K, N) | us per alpha | TFLOP/s done (of 2.5 PF) | TFLOP/s by the method's count |",
            "|---|---|---|---|"]
    for li, (name, K, N) in enumerate(SEARCH_PROFILE_LAYERS):
        sel = loss[li * 2 * n_alpha + n_alpha:(li + 1) * 2 * n_alpha]
        if not sel:
            continue
        t = float(np.median([us(r) for r in sel]))
        jt = K // 256
        tri = sum(min(256 * (J + 1), K) for J in range(jt)) * 256  # channels x columns contracted per n row
        done = 3 * 2 * N * tri
        meth = 2 * N * K * K
        out.append(f"| {name} ({K}, {N}) | {t:.1f} | {done / t * 1e-6:.0f} ({done / t * 1e-6 / 25:.1f} %) | "
                   f"{meth / t * 1e-6:.0f} ({meth / t * 1e-6 / 25:.1f} %) |")
    layer_of = search_call_layers([r[2] for r in rows])
    out += ["", "## HBM-bound phases", "",
            "| kernel | layer (K, N) | dispatches | mean us | algorithmic bytes | GB/s (of 8 TB/s) |",
            "|---|---|---|---|---|---|"]
    groups = defaultdict(list)
    for i, r in enumerate(rows):
        for key in ("stats_accumulate", "transpose_kernel", "quant_error_kernel", "pack_kernel"):
            if key in r[2] and layer_of[i] is not None:
                groups[(key, layer_of[i])].append(us(r))
    what = {"stats_accumulate": "X read", "transpose_kernel": "X read, X^T written",
            "quant_error_kernel": "W read, E hi/lo written (per alpha)", "pack_kernel": "W read; codes, scales, zeros written"}
    for key in ("stats_accumulate", "transpose_kernel", "quant_error_kernel", "pack_kernel"):
        for lay in SEARCH_PROFILE_LAYERS:
            v = groups.get((key, lay))
            if not v:
                continue
            name, K, N = lay
            alg = {"stats_accumulate": 2 * calib_rows * K, "transpose_kernel": 4 * calib_rows * K,
                   "quant_error_kernel": 6 * N * K,
                   "pack_kernel": 2 * N * K + N * K // 2 + N * K // 64 + N * ((K // 128 + 1) // 2)}[key]
            m = float(np.mean(v))
            out.append(f"| {key} ({what[key]}) | {name} ({K}, {N}) | {len(v)} | {m:.1f} | {alg} | "
                       f"{alg / m * 1e-3:.0f} ({alg / m * 1e-3 / 80:.1f} %) |")
    # the Gram of each call: gram_kernel plus its fix-up pass, summed
    gram_calls = defaultdict(float)
    starts = [i for i, r in enumerate(rows) if "stats_accumulate" in r[2]]
    for i, r in enumerate(rows):
        if is_gram_kernel(r[2]) and layer_of[i] is not None:
            gram_calls[(layer_of[i][1], max(c for c, i0 in enumerate(starts) if i0 <= i))] += us(r)
    out += ["", "## Gram (X^T X over the calibration rows, symmetric half of 2 M K^2 flops)", "",
            "Per awq_quantize call: gram_kernel, plus gram_fixup_kernel where the last round's tiles are split.", "",
            "| K | calls | mean us | TFLOP/s (of 2.5 PF) |", "|---|---|---|---|"]
    for K in sorted({K for _, K, _ in SEARCH_PROFILE_LAYERS}):
        v = [t for (k, _), t in gram_calls.items() if k == K]
        if v:
            m = float(np.mean(v))
            fl = calib_rows * K * K
            out.append(f"| {K} | {len(v)} | {m:.0f} | {fl / m * 1e-6:.0f} ({fl / m * 1e-6 / 25:.1f} %) |")
    out += ["", f"kernel sources (sha256[:16] of {' + '.join(SEARCH_SOURCES)}): {source_hash(SEARCH_SOURCES)}"]
    return out


def summarize_search_counters(dirs, n_alpha=20):
    """Markdown table of rocprofv3 --pmc passes over `--profile-mode search` restricted to the
    loss and Gram kernels: per layer (loss, the timed call's dispatches) and per K (Gram), the
    median of each counter over the dispatches, and ratios derived from them."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))  # (kernel, label) -> counter -> values
    for d in dirs:
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            disp = defaultdict(dict)
            names = {}
            for r in csv.DictReader(open(f)):
                did = int(r["Dispatch_Id"])
                disp[did][r["Counter_Name"]] = float(r["Counter_Value"])
                disp[did]["duration_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                names[did] = (r["Kernel_Name"], int(r.get("Grid_Size", "0")))
            loss_ids = sorted(i for i in disp if "loss_full" in names[i][0])
            for j, did in enumerate(loss_ids):
                li, call = divmod(j, 2 * n_alpha)
                if call >= n_alpha and li < len(SEARCH_PROFILE_LAYERS):  # the timed call
                    name, K, N = SEARCH_PROFILE_LAYERS[li]
                    for c, v in disp[did].items():
                        vals[("loss_full_kernel", f"{name} ({K}, {N})")][c].append(v)
            order = sorted(disp)
            layer_of = dict(zip(order, search_call_layers([names[i][0] for i in order])))
            for did in order:
                if "gram_kernel" in names[did][0] and layer_of[did] is not None:
                    for c, v in disp[did].items():
                        vals[("gram_kernel", f"K = {layer_of[did][1]}")][c].append(v)
    keys = sorted(vals, key=lambda k: (k[0], k[1]))
    counters = sorted({c for k in keys for c in vals[k]})
    med = {k: {c: float(np.median(vals[k][c])) for c in vals[k]} for k in keys}
    out = ["| counter | " + " | ".join(f"{k[0]} {k[1]}" for k in keys) + " |",
           "|---|" + "---|" * len(keys)]
    for c in counters:
        out.append(f"| {c} | " + " | ".join(f"{med[k][c]:.4g}" if c in med[k] else "-" for k in keys) + " |")
    derived = [
        ("vector instructions per MFMA", lambda m: m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"]),
        ("LDS instructions per MFMA", lambda m: m["SQ_INSTS_LDS"] / m["SQ_INSTS_MFMA"]),
        ("MFMA-busy cycles / (1024 SIMDs x duration at 2.4 GHz)",
         lambda m: m["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * m["duration_us"] * 2400)),
        ("waiting / wave cycles (SQ_WAIT_ANY / SQ_WAVE_CYCLES)", lambda m: m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]),
        ("L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))", lambda m: m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"])),
        ("fabric reads per dispatch, MB (FETCH_SIZE KiB x 1024 x 2: copy-calibrated factor 0.5)",
         lambda m: m["FETCH_SIZE"] * 1024 * 2 / 1e6),
        ("LDS bank-conflict cycles / LDS-active cycles", lambda m: m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"]),
    ]
    out += ["", "| derived | " + " | ".join(f"{k[0]} {k[1]}" for k in keys) + " |", "|---|" + "---|" * len(keys)]
    for label, fn in derived:
        cells = []
        for k in keys:
            try:
                cells.append(f"{fn(med[k]):.3g}")
            except (KeyError, ZeroDivisionError):
                cells.append("-")
        out.append(f"| {label} | " + " | ".join(cells) + " |")
    return out


def summarize_sq_counters(dirs, pattern, units_per_wave=0):
    """Markdown table of rocprofv3 --pmc passes (one output directory each) over the dispatches
    whose kernel name contains `pattern`: the median of each counter, then per-wave, per-unit
    ratios when `units_per_wave` (the pipeline stages or groups a wave runs) is given."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(list)
    for d in dirs:
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if pattern in r["Kernel_Name"]:
                    vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    med = {c: float(np.median(v)) for c, v in vals.items()}
    out = [f"dispatches per counter: {max((len(v) for v in vals.values()), default=0)}", "",
           "| counter | value |", "|---|---|"]
    out += [f"| {c} | {med[c]:.6g} |" for c in sorted(med)]
    derived = [
        ("LDS bank-conflict cycles / LDS-active cycles", lambda m: m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"]),
        ("MFMA-busy cycles / (4 x busy CU cycles)", lambda m: m["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * m["SQ_BUSY_CU_CYCLES"])),
        ("MFMA co-executing with vector ALU / MFMA-busy cycles",
         lambda m: m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"]),
        ("waiting / wave cycles (SQ_WAIT_ANY / SQ_WAVE_CYCLES)", lambda m: m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]),
    ]
    if units_per_wave:
        per = lambda c: (lambda m: m[c] / (m["SQ_WAVES"] * units_per_wave))
        derived += [(f"{c} per wave and unit", per(c))
                    for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM")]
    out += ["", "| derived | value |", "|---|---|"]
    for label, fn in derived:
        try:
            out.append(f"| {label} | {fn(med):.4g} |")
        except (KeyError, ZeroDivisionError):
            out.append(f"| {label} | - |")
    return out


def profile_mode(args, torch, awq, dev):
    """Short runs for rocprofv3: the headline decode step graphs alone, a plain copy (counter
    scale), one GEMM or decode-ring layer, or the ceiling kernels."""
    if args.profile_mode == "copy":
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(profile_mode="copy", bytes_per_copy=n, launches=5)))
        return
    if args.profile_mode == "ceilings":
        print(json.dumps(dict(profile_mode="ceilings", **run_ceilings(args, torch, dev))))
        return
    if args.profile_mode == "search":
        # one awq_quantize per layer shape class of the 7B block (65,536 calibration rows,
        # 20 alphas), each after a warm-up call on the same workspace
        from gen import activations_fp16, normal_fp16, seed_for
        M, out = 65536, {}
        for li, (name, K, N) in enumerate(SEARCH_PROFILE_LAYERS):
            X = torch.from_numpy(activations_fp16(M, K, seed=seed_for(5, 10 + li), lognormal=True)).to(dev)
            W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=seed_for(5, 100 + li))).to(dev)
            ws = torch.empty((awq.awq_quantize_workspace_bytes(N, K, M, 128, 20),), dtype=torch.uint8, device=dev)
            awq.awq_quantize(W, X, None, workspace=ws)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            r = awq.awq_quantize(W, X, None, workspace=ws)
            b.record()
            torch.cuda.synchronize()
            out[name] = dict(K=K, N=N, ms=round(a.elapsed_time(b), 2), alpha_index=int(r["best_alpha"].item()))
            del X, W, ws, r
            torch.cuda.empty_cache()
        print(json.dumps(dict(profile_mode="search", calib_rows=M, layers=out)))
        return
    if args.profile_mode in ("gemm", "ring"):
        # one layer, 20 launches: the M = 256 GEMM on (4096, 11008), or the M = 16 decode
        # ring kernel on (8192, 28672)
        from gen import activations_fp16, normal_fp16
        K, N, M = (4096, 11008, 256) if args.profile_mode == "gemm" else (8192, 28672, 16)
        W = torch.from_numpy(normal_fp16((N, K), 0.02, seed=K + N)).to(dev)
        p, sc, z = awq.awq_pack(W)
        del W
        x = torch.from_numpy(activations_fp16(M, K, seed=K)).to(dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        for _ in range(20):
            awq.awq_gemm(x, p, sc, z, out=y)
        torch.cuda.synchronize()
        print(json.dumps(dict(profile_mode=args.profile_mode, K=K, N=N, M=M, launches=20)))
        return
    # decode: the headline's step graphs only (warm-up and timed replays, as in the default run)
    r = run_decode(args, torch, awq, dev, per_layer=False)
    print(json.dumps(dict(profile_mode="decode", alg_bytes_per_launch=r["bytes_per_launch"],
                          ms_per_step=r["ms_per_step"], avg_launch_us=round(r["kern_ms"] * 1e3, 3),
                          steps=args.steps, warmup=args.warmup, launches_per_step=len(LAYERS_7B))))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)  # ~70 ms of decode steps: clocks settle first
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-search", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-decode-legs", action="store_true",
                    help="skip the fused, scaled-input and 3-bit decode legs (the headline step only)")
    ap.add_argument("--profile-mode", choices=["decode", "copy", "gemm", "ring", "ceilings", "search"], default=None)
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--oracle-timings", action="store_true",
                    help="also time the C++ oracle on the M = 256 product and one search layer per shape class "
                         "(minutes of host CPU time)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV", default=None,
                    help="print the dispatch statistics of a rocprofv3 kernel_trace.csv (no GPU) and exit")
    ap.add_argument("--summarize-search-trace", metavar="KERNEL_TRACE_CSV", default=None,
                    help="print the markdown tables of profiles/search_llama2_7b_block_trace.md from the kernel "
                         "trace of --profile-mode search, and exit")
    ap.add_argument("--summarize-decode-counters", metavar="PMC_DIR", nargs=4, default=None,
                    help="print profiles/gemv_llama2_7b_decode_m1_counters.txt's body from the FETCH_SIZE and "
                         "WRITE_SIZE passes over --profile-mode decode and --profile-mode copy, and exit")
    ap.add_argument("--summarize-search-counters", metavar="PMC_DIR", nargs="+", default=None,
                    help="print the counter tables of profiles/search_loss_gram_sq_counters.md from rocprofv3 --pmc "
                         "output directories of --profile-mode search, and exit")
    ap.add_argument("--summarize-sq-counters", metavar="PMC_DIR", nargs="+", default=None,
                    help="print the median of each counter over the --kernel dispatches of rocprofv3 --pmc output "
                         "directories (e.g. of --profile-mode ring or gemm), and exit")
    ap.add_argument("--units-per-wave", type=int, default=0,
                    help="--summarize-sq-counters: pipeline stages (or groups) each wave runs, for per-unit ratios")
    ap.add_argument("--kernel", default="gemv_kernel",
                    help="kernel-name substring for --summarize-trace and --summarize-sq-counters")
    ap.add_argument("--last", type=int, default=0, help="--summarize-trace: only the last N matching dispatches")
    args = ap.parse_args()
    if args.summarize_trace:
        print("\n".join(summarize_trace(args.summarize_trace, args.kernel, [], args.last)))
        return
    if args.summarize_search_trace:
        print("\n".join(summarize_search_trace(args.summarize_search_trace)))
        return
    if args.summarize_decode_counters:
        print("\n".join(summarize_decode_counters(*args.summarize_decode_counters)))
        return
    if args.summarize_search_counters:
        print("\n".join(summarize_search_counters(args.summarize_search_counters)))
        return
    if args.summarize_sq_counters:
        print("\n".join(summarize_sq_counters(args.summarize_sq_counters, args.kernel, args.units_per_wave)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the W4A16 kernels are measured on one MI355X; "
              f"--gpus {args.gpus} is not supported: column-parallel layers would shard N and row-parallel ones K, "
              f"with one all-reduce of y, and that path is not built", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_quantization_gemm_amd as awq

    awq.load()  # fails loudly if libawq.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_mode:
        profile_mode(args, torch, awq, dev)
        return

    log("decode: building 7B-block layers and graphs")
    dec = run_decode(args, torch, awq, dev)
    value = dec["step_bytes"] / (dec["ms_per_step"] * 1e-3) / 1e9
    log(f"decode: {dec['ms_per_step'] * 1e3:.2f} us/step, {value:.1f} GB/s; per launch {dec['kern_ms'] * 1e3:.2f} us")
    dec.pop("layers")
    torch.cuda.empty_cache()

    legs = {}
    if not args.no_decode_legs:
        log("decode, q/k/v and gate/up fused by concatenated rows (4 launches)")
        legs["decode_fused_qkv_gateup"] = run_decode_fused(args, torch, awq, dev)
        torch.cuda.empty_cache()
        log("decode, x divided by s on the device (a scaling launch before each product)")
        legs["decode_llama2_7b_scaled_input"] = run_decode_scaled(args, torch, awq, dev)
        torch.cuda.empty_cache()
        log("decode, 3-bit weights (7 launches)")
        legs["decode_llama2_7b_3bit"] = run_decode_3bit(args, torch, awq, dev)
        torch.cuda.empty_cache()
    if not args.no_ceilings:
        log("ceilings: streaming read and fp16 matrix-core loop")
        legs["ceilings"] = run_ceilings(args, torch, dev)
        torch.cuda.empty_cache()
    if not args.no_sweep:
        log("sweep: (4096, 11008) at M = 1..1024")
        legs["batch_sweep_4096x11008"] = run_sweep(args, torch, awq, dev)
        m256 = legs["batch_sweep_4096x11008"]["256"]
        legs["gemm_m256_4096x11008"] = dict(TFLOPs=m256["TFLOPs"], mfma_frac=m256["mfma_frac"], us=m256["us"])
        torch.cuda.empty_cache()
        log("sweep: (4096, 11008) with 3-bit codes at M = 1..1024")
        legs["batch_sweep_4096x11008_3bit"] = run_sweep3(args, torch, awq, dev)
        torch.cuda.empty_cache()
        log("70B layers: q/k/v, o, gate, up, down at M = 1, 8, 16")
        legs["llama2_70b_layers"] = run_70b(args, torch, awq, dev)
        torch.cuda.empty_cache()
    if not args.no_search:
        log("search: awq_quantize over a 7B block, 65,536 calibration rows")
        legs["search_llama2_7b_block"] = run_search(args, torch, awq, dev)
        torch.cuda.empty_cache()
        log("search: joint (one s per input: q/k/v, o, gate/up, down)")
        legs["search_llama2_7b_block_joint"] = run_search_joint(args, torch, awq, dev)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        cpu = run_cpu_baseline(LAYERS_7B, args.cpu_budget)
    if args.oracle_timings:
        log("oracle timings: M = 256 product and one search layer per shape class on the host cores")
        legs["oracle_cpu_timings"] = run_oracle_timings(args)

    traffic = measured_traffic(dec["bytes_per_launch"])
    trace = trace_summary_for_roofline()
    # The roofline's launch duration is the committed trace's per-dispatch mean over the same
    # step graphs when it was taken on the current GEMV source (each launch timed alone by the
    # profiler); the timed region divided by its launches, where back-to-back launches overlap
    # one kernel's drain with the next one's start, is reported beside it.
    live_us = dec["kern_ms"] * 1e3
    launch_us = trace["mean_launch_us"] if trace else live_us
    achieved = dec["bytes_per_launch"] / (launch_us * 1e-6) / 1e9
    # The measured floor of a kernel that reads each layer's bytes and ends every block with a
    # dependent store (the ceiling leg, same run), averaged over the step's launches.
    floor = None
    srs = legs.get("ceilings", {}).get("stream_read_store", {})
    by_bytes = {v["bytes"]: v["us"] for v in srs.values()}
    if all(gemv_bytes(1, K, N) in by_bytes for _, K, N in LAYERS_7B):
        f_us = sum(by_bytes[gemv_bytes(1, K, N)] for _, K, N in LAYERS_7B) / len(LAYERS_7B)
        floor = {"kind": "streaming read of each layer's bytes, every block ending in one dependent store "
                         "(legs.ceilings.stream_read_store, this run)",
                 "us_per_launch": round(f_us, 3), "frac_of_floor": round(f_us / launch_us, 4),
                 "region_frac_of_floor": round(f_us / live_us, 4)}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama2_7b_decode_m1", "M": 1, "weights": "int4 g128 (fp16 scales, 4-bit zeros)",
                   "layers_KN": [[K, N] for _, K, N in LAYERS_7B], "bytes_per_step": dec["step_bytes"],
                   "rotating_weight_copies": dec["copies"], "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 0),
                     "kernel": "awq::gemv_kernel (M=1)", "avg_launch_us": round(launch_us, 3),
                     "alg_bytes_per_launch": round(dec["bytes_per_launch"], 1),
                     "timing": ("rocprofv3 per-dispatch mean over the timed step graphs (" + trace["file"] + ")")
                     if trace else "HIP events on the replay stream around the timed graph replays / launches",
                     "region_us_per_launch": round(live_us, 3),
                     "region_frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
                     "trace": trace, "floor": floor},
        "cpu_baseline": cpu,
        "per_layer": dec["per_layer"],
        "legs": legs,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
