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


def run_decode(args, torch, awq, dev):
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

    # per layer: a graph of `copies` launches of that layer alone (each weight copy once)
    detail = {}
    for L in layers:
        def one(L=L):
            for c in range(copies):
                p, s, z = L.copies[c]
                awq.awq_gemm(L.x, p, s, z, out=L.y)
        g = graph_of(torch, one)
        ms = time_replays(torch, [g], max(5, args.steps // copies), 2) / copies
        detail[L.name] = dict(K=L.K, N=L.N, bytes=L.bytes, us=round(ms * 1e3, 3),
                              GBs=round(L.bytes / (ms * 1e-3) / 1e9, 1))
        del g
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
    (as x * inv_s, inv_s = 1/s from awq_inverse_scale) inside the GEMV's x load on the
    4096 x 4096 layers and with a separate scaling launch on the larger ones.  Bytes per
    step add inv_s (4 K per layer).  s is a^0.5 of a lognormal channel profile."""
    from gen import activations_fp16
    step_bytes = sum(gemv_bytes(1, K, N) + 4 * K for _, K, N in LAYERS_7B)
    copies = max(2, int(np.ceil((1 << 30) / step_bytes)) + 1)
    layers = [Layer(n, K, N, torch, awq, copies, dev) for n, K, N in LAYERS_7B]
    for L in layers:
        g = np.random.default_rng(2200 + L.K)
        sv = np.sqrt(np.exp(g.normal(0.0, 0.8, L.K))).astype(np.float32)
        L.inv = awq.awq_inverse_scale(torch.from_numpy(sv).to(dev))
        L.ws = torch.empty(max(awq.awq_gemm_scaled_workspace_bytes(1, L.N, L.K), 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(c):
        for L in layers:
            p, s, z = L.copies[c]
            awq.awq_gemm_scaled(L.x, L.inv, p, s, z, out=L.y, workspace=L.ws)

    ms = time_steps(torch, step, copies, args.steps, args.warmup)
    del layers
    fused = [n for n, K, N in LAYERS_7B if awq.awq_gemm_scaled_workspace_bytes(1, N, K) == 0]
    return dict(us_per_step=round(ms * 1e3, 3), GBs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
                hbm_frac=round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), bytes_per_step=step_bytes,
                launches=len(LAYERS_7B) + len(LAYERS_7B) - len(fused), fused_layers=fused)


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
                           kernel="gemv_dot2" if M <= 2 else ("ring_mfma" if M <= 16 else "mfma_gemm"))
    return out


def run_sweep3(args, torch, awq, dev):
    """The same (K=4096, N=11008) layer with 3-bit codes at M = 1..1024 (decode batch sizes, and
    M = 64 on the matrix-core ring kernel with four x tiles per stage) and prefill sizes 256 and 1024
    on the pipelined matrix-core GEMM."""
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
                           kernel="gemv3_dot2" if M <= 2 else "ring_mfma" if M <= 64 else "gemm_pipe_mfma")
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
                             hbm_frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4))
            step_us += us
            step_bytes += nbytes
        out[str(M)] = dict(step_us=round(step_us, 3), GBs=round(step_bytes / step_us / 1e3, 1),
                           hbm_frac=round(step_bytes / step_us / 1e3 / HBM_PEAK_GBS, 4),
                           kernel="gemv_dot2" if M <= 2 else "ring_mfma", layers=per)
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


def search_roofline_ms(M, K, N, n_alpha=20, statistics=True):
    """Composite roofline of one awq_quantize call, sum over its phases of
    max(bytes / 8 TB/s, flops / 2.5 PFLOP/s), algorithmic amounts: statistics read X
    once (2 M K bytes); the Gram is a symmetric product (M K (K + 1) flops); each alpha
    reads W and writes its error as an fp16 hi/lo pair (6 N K bytes) and forms the
    quadratic form as the three-term fp16 split (3 x 2 N K^2 flops); the pack reads W
    and writes the packed layer."""
    bw, pk = HBM_PEAK_GBS * 1e9, 2.5e15
    t = 0.0
    if statistics:  # without: taken from an earlier call on the same input
        t += 2.0 * M * K / bw
        t += M * K * (K + 1) / pk
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
    roof_shared = sum(search_roofline_ms(M, Ks[l][0], Ks[l][1], statistics=j == 0)
                      for group in by_src.values() for j, (_, l) in enumerate(group))
    for lname, r_ in res.items():
        r_["roofline_ms"] = round(search_roofline_ms(M, r_["K"], r_["N"]), 3)
    return dict(layers=res, s_per_layer=round(total_ms / 7 / 1e3, 4), total_s=round(total_ms / 1e3, 3),
                calib_rows=M, n_alpha=20, composite_roofline_s=round(roof / 1e3, 4),
                composite_roofline_frac=round(roof / total_ms, 4),
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


def run_cpu_baseline(layers_spec, budget_s: float):
    """The oracle's fp64 W4A16 product over the 7 decode layers, on the host cores."""
    import oracle
    from gen import activations_fp16, normal_fp16
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    prepared = []
    for name, K, N in layers_spec:
        W = normal_fp16((N, K), 0.02, seed=2000 + K + N)
        q, z, sc = oracle.quantize_groups(W.astype(np.float32))
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
                sample=f"{steps} full decode steps (7 layers of the 7B block, M=1) through oracle.gemm "
                       f"(fp64 dequantize + matmul), {dt:.1f} s")


def profile_mode(args, torch, awq, dev):
    """Short runs for rocprofv3 counter passes: the decode GEMVs, a plain copy, or one GEMM / decode layer."""
    if args.profile_mode == "copy":
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(profile_mode="copy", bytes_per_copy=n, launches=5)))
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
    r = run_decode(args, torch, awq, dev)
    print(json.dumps(dict(profile_mode="gemv", alg_bytes_per_launch=r["bytes_per_launch"], kern_ms=r["kern_ms"],
                          per_layer=r["per_layer"])))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-search", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-decode-legs", action="store_true",
                    help="skip the fused, scaled-input and 3-bit decode legs (the headline step only)")
    ap.add_argument("--profile-mode", choices=["gemv", "copy", "gemm", "ring"], default=None)
    args = ap.parse_args()
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
        log("decode, x divided by s on the device (fused into the GEMV on 4096 x 4096 layers)")
        legs["decode_llama2_7b_scaled_input"] = run_decode_scaled(args, torch, awq, dev)
        torch.cuda.empty_cache()
        log("decode, 3-bit weights (7 launches)")
        legs["decode_llama2_7b_3bit"] = run_decode_3bit(args, torch, awq, dev)
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

    traffic = measured_traffic(dec["bytes_per_launch"])
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
        "roofline": {"bound": "hbm", "achieved": round(dec["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 0),
                     "kernel": "awq::gemv_kernel (M=1)", "avg_launch_us": round(dec["kern_ms"] * 1e3, 3),
                     "alg_bytes_per_launch": round(dec["bytes_per_launch"], 1),
                     "timing": "HIP events around the timed graph replays / launches in the region"},
        "cpu_baseline": cpu,
        "per_layer": dec["per_layer"],
        "legs": legs,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
