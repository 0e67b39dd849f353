#!/usr/bin/env python3
"""Benchmark of the InfLLM-V2 sparse-attention forward path on one MI355X.

Default workload (the headline line): MiniCPM-style GQA layer prefill at 32k
tokens (b=1, n=32768, h_q=32, h_kv=2, d=128, bf16, B=64, l_C1=32, s_C1=16,
l=5, s=4, N_init=1, N_local=2, k=16) on seeded synthetic inputs with planted
needle blocks.  One step = the whole hot path: compress_k -> block_scores ->
topk_select -> sparse_attn (decode: select_blocks_append -- the step's new
K^C1 kernel formed inside the selection's score sweep, the top-k fused into
the pooling -- then sparse_attn), inputs resident in HBM, outputs
preallocated.
The same JSON line also carries the 128k prefill and the 16-sequence decode
step (both secondary, fewer steps), the dense-attention time on the same
input, the roofline of the dominant kernel, and the fp64 CPU oracle timed on a
bounded sample of the workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extra] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import trainable_block_sparse_amd as tbs  # noqa: E402
from synth import CONFIGS, make_inputs, paged_cache, varlen_lengths  # noqa: E402

METRIC = "sparse-attn prefill tokens/s at 32k/128k + decode µs/token; % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "trainable_block_sparse_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def problem_of(cfg, **kw) -> tbs.Problem:
    n_q = 1 if cfg.decode else cfg.n_kv
    p = dict(batch=cfg.batch, n_q=n_q, n_kv=cfg.n_kv, h_kv=cfg.h_kv, G=cfg.G, d=cfg.d,
             q_pos0=cfg.n_kv - n_q, B=cfg.B, l_C1=cfg.l_C1, s_C1=cfg.s_C1, l=cfg.l, s=cfg.s,
             k=cfg.k, N_init=cfg.N_init, N_local=cfg.N_local, dtype=cfg.io)
    p.update(kw)
    return tbs.Problem(**p)


# --------------------------------------------------------------------------
# algorithmic work (what the method must do; no padding, masking or re-sweeps)
# --------------------------------------------------------------------------

def visible_kernels(p, l_C1=32, s_C1=16):
    return np.where(p >= l_C1 - 1, (p - l_C1 + 1) // s_C1 + 1, 0)


def selection_flops_per_pass(cfg, positions, l_len=None, s_len=None):
    """b * h_q * 2d * sum_p |V(p)|  (one pass over the visible kernels of
    length l_len and stride s_len: K^C1's by default)."""
    vis = visible_kernels(positions, l_len or cfg.l_C1, s_len or cfg.s_C1)
    return float(cfg.batch * cfg.h_q * 2 * cfg.d * vis.sum())


def selection_flops_approx(cfg, positions):
    """The LSE approximation: the coarse sweep (kernels of 4 l_C1 at stride
    4 s_C1), one sweep over K^C1, and a second fine sweep for the positions
    that see no coarse kernel (they keep the exact LSE)."""
    early = positions[positions < 4 * cfg.l_C1 - 1]
    return (selection_flops_per_pass(cfg, positions, 4 * cfg.l_C1, 4 * cfg.s_C1) +
            selection_flops_per_pass(cfg, positions) + selection_flops_per_pass(cfg, early))


def attention_flops(cfg, positions, budget):
    """b * h_q * 4d * sum_p keys(p), keys(p) = (|I(p)|-1)*B + (p mod B) + 1."""
    b_p = positions // cfg.B
    nsel = np.minimum(b_p + 1, budget)
    keys = (nsel - 1) * cfg.B + positions % cfg.B + 1
    return float(cfg.batch * cfg.h_q * 4 * cfg.d * keys.sum())


def decode_bytes(cfg, budget, lse_approx=False):
    """Algorithmic HBM bytes of one decode step: K^C1 of every visible kernel
    (and K^C2 of every visible coarse kernel with the LSE approximation), the
    selected K and V blocks, Q and O."""
    L = cfg.n_kv
    n_c1 = (L - cfg.l_C1) // cfg.s_C1 + 1
    n_c2 = (L - 4 * cfg.l_C1) // (4 * cfg.s_C1) + 1 if lse_approx else 0
    nsel = min((L - 1) // cfg.B + 1, budget)
    kc = (n_c1 + n_c2) * cfg.d * 2
    kv = nsel * cfg.B * cfg.d * 2 * 2
    qo = 2 * cfg.G * cfg.d * 2
    return float(cfg.batch * cfg.h_kv * (kc + kv + qo))


def decode_varlen_bytes(cfg, lens, budget):
    """decode_bytes summed over a varlen batch: each sequence's own K^C1 and
    selected blocks (a short sequence selects all of its causal blocks)."""
    total = 0.0
    for L in lens:
        L = int(L)
        n_c1 = (L - cfg.l_C1) // cfg.s_C1 + 1 if L >= cfg.l_C1 else 0
        nsel = min((L - 1) // cfg.B + 1, budget)
        total += cfg.h_kv * (n_c1 * cfg.d * 2 + nsel * cfg.B * cfg.d * 2 * 2 + 2 * cfg.G * cfg.d * 2)
    return total


# the sources each kernel is built from (its own file and the headers it uses)
KERNEL_SOURCES = {
    "compress_k_kernel": ["compress.hip", "common.hpp", "kc1_mean.hpp"],
    "scores_": ["scores.hip", "common.hpp", "kc1_mean.hpp", "select_merge.hpp"],
    "topk_kernel": ["topk.hip", "common.hpp"],
    "kv_pack_kernel": ["attn.hip", "attn_layout.hpp", "common.hpp", "select_merge.hpp"],
    "attn_bwd": ["attn_bwd.hip", "attn_layout.hpp", "common.hpp"],
    "bwd_": ["attn_bwd.hip", "attn_layout.hpp", "common.hpp"],
    "attn_": ["attn.hip", "attn_layout.hpp", "common.hpp", "select_merge.hpp"],
}


def _code_only(text):
    """Source text without comments and whitespace (a comment edit does not
    change a kernel)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def kernel_source_hash(kernel=None):
    """sha256 prefix of the code of the sources a kernel is built from (all
    sources when the kernel is not listed)."""
    files = sorted(os.listdir(CSRC))
    if kernel is not None:
        for prefix, fs in KERNEL_SOURCES.items():
            if kernel.startswith(prefix):
                files = fs
                break
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# timed runs
# --------------------------------------------------------------------------

class StageTimer:
    """Per-stage HIP events on the stream the kernels are launched on."""

    def __init__(self, names):
        self.names = names
        self.ms = {n: 0.0 for n in names}
        self.pending = []

    def step(self, fns):
        s = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        evs[0].record(s)
        for i, fn in enumerate(fns):
            fn()
            evs[i + 1].record(s)
        self.pending.append(evs)

    def collect(self):
        torch.cuda.synchronize()
        for evs in self.pending:
            for i, n in enumerate(self.names):
                self.ms[n] += evs[i].elapsed_time(evs[i + 1])
        steps = len(self.pending)
        self.pending = []
        return {n: v / steps for n, v in self.ms.items()}


def bench_pipelined(lp, Q, K, V, Kc1, O_ref, lse_ref, steps, warmup, n_chunks, Kc2=None):
    """The same prefill as a two-stream pipeline over query ranges (selection
    of range i+1 beside attention of range i); checks it reproduces the serial
    outputs bitwise."""
    pipe = tbs.PrefillPipeline(lp, n_chunks)
    O2, lse2 = torch.empty_like(O_ref), torch.empty_like(lse_ref)
    for _ in range(warmup):
        pipe.run(Q, K, V, Kc1, O2, lse2, Kc2=Kc2)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        pipe.run(Q, K, V, Kc1, O2, lse2, Kc2=Kc2)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"n_ranges": len(pipe.chunks), "ms_per_step": ms,
            "tokens_per_s": lp.batch * lp.n_q / (ms / 1e3),
            "same_output_as_serial": bool(torch.equal(O2, O_ref) and torch.equal(lse2, lse_ref))}


def bench_prefill(cfg, steps, warmup, with_dense=True, dense_steps=None, pipeline_chunk=8192,
                  lse_approx=False):
    log(f"[bench] {cfg.name}{' (LSE approximation)' if lse_approx else ''}: generating inputs")
    x = make_inputs(cfg)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    del x
    lp = problem_of(cfg, lse_approx=lse_approx)
    n_blk, bud, n_c1 = tbs.n_blocks(lp), tbs.budget(lp), tbs.n_kernels(lp)
    Kc1 = torch.empty((lp.batch, lp.h_kv, n_c1, lp.d), dtype=Q.dtype, device=dev)
    n_c2 = tbs.n_coarse_kernels(lp)
    Kc2 = (torch.empty((lp.batch, lp.h_kv, n_c2, lp.d), dtype=Q.dtype, device=dev)
           if lse_approx else None)
    S = torch.empty((lp.batch, lp.h_kv, lp.n_q, n_blk), dtype=torch.float32, device=dev)
    idx = torch.empty((lp.batch, lp.h_kv, lp.n_q, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((lp.batch, lp.h_kv, lp.n_q), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((lp.batch, lp.h_q, lp.n_q), dtype=torch.float32, device=dev)
    ws_s = torch.empty(max(tbs.block_scores_workspace(lp), 16), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(tbs.sparse_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)
    fns = [
        lambda: tbs.compress_k(lp, K, Kc1),
        lambda: tbs.block_scores(lp, Q, Kc1, S, ws_s, Kc2=Kc2),
        lambda: tbs.topk_select(lp, S, idx, nsel),
        lambda: tbs.sparse_attn(lp, Q, K, V, idx, nsel, O, lse, ws_a),
    ]
    names = ["compress_k", "block_scores", "topk_select", "sparse_attn"]
    if lse_approx:
        fns.insert(1, lambda: tbs.compress_k2(lp, K, Kc2))
        names.insert(1, "compress_k2")
    log(f"[bench] {cfg.name}: warmup {warmup}")
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    timer = StageTimer(names)
    log(f"[bench] {cfg.name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        timer.step(fns)
    stage = timer.collect()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms = sum(stage.values())
    pos = np.arange(cfg.n_kv)
    out = dict(ms_per_step=ms, wall_ms_per_step=wall, stages_ms=stage,
               tokens_per_s=cfg.batch * cfg.n_q / (ms / 1e3),
               attn_flops=attention_flops(cfg, pos, bud))
    if lse_approx:
        # one sweep over K^C1 plus the coarse sweep over K^C2 (1/4 the kernels)
        out["lse_approx"] = True
        out["sel_flops"] = selection_flops_approx(cfg, pos)
    else:
        out["sel_flops"] = out["sel_flops_2pass"] = 2 * selection_flops_per_pass(cfg, pos)
    out["algo_tflops"] = (out["sel_flops"] + out["attn_flops"]) / (ms / 1e3) / 1e12
    out["frac_of_bf16_peak"] = out["algo_tflops"] / PEAK_BF16_TFLOPS
    if pipeline_chunk and lp.batch == 1 and lp.n_q > pipeline_chunk:
        out["pipelined"] = bench_pipelined(lp, Q, K, V, Kc1, O, lse, steps, warmup,
                                           lp.n_q // pipeline_chunk, Kc2=Kc2)
    if with_dense:
        dsteps = dense_steps or max(1, steps // 2)
        ws_d = torch.empty(max(tbs.dense_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)
        Od = torch.empty_like(Q)
        log(f"[bench] {cfg.name}: dense attention x{dsteps}")
        tbs.dense_attn(lp, Q, K, V, Od, lse, ws_d)
        dt = StageTimer(["dense_attn"])
        for _ in range(dsteps):
            dt.step([lambda: tbs.dense_attn(lp, Q, K, V, Od, lse, ws_d)])
        out["dense_ms"] = dt.collect()["dense_attn"]
        out["speedup_vs_dense"] = out["dense_ms"] / ms
    del Q, K, V, S, O
    torch.cuda.empty_cache()
    return out


def bench_backward(cfg, steps, warmup, with_dense=True):
    """Training-side record: the backward of the block-sparse attention (dQ,
    dK, dV with the selected sets fixed) after one forward on the same
    inputs; algorithmic work = 2.5x the forward attention flops (recomputed
    scores and dP: 2d each, dV, dK, dQ: 2d each per (token, head, key))."""
    log(f"[bench] {cfg.name}: backward")
    x = make_inputs(cfg)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    del x
    lp = problem_of(cfg)
    bud = tbs.budget(lp)
    gen = torch.Generator().manual_seed(cfg.seed)
    dO = torch.randn(Q.shape, generator=gen).to(Q.dtype).to(dev)
    Kc1 = tbs.compress_k(lp, K)
    idx, nsel = tbs.topk_select(lp, tbs.block_scores(lp, Q, Kc1))
    O, lse = tbs.sparse_attn(lp, Q, K, V, idx, nsel)
    dQ = torch.empty(Q.shape, dtype=torch.float32, device=dev)
    dK = torch.empty((lp.batch, lp.n_kv, lp.h_kv, lp.d), dtype=torch.float32, device=dev)
    dV = torch.empty_like(dK)
    ws = torch.empty(max(tbs.sparse_attn_bwd_workspace(lp), tbs.dense_attn_bwd_workspace(lp), 16),
                     dtype=torch.uint8, device=dev)
    fn = lambda: tbs.sparse_attn_bwd(lp, Q, K, V, idx, nsel, O, lse, dO, dQ, dK, dV, ws)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t = StageTimer(["sparse_attn_bwd"])
    for _ in range(steps):
        t.step([fn])
    ms = t.collect()["sparse_attn_bwd"]
    pos = np.arange(cfg.n_kv)
    flops = 2.5 * attention_flops(cfg, pos, bud)
    out = dict(ms=ms, tokens_per_s=cfg.batch * cfg.n_q / (ms / 1e3), algo_flops=flops,
               algo_tflops=flops / (ms / 1e3) / 1e12,
               workspace_bytes=tbs.sparse_attn_bwd_workspace(lp))
    out["frac_of_bf16_peak"] = out["algo_tflops"] / PEAK_BF16_TFLOPS
    if with_dense:
        Od, lsed = tbs.dense_attn(lp, Q, K, V)
        fd = lambda: tbs.dense_attn_bwd(lp, Q, K, V, Od, lsed, dO, dQ, dK, dV, ws)
        fd()
        td = StageTimer(["dense_attn_bwd"])
        for _ in range(max(1, steps // 2)):
            td.step([fd])
        out["dense_bwd_ms"] = td.collect()["dense_attn_bwd"]
        out["speedup_vs_dense_bwd"] = out["dense_bwd_ms"] / ms
    del Q, K, V, O, dO, dQ, dK, dV, ws
    torch.cuda.empty_cache()
    return out


def bench_decode_varlen(cfg, steps, warmup):
    """Serving-style decode step: 16 sequences of seeded lengths up to 131072
    (the first at full length), K/V in a shuffled page pool with a block
    table; the step appends each sequence's newest kernel, selects and
    attends through the varlen calls; timed as one HIP graph replay."""
    lens = varlen_lengths(cfg.batch, cfg.n_kv, seed=cfg.seed + 100, must=(cfg.n_kv,))
    log(f"[bench] {cfg.name} varlen paged: lengths {lens.tolist()}")
    x = make_inputs(cfg)
    dev = torch.device("cuda:0")
    kp, vp, table = paged_cache(x["k"], x["v"], lens, cfg.B, cfg.seed + 101)
    Q, K, V, table = x["q"].to(dev), kp.to(dev), vp.to(dev), table.to(dev)
    del x, kp, vp
    lp = problem_of(cfg, n_kv=cfg.n_kv, q_pos0=0)
    bud = tbs.budget(lp)
    seq = torch.tensor(lens, device=dev)
    Kc1 = torch.empty((lp.batch, lp.h_kv, tbs.n_kernels(lp), lp.d), dtype=Q.dtype, device=dev)
    tbs.compress_k_varlen(lp, K, seq - 1, Kc1, block_table=table)       # the cache before
    idx = torch.empty((lp.batch, lp.h_kv, 1, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((lp.batch, lp.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((lp.batch, lp.h_q, 1), dtype=torch.float32, device=dev)
    ws_s = torch.empty(max(tbs.select_blocks_varlen_workspace(lp), 16), dtype=torch.uint8,
                       device=dev)
    ws_a = torch.empty(max(tbs.sparse_attn_varlen_workspace(lp), 16), dtype=torch.uint8,
                       device=dev)
    fns = [
        lambda: tbs.compress_k_varlen(lp, K, seq, Kc1, block_table=table, last_n=1),
        lambda: tbs.select_blocks_varlen(lp, Q, Kc1, seq, idx, nsel, ws_s),
        lambda: tbs.sparse_attn_varlen(lp, Q, K, V, seq, idx, nsel, block_table=table, O=O,
                                       lse=lse, ws=ws_a),
    ]
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h0 = time.perf_counter()
    for _ in range(steps):
        for fn in fns:
            fn()
    host_ms = (time.perf_counter() - h0) * 1e3 / steps
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for fn in fns:
            fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    step_ms = min(eager_ms, graph_ms)
    nbytes = decode_varlen_bytes(cfg, lens, bud)
    out = dict(step_us=step_ms * 1e3, us_per_token=step_ms * 1e3 / cfg.batch,
               timing=("eager launches, steps back to back" if eager_ms <= graph_ms
                       else "HIP graph replay of the whole step"),
               eager_step_us=eager_ms * 1e3, graph_step_us=graph_ms * 1e3,
               host_enqueue_us=host_ms * 1e3, lengths=lens.tolist(),
               algo_bytes=nbytes, algo_GBps=nbytes / (step_ms / 1e3) / 1e9)
    out["frac_of_hbm_peak"] = out["algo_GBps"] / PEAK_HBM_GBS
    del Q, K, V, Kc1, O, ws_s, ws_a
    torch.cuda.empty_cache()
    return out


def bench_decode(cfg, steps, warmup, lse_approx=False):
    log(f"[bench] {cfg.name}{' (LSE approximation)' if lse_approx else ''}: "
        "generating the KV cache")
    x = make_inputs(cfg)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    del x
    lp = problem_of(cfg, lse_approx=lse_approx)
    prev = problem_of(cfg, n_kv=cfg.n_kv - 1, q_pos0=cfg.n_kv - 2, kv_cap=cfg.n_kv,
                      lse_approx=lse_approx)
    n_blk, bud, n_c1 = tbs.n_blocks(lp), tbs.budget(lp), tbs.n_kernels(lp)
    n_prev = tbs.n_kernels(prev)
    lp.c1_cap = prev.c1_cap = n_c1
    Kc1 = torch.empty((lp.batch, lp.h_kv, n_c1, lp.d), dtype=Q.dtype, device=dev)
    tbs.compress_k(prev, K, Kc1)           # the cache before this step
    Kc2, n_c2, n_prev2 = None, tbs.n_coarse_kernels(lp), tbs.n_coarse_kernels(prev)
    if lse_approx:
        lp.c2_cap = prev.c2_cap = n_c2
        Kc2 = torch.empty((lp.batch, lp.h_kv, n_c2, lp.d), dtype=Q.dtype, device=dev)
        tbs.compress_k2(prev, K, Kc2)
    S = torch.empty((lp.batch, lp.h_kv, 1, n_blk), dtype=torch.float32, device=dev)
    idx = torch.empty((lp.batch, lp.h_kv, 1, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((lp.batch, lp.h_kv, 1), dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((lp.batch, lp.h_q, 1), dtype=torch.float32, device=dev)
    ws_s = torch.empty(max(tbs.select_blocks_workspace(lp), tbs.block_scores_workspace(lp), 16),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(tbs.sparse_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)
    # the step as three calls: the append, scores and top-k in one call (the
    # top-k fused into the pooling kernel; S^cmp is not stored), attention
    fns3 = [
        lambda: tbs.compress_k(lp, K, Kc1, c1_begin=n_prev, c1_end=n_c1),
        lambda: tbs.select_blocks(lp, Q, Kc1, None, idx, nsel, ws_s, Kc2=Kc2),
        lambda: tbs.sparse_attn(lp, Q, K, V, idx, nsel, O, lse, ws_a),
    ]
    names3 = ["compress_append", "select_blocks", "sparse_attn"]
    if lse_approx and n_c2 > n_prev2:
        # this step also completes a coarse kernel (every 64th token)
        fns3.insert(1, lambda: tbs.compress_k2(lp, K, Kc2, c2_begin=n_prev2, c2_end=n_c2))
        names3.insert(1, "compress2_append")
    # the same step with the separate score and top-k calls, for comparison
    fns_sep = fns3[:-2] + [lambda: tbs.block_scores(lp, Q, Kc1, S, ws_s, Kc2=Kc2),
                           lambda: tbs.topk_select(lp, S, idx, nsel), fns3[-1]]
    # the step as two calls: the append inside the selection's score sweep,
    # then the attention
    fns2 = [
        lambda: tbs.select_blocks_append(lp, Q, K, Kc1, n_prev, n_c1, idx, nsel, ws_s),
        fns3[-1],
    ]
    if lse_approx:
        fns, names = fns3, names3
    else:
        # the timed step: one call (infv2_decode_step: the two calls' work,
        # with the selection's list merge inside the attention launch)
        ws_d = torch.empty(tbs.decode_step_workspace(lp), dtype=torch.uint8, device=dev)
        fns = [lambda: tbs.decode_step(lp, Q, K, V, Kc1, n_prev, n_c1, idx, nsel, O, lse, ws_d)]
        names = ["decode_step"]
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    timer = StageTimer(names)
    log(f"[bench] {cfg.name}: timing {steps} steps (per-stage events)")
    for _ in range(steps):
        timer.step(fns)
    stage = timer.collect()
    # the whole step, eager, without events in between
    # (host_ms: the host's enqueue time per step; the eager figure is the GPU's
    # own only while this stays below it)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    h0 = time.perf_counter()
    for _ in range(steps):
        for fn in fns:
            fn()
    host_ms = (time.perf_counter() - h0) * 1e3 / steps
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    # the step captured once in a HIP graph and replayed (how a serving loop
    # issues it: one launch, no host gaps between the kernels)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for fn in fns:
            fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    three_ms = None
    if fns is not fns3:
        for _ in range(warmup):
            for fn in fns3:
                fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            for fn in fns3:
                fn()
        e1.record()
        torch.cuda.synchronize()
        three_ms = e0.elapsed_time(e1) / steps
    two_ms = None
    if not lse_approx:
        for _ in range(warmup):
            for fn in fns2:
                fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            for fn in fns2:
                fn()
        e1.record()
        torch.cuda.synchronize()
        two_ms = e0.elapsed_time(e1) / steps
    graph_sep = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_sep):
        for fn in fns_sep:
            fn()
    for _ in range(warmup):
        graph_sep.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph_sep.replay()
    e1.record()
    torch.cuda.synchronize()
    sep_ms = e0.elapsed_time(e1) / steps
    nbytes = decode_bytes(cfg, bud, lse_approx)
    # the step as a serving loop would issue it: the faster of eager launches
    # (the host enqueues ahead of the GPU) and one graph replay per step
    graph_ms = step_ms
    step_ms = min(eager_ms, graph_ms)
    out = dict(step_us=step_ms * 1e3, us_per_token=step_ms * 1e3 / cfg.batch,
               eager_step_us=eager_ms * 1e3, graph_step_us=graph_ms * 1e3,
               host_enqueue_us=host_ms * 1e3,
               timing=("eager launches, steps back to back" if eager_ms <= graph_ms
                       else "HIP graph replay of the whole step"),
               separate_topk_step_us=sep_ms * 1e3,
               three_call_step_us=None if three_ms is None else three_ms * 1e3,
               two_call_step_us=None if two_ms is None else two_ms * 1e3,
               stages_us_eager={k: v * 1e3 for k, v in stage.items()}, algo_bytes=nbytes,
               algo_GBps=nbytes / (step_ms / 1e3) / 1e9)
    out["frac_of_hbm_peak"] = out["algo_GBps"] / PEAK_HBM_GBS
    del Q, K, V
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, as it stands, on a bounded sample
# --------------------------------------------------------------------------

_CPU = {}


def _cpu_rows(rows):
    """Worker: the oracle's selection, top-k and attention for some rows."""
    import oracle as orc
    from threadpoolctl import threadpool_limits
    c = _CPU
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        orc.forward_rows(c["Q"], c["K"], c["V"], np.asarray(rows), c["op"], Kc1=c["Kc1"],
                         mode="sparse")
    return len(rows), time.perf_counter() - t0


def cpu_baseline(cfg, budget_s=15.0):
    """The oracle as it stands (fp64 numpy), timed on the host's cores: one
    worker process per usable core (at most 16), each with one BLAS thread,
    over a stratified sample of query rows that takes about budget_s of wall
    time; compress_k runs once over all keys.  Extrapolated to every row."""
    import multiprocessing as mp
    import oracle as orc
    x = make_inputs(cfg)
    op = orc.Problem(G=cfg.G, h_kv=cfg.h_kv, d=cfg.d, B=cfg.B, l_C1=cfg.l_C1, s_C1=cfg.s_C1,
                     l=cfg.l, s=cfg.s, k=cfg.k, N_init=cfg.N_init, N_local=cfg.N_local,
                     io=cfg.io)
    Q = x["q"][0].double().numpy()
    K = x["k"][0].double().numpy()
    V = x["v"][0].double().numpy()
    t0 = time.perf_counter()
    Kc1 = orc.compress_k(K[None], op)[0]
    t_comp = time.perf_counter() - t0
    _CPU.update(Q=Q, K=K, V=V, Kc1=Kc1, op=op)
    nproc = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0))
    workers = max(1, min(usable, 16))
    # calibrate: the cost of a row grows with its position, so rows are
    # stratified over the sequence (one per stratum, jittered)
    n_cal = 16
    rng = np.random.default_rng(0)
    cal = np.sort(rng.choice(cfg.n_q, size=n_cal, replace=False))
    _, t_cal = _cpu_rows(cal)
    per_row = t_cal / n_cal
    n_rows = int(max(workers * 8, min(cfg.n_q, budget_s * workers / per_row)))
    edges = np.linspace(0, cfg.n_q, n_rows + 1).astype(np.int64)
    rows = np.unique(np.minimum(edges[:-1] + rng.integers(0, np.maximum(1, np.diff(edges))),
                                cfg.n_q - 1))
    chunks = [rows[i::workers * 4] for i in range(workers * 4)]
    ctx = mp.get_context("fork")
    t1 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        done = pool.map(_cpu_rows, chunks)
    t_rows = time.perf_counter() - t1
    rows_done = sum(n for n, _ in done)
    total = t_comp + t_rows / rows_done * cfg.n_q * cfg.batch
    return {"value": cfg.batch * cfg.n_q / total, "unit": "tokens/s", "cores": workers,
            "kind": "oracle", "nproc": nproc, "usable_cpus": usable,
            "sample": (f"{cfg.name}: compress_k over all {cfg.n_kv} keys ({t_comp:.1f} s, one "
                       f"process) + {rows_done} query rows stratified over the sequence "
                       f"(selection, top-k, attention) on {workers} worker processes with one "
                       f"BLAS thread each ({t_rows:.1f} s wall), extrapolated to "
                       f"{cfg.batch * cfg.n_q} rows; host nproc {nproc}")}


def cpu_baseline_child():
    """cpu_baseline run in a fresh child process (this process holds the
    GPU; the child only uses the CPU)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only"],
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        log("[bench] cpu baseline failed:", r.stderr[-2000:])
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


# the kernels one call of each prefill stage can launch (rocprofv3 name
# prefixes; which of them run depends on the shape: the key-range split of the
# attention from 1024 blocks on)
STAGE_KERNELS = {
    "compress_k": ["compress_k_kernel"],
    "block_scores": ["scores_prefill_kernel", "scores_exact_kernel"],
    "topk_select": ["topk_kernel"],
    "sparse_attn": ["kv_pack_kernel", "attn_prefill_kernel", "attn_prefill_seq_kernel",
                    "attn_range_kernel", "attn_range_merge_kernel"],
}

# the kernels one call of each decode stage launches
DECODE_STAGE_KERNELS = {
    "compress_append": ["compress_k_kernel"],
    # (the profiled run also times the three-call step, so the logits
    # kernel's two instances are named apart)
    "select_blocks": ["scores_split_logits_kernel<false,false>", "scores_split_pool_kernel",
                      "scores_select_merge_kernel"],
    "select_blocks_append": ["scores_split_logits_kernel<false,true>",
                             "scores_split_pool_kernel", "scores_select_merge_kernel"],
    "sparse_attn": ["attn_split_kernel", "attn_merge_kernel"],
    "decode_step": ["scores_split_logits_kernel<false,true>", "scores_split_pool_kernel",
                    "attn_split_select_kernel", "attn_merge_kernel"],
}


def stage_traffic(workload, prefixes):
    """(HBM bytes of one stage call, the kernels counted) from the committed
    rocprofv3 counter summary: every kernel of the workload's profiled run
    whose name starts with one of the prefixes, each entry's bytes per launch
    times its launches per call.  None when an entry was taken on other kernel
    sources than the current ones, or when none is there."""
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None, []
    total, kernels = 0.0, []
    for key, ent in tr.items():
        if not key.startswith(workload + "/"):
            continue
        kern = key.split("/", 1)[1]
        if not any(kern.startswith(pre) for pre in prefixes):
            continue
        if ent.get("source_hash") != kernel_source_hash(kern):
            return None, []
        total += ent.get("bytes_per_call", ent.get("bytes_per_launch", 0.0))
        kernels.append(kern)
    return (total, kernels) if kernels else (None, [])


def traffic_for(stage, workload):
    return stage_traffic(workload, STAGE_KERNELS.get(stage, [stage]))[0]


def prefill_roofline(res, workload):
    """Roofline object of the dominant stage of a prefill record: algorithmic
    flops of that stage over its event-timed duration (one launch per kernel
    per call) against the bf16 MFMA peak; traffic = the committed counter
    bytes of the stage's launches when they were taken on the current
    kernel sources, else null."""
    stages = res["stages_ms"]
    dom = max(stages, key=stages.get)
    flops = {"block_scores": res.get("sel_flops_2pass"), "sparse_attn": res["attn_flops"]}.get(dom)
    if flops is None:
        return {"kernel": dom, "bound": "mfma", "achieved": None, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": None, "traffic": None}
    ach = flops / (stages[dom] / 1e3) / 1e12
    traffic, kernels = stage_traffic(workload, STAGE_KERNELS.get(dom, [dom]))
    return {"kernel": dom, "launches": kernels or STAGE_KERNELS.get(dom, [dom]), "bound": "mfma",
            "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic,
            "per_launch_algorithmic": flops, "avg_launch_ms": stages[dom]}


def decode_roofline(res, cfg, budget, workload="decode"):
    """Roofline object of the decode step's dominant stage (HBM-bound):
    algorithmic bytes of that stage (select_blocks: every visible K^C1 row
    and Q; sparse_attn: the selected K/V blocks, Q and O; decode_step, the
    one-call step: both) over its event-timed duration against the HBM
    peak."""
    st = res["stages_us_eager"]
    dom = max(st, key=st.get)
    L = cfg.n_kv
    n_c1 = (L - cfg.l_C1) // cfg.s_C1 + 1
    nsel = min((L - 1) // cfg.B + 1, budget)
    qo = cfg.G * cfg.d * 2
    per = {"select_blocks": n_c1 * cfg.d * 2 + qo,
           # the selection's bytes plus the appended kernel's keys and its row
           "select_blocks_append": n_c1 * cfg.d * 2 + qo + cfg.l_C1 * cfg.d * 2 + cfg.d * 2,
           "sparse_attn": nsel * cfg.B * cfg.d * 2 * 2 + 2 * qo,
           "compress_append": cfg.l_C1 * cfg.d * 2 + cfg.d * 2}
    # the one-call step: the append's selection and the attention together
    per["decode_step"] = per["select_blocks_append"] + per["sparse_attn"]
    per = per[dom]
    nbytes = float(cfg.batch * cfg.h_kv * per)
    ach = nbytes / (st[dom] / 1e6) / 1e9
    traffic, kernels = stage_traffic(workload, DECODE_STAGE_KERNELS[dom])
    return {"kernel": dom, "launches": kernels or DECODE_STAGE_KERNELS[dom], "bound": "hbm",
            "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
            "traffic": traffic, "per_launch_algorithmic": nbytes,
            "avg_launch_us": st[dom]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="skip the 128k and decode lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the two-stream range-pipeline record of the 128k prefill")
    ap.add_argument("--only", choices=["prefill32k", "prefill128k", "decode", "dense_switch",
                                       "copy", "backward32k", "backward128k",
                                       "decode_varlen"],
                    help="run one workload alone and print its record (profiling runs); "
                         "'copy' is a plain 256 MiB device copy used to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--lse-approx", action="store_true",
                    help="with --only: the LSE approximation instead of the exact LSE")
    ap.add_argument("--no-approx", action="store_true",
                    help="skip the LSE-approximation records")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="only the CPU oracle baseline (no GPU use); prints its JSON object")
    args = ap.parse_args()
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline(CONFIGS["prefill32k"])), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU and has no multi-GPU path (the work would shard by "
              "KV group, batch or query range with the same kernels); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tbs.lib()
    if args.only:
        if args.only == "copy":
            n = 256 << 20
            src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(args.steps):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(json.dumps({"workload": "copy", "bytes_read": n, "bytes_written": n}), flush=True)
            return
        if args.only == "decode_varlen":
            rec = bench_decode_varlen(CONFIGS["decode"], args.steps, args.warmup)
            print(json.dumps({"workload": args.only, **rec}), flush=True)
            return
        if args.only.startswith("backward"):
            c = CONFIGS["prefill" + args.only[len("backward"):]]
            rec = bench_backward(c, args.steps, args.warmup, with_dense=not args.no_dense)
            print(json.dumps({"workload": args.only, **rec}), flush=True)
            return
        c = CONFIGS[args.only]
        if args.only == "decode":
            rec = bench_decode(c, args.steps, args.warmup, lse_approx=args.lse_approx)
        elif args.only == "dense_switch":
            rec = bench_dense_switch(c, args.steps, args.warmup)
        else:
            pipe = 0 if (args.no_pipeline or args.only == "prefill32k") else 8192
            rec = bench_prefill(c, args.steps, args.warmup, with_dense=not args.no_dense,
                                pipeline_chunk=pipe, lse_approx=args.lse_approx)
        name = args.only + ("_lse_approx" if args.lse_approx else "")
        print(json.dumps({"workload": name, **rec}), flush=True)
        return

    cfg = CONFIGS["prefill32k"]
    # the headline is the one-shot path (one launch per kernel per step, as
    # the rocprofv3 summaries see it); the 128k line adds the range pipeline
    main_res = bench_prefill(cfg, args.steps, args.warmup, with_dense=not args.no_dense,
                             pipeline_chunk=0)
    log(f"[bench] prefill32k: {main_res['ms_per_step']:.3f} ms/step, stages {main_res['stages_ms']}")

    # roofline of the dominant kernel
    roof = prefill_roofline(main_res, "prefill32k")

    extra = {}
    if not args.no_extra:
        c3 = CONFIGS["prefill128k"]
        r3 = bench_prefill(c3, max(2, args.steps // 5), 1, with_dense=not args.no_dense,
                           dense_steps=1, pipeline_chunk=0 if args.no_pipeline else 8192)
        r3["roofline"] = prefill_roofline(r3, "prefill128k")
        extra["prefill128k"] = {k: v for k, v in r3.items()}
        log(f"[bench] prefill128k: {r3['ms_per_step']:.3f} ms/step")
        c4 = CONFIGS["decode"]
        r4 = bench_decode(c4, max(20, args.steps * 5), args.warmup)
        r4["roofline"] = decode_roofline(r4, c4, 19)
        extra["decode"] = r4
        log(f"[bench] decode: {r4['step_us']:.1f} us/step")
        rv = bench_decode_varlen(c4, max(20, args.steps * 5), args.warmup)
        extra["decode_varlen_paged"] = rv
        log(f"[bench] decode varlen paged: {rv['step_us']:.1f} us/step")
        c5 = CONFIGS["dense_switch"]
        r5 = bench_dense_switch(c5, args.steps, args.warmup)
        extra["dense_switch"] = r5
        rbw = bench_backward(cfg, args.steps, args.warmup, with_dense=not args.no_dense)
        extra["prefill32k_backward"] = rbw
        log(f"[bench] prefill32k backward: {rbw['ms']:.3f} ms")
        if not args.no_approx:
            # the pages' default selection: the LSE approximation (its own
            # oracle mode and parity tests)
            ra = bench_prefill(cfg, args.steps, args.warmup, with_dense=False, pipeline_chunk=0,
                               lse_approx=True)
            extra["prefill32k_lse_approx"] = ra
            log(f"[bench] prefill32k (LSE approx): {ra['ms_per_step']:.3f} ms/step")
            rb = bench_prefill(c3, max(2, args.steps // 5), 1, with_dense=False,
                               pipeline_chunk=0 if args.no_pipeline else 8192, lse_approx=True)
            extra["prefill128k_lse_approx"] = rb
            log(f"[bench] prefill128k (LSE approx): {rb['ms_per_step']:.3f} ms/step")
            rc = bench_decode(c4, max(20, args.steps * 5), args.warmup, lse_approx=True)
            extra["decode_lse_approx"] = rc
            log(f"[bench] decode (LSE approx): {rc['step_us']:.1f} us/step")

    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle, child process)")
        cpu = cpu_baseline_child()

    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, 32 planted needle blocks)",
        "config": {"workload": "prefill32k: b=1 n=32768 h_q=32 h_kv=2 d=128 bf16 B=64 "
                               "l_C1=32 s_C1=16 l=5 s=4 N_init=1 N_local=2 k=16",
                   "global_batch": cfg.batch, "seq_len": cfg.n_kv, "parallelism": "none (1 GPU)"},
        "stages_ms": main_res["stages_ms"],
        "algo_tflops": main_res["algo_tflops"],
        "frac_of_bf16_peak": main_res["frac_of_bf16_peak"],
        "dense_ms": main_res.get("dense_ms"),
        "speedup_vs_dense": main_res.get("speedup_vs_dense"),
        "roofline": roof,
        "cpu_baseline": cpu,
        "library": tbs.library_info(),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def bench_dense_switch(cfg, steps, warmup):
    """Short sequences: the switch selects dense attention.  The sparse path
    (compress_k, block_scores, topk_select, sparse_attn, whose selection
    then covers every causal block) is timed beside it on the same input,
    and the two outputs are compared."""
    log(f"[bench] {cfg.name}: inputs")
    x = make_inputs(cfg)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("q", "k", "v"))
    lp = problem_of(cfg)
    assert tbs.use_dense(lp)
    ws_d = torch.empty(max(tbs.dense_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)
    O = torch.empty_like(Q)
    lse = torch.empty((lp.batch, lp.h_q, lp.n_q), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        tbs.dense_attn(lp, Q, K, V, O, lse, ws_d)
    t = StageTimer(["dense_attn"])
    for _ in range(steps):
        t.step([lambda: tbs.dense_attn(lp, Q, K, V, O, lse, ws_d)])
    dense_ms = t.collect()["dense_attn"]
    # the sparse path on the same input
    n_blk, bud, n_c1 = tbs.n_blocks(lp), tbs.budget(lp), tbs.n_kernels(lp)
    Kc1 = torch.empty((lp.batch, lp.h_kv, n_c1, lp.d), dtype=Q.dtype, device=dev)
    S = torch.empty((lp.batch, lp.h_kv, lp.n_q, n_blk), dtype=torch.float32, device=dev)
    idx = torch.empty((lp.batch, lp.h_kv, lp.n_q, bud), dtype=torch.int32, device=dev)
    nsel = torch.empty((lp.batch, lp.h_kv, lp.n_q), dtype=torch.int32, device=dev)
    Os = torch.empty_like(Q)
    lses = torch.empty_like(lse)
    ws_s = torch.empty(max(tbs.block_scores_workspace(lp), 16), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(tbs.sparse_attn_workspace(lp), 16), dtype=torch.uint8, device=dev)
    fns = [lambda: tbs.compress_k(lp, K, Kc1),
           lambda: tbs.block_scores(lp, Q, Kc1, S, ws_s),
           lambda: tbs.topk_select(lp, S, idx, nsel),
           lambda: tbs.sparse_attn(lp, Q, K, V, idx, nsel, Os, lses, ws_a)]
    names = ["compress_k", "block_scores", "topk_select", "sparse_attn"]
    for _ in range(warmup):
        for fn in fns:
            fn()
    ts = StageTimer(names)
    for _ in range(steps):
        ts.step(fns)
    sp_stages = ts.collect()
    sparse_ms = sum(sp_stages.values())
    diff = float((Os.float() - O.float()).abs().max().item())
    flops = attention_flops(cfg, np.arange(cfg.n_kv), 10 ** 9)
    out = {"dense_ms": dense_ms, "tokens_per_s": cfg.batch * cfg.n_q / (dense_ms / 1e3),
           "algo_tflops": flops / (dense_ms / 1e3) / 1e12,
           "sparse_ms": sparse_ms, "sparse_stages_ms": sp_stages,
           "sparse_over_dense": sparse_ms / dense_ms,
           "sparse_attn_over_dense_attn": sp_stages["sparse_attn"] / dense_ms,
           "sparse_vs_dense_max_abs_O": diff}
    del Q, K, V, O, Os, S, Kc1
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
