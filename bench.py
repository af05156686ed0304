"""Benchmark of masked scaled dot-product attention over a CSR mask on one MI355X.

A step is one pass of the CSR path over one batch of synthetic input: SDDMM, sparse
softmax and SpMM (scores, weights and context), replayed from a HIP graph of several steps,
on the Longformer-style workload (12 heads, n=4096, d=64, bf16, window |i-j|<=128 plus
global tokens 0 and 1).
The row plan (a function of the mask alone) is built once before timing and reported
separately. Inputs are resident in HBM before timing starts. The JSON line reports attended pairs/s
(value), per-kernel durations from HIP events recorded on the stream the kernels run
on, the roofline of the dominant kernel, the other fused variants measured on their own
workloads, and the fp64 CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-extra] [--workload NAME]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
VALU_FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 vector peak (packed), TFLOP/s
METRIC = "attended (i,j) pairs/sec and % of HBM/MFMA roofline, 1×MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_BYTES = 256 << 20          # size of the calibration copy (--profile copy)
CSRC = os.path.join(ROOT, "masked_scaled_dot_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="longformer_n4096",
                    choices=["longformer_n4096", "random_n8192"])
    ap.add_argument("--streams", type=int, default=2,
                    help="independent batches in flight, one HIP stream (and graph) each")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the fused/BSR/bias rows")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    ap.add_argument("--profile", choices=["pipeline", "backward", "fused_csr", "fused_bsr", "fused_dense",
                                          "fused_backward", "fused_backward_cover", "copy"],
                    help="run only this kernel family (steps iterations after warmup) and exit; "
                         "for rocprofv3 runs")
    return ap.parse_args()


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------------ device setup

def to_device(p, torch, sa, element=True):
    dev = torch.device("cuda:0")

    def qkv(w):
        bits = getattr(p, w + "_bits")
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(getattr(p, w)).to(dev)

    rp, ci, block = p.row_ptr, p.col_idx, p.block
    if element and rp is not None and block != 1:
        rp, ci = p.element_csr()
        rp, ci, block = rp.astype(np.int32), ci.astype(np.int32), 1
    t = dict(q=qkv("q"), k=qkv("k"), v=qkv("v"),
             row_ptr=None if rp is None else torch.from_numpy(rp).to(dev),
             col_idx=None if ci is None else torch.from_numpy(ci).to(dev),
             bias=None if p.bias is None else torch.from_numpy(p.bias).to(dev),
             key_mask=None if p.key_mask is None else torch.from_numpy(p.key_mask).to(dev))
    nnz = 0 if rp is None else int(rp[-1])
    prob = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16 if p.dtype == "bf16" else sa.SA_F32,
                      t["row_ptr"], t["col_idx"], nnz, block=block, scale=p.scale,
                      bias=t["bias"], key_mask=t["key_mask"], key_mask_heads=p.key_mask_heads)
    return prob, t, nnz


class EventTimer:
    """Per-kernel HIP events on the current stream; durations summed per name."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def add(self, name, a, b, reps=1):
        """Events a, b bracket `reps` back-to-back launches of one kernel."""
        self.pending.append((name, a, b, reps))

    def result(self):
        self.torch.cuda.synchronize()
        out = {}
        for name, a, b, reps in self.pending:
            out.setdefault(name, []).append(a.elapsed_time(b) * 1e3 / reps)  # us per launch
        return {k: float(np.mean(v)) for k, v in out.items()}


# ------------------------------------------------------------------------------ algorithmic bytes

def bytes_pipeline(BH, n, d, nnz, elem):
    """Unique bytes each kernel must move (every gathered K/V row counted once)."""
    qkv = BH * n * d * elem
    csr = 4 * (n + 1) + 4 * nnz
    return {
        "plan": 4 * (n + 1) + 16 * (n + nnz // 512 + 1),
        "sddmm": 2 * qkv + csr + 4 * BH * nnz,
        "softmax": 4 * (n + 1) + 8 * BH * nnz,
        "spmm": 4 * BH * nnz + csr + qkv + 4 * BH * n * d,
    }


def bytes_fused(p, nnz_blocks=None):
    qkv = p.BH * p.n * p.d * (2 if p.dtype == "bf16" else 4)
    b = 3 * qkv + 4 * p.BH * p.n * p.d + 4 * p.BH * p.n  # q, k, v, out, lse
    if p.row_ptr is not None:
        b += 4 * len(p.row_ptr) + 4 * len(p.col_idx)
    if p.bias is not None:
        b += p.bias.nbytes
    if p.key_mask is not None:
        b += p.key_mask.nbytes
    return b


# ------------------------------------------------------------------------------ measurements

def run_pipeline_steps(torch, sa, prob, t, nnz, BH, n, d, steps, warmup, timer):
    """Build the row plan once (it depends on the mask only), then run `steps` passes of
    SDDMM -> sparse softmax -> SpMM launched one call at a time (the eager rate), time each
    kernel over `steps` back-to-back launches between HIP events (per-kernel durations), then
    run the steps again from a HIP graph of several steps (the step rate).
    Returns (wall seconds of the graph-launched steps, wall seconds of the eager steps,
    plan build us, steps per graph)."""
    scores = torch.empty(BH * nnz, device="cuda:0")
    weights = torch.empty_like(scores)
    out = torch.empty(BH, n, d, device="cuda:0")
    plan = torch.zeros(sa.sa_plan_bytes(prob) // 4 + 1, dtype=torch.int32, device="cuda:0")
    pt = EventTimer(torch)
    a = pt.mark()
    sa.sa_plan_build(prob, plan)
    b = pt.mark()
    pt.add("plan", a, b)
    plan_us = pt.result()["plan"]
    prob.set_plan(plan)

    calls = {"sddmm": lambda: sa.sa_sddmm(prob, t["q"], t["k"], scores),
             "softmax": lambda: sa.sa_sparse_softmax(prob, scores, weights),
             "spmm": lambda: sa.sa_spmm(prob, weights, t["v"], out)}

    def step(_=None):
        for f in calls.values():
            f()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    # per-kernel durations: each call `steps` times back to back between two HIP events on the
    # stream the kernels run on (the inputs are the pipeline's own: the step above left them),
    # so the launch gaps between calls stay hidden, as in a kernel trace
    for name, f in calls.items() if timer is not None else ():
        a = timer.mark()
        for _ in range(steps):
            f()
        b = timer.mark()
        timer.add(name, a, b, steps)

    # the same calls captured as a HIP graph of `chunk` steps (the kernels allocate nothing and
    # take no host decision after the plan is built; chunk is the largest divisor of `steps`
    # up to 10, so the replays run exactly `steps` steps), replayed steps / chunk times
    chunk = max(c for c in range(1, min(steps, 10) + 1) if steps % c == 0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(chunk):
            step()
    for _ in range(max(1, warmup // chunk)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // chunk):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, eager_wall, plan_us, chunk


def run_concurrent_steps(torch, sa, p, steps, warmup, streams):
    """`steps` pipeline steps split evenly over `streams` independent batches, each with its
    own copy of the inputs, its own plan and outputs, captured as a HIP graph of `chunk` steps
    on its own stream (default priority); the graphs are replayed round-robin so the streams'
    kernels overlap. Returns (wall seconds of all `steps` steps, steps per graph)."""
    per = steps // streams
    chunk = max(c for c in range(1, min(per, 10) + 1) if per % c == 0)
    lanes = []
    for _ in range(streams):
        prob, t, nnz = to_device(p, torch, sa)
        plan = torch.zeros(sa.sa_plan_bytes(prob) // 4 + 1, dtype=torch.int32, device="cuda:0")
        sa.sa_plan_build(prob, plan)
        prob.set_plan(plan)
        S = torch.empty(p.BH * nnz, device="cuda:0")
        W = torch.empty_like(S)
        O = torch.empty(p.BH, p.n, p.d, device="cuda:0")

        def step(prob=prob, t=t, S=S, W=W, O=O):
            sa.sa_sddmm(prob, t["q"], t["k"], S)
            sa.sa_sparse_softmax(prob, S, W)
            sa.sa_spmm(prob, W, t["v"], O)

        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(chunk):
                step()
        lanes.append((graph, torch.cuda.Stream(), (prob, t, plan, S, W, O)))

    def replay_all(rounds):
        for _ in range(rounds):
            for graph, stream, _ in lanes:
                with torch.cuda.stream(stream):
                    graph.replay()

    replay_all(max(1, warmup // chunk))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    replay_all(per // chunk)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, chunk


def run_backward_steps(torch, sa, prob, t, nnz, BH, n, d, steps, warmup, timer):
    """The backward pass of the CSR pipeline for an upstream gradient dO (bf16, N(0,1)):
    dW = SDDMM(dO, V) at scale 1, dS = softmax gradient (times the scale), dQ = SpMM(dS, K),
    dS and W gathered together into the transposed pattern's order (block read order),
    dK = SpMM^T(dS, Q), dV = SpMM^T(W, dO). The transposed pattern, its gather order and
    both row plans are built once per mask before timing; the forward weights come from one
    forward pass. Returns the wall seconds of `steps` eager backward steps; with a timer,
    each call is then also timed over `steps` back-to-back launches."""
    dtype = prob.c.dtype
    plan = torch.zeros(sa.sa_plan_bytes(prob) // 4 + 1, dtype=torch.int32, device="cuda:0")
    sa.sa_plan_build(prob, plan)
    prob.set_plan(plan)
    rpt = torch.empty(n + 1, dtype=torch.int32, device="cuda:0")
    cit = torch.empty(nnz, dtype=torch.int32, device="cuda:0")
    perm = torch.empty(nnz, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(sa.sa_transpose_workspace_bytes(prob), dtype=torch.uint8, device="cuda:0")
    sa.sa_csr_transpose(prob, rpt, cit, perm, ws)
    order = torch.empty(2 * nnz, dtype=torch.int32, device="cuda:0")
    sa.sa_gather_order_build(prob, perm, order, ws)
    del ws
    c = prob.c
    prob_dw = sa.Problem(c.B, c.H, n, d, dtype, t["row_ptr"], t["col_idx"], nnz, scale=1.0)
    prob_t = sa.Problem(c.B, c.H, n, d, dtype, rpt, cit, nnz, scale=c.scale)
    keep = []
    for pr in (prob_dw, prob_t):
        buf = torch.zeros(sa.sa_plan_bytes(pr) // 4 + 1, dtype=torch.int32, device="cuda:0")
        sa.sa_plan_build(pr, buf)
        pr.set_plan(buf)
        keep.append(buf)
    g = torch.Generator(device="cpu").manual_seed(77)
    dO = torch.randn(BH, n, d, generator=g).to("cuda:0", t["q"].dtype)
    S = torch.empty(BH * nnz, device="cuda:0")
    W = torch.empty_like(S)
    sa.sa_sddmm(prob, t["q"], t["k"], S)
    sa.sa_sparse_softmax(prob, S, W)
    dW, dS, Wt, dSt = (torch.empty_like(S) for _ in range(4))
    dQ, dK, dV = (torch.empty(BH, n, d, device="cuda:0") for _ in range(3))
    calls = {"sddmm_dO_V": lambda: sa.sa_sddmm(prob_dw, dO, t["v"], dW),
             "softmax_backward": lambda: sa.sa_sparse_softmax_backward(prob, W, dW, c.scale, dS),
             "spmm_dS_K": lambda: sa.sa_spmm(prob, dS, t["k"], dQ),
             "gather_dS_W": lambda: sa.sa_gather_entries_ordered(prob, order, dS, dSt, W, Wt),
             "spmmT_dS_Q": lambda: sa.sa_spmm(prob_t, dSt, t["q"], dK),
             "spmmT_W_dO": lambda: sa.sa_spmm(prob_t, Wt, dO, dV)}

    def step():
        for f in calls.values():
            f()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for name, f in calls.items() if timer is not None else ():
        a = timer.mark()
        for _ in range(steps):
            f()
        b = timer.mark()
        timer.add(name, a, b, steps)
    del keep
    return wall


def bytes_backward(BH, n, d, nnz, elem):
    """Unique bytes of each backward call (as bytes_pipeline: gathered rows counted once)."""
    qkv = BH * n * d * elem
    csr = 4 * (n + 1) + 4 * nnz
    e4 = 4 * BH * nnz
    spmm = e4 + csr + qkv + 4 * BH * n * d
    return {"sddmm_dO_V": 2 * qkv + csr + e4, "softmax_backward": 4 * (n + 1) + 3 * e4,
            "spmm_dS_K": spmm, "gather_dS_W": 4 * e4 + 8 * nnz,
            "spmmT_dS_Q": spmm, "spmmT_W_dO": spmm}


def _avg_us(torch, f, iters=10, warmup=2):
    """Average HIP-event time of f over `iters` back-to-back calls on the current stream."""
    for _ in range(warmup):
        f()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(iters):
        f()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / iters


def time_mask_construction(torch, sa, p):
    """Mask construction on the device: the workload's pattern given as shuffled COO pairs
    (COO -> CSR), a packed batch of 8 sequences of 4096 tokens in all (both varlen calls),
    key masks from 32 key lengths of 384 keys, a top-256-per-row mask from a 4096 x 4096
    score matrix, and the fused dense kernel on evoformer_l384
    with its key padding given as the mask vector, as per-batch key lengths, and absent."""
    import gen
    dev = "cuda:0"
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    order = np.random.default_rng(5).permutation(len(rows))
    R = torch.from_numpy(rows[order].astype(np.int32)).to(dev)
    C = torch.from_numpy(p.col_idx[order].astype(np.int32)).to(dev)
    rp = torch.empty(p.n + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(len(rows), dtype=torch.int32, device=dev)
    counts = torch.empty(3, dtype=torch.int32, device=dev)
    ws = torch.empty(sa.sa_mask_workspace_bytes(p.n, len(rows)), dtype=torch.uint8, device=dev)
    coo_us = _avg_us(torch, lambda: sa.sa_coo_to_csr(p.n, R, C, rp, ci, counts, ws))
    lens = np.random.default_rng(6).multinomial(4096 - 8, [1 / 8] * 8) + 1
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    vrp = torch.empty(4097, dtype=torch.int32, device=dev)
    vws = torch.empty(sa.sa_mask_workspace_bytes(4096, 0), dtype=torch.uint8, device=dev)
    sa.sa_varlen_row_ptr(8, 4096, cu, -1, vrp, vws)
    vnnz = int(vrp[-1].item())
    vci = torch.empty(vnnz, dtype=torch.int32, device=dev)
    varlen_us = _avg_us(torch, lambda: (sa.sa_varlen_row_ptr(8, 4096, cu, -1, vrp, vws),
                                        sa.sa_varlen_col_idx(8, 4096, cu, -1, vrp, vci)))
    seqlen = torch.from_numpy(np.random.default_rng(7).integers(320, 385, 32).astype(np.int32)).to(dev)
    km = torch.empty(32, 384, device=dev)
    km_us = _avg_us(torch, lambda: sa.sa_key_mask_from_lengths(32, 384, seqlen, km))
    # a mask generated at run time: the 256 largest of every row of a 4096 x 4096 score matrix
    # (q.k of one head of the workload)
    qh, kh = torch.from_numpy(p.q[0]).to(dev), torch.from_numpy(p.k[0]).to(dev)
    Sk = (qh @ kh.T).contiguous()
    trp = torch.empty(p.n + 1, dtype=torch.int32, device=dev)
    tci = torch.empty(p.n * 256, dtype=torch.int32, device=dev)
    topk_us = _avg_us(torch, lambda: sa.sa_topk_mask(p.n, 256, Sk, trp, tci))
    del Sk, qh, kh
    evo = gen.make("evoformer_l384")
    with_mask = time_fused(torch, sa, evo)
    without = time_fused(torch, sa, dataclasses.replace(evo, key_mask=None))
    evo_lens = np.isfinite(evo.key_mask[:, 0, :]).sum(axis=1)  # the same padding as lengths
    with_lens = time_fused(torch, sa, dataclasses.replace(evo, key_mask=None), seqlen_k=evo_lens)
    return {"coo_to_csr_" + p.name: {"pairs": len(rows), "us": round(coo_us, 2),
                                     "pairs_per_s": len(rows) / (coo_us * 1e-6)},
            "varlen_8_sequences_4096_tokens": {"nnz": vnnz, "us": round(varlen_us, 2),
                                               "entries_per_s": vnnz / (varlen_us * 1e-6)},
            "key_mask_from_lengths_32x384": {"us": round(km_us, 2)},
            "topk_mask_4096_k256": {"us": round(topk_us, 2), "scores_read_GB_s": round(p.n * p.n * 4 / (topk_us * 1e-6) / 1e9, 1)},
            "fused_evoformer_l384_key_padding": {"key_mask_vector_us": round(with_mask, 2),
                                                 "seqlen_k_us": round(with_lens, 2),
                                                 "no_padding_us": round(without, 2)}}


def time_fused(torch, sa, p, iters=20, warmup=3, element=False, seqlen_k=None):
    """Average HIP-event time of one fused forward over `iters` back-to-back launches; an
    element CSR gets its row plan first (built once per mask, as for the pipeline).
    seqlen_k: optional per-batch key lengths (host ints) read by the kernel."""
    prob, t, nnz = to_device(p, torch, sa, element=element)
    if seqlen_k is not None:
        t["seqlen_k"] = torch.tensor(np.asarray(seqlen_k, np.int32), device="cuda:0")
        prob.c.seqlen_k = t["seqlen_k"].data_ptr()
    if prob.c.row_ptr and prob.c.block == 1:
        t["plan"] = torch.zeros(sa.sa_plan_bytes(prob) // 4 + 1, dtype=torch.int32, device="cuda:0")
        sa.sa_plan_build(prob, t["plan"])
        prob.set_plan(t["plan"])
    out = torch.empty(p.BH, p.n, p.d, device="cuda:0")
    lse = torch.empty(p.BH, p.n, device="cuda:0")
    for _ in range(warmup):
        sa.sa_fused_forward(prob, t["q"], t["k"], t["v"], out, lse)
    tm = EventTimer(torch)
    a = tm.mark()
    for _ in range(iters):
        sa.sa_fused_forward(prob, t["q"], t["k"], t["v"], out, lse)
    b = tm.mark()
    tm.add("fused", a, b, iters)
    us = tm.result()["fused"]
    del t, out, lse
    return us


def time_fused_backward(torch, sa, p, iters=20, warmup=3, with_dscores=False):
    """Average HIP-event time of sa_fused_backward (dense or block CSR) over `iters`
    back-to-back calls, from one forward's O and lse and a N(0,1) bf16 upstream gradient."""
    prob, t, _ = to_device(p, torch, sa, element=False)
    dev = "cuda:0"
    shape = (p.BH, p.n, p.d)
    rpt = cit = None
    if p.row_ptr is not None:  # block CSR: the transposed block pattern, built once per mask
        nb = (p.n + 63) // 64
        bprob = sa.Problem(1, 1, nb, 32, sa.SA_BF16, t["row_ptr"], t["col_idx"], p.nnz)
        rpt = torch.empty(nb + 1, dtype=torch.int32, device=dev)
        cit = torch.empty(p.nnz, dtype=torch.int32, device=dev)
        perm = torch.empty_like(cit)
        ws0 = torch.empty(sa.sa_transpose_workspace_bytes(bprob), dtype=torch.uint8, device=dev)
        sa.sa_csr_transpose(bprob, rpt, cit, perm, ws0)
        del perm, ws0
    out = torch.empty(shape, device=dev)
    lse = torch.empty(p.BH, p.n, device=dev)
    sa.sa_fused_forward(prob, t["q"], t["k"], t["v"], out, lse)
    g = torch.Generator(device="cpu").manual_seed(78)
    dO = torch.randn(shape, generator=g).to(dev, torch.bfloat16)
    dq, dk, dv = (torch.empty(shape, device=dev) for _ in range(3))
    ws = torch.empty(p.BH * p.n, device=dev)
    ds = torch.empty(p.BH, p.n, p.n, device=dev) if with_dscores else None
    call = lambda: sa.sa_fused_backward(prob, t["q"], t["k"], t["v"], out, lse, dO, dq, dk, dv, ws,
                                        dscores=ds, t_row_ptr=rpt, t_col_idx=cit)
    us = _avg_us(torch, call, iters=iters, warmup=warmup)
    del t, out, lse, dO, dq, dk, dv, ws, ds
    return us


def time_fused_backward_cover(torch, sa, p, iters=20, warmup=3):
    """Element CSR: HIP-event time of building the block cover once (four calls, one
    read-back) and the average of `iters` back-to-back sa_fused_backward_cover calls."""
    prob, t, _ = to_device(p, torch, sa)
    dev = "cuda:0"
    shape = (p.BH, p.n, p.d)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    cover = sa.block_cover(prob, device=dev)
    b.record()
    torch.cuda.synchronize()
    build_us = a.elapsed_time(b) * 1000
    out = torch.empty(shape, device=dev)
    lse = torch.empty(p.BH, p.n, device=dev)
    sa.sa_fused_forward(prob, t["q"], t["k"], t["v"], out, lse)
    g = torch.Generator(device="cpu").manual_seed(79)
    dO = torch.randn(shape, generator=g).to(dev, torch.bfloat16)
    dq, dk, dv = (torch.empty(shape, device=dev) for _ in range(3))
    ws = torch.empty(p.BH * p.n, device=dev)
    call = lambda: sa.sa_fused_backward_cover(prob, cover, t["q"], t["k"], t["v"], out, lse, dO, dq, dk,
                                              dv, ws)
    us = _avg_us(torch, call, iters=iters, warmup=warmup)
    nblk = cover.nnz
    del t, out, lse, dO, dq, dk, dv, ws, cover
    return us, build_us, nblk


def cpu_baseline(p, budget_s):
    """The fp64 dense oracle (definition with -inf outside the mask), timed on whole heads
    until the budget is used; returns attended pairs/s on the host cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    pattern = ("csr", p.row_ptr, p.col_idx)
    done, t0 = 0, time.perf_counter()
    while done < p.BH:
        oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, pattern, heads=[done])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    pairs = done * p.nnz
    return {"value": pairs / dt, "unit": "pairs/s",
            "cores": blas_threads if blas_threads else len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{done} of {p.BH} heads of {p.name} (all rows of each), dense fp64 "
                      f"oracle with -inf outside the mask; {dt:.1f} s; exp and masking on one "
                      f"thread, GEMMs on {blas_threads} BLAS threads; "
                      f"{len(os.sched_getaffinity(0))} cores in the affinity mask"}


def load_traffic(kernel, src_hash):
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tr.get(kernel)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


def profile_only(args, torch, sa, gen):
    """Run one kernel family alone so that a profiler sees only its launches. "copy" is a
    plain device-to-device copy of 256 MiB, the reference for scaling the HBM byte counters."""
    if args.profile == "copy":
        src = torch.ones(COPY_BYTES // 4, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
    elif args.profile == "pipeline":
        p = gen.make(args.workload)
        prob, t, nnz = to_device(p, torch, sa)
        run_pipeline_steps(torch, sa, prob, t, nnz, p.BH, p.n, p.d, args.steps, args.warmup, None)
    elif args.profile == "backward":
        p = gen.make(args.workload)
        prob, t, nnz = to_device(p, torch, sa)
        run_backward_steps(torch, sa, prob, t, nnz, p.BH, p.n, p.d, args.steps, args.warmup, None)
    elif args.profile == "fused_backward":
        q = gen.make("evoformer_l384")
        us = time_fused_backward(torch, sa, q, iters=args.steps, warmup=args.warmup)
        log(f"fused_backward evoformer_l384: {us:.1f} us")
    elif args.profile == "fused_backward_cover":
        q = gen.make(args.workload)
        us, _, _ = time_fused_backward_cover(torch, sa, q, iters=args.steps, warmup=args.warmup)
        log(f"fused_backward_cover {args.workload}: {us:.1f} us")
    else:
        name = {"fused_csr": args.workload, "fused_bsr": "bsr_n16384",
                "fused_dense": "evoformer_l384"}[args.profile]
        q = gen.make(name)
        us = time_fused(torch, sa, q, iters=args.steps, warmup=args.warmup)
        log(f"{args.profile} {name}: {us:.1f} us")
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch

    import gen
    if not os.path.exists(os.path.join(ROOT, "masked_scaled_dot_amd", "libsa.so")):
        import __graft_entry__
        __graft_entry__.build()
    import masked_scaled_dot_amd as sa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile:
        return profile_only(args, torch, sa, gen)
    p = gen.make(args.workload)
    BH, n, d = p.BH, p.n, p.d
    prob, t, nnz = to_device(p, torch, sa)
    pairs = BH * nnz
    log(f"workload {p.name}: BH={BH} n={n} d={d} nnz/head={nnz} pairs/step={pairs}")

    timer = EventTimer(torch)
    wall, eager_wall, plan_us, chunk = run_pipeline_steps(torch, sa, prob, t, nnz, BH, n, d,
                                                          args.steps, args.warmup, timer)
    kern_us = timer.result()
    single_ms = wall * 1e3 / args.steps
    streams = args.streams if args.streams > 1 and args.steps % args.streams == 0 else 1
    if streams > 1:
        cwall, cchunk = run_concurrent_steps(torch, sa, p, args.steps, args.warmup, streams)
        launch = (f"{streams} streams, each a HIP graph of {cchunk} steps on its own inputs, plan "
                  f"and outputs, {args.steps // streams} steps per stream, replayed concurrently")
    else:
        cwall = wall
        launch = f"one stream: a HIP graph of {chunk} steps, replayed {args.steps // chunk} times"
    ms_per_step = cwall * 1e3 / args.steps
    value = pairs / (cwall / args.steps)
    log(f"pipeline: {ms_per_step * 1e3:.1f} us/step ({streams} streams), {single_ms * 1e3:.1f} us/step "
        f"(one stream, graph of {chunk} steps), {eager_wall * 1e6 / args.steps:.1f} us/step (eager)  " +
        "  ".join(f"{k}={v:.1f}us" for k, v in kern_us.items()))

    algo = bytes_pipeline(BH, n, d, nnz, 2 if p.dtype == "bf16" else 4)
    kernels = {"plan_build_once": {"us": round(plan_us, 2), "algo_bytes": algo["plan"],
                                   "note": "built once per mask, outside the timed step"}}
    for k, us in kern_us.items():
        gbs = algo[k] / (us * 1e-6) / 1e9
        kernels[k] = {"us": round(us, 2), "algo_bytes": algo[k], "GB_s": round(gbs, 1),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    total_bytes = sum(algo[k] for k in ("sddmm", "softmax", "spmm"))
    total_us = sum(kern_us[k] for k in ("sddmm", "softmax", "spmm"))
    dominant = max(("sddmm", "softmax", "spmm"), key=lambda k: kern_us[k])
    src_of = {"sddmm": ["sddmm.hip", "common.h", "tile.h", "plan_layout.h"],
              "softmax": ["softmax.hip", "common.h"],
              "spmm": ["spmm.hip", "common.h", "tile.h", "plan_layout.h"]}
    dom_hash = source_hash(src_of[dominant])
    achieved = algo[dominant] / (kern_us[dominant] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(dominant, dom_hash),
                "algo_bytes_per_launch": algo[dominant], "avg_launch_us": round(kern_us[dominant], 2),
                "source_hash": dom_hash,
                "pipeline_aggregate_frac": round(total_bytes / (total_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    extra = {}
    if not args.no_extra:
        fused_us = time_fused(torch, sa, p)
        flops = 4.0 * pairs * d
        extra["fused_csr_" + p.name] = {
            "us": round(fused_us, 2), "pairs_per_s": pairs / (fused_us * 1e-6),
            "TFLOP_s": round(flops / (fused_us * 1e-6) / 1e12, 2),
            # the tiles of this workload run on the matrix cores (bf16); the vector-ALU
            # fraction is the bound for tiles that take the vector path
            "mfma_frac": round(flops / (fused_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "valu_frac": round(flops / (fused_us * 1e-6) / 1e12 / VALU_FP32_PEAK_TFLOPS, 4),
            "hbm_frac": round(bytes_fused(p) / (fused_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del t
        # the backward pass of the CSR pipeline on the main workload
        bprob, bt, _ = to_device(p, torch, sa)
        btimer = EventTimer(torch)
        bwall = run_backward_steps(torch, sa, bprob, bt, nnz, BH, n, d, 20, 3, btimer)
        bk = btimer.result()
        balgo = bytes_backward(BH, n, d, nnz, 2 if p.dtype == "bf16" else 4)
        extra["backward_" + p.name] = {
            "us_per_step_eager": round(bwall * 1e6 / 20, 2), "pairs_per_s": pairs / (bwall / 20),
            "kernels_us": {k: round(v, 2) for k, v in bk.items()},
            "hbm_frac": {k: round(balgo[k] / (v * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for k, v in bk.items()},
            "aggregate_hbm_frac": round(sum(balgo.values()) / (sum(bk.values()) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"backward {p.name}: {bwall * 1e6 / 20:.1f} us/step (eager) " +
            "  ".join(f"{k}={v:.1f}us" for k, v in bk.items()))
        del bt, bprob
        # the random-row workload (rows of 32-512 random columns): every tile takes the
        # vector path, whose key/value row gathers bound it
        rq = gen.make("random_n8192")
        rprob, rt, rnnz = to_device(rq, torch, sa)
        rtimer = EventTimer(torch)
        _, reager, _, _ = run_pipeline_steps(torch, sa, rprob, rt, rnnz, rq.BH, rq.n, rq.d, 10, 2, rtimer)
        rk = rtimer.result()
        ralgo = bytes_pipeline(rq.BH, rq.n, rq.d, rnnz, 2)
        rpairs = rq.BH * rnnz
        extra["pipeline_" + rq.name] = {
            "us_per_step_eager": round(reager * 1e6 / 10, 2), "pairs_per_s": rpairs / (reager / 10),
            "kernels_us": {k: round(v, 2) for k, v in rk.items()},
            "hbm_frac": {k: round(ralgo[k] / (v * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for k, v in rk.items()}}
        fr = time_fused(torch, sa, rq)
        extra["fused_csr_" + rq.name] = {
            "us": round(fr, 2), "pairs_per_s": rpairs / (fr * 1e-6),
            "TFLOP_s": round(4.0 * rpairs * rq.d / (fr * 1e-6) / 1e12, 2),
            "hbm_frac": round(bytes_fused(rq) / (fr * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"random_n8192: pipeline {reager * 1e6 / 10:.1f} us/step (eager) " +
            "  ".join(f"{k}={v:.1f}us" for k, v in rk.items()) + f", fused {fr:.1f} us")
        del rt, rprob
        for name in ("bsr_n16384", "evoformer_l384"):
            q = gen.make(name)
            us = time_fused(torch, sa, q)
            pr = q.attended_pairs() if q.row_ptr is None else q.BH * int(q.element_csr()[0][-1])
            flops = 4.0 * pr * q.d
            extra["fused_" + name] = {
                "us": round(us, 2), "pairs_per_s": pr / (us * 1e-6),
                "TFLOP_s": round(flops / (us * 1e-6) / 1e12, 2),
                "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "hbm_frac": round(bytes_fused(q) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "warm": True}
            log(f"fused {name}: {us:.1f} us")
            # the backward of the fused forward (dS written out too for the dense pattern,
            # where it is [B*H, n, n]: the bias gradient's input)
            bus = time_fused_backward(torch, sa, q)
            bflops = 10.0 * pr * q.d  # S again, dP, dV, dK, dQ: five products of 2 pairs d
            row = {"us": round(bus, 2), "TFLOP_s": round(bflops / (bus * 1e-6) / 1e12, 2),
                   "mfma_frac": round(bflops / (bus * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                   "flops_model": "10 * attended pairs * d (five products of 2 * pairs * d)"}
            if q.row_ptr is None:
                row["us_with_dscores"] = round(time_fused_backward(torch, sa, q, with_dscores=True), 2)
            extra["fused_backward_" + name] = row
            log(f"fused backward {name}: {bus:.1f} us")
            del q

        # the backward of the fused element-CSR forward, on the pattern's 64x64 block cover
        bus, build_us, nblk = time_fused_backward_cover(torch, sa, p)
        pr = p.BH * p.nnz
        bflops = 10.0 * pr * p.d
        extra["fused_backward_cover_" + args.workload] = {
            "us": round(bus, 2), "TFLOP_s": round(bflops / (bus * 1e-6) / 1e12, 2),
            "mfma_frac": round(bflops / (bus * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_model": "10 * attended pairs * d", "cover_blocks_per_head": nblk,
            "computed_pairs_per_head": nblk * 64 * 64, "cover_build_us_once": round(build_us, 1)}
        log(f"fused backward over the block cover {args.workload}: {bus:.1f} us "
            f"({nblk} blocks per head; cover built once in {build_us:.0f} us)")

        mc = time_mask_construction(torch, sa, p)
        extra["mask_construction"] = mc
        log("mask construction: " + ", ".join(f"{k} {v.get('us', v)}" for k, v in mc.items()))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.3e} pairs/s ({cpu['sample']})")

    line = {
        "metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": {"workload": p.name, "B": p.B, "H": p.H, "n": n, "d": d, "nnz_per_head": nnz,
                   "pairs_per_step": pairs,
                   "step": "sddmm + sparse_softmax + spmm (scores, weights, context); the row plan "
                           "is built once per mask before timing",
                   "launch": launch, "streams": streams,
                   "single_stream_ms_per_step": round(single_ms, 5),
                   "eager_ms_per_step": round(eager_wall * 1e3 / args.steps, 5),
                   "inputs": "resident in HBM; caches not flushed between steps"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
