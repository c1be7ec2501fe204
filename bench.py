#!/usr/bin/env python3
"""Throughput of one MoE speculative verification step on one MI355X.

A step is one call of moe_verify_step: B sequences x (K+1) positions through
L MoE blocks (RMSNorm, top-6-of-64 router, 6 routed + 2 shared SwiGLU
experts, combine, residual), the final norm, the LM head with greedy arg-max
and the longest-prefix acceptance.  The headline is verified tokens per
second (B*(K+1) tokens per step); the dominant kernel is reported against the
HBM roofline, and the CPU oracle is timed on a bounded sample beside it.

Inputs are seeded synthetic data shaped like the pages' workloads (random
N(0, 0.02^2) weights, N(0,1) hidden states); they are resident in HBM before
the timed region.  Several independent weight copies are rotated so that no
weight byte of a step is served by the 256 MB last-level cache from an earlier
step.

The draft-head workloads (draft_b1, draft_b32, draft_b1_head32k) time one
moe_draft_step instead: K recursive applications of the dense draft block
for B sequences, reported as draft tokens per second (B*K per call) with the
draft's LM-head kernel against the HBM roofline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "verified tokens/s per MoE verify step (B×4 tokens); % HBM or MFMA peak"
DRAFT_METRIC = "draft tokens/s per draft call (B×K tokens, K recursive dense-block steps); % HBM peak"
EVERY = 8
EXPERT_BYTES = None  # filled per workload


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- HIP events

class HipEvents:
    """hipEvent_t handles through the HIP runtime torch has already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def record(self, ev: int, stream: int):
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, ev: int):
        self.hip.hipEventDestroy(ev)


# ---------------------------------------------------------- algorithmic work

def expert_bytes(w) -> int:
    return 3 * w.I * w.H * 2


def step_bytes(w, touched_per_layer) -> int:
    """Bytes the step must move: touched experts' weights, shared experts,
    router, activations in/out per block, LM head."""
    per = []
    for n in touched_per_layer:
        per.append(n * expert_bytes(w) + w.S * expert_bytes(w) + w.E * w.H * 2 + 2 * w.T * w.H * 2)
    lm = w.V * w.H * 2 if w.has_lm_head else 0
    return int(sum(per) + lm)


def attn_kv_bytes(w, positions) -> int:
    """Keys and values the step's queries read: per sequence and head the
    cache rows 0..p_b+K (256 B each for keys and for values)."""
    return int(sum(w.n_heads * (int(p) + w.K + 1) * 512 for p in positions))


def attn_step_bytes(w, positions) -> int:
    """Attention's share of a step: per layer the four projections, the cache
    rows read, the step's own keys and values written."""
    if not w.n_heads:
        return 0
    return w.L * (4 * w.H * w.H * 2 + attn_kv_bytes(w, positions) + w.T * w.n_heads * 512)


def step_flops(w) -> int:
    f = w.L * (w.T * (w.k + w.S) * 6 * w.H * w.I + 2 * w.T * w.E * w.H)
    if w.has_lm_head:
        f += 2 * w.T * w.H * w.V
    return int(f)


def lmhead_bytes(w) -> int:
    # weights once + final-norm activations in + one 8-byte key per token
    return w.V * w.H * 2 + w.T * w.H * 2 + w.T * 8


def draft_head_bytes(H, Vd, B) -> int:
    # head rows once + head-input rows in + one 8-byte key per row
    return Vd * H * 2 + B * H * 2 + B * 8


def draft_call_bytes(H, Id, Vd, B, K) -> int:
    """Bytes one draft call must move: per step the projection (2H x H), the
    dense SwiGLU (3 x Id x H) and the head rows, plus the rows it reads and
    writes (state and embedding rows, the drafts)."""
    per_step = 2 * H * H * 2 + 3 * Id * H * 2 + draft_head_bytes(H, Vd, B) + 2 * B * H * 2
    return K * per_step + B * H * 2 + B * K * 4


def draft_call_flops(H, Id, Vd, B, K) -> int:
    return K * B * 2 * (2 * H * H + 3 * Id * H + Vd * H)


# ------------------------------------------------------------ counter file

def kernel_source_hash(name: str) -> str:
    p = os.path.join(ROOT, "moe_decoder_speculative_amd", "csrc", name)
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "moe_decoder_speculative_amd", "csrc", "common.h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_file: str, workload: str):
    """HBM bytes per launch from committed counter summaries, or None when
    absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    return ent.get("bytes_per_launch")


# ---------------------------------------------------------------- CPU leg

def cpu_baseline(w, weights, hidden_np, drafts_np, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    import oracle
    shp = oracle.Shape(H=w.H, E=w.E, k=w.k, S=w.S, I=w.I, V=w.V, L=w.L, eps=w.eps, dtype=w.dtype)
    # sample: whole steps when small, else one sequence (K+1 tokens) per call
    if w.has_lm_head and w.n_heads:
        from oracle import attn_oracle as A
        from moe_decoder_speculative_amd import synth
        K = w.K
        ash = A.AttnShape(H=w.H, n_heads=w.n_heads, d_head=128, P=w.P, theta=w.rope_theta, eps=w.eps,
                          dtype=w.dtype)
        pos = synth.kv_positions(w)[:1]
        caches = []
        for l in range(w.L):
            k, v = synth.kv_prefix(w, l, 0, int(pos[0]))
            kc = np.zeros((1, w.n_heads, w.P, 128), np.float32)
            vc = np.zeros_like(kc)
            kc[0, :, :pos[0]] = oracle.as_f32(k)
            vc[0, :, :pos[0]] = oracle.as_f32(v)
            caches.append((kc, vc))
        h = hidden_np[: K + 1]
        d = drafts_np[:1]
        what = f"1 sequence x {K + 1} positions over a {int(pos[0])}-position cache per oracle step"
        tokens_per_call = K + 1

        def call():
            A.verify_step_attn(shp, ash, weights, h, d, pos, caches, 1, K)
    elif w.has_lm_head:
        seqs = w.B if w.T <= 8 else 1
        Bs, K = seqs, w.K
        h = hidden_np[: Bs * (K + 1)]
        d = drafts_np[:Bs]
        what = f"{Bs} sequence(s) x {K + 1} positions per oracle step"
        tokens_per_call = Bs * (K + 1)

        def call():
            oracle.verify_step(shp, weights, h, d, Bs, K)
    else:
        rows = min(w.T, 256)
        h = oracle.as_f32(hidden_np[:rows])
        what = f"{rows} token rows through {w.L} block(s) per oracle call"
        tokens_per_call = rows

        def call():
            x = h
            for l in range(w.L):
                x = oracle.moe_block(x, weights["layers"][l], shp).x_out
    t0 = time.perf_counter()
    n = 0
    while True:
        call()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tok_s = n * tokens_per_call / el
    return {"value": tok_s, "unit": "verified tokens/s" if w.has_lm_head else "tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{n} calls of {what} in {el:.1f} s (numpy float32, BLAS threads {threads})"}


# ---------------------------------------------------------------- decode-loop cost model

def cost_model(args, w0, weights, hidden_np, copies, torch, np, synth, binding, VerifyModel, to_device):
    """Verify-step cost against the number of drafts K, eager launches against
    a HIP-graph replay of the same step.  For each K in 0..3 on the
    workload's B sequences: the step time both ways, the committed tokens per
    sequence expected at per-draft acceptance p (sum of p^i, i = 0..K, the
    accepted prefix plus the bonus), c_K = t_K / t_0 (the verify step's cost in
    one-token steps, K = 0 being plain greedy decoding) and the speed-up over
    greedy decoding S_K = tau_K / c_K (the pages' c = tau / S, page "jina-ocr-v1 :
    Analyse de documents plus rapide sur des GPU a budget limite", section
    "Decodage speculatif sur un L4").

    When a draft workload is defined on this verify workload, the draft call
    of the same batch and shapes (K recursive dense-block steps, continuing
    from the step's own rows and counts) is timed the same two ways, and so is the whole decode-loop
    iteration, verify then draft on one stream: c_loop_K = t_loop_K / t_0 and
    S_loop_K = tau_K / c_loop_K are the figures that compare with the pages'
    (their c includes the draft head).  The drafts of random weights are never
    accepted, so tau_K is the expected count at acceptance p, not this run's."""
    from moe_decoder_speculative_amd.model import DraftModel
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    B = w0.B
    p = w0.accept_p
    model = VerifyModel(w0, weights, max_tokens=B * 4, copies=copies, max_seqs=B)
    positions = None
    if w0.n_heads:  # every copy's caches hold the same prompt rows
        pos_np = synth.kv_positions(w0)
        for l in range(w0.L):
            for b in range(B):
                k, v = synth.kv_prefix(w0, l, b, int(pos_np[b]))
                for c in range(copies):
                    model.kv_write(l, b, k, v, copy=c)
        positions = to_device(pos_np)

    def vstep(hidden, drafts, K, committed, counts, aux=None, c=0):
        if positions is not None:
            model.step_kv(hidden, drafts, positions, B, K, committed, counts, aux, stream=sh, copy=c)
        else:
            model.step(hidden, drafts, B, K, committed, counts, aux, stream=sh, copy=c)

    def vgraph(c, hidden, drafts, K, committed, counts):
        if positions is not None:
            return binding.moe_verify_graph_create_kv(model.ctxs[c], hidden, drafts, positions, B, K, committed,
                                                      counts, sh)
        return binding.moe_verify_graph_create(model.ctxs[c], hidden, drafts, B, K, committed, counts, sh)
    # the draft workload of the same batch and shapes (whole-vocabulary head unless --draft names one)
    dname = args.draft or next((n for n, d in synth.DRAFT_WORKLOADS.items()
                                if d.B == B and d.head_rows == 0 and synth.WORKLOADS[d.base].H == w0.H
                                and synth.WORKLOADS[d.base].V == w0.V), None)
    dms = []
    if dname:
        dwl = synth.DRAFT_WORKLOADS[dname]
        dw = synth.gen_draft_weights(dwl, w0, weights["lm_head"])
        dms = [DraftModel(model, dwl.Id, dw, max_batch=B, k_max=3, copy=c) for c in range(copies)]
        del dw
    ev = HipEvents()
    rows = []
    for K in range(4):
        T = B * (K + 1)
        hidden = to_device(hidden_np[:T])
        committed, counts = model.alloc_outputs(B, K)
        aux = model.alloc_aux(T, with_hidden=False)
        vstep(hidden, to_device(np.zeros((B, K), np.int32)) if K else None, K, committed, counts, aux)
        torch.cuda.synchronize()
        wk = w0.with_(K=K, T=T)
        drafts = to_device(synth.make_drafts(wk, aux["tstar"].cpu().numpy().reshape(B, K + 1))) if K else None
        del aux

        def timed(launch, n):
            for i in range(args.warmup):
                launch(i % copies)
            stream.synchronize()
            a, b = ev.create(), ev.create()
            ev.record(a, sh)
            for i in range(n):
                launch(i % copies)
            ev.record(b, sh)
            stream.synchronize()
            ms = ev.elapsed_ms(a, b) / n
            ev.destroy(a)
            ev.destroy(b)
            return ms * 1e3

        eager_us = timed(lambda c: vstep(hidden, drafts, K, committed, counts, c=c), args.steps)
        graphs = [vgraph(c, hidden, drafts, K, committed, counts) for c in range(copies)]
        try:
            graph_us = timed(lambda c: binding.moe_verify_graph_launch(graphs[c], sh), args.steps)
        finally:
            for g in graphs:
                binding.moe_verify_graph_destroy(g)
        row = {"K": K, "tokens_per_step": T, "eager_us": round(eager_us, 2), "graph_us": round(graph_us, 2),
               "committed_per_seq_expected": round(sum(p ** i for i in range(K + 1)), 4),
               "committed_per_seq_this_input": round(float(counts.sum().item()) / B, 4)}
        if dms and K > 0:
            row["draft_eager_us"] = round(timed(lambda c: dms[c].step(hidden, committed, counts, K + 1, B, K, drafts,
                                                                      stream=sh), args.steps), 2)
            graphs = [vgraph(c, hidden, drafts, K, committed, counts) for c in range(copies)]
            dgraphs = [binding.moe_draft_graph_create(dms[c].ctx, hidden, committed, counts, K + 1, B, K, drafts,
                                                      None, sh) for c in range(copies)]
            try:
                row["draft_graph_us"] = round(timed(lambda c: binding.moe_verify_graph_launch(dgraphs[c], sh),
                                                    args.steps), 2)

                def loop_eager(c):
                    vstep(hidden, drafts, K, committed, counts, c=c)
                    dms[c].step(hidden, committed, counts, K + 1, B, K, drafts, stream=sh)

                def loop_graph(c):
                    binding.moe_verify_graph_launch(graphs[c], sh)
                    binding.moe_verify_graph_launch(dgraphs[c], sh)

                row["loop_eager_us"] = round(timed(loop_eager, args.steps), 2)
                row["loop_graph_us"] = round(timed(loop_graph, args.steps), 2)
            finally:
                for g in graphs + dgraphs:
                    binding.moe_verify_graph_destroy(g)
        elif dms:
            row["loop_eager_us"], row["loop_graph_us"] = row["eager_us"], row["graph_us"]
        rows.append(row)
    for d in dms:
        d.close()
    model.close()
    for r in rows:
        for mode in ("eager", "graph"):
            c = r[f"{mode}_us"] / rows[0][f"{mode}_us"]
            r[f"c_{mode}"] = round(c, 4)
            r[f"S_{mode}"] = round(r["committed_per_seq_expected"] / c, 4)
            if dms:
                cl = r[f"loop_{mode}_us"] / rows[0][f"{mode}_us"]
                r[f"c_loop_{mode}"] = round(cl, 4)
                r[f"S_loop_{mode}"] = round(r["committed_per_seq_expected"] / cl, 4)
    print(json.dumps({"cost_model": {"workload": w0.name, "B": B, "p_accept": p, "weight_copies": copies,
                                     "draft_workload": dname, "steps": args.steps, "rows": rows}}))


# ---------------------------------------------------------------- draft head

def cpu_baseline_draft(dwl, base, dw, hidden_np, committed_np, counts_np, seconds: float):
    """The draft oracle, as it stands, on the same B rows (whole draft calls)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    from oracle import draft_oracle as D
    dshp = D.DraftShape(H=base.H, Id=dwl.Id, V=base.V, Vd=dwl.head_rows or base.V, dtype=base.dtype)
    h0, t0 = D.continue_from_verify(hidden_np, committed_np, counts_np, dwl.R)
    t_start = time.perf_counter()
    n = 0
    while True:
        D.draft_chain(h0, t0, dwl.K, dw, dshp)
        n += 1
        el = time.perf_counter() - t_start
        if el >= seconds:
            break
    return {"value": n * dwl.B * dwl.K / el, "unit": "draft tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} oracle draft calls of {dwl.B} sequence(s) x {dwl.K} steps in {el:.1f} s "
                      f"(numpy float32, BLAS threads {threads})"}


def bench_draft(args, name, torch, np, synth, binding, VerifyModel, to_device):
    from moe_decoder_speculative_amd.model import DraftModel
    dwl = synth.DRAFT_WORKLOADS[name]
    # the verifier context only lends the LM head: one block is enough
    base = synth.WORKLOADS[dwl.base].with_(L=1)
    B, K, H, V = dwl.B, dwl.K, base.H, base.V
    Vd = dwl.head_rows or V
    log(f"draft workload {name}: B={B} K={K} R={dwl.R} H={H} Id={dwl.Id} V={V} head rows={Vd}")
    t = time.time()
    weights = synth.gen_weights(base)
    dw = synth.gen_draft_weights(dwl, base, weights["lm_head"])
    hidden_np, committed_np, counts_np = synth.draft_inputs(dwl, base)
    log(f"generated weights in {time.time() - t:.1f}s")
    cbytes = draft_call_bytes(H, dwl.Id, Vd, B, K)
    # distinct weight bytes one call reads (the head is read once per step,
    # but from the same rows) decide how many copies keep calls out of the LLC
    distinct = 2 * H * H * 2 + 3 * dwl.Id * H * 2 + Vd * H * 2
    copies = args.copies or max(1, math.ceil(1.5e9 / distinct))
    vm = VerifyModel(base, weights, max_tokens=base.T, copies=copies)
    dms = [DraftModel(vm, dwl.Id, dw, max_batch=B, k_max=K, copy=c) for c in range(copies)]
    log(f"{copies} draft/verifier copies")
    hidden = to_device(hidden_np)
    committed = to_device(committed_np)
    counts = to_device(counts_np)
    drafts = torch.empty((B, K), dtype=torch.int32, device="cuda")

    def run(c):
        dms[c].step(hidden, committed, counts, dwl.R, B, K, drafts)

    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        run(i % copies)
    torch.cuda.synchronize()
    n = args.steps
    sampled = list(range(0, n, EVERY))
    before = [ev.create() for _ in sampled]
    after = [ev.create() for _ in sampled]
    g0, g1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(g0, stream)
    for i in range(n):
        c = i % copies
        if i % EVERY == 0:
            binding.moe_draft_set_stage_events(dms[c].ctx, binding.MOE_STAGE_LMHEAD, before[i // EVERY],
                                               after[i // EVERY])
        run(c)
    ev.record(g1, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_call = (t1 - t0) * 1e3 / n
    gpu_ms_call = ev.elapsed_ms(g0, g1) / n
    kern_ms = sorted(ev.elapsed_ms(b, a) for b, a in zip(before, after))
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    for e in before + after + [g0, g1]:
        ev.destroy(e)
    kname = "k_lmhead_stream" if B <= 16 else ("k_lmhead_wide" if B <= 128 else "k_lmhead_mfma")
    kbytes = draft_head_bytes(H, Vd, B)
    achieved = kbytes / (kern_avg_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profiles("k_lmhead.hip", name),
            "kernel": kname, "bytes_per_launch": kbytes, "avg_us": kern_avg_ms * 1e3,
            "median_us": kern_ms[len(kern_ms) // 2] * 1e3, "launches_timed": len(kern_ms)}
    cflops = draft_call_flops(H, dwl.Id, Vd, B, K)
    step = {"gpu_ms_per_call": gpu_ms_call, "algorithmic_bytes": cbytes,
            "hbm_frac": cbytes / (ms_call * 1e-3) / (HBM_PEAK_GBS * 1e9), "flops": cflops,
            "mfma_frac": cflops / (ms_call * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "drafts_first_sequence": drafts[0].cpu().tolist()}
    res = {
        "metric": DRAFT_METRIC,
        "value": B * K / (ms_call * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": ms_call,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "K": K, "rows_per_sequence": dwl.R, "hidden": H,
                   "draft_inter": dwl.Id, "vocab": V, "draft_head_rows": Vd, "weight_copies": copies},
        "roofline": roof,
        "step": step,
    }
    for d in dms:
        d.close()
    vm.close()
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline_draft(dwl, base, dw, hidden_np, committed_np, counts_np,
                                                 args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stack12_b32_zipf",
                    choices=["decode_b1", "decode_b32_zipf", "stack12_b32_zipf", "prefill_8pages",
                             "prefill_8pages_stack12", "stack12_b1", "draft_b1", "draft_b32", "draft_b1_head32k",
                             "attn_b1", "attn_b32_zipf", "attn_stack12_b1", "attn_stack12_b32_zipf"])
    ap.add_argument("--draft", default=None, help="draft workload of the cost model (default: same B, whole head)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for 1.5 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--cost-model", action="store_true",
                    help="only time the verify step for K = 0..3, eager and as a HIP graph (decode workloads)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the verification step runs on a single MI355X "
              "(data parallelism over sequences needs no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from moe_decoder_speculative_amd import synth, binding
    from moe_decoder_speculative_amd.model import VerifyModel, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # a copy kernel of known size: FETCH_SIZE and WRITE_SIZE of one
        # dispatch against 1 GiB give the counters' scale
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "dispatches": 5}))
        return
    if args.workload in synth.DRAFT_WORKLOADS:
        bench_draft(args, args.workload, torch, np, synth, binding, VerifyModel, to_device)
        return
    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} K={w.K} T={w.T} L={w.L} H={w.H} E={w.E} k={w.k} S={w.S} I={w.I} V={w.V}")
    t = time.time()
    weights = synth.gen_weights(w)
    noise = synth.HiddenNoise(w)
    offset = synth.hidden_offset(w, weights, noise)
    hidden_np = synth.to_storage(noise.draw(w.T) + offset, w.dtype)
    log(f"generated weights in {time.time() - t:.1f}s")

    copy_bytes = w.L * (w.E + w.S) * expert_bytes(w) + (w.V * w.H * 2 if w.has_lm_head else 0)
    copies = args.copies or max(1, math.ceil(1.5e9 / copy_bytes))
    if args.cost_model:
        if not w.has_lm_head:
            sys.exit("--cost-model needs a decode workload")
        # the bench's own rows (B x 4): at K = 3 the step is the benchmarked one
        cost_model(args, w, weights, hidden_np, copies, torch, np, synth, binding, VerifyModel, to_device)
        return
    prefill = not w.has_lm_head
    model = VerifyModel(w, weights, max_tokens=16 if prefill else w.T,
                        max_prefill_tokens=w.T if prefill else 0, copies=copies, max_seqs=max(w.B, 1))
    log(f"{copies} weight copies of {copy_bytes / 1e6:.0f} MB in HBM")
    positions_np = None
    if w.n_heads:
        positions_np = synth.kv_positions(w)
        t = time.time()
        for l in range(w.L):
            for b in range(w.B):
                k, v = synth.kv_prefix(w, l, b, int(positions_np[b]))
                for c in range(copies):
                    model.kv_write(l, b, k, v, copy=c)
        positions = to_device(positions_np)
        log(f"KV caches filled ({w.n_heads} heads, positions {int(positions_np.min())}..{int(positions_np.max())}) "
            f"in {time.time() - t:.1f}s")

    hidden = to_device(hidden_np)
    drafts_np = None
    committed_per_step = None
    if prefill:
        # the blocks in turn, residual stream ping-ponging between two buffers
        ys = [torch.empty_like(hidden), torch.empty_like(hidden)]
        aux = model.alloc_aux(w.T, layers=1, with_hidden=False)
        aux.pop("tstar")
        touched = []
        src = hidden
        for l in range(w.L):
            model.block_forward(l, src, w.T, ys[l % 2], aux)
            torch.cuda.synchronize()
            touched.append(int((aux["expert_count"][0] > 0).sum().item()))
            src = ys[l % 2]

        def run(c):
            x = hidden
            for l in range(w.L):
                model.block_forward(l, x, w.T, ys[l % 2], copy=c)
                x = ys[l % 2]
    else:
        # drafts: each correct with probability p against this step's own greedy picks
        committed, counts = model.alloc_outputs(w.B, w.K)
        aux = model.alloc_aux(w.T, with_hidden=False)

        def one(d, c=0, a=None):
            if w.n_heads:
                model.step_kv(hidden, d, positions, w.B, w.K, committed, counts, a, copy=c)
            else:
                model.step(hidden, d, w.B, w.K, committed, counts, a, copy=c)

        one(to_device(np.zeros((w.B, w.K), np.int32)), 0, aux)
        torch.cuda.synchronize()
        tstar = aux["tstar"].cpu().numpy()
        touched = [len(np.unique(aux["topk_idx"][l].cpu().numpy())) for l in range(w.L)]
        drafts_np = synth.make_drafts(w, tstar.reshape(w.B, w.K + 1))
        drafts = to_device(drafts_np)
        one(drafts)
        torch.cuda.synchronize()
        committed_per_step = int(counts.sum().item())

        def run(c):
            one(drafts, c)
    del aux

    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        run(i % copies)
    torch.cuda.synchronize()

    K = args.steps
    # the dominant kernel is bracketed by events on every EVERY-th step of the
    # timed region (each event record stalls the stream for a few us)
    sampled = list(range(0, K, EVERY))
    before = [ev.create() for _ in sampled]
    after = [ev.create() for _ in sampled]
    abefore = [ev.create() for _ in sampled] if w.n_heads else []
    aafter = [ev.create() for _ in sampled] if w.n_heads else []
    g0, g1 = ev.create(), ev.create()
    stage = binding.MOE_STAGE_LMHEAD if (w.L == 1 and not prefill) else binding.MOE_STAGE_EXPERT_UP
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(g0, stream)
    for i in range(K):
        c = i % copies
        if i % EVERY == 0:
            binding.moe_verify_set_stage_events(model.ctxs[c], stage, before[i // EVERY], after[i // EVERY])
            if w.n_heads:
                binding.moe_verify_set_stage_events(model.ctxs[c], binding.MOE_STAGE_ATTENTION,
                                                    abefore[i // EVERY], aafter[i // EVERY])
        run(c)
    ev.record(g1, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    gpu_ms_step = ev.elapsed_ms(g0, g1) / K
    kern_ms = sorted(ev.elapsed_ms(b, a) for b, a in zip(before, after))
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    attn_ms = sorted(ev.elapsed_ms(b, a) for b, a in zip(abefore, aafter))
    for e in before + after + abefore + aafter + [g0, g1]:
        ev.destroy(e)

    if prefill:
        # the gate+up GEMM: the persistent kernel from 16 reduction steps (H >= 512)
        kname = "k_gemm_up_persist" if w.H >= 512 else "k_grouped_gemm<up>"
        kfile = "k_prefill.hip"
        kflops = (w.T * w.k + w.S * w.T) * 2 * (2 * w.I * w.H)
        achieved = kflops / (kern_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic_from_profiles(kfile, w.name),
                "kernel": kname, "flops_per_launch": kflops}
    else:
        if stage == binding.MOE_STAGE_LMHEAD:
            kname = "k_lmhead_stream" if w.T <= 16 else ("k_lmhead_wide" if w.T <= 128 else "k_lmhead_mfma")
            kfile, kbytes = "k_lmhead.hip", lmhead_bytes(w)
        else:
            kname, kfile = "k_up_mfma", "k_experts.hip"
            kbytes = (touched[0] + w.S) * 2 * w.I * w.H * 2 + w.T * w.H * 2 + w.T * (w.k + w.S) * w.I * 2
        achieved = kbytes / (kern_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profiles(kfile, w.name),
                "kernel": kname, "bytes_per_launch": kbytes}
    roof.update({"avg_us": kern_avg_ms * 1e3, "median_us": kern_ms[len(kern_ms) // 2] * 1e3,
                 "launches_timed": len(kern_ms)})
    attn_roof = None
    if w.n_heads:
        abytes = attn_kv_bytes(w, positions_np) + w.T * w.H * 2
        aavg = sum(attn_ms) / len(attn_ms)
        aach = abytes / (aavg * 1e-3) / 1e9
        attn_roof = {"bound": "hbm", "achieved": aach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": aach / HBM_PEAK_GBS, "kernel": "k_attn_split", "bytes_per_launch": abytes,
                     "avg_us": aavg * 1e3, "median_us": attn_ms[len(attn_ms) // 2] * 1e3,
                     "launches_timed": len(attn_ms),
                     "traffic": traffic_from_profiles("k_attention.hip", f"{w.name}:k_attn_split")}
    sbytes = step_bytes(w, touched) + attn_step_bytes(w, positions_np)
    sflops = step_flops(w)
    if w.n_heads:  # projections and the q.k / p.v products over the cached rows
        sflops += w.L * (8 * w.T * w.H * w.H + 4 * 128 * w.n_heads * sum(
            (w.K + 1) * (int(p) + w.K + 1) for p in positions_np))
    step = {"gpu_ms_per_step": gpu_ms_step, "algorithmic_bytes": sbytes,
            "hbm_frac": sbytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9), "flops": sflops,
            "mfma_frac": sflops / (ms_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "experts_touched_per_layer": touched}
    # the whole step against the same peak, beside the dominant kernel's figure
    roof["step_frac"] = step["mfma_frac"] if prefill else step["hbm_frac"]
    if committed_per_step is not None:
        step["committed_tokens_per_step"] = committed_per_step
        step["committed_tokens_per_s"] = committed_per_step / (ms_step * 1e-3)

    res = {
        "metric": METRIC,
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s" if prefill else "verified tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "tokens_per_step": w.T, "layers": w.L,
                   "hidden": w.H, "routed_experts": w.E, "top_k": w.k, "shared_experts": w.S,
                   "inter": w.I, "vocab": w.V if w.has_lm_head else 0, "routing": w.routing,
                   "weight_copies": copies},
        "roofline": roof,
        "step": step,
    }
    if attn_roof:
        res["attention"] = attn_roof
        res["config"].update(heads=w.n_heads, kv_positions=[int(positions_np.min()), int(positions_np.max())],
                             kv_capacity=w.P)
    model.close()
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, weights, hidden_np, drafts_np, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
