"""Test-side assembly of seeded cases: synthetic inputs + the oracle's results.

Inputs come from moe_decoder_speculative_amd.synth (random numbers only).  The
oracle is run here to (1) redraw any hidden row whose top-k or arg-max margin is
below MARGIN, so discrete outputs are well separated, and (2) build drafts from
the oracle's greedy picks.  Expected values therefore come from the oracle only.
"""
from __future__ import annotations

import functools
import json
import os
from dataclasses import dataclass

import numpy as np

import oracle
from moe_decoder_speculative_amd import synth

MARGIN = 1e-3


def shape_of(w: synth.Workload) -> oracle.Shape:
    return oracle.Shape(H=w.H, E=w.E, k=w.k, S=w.S, I=w.I, V=w.V, L=w.L, eps=w.eps, dtype=w.dtype)


def row_margins(shp: oracle.Shape, weights: dict, x_rows: np.ndarray, has_lm_head: bool) -> np.ndarray:
    """Smallest top-k margin over all layers and (optionally) the arg-max margin, per row."""
    x = x_rows
    worst = np.full(x.shape[0], np.inf, dtype=np.float64)
    for l in range(shp.L):
        r = oracle.moe_block(x, weights["layers"][l], shp)
        worst = np.minimum(worst, oracle.topk_margin(r.z, shp.k))
        x = r.x_out
    if has_lm_head:
        store = oracle.storage_round(shp.dtype)
        lg = oracle.lm_head_logits(x, weights["final_gamma"], weights["lm_head"], shp.eps, store)
        worst = np.minimum(worst, oracle.argmax_margin(lg))
    return worst


@dataclass
class Case:
    w: synth.Workload
    shp: oracle.Shape
    weights: dict
    hidden: np.ndarray          # [T, H] storage (uint16 bf16 bits or float32)
    drafts: np.ndarray          # [B, K] int32 (empty for prefill)
    ref: oracle.StepResult
    redrawn_rows: int


def build_case(w: synth.Workload, margin: float = MARGIN, max_rounds: int = 100) -> Case:
    shp = shape_of(w)
    weights = synth.gen_weights(w)
    noise = synth.HiddenNoise(w)
    offset = synth.hidden_offset(w, weights, noise)
    raw = noise.draw(w.T)
    hidden = synth.to_storage(raw + offset, w.dtype)
    todo = np.arange(w.T)
    redrawn = 0
    for _ in range(max_rounds):
        m = row_margins(shp, weights, hidden[todo], w.has_lm_head)
        bad = todo[m < margin]
        if bad.size == 0:
            break
        redrawn += bad.size
        raw[bad] = noise.draw(bad.size)
        hidden[bad] = synth.to_storage(raw[bad] + offset, w.dtype)
        todo = bad
    else:
        raise RuntimeError("margin rejection did not converge")

    if w.has_lm_head:
        B, K = w.B, w.K
        ref = oracle.verify_step(shp, weights, hidden, np.zeros((B, K), np.int32), B, K)
        drafts = synth.make_drafts(w, ref.tstar.reshape(B, K + 1))
        if K > 0:
            ref.committed, ref.counts = oracle.accept_prefix(ref.tstar.reshape(B, K + 1), drafts)
    else:
        drafts = np.zeros((0, 0), np.int32)
        ref = oracle.verify_step(shp, weights, hidden, None, w.T, 0, has_lm_head=False)
    return Case(w, shp, weights, hidden, drafts, ref, redrawn)


@functools.lru_cache(maxsize=4)
def cached_case(name: str, **overrides) -> Case:
    w = synth.WORKLOADS[name]
    if overrides:
        w = w.with_(**overrides)
    return build_case(w)


def small_bf16(name="small_bf16", B=5, K=3, H=256, E=16, k=4, S=2, I=128, V=1000, L=2,
               routing="uniform", seed_id=11) -> synth.Workload:
    """A bf16 workload the oracle finishes in well under a second but which still
    spans several kernel tiles and a ragged vocabulary / token tail."""
    return synth.Workload(name=name, H=H, E=E, k=k, S=S, I=I, V=V, L=L, B=B, K=K,
                          T=B * (K + 1), dtype="bf16", routing=routing,
                          drafts="independent", has_lm_head=True, seed_id=seed_id)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def margin_rows_case(name: str) -> Case:
    """A stacked workload on rows whose top-k and arg-max gaps leave room for
    the drift of a second float32 evaluation at every block: the stream
    positions written by tests/golden/make_margin_rows.py (which uses only
    the oracle and the seeded generator) select rows of the workload's own
    hidden-noise stream; the expected outputs are the oracle's step on them."""
    with open(os.path.join(GOLDEN, f"{name}_rows.json")) as f:
        spec = json.load(f)
    w = synth.WORKLOADS[name]
    shp = shape_of(w)
    weights = synth.gen_weights(w)
    noise = synth.HiddenNoise(w)
    offset = synth.hidden_offset(w, weights, noise)
    rows = np.asarray(spec["rows"], dtype=np.int64)
    assert rows.size == w.T
    n = 0
    chunks = []
    while n <= rows.max():
        chunks.append(noise.draw(spec["chunk"]))
        n += spec["chunk"]
    raw = np.concatenate(chunks)[rows]
    hidden = synth.to_storage(raw + offset, w.dtype)
    B, K = w.B, w.K
    ref = oracle.verify_step(shp, weights, hidden, np.zeros((B, K), np.int32), B, K)
    # the rows meet the stored schedule along the oracle's own trajectory
    for l, blk in enumerate(ref.blocks):
        assert oracle.topk_margin(blk.z, w.k).min() >= spec["router_margin"][l], f"block {l}: margin below schedule"
    drafts = synth.make_drafts(w, ref.tstar.reshape(B, K + 1))
    ref.committed, ref.counts = oracle.accept_prefix(ref.tstar.reshape(B, K + 1), drafts)
    return Case(w, shp, weights, hidden, drafts, ref, 0)


@dataclass
class AttnSeqCase:
    w: synth.Workload            # the workload reshaped to the stored sequences (B = n, K = 0)
    base: synth.Workload         # the workload the sequences were drawn from
    weights: dict
    hidden: np.ndarray           # [n, H] storage dtype
    positions: np.ndarray        # [n] cache length of each sequence
    cands: list                  # candidate (stream position and cache seed) of each sequence
    ref: object                  # the oracle's step (attn_oracle.AttnStepResult)


def attn_margin_seqs_case(gen_weights=synth.gen_weights) -> AttnSeqCase:
    """The 12-layer step with attention on the single-row sequences written by
    tests/golden/make_attn_margin_rows.py (oracle and seeded generators only):
    hidden row c of the workload's noise stream, the cache of sequence c at
    its stored length.  Asserts the stored gap schedule (every layer's top-k
    gap, the head's arg-max gap) along the oracle's own trajectory."""
    from oracle import attn_oracle as A
    with open(os.path.join(GOLDEN, "attn_stack12_b32_zipf_seqs.json")) as f:
        spec = json.load(f)
    base = synth.WORKLOADS[spec["workload"]]
    seqs = spec["sequences"]
    n = len(seqs)
    cands = [int(q["candidate"]) for q in seqs]
    positions = np.array([int(q["length"]) for q in seqs], np.int32)
    w = base.with_(name=base.name + "_margin_seqs", B=n, K=0, T=n)
    weights = gen_weights(base)
    noise = synth.HiddenNoise(base)
    offset = synth.hidden_offset(base, weights, noise)
    chunk = spec["chunk"]
    raw = np.concatenate([noise.draw(chunk) for _ in range(max(cands) // chunk + 1)])[cands]
    hidden = synth.to_storage(raw + offset, w.dtype)
    caches = []
    for l in range(w.L):
        kc = np.zeros((n, w.n_heads, w.P, 128), np.float32)
        vc = np.zeros_like(kc)
        for i, c in enumerate(cands):
            k, v = synth.kv_prefix(base, l, c, int(positions[i]))
            kc[i, :, :positions[i]] = oracle.as_f32(k)
            vc[i, :, :positions[i]] = oracle.as_f32(v)
        caches.append((kc, vc))
    shp = shape_of(w)
    ash = A.AttnShape(H=w.H, n_heads=w.n_heads, d_head=128, P=w.P, theta=w.rope_theta, eps=w.eps, dtype=w.dtype)
    ref = A.verify_step_attn(shp, ash, weights, hidden, np.zeros((n, 0), np.int32), positions, caches, n, 0)
    for l, blk in enumerate(ref.blocks):
        assert oracle.topk_margin(blk.z, w.k).min() >= spec["router_margin"][l], f"layer {l}: margin below schedule"
    lg = oracle.lm_head_logits(ref.hidden_out, weights["final_gamma"], weights["lm_head"], w.eps,
                               oracle.storage_round(w.dtype))
    assert oracle.argmax_margin(lg).min() >= spec["head_margin"], "head margin below schedule"
    return AttnSeqCase(w, base, weights, hidden, positions, cands, ref)
