"""Test-side assembly of seeded cases: synthetic inputs + the oracle's results.

Inputs come from moe_decoder_speculative_amd.synth (random numbers only).  The
oracle is run here to (1) redraw any hidden row whose top-k or arg-max margin is
below MARGIN, so discrete outputs are well separated, and (2) build drafts from
the oracle's greedy picks.  Expected values therefore come from the oracle only.
"""
from __future__ import annotations

import functools
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
