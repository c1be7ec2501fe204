"""Select single-row sequences of the 12-layer verify step with attention
(attention + MoE in every layer, a KV cache part-way through a page) whose
discrete outputs are decided with room to spare at every layer, and store
them: each candidate's position in the workload's hidden-noise stream, its
cache length and its cache seed.

Run from the repository root:
    python tests/golden/make_attn_margin_rows.py attn_stack12_b32_zipf

Why.  As for the MoE-only stack (make_margin_rows.py): two float32
evaluations of the same stack, the oracle and the GPU kernels, resolve a few
bfloat16 roundings differently after the first layer, and the router logits
of the two trajectories drift apart with depth.  A sequence is kept when, at
every layer l, its row's top-k gap z_(k) - z_(k+1) is at least
ROUTER_MARGIN[l], and the head's arg-max gap at least HEAD_MARGIN, along the
oracle's own trajectory.  A sequence here is one row (K = 0, plain greedy
decoding through the full stack): its rows would otherwise attend to each
other, and all of them would have to meet the schedule together.

Candidate c: hidden row c of the workload's noise stream (plus its routing
offset), cache length PAGE_PROMPT + U{0 .. PAGE_OUTPUT - 1} from
SeedSequence([8100 + seed_id]) (the c-th draw), cached keys and values
synth.kv_prefix(w, l, c, length) (the cache of sequence c).  Only the oracle
and the seeded generators are used.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import attn_oracle as A  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from moe_decoder_speculative_amd import synth  # noqa: E402

N_SEQS = 6
BASE, PER_LAYER, HEAD = 1.5e-3, 6e-3, 9e-2   # 1.5 x the MoE-only stack's schedule


def candidate_lengths(w, n: int) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([8100 + w.seed_id]))
    return (synth.PAGE_PROMPT + g.integers(0, synth.PAGE_OUTPUT, size=n)).astype(np.int32)


_CTX = {}


def _keep(job) -> bool:
    """One candidate through the oracle's layers, stopping at the first gap
    below the schedule."""
    c, n, x = job
    w, shp, ash, weights, sched, store = (_CTX[k] for k in ("w", "shp", "ash", "weights", "sched", "store"))
    x = x[None, :]
    for l in range(w.L):
        k, v = synth.kv_prefix(w, l, c, n)
        kc = np.zeros((1, w.n_heads, w.P, 128), np.float32)
        vc = np.zeros_like(kc)
        kc[0, :, :n] = O.as_f32(k)
        vc[0, :, :n] = O.as_f32(v)
        a = A.attn_sublayer(x, np.array([n], np.int32), 1, 0, kc, vc, weights["layers"][l], ash)
        blk = O.moe_block(a.x_out, weights["layers"][l], shp)
        if O.topk_margin(blk.z, shp.k)[0] < sched[l]:
            return False
        x = blk.x_out
    lg = O.lm_head_logits(x, weights["final_gamma"], weights["lm_head"], shp.eps, store)
    return bool(O.argmax_margin(lg)[0] >= HEAD)


def select(name: str, max_candidates: int = 20000, procs: int = 8):
    import multiprocessing as mp
    w = synth.WORKLOADS[name]
    shp = O.Shape(H=w.H, E=w.E, k=w.k, S=w.S, I=w.I, V=w.V, L=w.L, eps=w.eps, dtype=w.dtype)
    ash = A.AttnShape(H=w.H, n_heads=w.n_heads, d_head=128, P=w.P, theta=w.rope_theta, eps=w.eps, dtype=w.dtype)
    weights = synth.gen_weights(w)
    noise = synth.HiddenNoise(w)
    offset = synth.hidden_offset(w, weights, noise)
    _CTX.update(w=w, shp=shp, ash=ash, weights=weights, sched=[BASE + PER_LAYER * l for l in range(w.L)],
                store=O.storage_round(shp.dtype))
    lengths = candidate_lengths(w, max_candidates)
    kept = []
    t0 = time.time()
    chunk = 256
    c = 0
    # candidates are independent: worker processes forked after the weights
    # exist share them, one BLAS thread each
    with mp.get_context("fork").Pool(procs) as pool:
        while len(kept) < N_SEQS and c < max_candidates:
            xs = O.as_f32(synth.to_storage(noise.draw(chunk) + offset, w.dtype))
            jobs = [(c + i, int(lengths[c + i]), xs[i]) for i in range(chunk)]
            for (cc, n, _), ok in zip(jobs, pool.map(_keep, jobs, chunksize=4)):
                if ok and len(kept) < N_SEQS:
                    kept.append({"candidate": cc, "length": n})
            c += chunk
            print(f"[attn rows] {name}: {c} candidates, kept {len(kept)}/{N_SEQS} ({time.time() - t0:.0f} s)",
                  flush=True)
    return w, _CTX["sched"], kept, c


def main():
    name = sys.argv[1] if len(sys.argv) > 1 else "attn_stack12_b32_zipf"
    w, sched, kept, drawn = select(name)
    out = {
        "_source": ("Single-row sequences kept by tests/golden/make_attn_margin_rows.py: along the oracle's own "
                    "trajectory through the twelve layers of attention and MoE, every layer's top-k gap and the "
                    "head's arg-max gap exceed a schedule 1.5 times the MoE-only stack's (the pages fix the "
                    "12-layer depth: page 'Jina AI releases lightweight OCR model with built-in speculative "
                    "decoding', section 'Lean architecture with a compressed encoder')."),
        "workload": name,
        "chunk": 256,
        "router_margin": sched,
        "head_margin": HEAD,
        "candidates_drawn": drawn,
        "sequences": kept,
        "numpy": np.__version__,
    }
    path = os.path.join(HERE, f"{name}_seqs.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
