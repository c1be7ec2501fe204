"""Seeded synthetic inputs for the MoE verification step.

This module draws random numbers and shapes them; it holds none of the step's
arithmetic (no normalisation, routing, expert or head computation).  The HIP
library's tests, the benchmark and the CPU oracle's tests all take their inputs
from here, so both sides see identical bytes for a given seed.

The workloads mirror the pages' shapes:
  * the decoder routes each token to 6 of 64 experts plus 2 shared experts over
    12 layers ("Jina AI releases lightweight OCR model with built-in speculative
    decoding", section "Lean architecture with a compressed encoder");
  * a verification step carries the last committed token plus K = 3 FastMTP
    drafts per sequence (same page, "Speculative decoding without accuracy
    loss"), at batch 1 and at concurrency 32 (same page, "High throughput on
    cheap hardware");
  * a page is at most 1,156 visual tokens (256 global + 9 tiles of 100; same
    page, "Lean architecture with a compressed encoder").
Hidden size, SwiGLU width and vocabulary are not on the pages; the values
below (1280, 896, 129280) are this library's reading of a DeepSeek-3B-MoE-sized
decoder.  Weights are random N(0, 0.02^2); no trained checkpoint is used.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
import os

import numpy as np

WEIGHT_STD = 0.02
ZIPF_S = 1.1
# strength of the router-logit shift that produces Zipf-skewed expert
# popularity; chosen so the top-1 frequency over popularity ranks falls off
# with a log-log slope near -1.1 at the first layer (checked by the tests).
ZIPF_ALPHA = 0.33
DRAFT_ACCEPT_P = 0.576


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    E: int
    k: int
    S: int
    I: int
    V: int
    L: int
    B: int          # sequences (0 for a prefill workload)
    K: int          # drafts per sequence
    T: int          # tokens per step
    dtype: str      # 'bf16' or 'f32'
    routing: str    # 'uniform' or 'zipf'
    drafts: str     # 'independent', 'replace_pos2' or 'none'
    has_lm_head: bool
    seed_id: int
    eps: float = 1e-6
    accept_p: float = DRAFT_ACCEPT_P
    n_heads: int = 0        # attention heads of 128 (0: MoE-only blocks)
    P: int = 0              # KV-cache positions per sequence
    rope_theta: float = 10000.0

    @property
    def weight_seed(self) -> int:
        return 1000 + self.seed_id

    @property
    def input_seed(self) -> int:
        return 2000 + self.seed_id

    @property
    def draft_seed(self) -> int:
        return 3000 + self.seed_id

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


PAGE_PROMPT = 1156 + 64     # visual tokens of a page at most, plus the prompt
PAGE_OUTPUT = 1085          # output tokens per page
ATTN_P = 2368               # >= PAGE_PROMPT + PAGE_OUTPUT + 8, a multiple of 64
KV_STD = 0.7                # cached keys / values ~ the scale of W x at N(0, 0.02^2) weights


def _verify(name, seed_id, B, **kw):
    base = dict(H=1280, E=64, k=6, S=2, I=896, V=129280, L=1, K=3, dtype="bf16",
                routing="uniform", drafts="independent", has_lm_head=True)
    base.update(kw)
    return Workload(name=name, B=B, T=B * (base["K"] + 1), seed_id=seed_id, **base)


WORKLOADS = {
    # tiny fp32 block: 8 experts top-2, 1 shared; drafts are the greedy picks
    # with the second draft replaced by a wrong token
    "tiny_fp32": Workload("tiny_fp32", H=256, E=8, k=2, S=1, I=128, V=1024, L=1,
                          B=2, K=3, T=8, dtype="f32", routing="uniform",
                          drafts="replace_pos2", has_lm_head=True, seed_id=1),
    # batch-1 decode analogue: one block at the pages' routing shape
    "decode_b1": _verify("decode_b1", 2, B=1),
    # concurrency-32 analogue with Zipf-skewed expert popularity
    "decode_b32_zipf": _verify("decode_b32_zipf", 3, B=32, routing="zipf"),
    # prefill: 8 pages x (1,156 visual + 64 prompt tokens), no LM head
    "prefill_8pages": Workload("prefill_8pages", H=1280, E=64, k=6, S=2, I=896,
                               V=129280, L=1, B=0, K=0, T=8 * (1156 + 64),
                               dtype="bf16", routing="uniform", drafts="none",
                               has_lm_head=False, seed_id=4),
    # 12 blocks with residual between them, then the LM head
    "stack12_b32_zipf": _verify("stack12_b32_zipf", 5, B=32, L=12, routing="zipf"),
    # batch 1 through the 12 blocks + LM head (the decode-loop cost model's verifier)
    "stack12_b1": _verify("stack12_b1", 7, B=1, L=12),
    # attention + MoE layers with a KV cache: each sequence part-way through
    # one page (1,156 visual + 64 prompt tokens, then up to 1,085 generated)
    "attn_b1": _verify("attn_b1", 8, B=1, n_heads=10, P=ATTN_P),
    "attn_b32_zipf": _verify("attn_b32_zipf", 9, B=32, routing="zipf", n_heads=10, P=ATTN_P),
    "attn_stack12_b1": _verify("attn_stack12_b1", 10, B=1, L=12, n_heads=10, P=ATTN_P),
    "attn_stack12_b32_zipf": _verify("attn_stack12_b32_zipf", 11, B=32, L=12, routing="zipf", n_heads=10, P=ATTN_P),
    # the 8-page prefill through the same 12-block stack (no LM head)
    "prefill_8pages_stack12": Workload("prefill_8pages_stack12", H=1280, E=64, k=6, S=2, I=896,
                                       V=129280, L=12, B=0, K=0, T=8 * (1156 + 64),
                                       dtype="bf16", routing="uniform", drafts="none",
                                       has_lm_head=False, seed_id=6),
}


# --------------------------------------------------------------------------
# storage helpers (no arithmetic of the step)
# --------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in the workload's storage type (uint16 bits for bf16)."""
    if dtype == "bf16":
        return to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _rng(seed_seq) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq))


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

_TENSORS = ("router", "gate", "up", "down", "s_gate", "s_up", "s_down")


def _tensor_shape(w: Workload, name: str):
    return {
        "router": (w.E, w.H),
        "gate": (w.E, w.I, w.H),
        "up": (w.E, w.I, w.H),
        "down": (w.E, w.H, w.I),
        "s_gate": (w.S, w.I, w.H),
        "s_up": (w.S, w.I, w.H),
        "s_down": (w.S, w.H, w.I),
        "lm_head": (w.V, w.H),
    }[name]


def _draw_tensor(w: Workload, child, name: str) -> np.ndarray:
    shape = _tensor_shape(w, name)
    n = int(np.prod(shape))
    vals = _rng(child).standard_normal(n, dtype=np.float32)
    vals *= np.float32(WEIGHT_STD)
    return to_storage(vals.reshape(shape), w.dtype)


def gen_weights(w: Workload, layers=None, threads: int | None = None) -> dict:
    """Seeded weights: each (layer, tensor) has its own spawned child of
    SeedSequence(weight_seed), so any tensor is reproducible on its own.

    Returns {'layers': [dict(gamma, router, gate, up, down, s_gate, s_up,
    s_down)], 'final_gamma', 'lm_head'} with float32 arrays for 'f32' and
    uint16 bfloat16 bit patterns for 'bf16'.  Norm gains are 1.
    """
    children = np.random.SeedSequence(w.weight_seed).spawn(w.L * len(_TENSORS) + 1)
    layer_ids = list(range(w.L)) if layers is None else list(layers)
    jobs = []
    for l in layer_ids:
        for i, name in enumerate(_TENSORS):
            jobs.append((l, name, children[l * len(_TENSORS) + i]))
    if w.has_lm_head:
        jobs.append((None, "lm_head", children[w.L * len(_TENSORS)]))
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        outs = list(ex.map(lambda j: _draw_tensor(w, j[2], j[1]), jobs))
    one = to_storage(np.ones(w.H, np.float32), w.dtype)
    res = {"layers": [dict(gamma=one.copy()) for _ in layer_ids],
           "final_gamma": one.copy(), "lm_head": None}
    pos = {l: i for i, l in enumerate(layer_ids)}
    for (l, name, _), arr in zip(jobs, outs):
        if l is None:
            res["lm_head"] = arr
        else:
            res["layers"][pos[l]][name] = arr
    if w.n_heads > 0:
        for l, lw in zip(layer_ids, res["layers"]):
            lw.update(gen_attn_layer(w, l))
    return res


def gen_attn_layer(w: Workload, l: int) -> dict:
    """Layer l's attention weights from their own seed (SeedSequence(7000+id),
    one child per layer): attn_gamma = 1 + U(-0.1, 0.1), w_q, w_k, w_v, w_o
    N(0, 0.02^2)."""
    ch = np.random.SeedSequence(7000 + w.seed_id).spawn(w.L)[l].spawn(5)
    out = {"attn_gamma": to_storage((1.0 + 0.1 * _rng(ch[0]).uniform(-1, 1, w.H)).astype(np.float32), w.dtype)}
    for c, name in zip(ch[1:], ("w_q", "w_k", "w_v", "w_o")):
        vals = _rng(c).standard_normal(w.H * w.H, dtype=np.float32)
        vals *= np.float32(WEIGHT_STD)
        out[name] = to_storage(vals.reshape(w.H, w.H), w.dtype)
    return out


def kv_positions(w: Workload, B: int | None = None) -> np.ndarray:
    """Cache length of each sequence before the step: part-way through one
    page, PAGE_PROMPT + U{0 .. PAGE_OUTPUT - 1}, capped so the step fits; a
    workload whose cache is shorter than a page draws uniformly over what fits."""
    B = w.B if B is None else B
    g = _rng(np.random.SeedSequence(8000 + w.seed_id).spawn(1)[0])
    top = w.P - (w.K + 1)
    if top >= PAGE_PROMPT + PAGE_OUTPUT:
        return (PAGE_PROMPT + g.integers(0, PAGE_OUTPUT, size=B)).astype(np.int32)
    return g.integers(0, top + 1, size=B).astype(np.int32)


def kv_prefix(w: Workload, l: int, b: int, n: int):
    """Cached keys and values of layer l, sequence b at positions 0..n-1:
    N(0, KV_STD^2) in the storage type, [n_heads, n, 128] each, from child
    (l, b) of SeedSequence(9000+id) (so any one sequence is reproducible)."""
    ss = np.random.SeedSequence([9000 + w.seed_id, l, b])
    g = _rng(ss)
    shape = (w.n_heads, n, 128)
    k = g.standard_normal(shape, dtype=np.float32) * np.float32(KV_STD)
    v = g.standard_normal(shape, dtype=np.float32) * np.float32(KV_STD)
    return to_storage(k, w.dtype), to_storage(v, w.dtype)


# --------------------------------------------------------------------------
# hidden states
# --------------------------------------------------------------------------

class HiddenNoise:
    """Sequential stream of N(0,1) hidden-state rows from SeedSequence(input_seed).

    Rows are drawn in order; redrawing a row takes the next rows of the same
    stream, so a fixed sequence of redraw requests gives fixed bytes."""

    def __init__(self, w: Workload):
        ss = np.random.SeedSequence(w.input_seed)
        noise_ss, self._perm_ss = ss.spawn(2)
        self._rng = _rng(noise_ss)
        self.H = w.H

    def draw(self, n_rows: int) -> np.ndarray:
        return self._rng.standard_normal((n_rows, self.H), dtype=np.float32)

    def zipf_permutations(self, L: int, E: int):
        """One seeded permutation per layer: popularity rank -> expert id."""
        g = _rng(self._perm_ss)
        return [g.permutation(E) for _ in range(L)]


def zipf_offset(w: Workload, routers_f32, perms, alpha: float = ZIPF_ALPHA) -> np.ndarray:
    """A fixed hidden-state offset v that shifts every layer's router logits
    towards a Zipf(s) popularity profile.

    Target shift per layer: s_l[e] = alpha * (log p_rank(e) - mean), with
    p_r proportional to r^-s over ranks r = 1..E and rank(e) given by the
    layer's permutation.  v is the minimum-norm solution of R v = concat_l s_l,
    R being the stacked router matrices (full row rank for these shapes).
    """
    E = w.E
    logp = -ZIPF_S * np.log(np.arange(1, E + 1, dtype=np.float64))
    logp -= logp.mean()
    rows, rhs = [], []
    for R_l, pi in zip(routers_f32, perms):
        shift = np.empty(E)
        shift[pi] = alpha * logp          # expert pi[r] has popularity rank r+1
        rows.append(np.asarray(R_l, dtype=np.float64))
        rhs.append(shift)
    R = np.concatenate(rows, axis=0)
    s = np.concatenate(rhs)
    v, *_ = np.linalg.lstsq(R, s, rcond=None)
    return v.astype(np.float32)


def hidden_offset(w: Workload, weights: dict, noise: HiddenNoise) -> np.ndarray:
    """Per-row additive offset of the workload: zero for uniform routing, the
    Zipf offset otherwise."""
    if w.routing != "zipf":
        return np.zeros(w.H, dtype=np.float32)
    routers = [bits_to_f32(lw["router"]) if lw["router"].dtype == np.uint16 else lw["router"]
               for lw in weights["layers"]]
    perms = noise.zipf_permutations(w.L, w.E)
    return zipf_offset(w, routers, perms)


# --------------------------------------------------------------------------
# drafts
# --------------------------------------------------------------------------

def draft_randoms(w: Workload, B: int | None = None, K: int | None = None):
    """Random numbers that decide the drafts: u [B,K] uniform in [0,1) and
    r [B,K] uniform over {0..V-2} (a wrong token is r, skipping the correct one)."""
    B = w.B if B is None else B
    K = w.K if K is None else K
    g = _rng(np.random.SeedSequence(w.draft_seed))
    u = g.random((B, K))
    r = g.integers(0, w.V - 1, size=(B, K))
    return u, r


def wrong_token(correct: np.ndarray, r: np.ndarray) -> np.ndarray:
    """A token different from `correct`: r in {0..V-2} mapped past it."""
    r = np.asarray(r, dtype=np.int64)
    return np.where(r < correct, r, r + 1).astype(np.int32)


def make_drafts(w: Workload, tstar_bk1: np.ndarray, u=None, r=None) -> np.ndarray:
    """Drafts [B, K] given the verifier's picks tstar [B, K+1].

    'independent': draft j equals tstar[b, j] with probability accept_p,
    otherwise a uniformly random wrong token.
    'replace_pos2': drafts are the picks with the second draft (position 2 of
    the K+1 frame) replaced by a random wrong token.
    """
    tstar_bk1 = np.asarray(tstar_bk1)
    B, K1 = tstar_bk1.shape
    K = K1 - 1
    if K == 0:
        return np.zeros((B, 0), dtype=np.int32)
    if u is None or r is None:
        u, r = draft_randoms(w, B, K)
    correct = tstar_bk1[:, :K].astype(np.int32)
    if w.drafts == "replace_pos2":
        d = correct.copy()
        d[:, 1] = wrong_token(correct[:, 1], r[:, 1])
        return d
    if w.drafts == "independent":
        return np.where(u < w.accept_p, correct, wrong_token(correct, r)).astype(np.int32)
    raise ValueError(f"workload {w.name} has no drafts")


# --------------------------------------------------------------------------
# draft head
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class DraftWorkload:
    """A draft-head workload on top of a verify workload, whose hidden size,
    vocabulary and LM head it shares.

    The pages fix one dense block applied recursively for K = 3 steps ("Jina
    AI releases lightweight OCR model with built-in speculative decoding",
    section "Speculative decoding without accuracy loss") but not its width:
    Id = (k + S) * I = 7168, the SwiGLU width a verifier block activates per
    token, is this library's reading.  head_rows = 0 drafts over the whole
    vocabulary; a positive value restricts the draft head to that many rows
    (a seeded subset of token ids)."""

    name: str
    base: str
    Id: int
    head_rows: int
    B: int
    K: int
    R: int          # verifier rows per sequence handed to the draft (K + 1)
    seed_id: int

    @property
    def weight_seed(self) -> int:
        return 5000 + self.seed_id

    @property
    def input_seed(self) -> int:
        return 6000 + self.seed_id

    def with_(self, **kw) -> "DraftWorkload":
        return replace(self, **kw)


DRAFT_WORKLOADS = {
    "draft_b1": DraftWorkload("draft_b1", "decode_b1", Id=7168, head_rows=0, B=1, K=3, R=4, seed_id=1),
    "draft_b32": DraftWorkload("draft_b32", "decode_b32_zipf", Id=7168, head_rows=0, B=32, K=3, R=4, seed_id=2),
    "draft_b1_head32k": DraftWorkload("draft_b1_head32k", "decode_b1", Id=7168, head_rows=32768, B=1, K=3, R=4,
                                      seed_id=3),
}

DRAFT_GAIN_SPREAD = 0.1


def gen_draft_weights(dw: DraftWorkload, base: Workload, lm_head: np.ndarray) -> dict:
    """Seeded draft-head weights in the base workload's storage type.

    embed [V, H], w_proj [H, 2H], w_gate / w_up [Id, H], w_down [H, Id] are
    N(0, 0.02^2); the four RMSNorm gains are 1 + U(-0.1, 0.1) (distinct, so a
    gain used in the wrong place shows); head is lm_head itself or its rows
    head_ids (a sorted seeded subset)."""
    H, V, Id = base.H, base.V, dw.Id
    ch = np.random.SeedSequence(dw.weight_seed).spawn(10)

    def normal(c, shape):
        vals = _rng(c).standard_normal(int(np.prod(shape)), dtype=np.float32)
        vals *= np.float32(WEIGHT_STD)
        return to_storage(vals.reshape(shape), base.dtype)

    def gain(c):
        return to_storage((1.0 + DRAFT_GAIN_SPREAD * _rng(c).uniform(-1, 1, H)).astype(np.float32), base.dtype)

    out = dict(embed=normal(ch[0], (V, H)), gamma_h=gain(ch[1]), gamma_e=gain(ch[2]), gamma_f=gain(ch[3]),
               gamma_o=gain(ch[4]), w_proj=normal(ch[5], (H, 2 * H)), w_gate=normal(ch[6], (Id, H)),
               w_up=normal(ch[7], (Id, H)), w_down=normal(ch[8], (H, Id)))
    if dw.head_rows > 0:
        ids = np.sort(_rng(ch[9]).choice(V, size=dw.head_rows, replace=False)).astype(np.int32)
        out["head"] = np.ascontiguousarray(lm_head[ids])
        out["head_ids"] = ids
    else:
        out["head"] = lm_head
    return out


def draft_inputs(dw: DraftWorkload, base: Workload, B: int | None = None):
    """What a draft call continues from: hidden [B*R, H] N(0, 1) rows in the
    storage type, committed [B, R] token ids uniform over [0, V), counts [B]
    uniform over 1..R."""
    B = dw.B if B is None else B
    g = _rng(np.random.SeedSequence(dw.input_seed))
    hidden = to_storage(g.standard_normal((B * dw.R, base.H), dtype=np.float32), base.dtype)
    committed = g.integers(0, base.V, size=(B, dw.R)).astype(np.int32)
    counts = g.integers(1, dw.R + 1, size=B).astype(np.int32)
    return hidden, committed, counts
