"""CPU oracle for one speculative verification step of a mixture-of-experts decoder.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, header, table or
helper with the HIP library; the only thing the two sides have in common is the
seeded input generator, which holds none of the arithmetic below.

Sources (the pages this oracle follows; cited by short key below):

  [JINA-FR]  "jina-ocr-v1 : Analyse de documents plus rapide sur des GPU a budget
             limite" (jina.ai news page, French).
  [CLAWPIT]  "Jina AI releases lightweight OCR model with built-in speculative
             decoding" (clawpit.io).
  [NULLBOT]  "Jina AI lance jina-ocr-v1, parseur de documents GPU low-cost avec
             MoE et decodage speculatif" (nullbot.ai).
  [D9249]    d9249.github.io blog post on jina-ocr-v1 low-budget document
             parsing (Korean).

What the pages fix, in their own terms:
  * the decoder is a mixture of experts with 64 routed experts, two shared
    experts and top-6 routing, 12 layers ([CLAWPIT] "Lean architecture with a
    compressed encoder");
  * the verifier checks each draft greedily, accepts the longest prefix on which
    draft and verifier agree, and commits one extra token of its own, so the
    committed text equals plain greedy decoding ([CLAWPIT] "Speculative decoding
    without accuracy loss"; [JINA-FR] "Modele et entrainement"; [D9249] core-idea
    section).

What the pages leave open and this oracle reads plainly (every reading is also
listed in the design notes of the repository):
  * pre-norm block x <- x + MoE(RMSNorm(x)) with RMSNorm x / sqrt(mean(x^2)+eps) * gamma;
  * router logits z = W_r xh; the k largest by (z descending, expert ascending);
    gate weights are the softmax over the k selected logits (they sum to 1);
  * experts are bias-free SwiGLU MLPs: Wd (silu(Wg xh) * (Wu xh)), silu(v) = v/(1+e^-v);
  * shared experts are always on with weight 1;
  * combine order is fixed: shared experts in index order, then the routed
    experts of the token in ascending expert index;
  * a final RMSNorm precedes the LM head; the greedy pick is the arg-max logit,
    lowest token id on ties;
  * draft j of a sequence is compared with the verifier's pick after input
    position j; the pick after the last position is the bonus token.

Precision: all arithmetic is float32 (numpy, BLAS for matrix products).  When the
storage type is bfloat16, values are rounded to bfloat16 (round to nearest,
ties to even) at exactly three points, and nowhere else:
  R1  the normalised activations xh (and the final-norm activations),
  R2  the SwiGLU activation a = silu(g) * u,
  R3  the block output x' = x + m.
When the storage type is float32 nothing is rounded.

Parity status of each function is stated in its docstring; the pins live in
tests/test_oracle_pins.py.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32


# --------------------------------------------------------------------------
# bfloat16 storage
# --------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value, ties to even.

    The result is returned as float32 (bfloat16 values are exactly
    representable in float32).  NaN stays NaN, infinities stay infinities and
    finite values past the largest bfloat16 round to infinity, as IEEE
    round-to-nearest-even requires.

    Pinned: against torch's float32 -> bfloat16 conversion on every high half
    and a set of low halves that covers every rounding case.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    bits = a.view(np.uint32).astype(np.uint64)
    # keep bit 16 (the lowest bit that survives) to break exact ties to even
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(F32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def as_f32(a) -> np.ndarray:
    """A weight or activation as float32: bfloat16 bit patterns are widened."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return a.astype(F32, copy=False)


def storage_round(dtype: str):
    """The rounding applied at R1/R2/R3 for a storage type ('bf16' or 'f32')."""
    if dtype == "bf16":
        return bf16_round
    if dtype == "f32":
        return lambda v: np.asarray(v, dtype=F32)
    raise ValueError(f"unknown storage type {dtype!r}")


# --------------------------------------------------------------------------
# Shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    """Block shape.  H hidden, E routed experts, k routed per token, S shared,
    I SwiGLU width, V vocabulary, L layers.  64 routed + 2 shared, top-6 and 12
    layers are the pages' decoder ([CLAWPIT] "Lean architecture with a
    compressed encoder"); H, I and V are not on the pages."""

    H: int
    E: int
    k: int
    S: int
    I: int
    V: int
    L: int = 1
    eps: float = 1e-6
    dtype: str = "bf16"


# --------------------------------------------------------------------------
# The step, one operation at a time
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, store) -> np.ndarray:
    """R1: xh = store(x / sqrt(mean(x^2) + eps) * gamma), row-wise, float32.

    Not on the pages (they give no layer internals); plain RMSNorm reading.
    Pinned: torch.nn.functional.rms_norm on the CPU, closed form for constant
    rows, scale invariance.
    """
    x = as_f32(x)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    y = x / np.sqrt(ms + F32(eps)) * as_f32(gamma)
    return store(y.astype(F32, copy=False))


def router_logits(xh: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """z[t, e] = sum_h xh[t, h] * W_r[e, h], float32 (one logit per routed expert)."""
    return (as_f32(xh) @ as_f32(w_router).T).astype(F32, copy=False)


def topk_select(z: np.ndarray, k: int):
    """Top-k routing ([CLAWPIT] "Lean architecture...": top-6 of 64 routed experts).

    Returns (idx, w): idx[t] holds the k experts with the largest logits, in
    order of descending logit with the lower expert index first on equal logits;
    w[t] is the softmax over the k selected logits (max-subtracted), so each
    row sums to 1.  Pinned: brute-force subset enumeration, the separation
    certificate, torch.topk, torch.softmax and the closed-form weight ratios.
    """
    z = np.asarray(z, dtype=F32)
    T, E = z.shape
    # a stable sort of the negated logits puts equal logits in expert order
    order = np.argsort(-z, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    zs = np.take_along_axis(z, idx, axis=1)
    zmax = zs[:, :1]
    ex = np.exp(zs - zmax)
    den = np.zeros((T, 1), dtype=F32)
    for j in range(k):  # sequential, in selection order
        den = den + ex[:, j:j + 1]
    w = (ex / den).astype(F32)
    return idx, w


def counting_sort(idx_flat: np.ndarray, E: int):
    """Stable counting sort of the (token, slot) pairs p = t*k + j by expert.

    Returns (cnt[E], off[E+1], perm[P]): cnt the pairs per expert, off the
    exclusive prefix sum, perm the pair ids grouped by expert in increasing
    pair order.  The pages only say that each token activates a few experts
    ([NULLBOT] "Architecture MoE et economies de parametres"); grouping tokens by
    expert is how a sparse dispatch gathers them.  Pinned: numpy's stable
    argsort, bincount.
    """
    idx_flat = np.asarray(idx_flat).ravel()
    P = idx_flat.size
    cnt = np.zeros(E, dtype=np.int32)
    for p in range(P):
        cnt[idx_flat[p]] += 1
    off = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        off[e + 1] = off[e] + cnt[e]
    nxt = off[:E].copy()
    perm = np.empty(P, dtype=np.int32)
    for p in range(P):
        e = idx_flat[p]
        perm[nxt[e]] = p
        nxt[e] += 1
    return cnt, off, perm


def swiglu_expert(xh_rows, w_gate, w_up, w_down, store) -> np.ndarray:
    """One expert on a set of token rows: y = Wd store(silu(Wg xh) * (Wu xh)).

    R2 rounds the activation a.  silu(v) = v / (1 + exp(-v)).  Pinned: the
    single-expert special case equals a textbook SwiGLU MLP built from
    torch.nn.functional.silu on the CPU.
    """
    xh_rows = as_f32(xh_rows)
    g = xh_rows @ as_f32(w_gate).T
    u = xh_rows @ as_f32(w_up).T
    a = store((g / (F32(1.0) + np.exp(-g)) * u).astype(F32))
    return (a @ as_f32(w_down).T).astype(F32, copy=False)


@dataclass
class BlockResult:
    x_out: np.ndarray   # [T, H] block output (R3)
    m: np.ndarray       # [T, H] float32 MoE output before the residual add
    idx: np.ndarray     # [T, k] int32 selected experts, descending logit
    w: np.ndarray       # [T, k] float32 gate weights
    z: np.ndarray       # [T, E] float32 router logits
    cnt: np.ndarray
    off: np.ndarray
    perm: np.ndarray


def moe_block(x, lw: dict, shp: Shape) -> BlockResult:
    """One MoE-FFN block, sparse dispatch: x' = store(x + MoE(RMSNorm(x))).

    lw holds this layer's tensors: gamma [H], router [E,H], gate/up [E,I,H],
    down [E,H,I], s_gate/s_up [S,I,H], s_down [S,H,I].
    Shared experts see every token with weight 1; each token's routed experts
    are combined with their gate weights, in ascending expert order, after the
    shared experts ([CLAWPIT] "Lean architecture...": routed and shared
    experts, top-6).
    """
    store = storage_round(shp.dtype)
    x = as_f32(x)
    T = x.shape[0]
    k = shp.k
    xh = rmsnorm(x, lw["gamma"], shp.eps, store)                  # R1
    z = router_logits(xh, lw["router"])
    idx, w = topk_select(z, k)
    cnt, off, perm = counting_sort(idx.ravel(), shp.E)

    y_routed = np.zeros((T * k, shp.H), dtype=F32)
    for e in range(shp.E):
        pairs = perm[off[e]:off[e + 1]]
        if pairs.size == 0:
            continue
        tokens = pairs // k
        y_routed[pairs] = swiglu_expert(xh[tokens], lw["gate"][e], lw["up"][e],
                                        lw["down"][e], store)

    m = np.zeros((T, shp.H), dtype=F32)
    for s in range(shp.S):
        m = m + swiglu_expert(xh, lw["s_gate"][s], lw["s_up"][s], lw["s_down"][s], store)
    # routed contributions of each token in ascending expert order
    asc = np.argsort(idx, axis=1, kind="stable")
    rows = np.arange(T)
    for jj in range(k):
        j = asc[:, jj]
        m = m + w[rows, j][:, None] * y_routed[rows * k + j]
    x_out = store((x + m).astype(F32))                            # R3
    return BlockResult(x_out, m.astype(F32), idx, w, z, cnt, off, perm)


def moe_block_dense(x, lw: dict, shp: Shape):
    """The same block computed densely: every expert on every token, times a
    gate matrix that is zero outside each token's selection, summed in
    ascending expert order.  Used only to pin moe_block (the sparse dispatch
    must give the same m)."""
    store = storage_round(shp.dtype)
    x = as_f32(x)
    T = x.shape[0]
    xh = rmsnorm(x, lw["gamma"], shp.eps, store)
    z = router_logits(xh, lw["router"])
    idx, w = topk_select(z, shp.k)
    G = np.zeros((T, shp.E), dtype=F32)
    np.put_along_axis(G, idx, w, axis=1)
    m = np.zeros((T, shp.H), dtype=F32)
    for s in range(shp.S):
        m = m + swiglu_expert(xh, lw["s_gate"][s], lw["s_up"][s], lw["s_down"][s], store)
    for e in range(shp.E):
        y = swiglu_expert(xh, lw["gate"][e], lw["up"][e], lw["down"][e], store)
        m = m + G[:, e:e + 1] * y
    return store((x + m).astype(F32)), m


def lm_head_logits(x, gamma_f, w_lm, eps: float, store) -> np.ndarray:
    """Final RMSNorm (R1) then logits l[t, v] = sum_h xf[t, h] * W_lm[v, h], float32."""
    xf = rmsnorm(x, gamma_f, eps, store)
    return (xf @ as_f32(w_lm).T).astype(F32, copy=False)


def greedy_pick(logits: np.ndarray) -> np.ndarray:
    """The verifier's greedy token: arg-max logit, lowest token id on ties
    ([JINA-FR] "Modele et entrainement": the verifier checks greedily)."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def accept_prefix(tstar: np.ndarray, drafts: np.ndarray):
    """Longest-prefix acceptance plus one verifier token.

    tstar [B, K+1]: verifier picks after each of the K+1 input positions;
    drafts [B, K]: draft j proposes the token at input position j+1.
    a_b = number of leading j with drafts[b, j] == tstar[b, j];
    committed[b, :a_b+1] = tstar[b, :a_b+1], the rest -1; counts[b] = a_b + 1.
    When all K drafts match, the extra token tstar[b, K] is the bonus
    ([CLAWPIT] "Speculative decoding without accuracy loss").
    Pinned: exhaustive enumeration of all 2^K correctness patterns, K = 0,
    and greedy-equivalence of a toy decode loop.
    """
    tstar = np.asarray(tstar, dtype=np.int64)
    drafts = np.asarray(drafts, dtype=np.int64)
    B, K1 = tstar.shape
    K = K1 - 1
    committed = np.full((B, K1), -1, dtype=np.int32)
    counts = np.zeros(B, dtype=np.int32)
    for b in range(B):
        a = 0
        while a < K and drafts[b, a] == tstar[b, a]:
            a += 1
        committed[b, :a + 1] = tstar[b, :a + 1]
        counts[b] = a + 1
    return committed, counts


@dataclass
class StepResult:
    committed: np.ndarray       # [B, K+1] int32
    counts: np.ndarray          # [B] int32
    tstar: np.ndarray           # [T] int32 (None without an LM head)
    blocks: list                # BlockResult per layer
    hidden_out: np.ndarray      # [T, H] residual stream after the last block
    logits: np.ndarray | None   # [T, V] float32 when kept


def verify_step(shp: Shape, weights: dict, hidden, drafts, B: int, K: int,
                keep_logits: bool = False, has_lm_head: bool = True) -> StepResult:
    """One speculative verification step over B sequences x (K+1) positions.

    hidden [B*(K+1), H]: the residual stream entering the first MoE block for
    the last committed token and the K drafts of each sequence; drafts [B, K].
    Runs L blocks, the final norm, the LM head and greedy pick, and prefix
    acceptance.  weights: 'layers' (list of per-layer dicts, see moe_block),
    'final_gamma' [H], 'lm_head' [V, H].
    """
    x = as_f32(hidden)
    assert x.shape == (B * (K + 1), shp.H)
    blocks = []
    for l in range(shp.L):
        r = moe_block(x, weights["layers"][l], shp)
        blocks.append(r)
        x = r.x_out
    if not has_lm_head:
        return StepResult(None, None, None, blocks, x, None)
    store = storage_round(shp.dtype)
    logits = lm_head_logits(x, weights["final_gamma"], weights["lm_head"], shp.eps, store)
    tstar = greedy_pick(logits)
    if K > 0:
        committed, counts = accept_prefix(tstar.reshape(B, K + 1), np.asarray(drafts).reshape(B, K))
    else:
        committed, counts = accept_prefix(tstar.reshape(B, 1), np.zeros((B, 0), np.int32))
    return StepResult(committed, counts, tstar, blocks, x, logits if keep_logits else None)


# --------------------------------------------------------------------------
# Margins (used to seed inputs whose discrete outputs are well separated)
# --------------------------------------------------------------------------

def topk_margin(z: np.ndarray, k: int) -> np.ndarray:
    """z_(k) - z_(k+1) per row: the gap between the last selected and the first
    unselected logit."""
    zs = -np.sort(-np.asarray(z, dtype=F32), axis=1)
    return zs[:, k - 1] - zs[:, k]


def argmax_margin(logits: np.ndarray) -> np.ndarray:
    """l_(1) - l_(2) per row."""
    part = -np.partition(-np.asarray(logits, dtype=F32), 1, axis=1)[:, :2]
    return part[:, 0] - part[:, 1]


# --------------------------------------------------------------------------
# Decode-loop measures as the pages define them
# --------------------------------------------------------------------------

def tau(counts) -> float:
    """Mean tokens committed per speculative step, bonus token included
    ([JINA-FR] "Decodage speculatif sur un L4", caption of the lost table)."""
    return float(np.mean(np.asarray(counts, dtype=np.float64)))


def acceptance_rate(tau_value: float, K: int) -> float:
    """Accepted drafts over proposed drafts, (tau - 1) / K.  With the pages'
    tau = 2.73 at K = 3 this is the 57.6 % quoted with the L4 speed-up
    ([CLAWPIT] "High throughput on cheap hardware")."""
    return (tau_value - 1.0) / K


def step_cost(tau_value: float, speedup: float) -> float:
    """c = tau / S: the cost of a speculative step in autoregressive-step
    units, S being the speed-up over greedy decoding ([JINA-FR] "Decodage
    speculatif sur un L4"; S is not defined on the page, the printed c values
    fix it as the speed-up)."""
    return tau_value / speedup


def expected_counts_independent(p: float, K: int) -> float:
    """E[counts] when each draft is correct independently with probability p:
    1 + p + p^2 + ... + p^K."""
    return float(sum(p ** i for i in range(K + 1)))
