"""CPU oracle for the FastMTP draft head: one dense block applied recursively.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library.

What the pages fix (short keys as in moe_oracle):
  * one dense ("compressed") draft block is applied recursively for K = 3
    prediction steps, so the draft parameters do not grow with the depth
    ([CLAWPIT] "Speculative decoding without accuracy loss"; [JINA-FR] "Modele
    et entrainement");
  * the block was trained with recursive hidden-state feedback: each draft step
    continues from the block's own previous output, it is not reset onto the
    verifier's state at every step (the serving engine must register it as an
    eagle-style head rather than an MTP head; [JINA-FR] "Pour commencer");
  * the verifier checks the drafts greedily and commits the longest agreeing
    prefix plus one token of its own ([CLAWPIT] same section).

What the pages leave open and this oracle reads plainly (each reading is also
listed in the repository's design notes):
  * a draft step takes the hidden state h it continues from and the token t
    whose successor it predicts, normalises both (separate RMSNorm gains; the
    token enters through an embedding table), projects their concatenation
    [norm(h); norm(E[t])] from 2H to H, and runs a pre-norm dense SwiGLU FFN
    with a residual add on the result; attention is not part of the block
    here (the verifier's attention is not on the pages either);
  * the step's output v is the next step's h; its token is the arg-max of the
    verifier's LM head (shared weights) over RMSNorm(v) with the draft's own
    output gain, lowest row on ties; an optional list of vocabulary rows
    restricts the draft head to those rows (the pick is the row's token id);
  * the first step continues from the verifier: h is the verifier's residual
    stream after its last block at the position whose greedy pick was the last
    committed token, t is that token;
  * a token id outside [0, V) embeds as the zero vector.

Precision, as in moe_oracle: float32 arithmetic; with bfloat16 storage the
values are rounded to bfloat16 at these points only:
  R1  every normalised activation (norm(h), norm(E[t]), the FFN input, the
      head input),
  R2  the SwiGLU activation,
  R3  the projected state u and the step output v (residual-stream values).

Pins live in tests/test_draft_oracle_pins.py.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .moe_oracle import F32, as_f32, greedy_pick, rmsnorm, storage_round


@dataclass(frozen=True)
class DraftShape:
    """H hidden, Id dense SwiGLU width, V verifier vocabulary (embedding rows),
    Vd draft-head rows (V when the head is the verifier's whole LM head)."""

    H: int
    Id: int
    V: int
    Vd: int
    eps: float = 1e-6
    dtype: str = "bf16"


def embed(tokens, table) -> np.ndarray:
    """E[t] per token; ids outside [0, V) give the zero vector (the library's
    rule for an invalid id, not on the pages)."""
    tokens = np.asarray(tokens, dtype=np.int64).ravel()
    table = as_f32(table)
    V, H = table.shape
    out = np.zeros((tokens.size, H), dtype=F32)
    ok = (tokens >= 0) & (tokens < V)
    out[ok] = table[tokens[ok]]
    return out


def head_pick(v, dw: dict, shp: DraftShape, store):
    """Token predicted from step output v: RMSNorm with the output gain (R1),
    logits over the draft head's rows, arg-max (lowest row on ties), mapped to
    the row's token id.  Returns (tokens, logits)."""
    xf = rmsnorm(v, dw["gamma_o"], shp.eps, store)
    logits = (xf @ as_f32(dw["head"]).T).astype(F32, copy=False)
    rows = greedy_pick(logits)
    ids = dw.get("head_ids")
    tok = rows if ids is None else np.asarray(ids, dtype=np.int32)[rows]
    return tok.astype(np.int32), logits


@dataclass
class DraftStepResult:
    u: np.ndarray        # [B, H] projected state (R3)
    v: np.ndarray        # [B, H] step output, the next step's h (R3)
    tokens: np.ndarray   # [B] int32 predicted tokens
    logits: np.ndarray   # [B, Vd] float32


def draft_block(h, tokens, dw: dict, shp: DraftShape) -> DraftStepResult:
    """One application of the draft block ([CLAWPIT] "Speculative decoding
    without accuracy loss": one block, applied once per prediction step).

    dw: embed [V, H], gamma_h, gamma_e, gamma_f, gamma_o [H], w_proj [H, 2H]
    (columns 0..H-1 act on norm(h), H..2H-1 on norm(E[t])), w_gate, w_up
    [Id, H], w_down [H, Id], head [Vd, H], head_ids [Vd] or absent.
    """
    store = storage_round(shp.dtype)
    h = as_f32(h)
    a = rmsnorm(h, dw["gamma_h"], shp.eps, store)                        # R1
    e = rmsnorm(embed(tokens, dw["embed"]), dw["gamma_e"], shp.eps, store)  # R1
    x = np.concatenate([a, e], axis=1)
    u = store((x @ as_f32(dw["w_proj"]).T).astype(F32))                  # R3
    uh = rmsnorm(u, dw["gamma_f"], shp.eps, store)                       # R1
    g = uh @ as_f32(dw["w_gate"]).T
    up = uh @ as_f32(dw["w_up"]).T
    act = store((g / (F32(1.0) + np.exp(-g)) * up).astype(F32))          # R2
    v = store((u + act @ as_f32(dw["w_down"]).T).astype(F32))            # R3
    tok, logits = head_pick(v, dw, shp, store)
    return DraftStepResult(u, v, tok, logits)


@dataclass
class DraftChainResult:
    drafts: np.ndarray   # [B, K] int32: draft j proposes the token after position j
    states: list         # DraftStepResult per step


def draft_chain(h0, t0, K: int, dw: dict, shp: DraftShape) -> DraftChainResult:
    """K recursive draft steps with hidden-state feedback ([JINA-FR] "Pour
    commencer": each step continues from the block's own previous output).

    Step 1 takes (h0, t0); step j+1 takes step j's output v and its token.
    """
    h, t = as_f32(h0), np.asarray(t0, dtype=np.int32).ravel()
    B = h.shape[0]
    drafts = np.zeros((B, K), dtype=np.int32)
    states = []
    for j in range(K):
        r = draft_block(h, t, dw, shp)
        states.append(r)
        drafts[:, j] = r.tokens
        h, t = r.v, r.tokens
    return DraftChainResult(drafts, states)


def continue_from_verify(hidden_rows, committed, counts, R: int):
    """The state the first draft step continues from, per sequence b:
    position j = counts[b] - 1 (clamped into [0, R-1]) of the verifier's R
    positions, i.e. the position whose greedy pick was the last committed
    token; h = hidden_rows[b*R + j], t = committed[b, j].  counts None means
    j = R - 1.  (The pages say the verifier commits the agreeing prefix plus
    its own next token; which verifier state the next draft round starts from
    is this library's reading.)"""
    hidden_rows = as_f32(hidden_rows)
    committed = np.asarray(committed, dtype=np.int32).reshape(-1, R)
    B = committed.shape[0]
    if counts is None:
        j = np.full(B, R - 1, dtype=np.int64)
    else:
        j = np.clip(np.asarray(counts, dtype=np.int64) - 1, 0, R - 1)
    rows = np.arange(B) * R + j
    return hidden_rows[rows], committed[np.arange(B), j]
