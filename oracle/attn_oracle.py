"""CPU oracle for the attention sublayer and KV cache of the verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library.

What the pages fix: the decoder is DeepSeek-3B-MoE with 12 layers, 64 routed
and 2 shared experts, and a position limit of 32,768 ([CLAWPIT] "Lean
architecture with a compressed encoder"); a verify step checks K drafts per
sequence after the last committed token ([CLAWPIT] "Speculative decoding
without accuracy loss").  Nothing about attention is on the pages.

Readings (each also listed in the repository's design notes):
  * every layer is attention then MoE, both pre-norm with a residual add:
    x <- x + Attn(RMSNorm(x; gamma_a)); x <- x + MoE(RMSNorm(x));
  * multi-head attention with full-width projections W_q, W_k, W_v, W_o
    (H x H each): with them the decoder activates 0.574 B parameters per
    token, the pages' ~570 M ([CLAWPIT] same section), without them 0.50 B;
    heads of 128 (10 at H = 1280);
  * rotary position embedding in its original form: dimension pairs
    (2i, 2i+1) of every head rotated by pos * theta^(-2i/d), theta = 10,000;
  * a KV cache per layer and sequence: entries 0..P-1 hold the keys and
    values of the sequence's earlier positions; a verify step of sequence b
    starting at position p_b writes its K+1 keys and values at p_b..p_b+K and
    query j attends causally to positions 0..p_b+j; scores are q.k/sqrt(d),
    softmax in float32;
  * precision as in moe_oracle, float32 arithmetic, with bfloat16 storage
    rounding at: the normalised input (R1), q, k and v after the rotation
    (R4: k and v are what the cache holds), the attention output per head
    before W_o (R2), and the sublayer output x + o (R3).
  * angles: inverse frequencies computed in float64 and rounded to float32,
    angle = float32(float32(pos) * inv_freq), its cosine and sine evaluated
    accurately and rounded to float32.

Pins live in tests/test_attn_oracle_pins.py.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .moe_oracle import F32, Shape, accept_prefix, as_f32, greedy_pick, lm_head_logits, moe_block, rmsnorm, \
    storage_round


@dataclass(frozen=True)
class AttnShape:
    """H hidden, n_heads x d_head = H, P cache positions per sequence."""

    H: int
    n_heads: int
    d_head: int
    P: int
    theta: float = 10000.0
    eps: float = 1e-6
    dtype: str = "bf16"


def rope_angles(pos, d: int, theta: float) -> np.ndarray:
    """float32 angles [len(pos), d/2]: float32(pos) * float32(theta^(-2i/d))."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = (theta ** (-2.0 * i / d)).astype(F32)
    return (np.asarray(pos, dtype=F32)[:, None] * inv[None, :]).astype(F32)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate pairs (2i, 2i+1) of every head: x [T, nh, d], pos [T]."""
    x = as_f32(x)
    T, nh, d = x.shape
    ang = rope_angles(pos, d, theta).astype(np.float64)
    c = np.cos(ang).astype(F32)[:, None, :]
    s = np.sin(ang).astype(F32)[:, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def attend(q, kc, vc, n: int, d: int) -> np.ndarray:
    """One query row of one head over cache rows 0..n-1: softmax(K q / sqrt(d)) V,
    float32 (max-subtracted)."""
    s = (as_f32(kc[:n]) @ as_f32(q)).astype(F32) * F32(1.0 / np.sqrt(d))
    s = s - s.max()
    e = np.exp(s).astype(F32)
    w = e / e.sum(dtype=F32)
    return (w @ as_f32(vc[:n])).astype(F32)


@dataclass
class AttnResult:
    x_out: np.ndarray    # [T, H] sublayer output (R3)
    q: np.ndarray        # [T, H] rotated queries (R4)
    k: np.ndarray        # [T, H] rotated keys written to the cache (R4)
    v: np.ndarray        # [T, H] values written to the cache (R4)
    ctx: np.ndarray      # [T, H] attention output before W_o (R2)
    o: np.ndarray        # [T, H] float32 W_o ctx


def attn_sublayer(x, positions, B: int, K: int, kcache, vcache, lw: dict, ash: AttnShape) -> AttnResult:
    """x [B*(K+1), H] rows b*(K+1)+j; positions [B]; kcache / vcache [B, nh, P, d]
    (float32 values, updated in place at p_b..p_b+K); lw: attn_gamma [H], w_q,
    w_k, w_v, w_o [H, H]."""
    store = storage_round(ash.dtype)
    x = as_f32(x)
    T = B * (K + 1)
    nh, d = ash.n_heads, ash.d_head
    pos = (np.asarray(positions, dtype=np.int64)[:, None] + np.arange(K + 1)[None, :]).ravel()
    xh = rmsnorm(x, lw["attn_gamma"], ash.eps, store)                              # R1
    qf = (xh @ as_f32(lw["w_q"]).T).astype(F32).reshape(T, nh, d)
    kf = (xh @ as_f32(lw["w_k"]).T).astype(F32).reshape(T, nh, d)
    vf = (xh @ as_f32(lw["w_v"]).T).astype(F32).reshape(T, nh, d)
    q = store(rope(qf, pos, ash.theta))                                           # R4
    k = store(rope(kf, pos, ash.theta))
    v = store(vf)
    for t in range(T):
        b = t // (K + 1)
        kcache[b, :, pos[t]] = k[t]
        vcache[b, :, pos[t]] = v[t]
    ctx = np.zeros((T, nh, d), dtype=F32)
    for t in range(T):
        b = t // (K + 1)
        for h in range(nh):
            ctx[t, h] = attend(q[t, h], kcache[b, h], vcache[b, h], int(pos[t]) + 1, d)
    ctx = store(ctx.reshape(T, nh * d))                                             # R2
    o = (ctx @ as_f32(lw["w_o"]).T).astype(F32)
    x_out = store((x + o).astype(F32))                                              # R3
    return AttnResult(x_out, q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1), ctx, o)


@dataclass
class AttnStepResult:
    committed: np.ndarray
    counts: np.ndarray
    tstar: np.ndarray
    attn: list = field(default_factory=list)    # AttnResult per layer
    blocks: list = field(default_factory=list)  # moe_oracle.BlockResult per layer
    hidden_out: np.ndarray | None = None


def verify_step_attn(shp: Shape, ash: AttnShape, weights: dict, hidden, drafts, positions, caches: list,
                     B: int, K: int) -> AttnStepResult:
    """One verify step through L layers of attention + MoE, the final norm, the
    LM head and the acceptance.  caches[l] = (kcache, vcache) float32 arrays
    [B, nh, P, d], updated in place.  weights['layers'][l] holds the MoE
    tensors and attn_gamma, w_q, w_k, w_v, w_o."""
    x = as_f32(hidden)
    res = AttnStepResult(None, None, None)
    for l in range(shp.L):
        lw = weights["layers"][l]
        a = attn_sublayer(x, positions, B, K, caches[l][0], caches[l][1], lw, ash)
        res.attn.append(a)
        blk = moe_block(a.x_out, lw, shp)
        res.blocks.append(blk)
        x = blk.x_out
    res.hidden_out = x
    store = storage_round(shp.dtype)
    logits = lm_head_logits(x, weights["final_gamma"], weights["lm_head"], shp.eps, store)
    res.tstar = greedy_pick(logits)
    d = np.asarray(drafts, dtype=np.int32).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int32)
    res.committed, res.counts = accept_prefix(res.tstar.reshape(B, K + 1), d)
    return res
