"""Pins of the draft-head oracle (oracle/draft_oracle.py) to things other than
itself: constructions whose drafts follow in closed form, torch's own layer
routines, brute force, and the verify oracle.  No GPU needed.

The permutation construction: embedding rows are orthogonal with mean square 1
(so RMSNorm with unit gain leaves them unchanged), the head is the embedding
table, and one half of the projection maps row v's direction onto row
sigma(v)'s.  With the FFN's down projection zero the block's output is then
E[sigma(.)] and the head picks sigma(.) by a wide margin, so the K drafts are
sigma, sigma^2, sigma^3 of the input -- only if every step continues from the
block's own previous output (and token), not from the verifier's state.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import draft_oracle as D

rng = np.random.default_rng(4242)
F = torch.nn.functional


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _random_draft(H=128, Id=256, V=300, subset=None, dtype="bf16", scale=0.05):
    dw = dict(embed=rng.standard_normal((V, H)).astype(np.float32),
              gamma_h=(1 + 0.2 * rng.uniform(-1, 1, H)).astype(np.float32),
              gamma_e=(1 + 0.2 * rng.uniform(-1, 1, H)).astype(np.float32),
              gamma_f=(1 + 0.2 * rng.uniform(-1, 1, H)).astype(np.float32),
              gamma_o=(1 + 0.2 * rng.uniform(-1, 1, H)).astype(np.float32),
              w_proj=(rng.standard_normal((H, 2 * H)) * scale).astype(np.float32),
              w_gate=(rng.standard_normal((Id, H)) * scale).astype(np.float32),
              w_up=(rng.standard_normal((Id, H)) * scale).astype(np.float32),
              w_down=(rng.standard_normal((H, Id)) * scale).astype(np.float32),
              lm=(rng.standard_normal((V, H)) * scale).astype(np.float32))
    if dtype == "bf16":
        dw = {k: _bf16(v) for k, v in dw.items()}
    lm = dw.pop("lm")
    if subset is None:
        dw["head"] = lm
        Vd = V
    else:
        ids = np.sort(rng.choice(V, size=subset, replace=False)).astype(np.int32)
        dw["head"], dw["head_ids"] = lm[ids], ids
        Vd = subset
    return dw, D.DraftShape(H=H, Id=Id, V=V, Vd=Vd, dtype=dtype), lm


# ------------------------------------------------- permutation construction ----

def _perm_setup(H=64, V=40, half="h", seed=0):
    r = np.random.default_rng(seed)
    q, _ = np.linalg.qr(r.standard_normal((H, H)))
    E = (q[:V] * np.sqrt(H)).astype(np.float32)          # orthogonal rows, mean square 1
    sigma = r.permutation(V)
    P = sum(np.outer(E[sigma[v]], E[v]) for v in range(V)) / H   # P E[v] = E[sigma(v)]
    Z = np.zeros((H, H))
    w_proj = np.concatenate([P, Z] if half == "h" else [Z, P], axis=1).astype(np.float32)
    one = np.ones(H, np.float32)
    Id = 32
    dw = dict(embed=E, gamma_h=one, gamma_e=one, gamma_f=one, gamma_o=one, w_proj=w_proj,
              w_gate=r.standard_normal((Id, H)).astype(np.float32),
              w_up=r.standard_normal((Id, H)).astype(np.float32),
              w_down=np.zeros((H, Id), np.float32), head=E)
    return dw, D.DraftShape(H=H, Id=Id, V=V, Vd=V, dtype="bf16"), E, sigma


def _sigma_pow(sigma, t, j):
    for _ in range(j):
        t = sigma[t]
    return t


@pytest.mark.parametrize("K", [1, 2, 3, 5])
def test_hidden_feedback_gives_sigma_powers(K):
    """Projection acts on the h half only: drafts are sigma^j(t*) for h0 along
    E[t*], whatever the input tokens are."""
    dw, shp, E, sigma = _perm_setup(half="h")
    B = 6
    tstar = rng.integers(0, shp.V, B)
    h0 = E[tstar] * rng.uniform(0.5, 3.0, (B, 1)).astype(np.float32)   # any positive scale
    t0 = rng.integers(0, shp.V, B)
    got = D.draft_chain(h0, t0, K, dw, shp).drafts
    want = np.array([[_sigma_pow(sigma, t, j + 1) for j in range(K)] for t in tstar])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("K", [1, 3])
def test_token_feedback_gives_sigma_powers(K):
    """Projection acts on the token half only: drafts are sigma^j(t0); the
    hidden input is irrelevant and each step embeds the previous step's pick."""
    dw, shp, E, sigma = _perm_setup(half="e", seed=1)
    B = 5
    t0 = rng.integers(0, shp.V, B)
    h0 = rng.standard_normal((B, shp.H)).astype(np.float32)
    got = D.draft_chain(h0, t0, K, dw, shp).drafts
    want = np.array([[_sigma_pow(sigma, t, j + 1) for j in range(K)] for t in t0])
    assert np.array_equal(got, want)


# ------------------------------------------------------ torch layer routines ----

def _torch_step(h, tok, dw, shp):
    T = lambda a: torch.from_numpy(np.asarray(a, np.float32))
    rb = (lambda t: t.to(torch.bfloat16).to(torch.float32)) if shp.dtype == "bf16" else (lambda t: t)
    H = shp.H
    tk = torch.from_numpy(np.asarray(tok, np.int64))
    emb = F.embedding(tk.clamp(0, shp.V - 1), T(dw["embed"])) * ((tk >= 0) & (tk < shp.V)).float()[:, None]
    a = rb(F.rms_norm(T(h), (H,), T(dw["gamma_h"]), shp.eps))
    e = rb(F.rms_norm(emb, (H,), T(dw["gamma_e"]), shp.eps))
    u = rb(F.linear(torch.cat([a, e], 1), T(dw["w_proj"])))
    uh = rb(F.rms_norm(u, (H,), T(dw["gamma_f"]), shp.eps))
    act = rb(F.silu(F.linear(uh, T(dw["w_gate"]))) * F.linear(uh, T(dw["w_up"])))
    v = rb(u + F.linear(act, T(dw["w_down"])))
    logits = F.linear(rb(F.rms_norm(v, (H,), T(dw["gamma_o"]), shp.eps)), T(dw["head"]))
    return u.numpy(), v.numpy(), logits.numpy()


def _close(got, ref, dtype):
    if dtype == "f32":
        np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-5)
    else:
        # rounding points may fall on the other side of a bf16 tie now and then
        rel = np.abs(got - ref).mean() / np.abs(ref).mean()
        assert rel < 2e-3, rel
        assert np.mean(np.abs(got - ref) > 1e-2 * np.abs(ref) + 1e-3) < 0.01


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_matches_torch_layers(dtype):
    dw, shp, _ = _random_draft(dtype=dtype)
    B = 24
    h = rng.standard_normal((B, shp.H)).astype(np.float32)
    if dtype == "bf16":
        h = _bf16(h)
    tok = rng.integers(0, shp.V, B)
    tok[:2] = [-1, shp.V]                                  # the zero-embedding rule
    r = D.draft_block(h, tok, dw, shp)
    u, v, logits = _torch_step(h, tok, dw, shp)
    _close(r.u, u, dtype)
    _close(r.v, v, dtype)
    _close(r.logits, logits, dtype)
    decided = O.argmax_margin(logits) > 1e-2
    assert decided.sum() > B // 2
    assert np.array_equal(r.tokens[decided], np.argmax(logits, 1)[decided])


def test_invalid_token_is_a_zero_embedding():
    """An id outside [0, V) contributes nothing: the same as a valid token with
    the token half of the projection zeroed."""
    dw, shp, _ = _random_draft(dtype="f32")
    h = rng.standard_normal((3, shp.H)).astype(np.float32)
    bad = D.draft_block(h, np.array([-1, shp.V, 10 ** 6]), dw, shp)
    dz = dict(dw, w_proj=np.concatenate([dw["w_proj"][:, :shp.H], np.zeros((shp.H, shp.H), np.float32)], 1))
    ref = D.draft_block(h, np.array([0, 1, 2]), dz, shp)
    np.testing.assert_array_equal(bad.u, ref.u)
    np.testing.assert_array_equal(bad.v, ref.v)


# ---------------------------------------------------------- head subset ----

def test_head_subset_pick_is_bruteforce_best_row():
    dw, shp, lm = _random_draft(subset=97)
    B = 16
    h = _bf16(rng.standard_normal((B, shp.H)).astype(np.float32))
    tok = rng.integers(0, shp.V, B)
    r = D.draft_block(h, tok, dw, shp)
    xf = O.rmsnorm(r.v, dw["gamma_o"], shp.eps, O.bf16_round).astype(np.float64)
    for b in range(B):
        best, arg = -np.inf, -1
        for i, t in enumerate(dw["head_ids"]):          # rows in subset order, first best wins
            s = float(xf[b] @ lm[t].astype(np.float64))
            if s > best + 1e-4:
                best, arg = s, int(t)
        if O.argmax_margin(r.logits[b:b + 1])[0] > 1e-3:
            assert r.tokens[b] == arg


def test_head_ties_go_to_the_lower_row():
    dw, shp, lm = _random_draft(subset=50, dtype="f32")
    dw["head"] = dw["head"].copy()
    h = rng.standard_normal((4, shp.H)).astype(np.float32)
    r0 = D.draft_block(h, np.zeros(4, np.int64), dw, shp)
    rows = np.argmax(r0.logits, 1)
    # duplicate each winning row to every later row position: ties everywhere after it
    dup = dict(dw, head=np.repeat(dw["head"][rows[:1]], shp.Vd, axis=0))
    r1 = D.draft_block(h[:1], np.zeros(1, np.int64), dup, shp)
    assert r1.tokens[0] == dw["head_ids"][0]


def test_full_head_equals_subset_with_every_row():
    dw, shp, lm = _random_draft(dtype="bf16")
    sub = dict(dw, head_ids=np.arange(shp.V, dtype=np.int32))
    h = _bf16(rng.standard_normal((8, shp.H)).astype(np.float32))
    tok = rng.integers(0, shp.V, 8)
    a = D.draft_chain(h, tok, 3, dw, shp).drafts
    b = D.draft_chain(h, tok, 3, sub, shp).drafts
    assert np.array_equal(a, b)


# --------------------------------------------------- hand-off from verify ----

def test_continue_from_verify_takes_the_row_of_the_last_pick():
    """The token handed to the draft is the verifier's greedy pick at the
    hidden row handed over: recompute it from that row through the verifier's
    own final norm and LM head."""
    H, V, B, K = 64, 200, 12, 3
    shp = O.Shape(H=H, E=4, k=2, S=1, I=32, V=V, dtype="bf16")
    lw = {k: _bf16(v) for k, v in dict(
        gamma=np.ones(H, np.float32),
        router=rng.standard_normal((4, H)).astype(np.float32) * 0.1,
        gate=rng.standard_normal((4, 32, H)).astype(np.float32) * 0.1,
        up=rng.standard_normal((4, 32, H)).astype(np.float32) * 0.1,
        down=rng.standard_normal((4, H, 32)).astype(np.float32) * 0.1,
        s_gate=rng.standard_normal((1, 32, H)).astype(np.float32) * 0.1,
        s_up=rng.standard_normal((1, 32, H)).astype(np.float32) * 0.1,
        s_down=rng.standard_normal((1, H, 32)).astype(np.float32) * 0.1).items()}
    weights = dict(layers=[lw], final_gamma=np.ones(H, np.float32),
                   lm_head=_bf16(rng.standard_normal((V, H)).astype(np.float32)))
    x = _bf16(rng.standard_normal((B * (K + 1), H)).astype(np.float32))
    first = O.verify_step(shp, weights, x, np.zeros((B, K), np.int32), B, K)
    # drafts equal to the greedy picks for a random number of leading positions
    n_ok = rng.integers(0, K + 1, B)
    ts = first.tstar.reshape(B, K + 1)
    drafts = np.where(np.arange(K)[None, :] < n_ok[:, None], ts[:, :K], (ts[:, :K] + 1) % V).astype(np.int32)
    res = O.verify_step(shp, weights, x, drafts, B, K)
    assert np.array_equal(res.counts, n_ok + 1)
    h, t = D.continue_from_verify(res.hidden_out, res.committed, res.counts, K + 1)
    logits = O.lm_head_logits(h, weights["final_gamma"], weights["lm_head"], shp.eps, O.bf16_round)
    assert np.array_equal(t, O.greedy_pick(logits))
    assert np.array_equal(t, res.committed[np.arange(B), res.counts - 1])
    # without counts: the last position of each sequence
    h2, t2 = D.continue_from_verify(res.hidden_out, res.tstar.reshape(B, K + 1), None, K + 1)
    assert np.array_equal(h2, res.hidden_out[np.arange(B) * (K + 1) + K])


# ---------------------------------------------------------- sensitivity ----

def test_sensitivity_pins_reject_planted_mistakes():
    """Plausible mistakes, planted in copies of the oracle's steps, fail the pins."""
    dw, shp, E, sigma = _perm_setup(half="h")
    B, K = 6, 3
    tstar = rng.integers(0, shp.V, B)
    h0 = E[tstar]
    t0 = rng.integers(0, shp.V, B)
    want = np.array([[_sigma_pow(sigma, t, j + 1) for j in range(K)] for t in tstar])
    # (1) every step reset onto the verifier's state (MTP semantics)
    reset = np.stack([D.draft_block(h0, t0, dw, shp).tokens for _ in range(K)], 1)
    assert not np.array_equal(reset, want)
    # (2) projection halves swapped: the h half acts on the token embedding
    swapped = dict(dw, w_proj=np.concatenate([dw["w_proj"][:, shp.H:], dw["w_proj"][:, :shp.H]], 1))
    assert not np.array_equal(D.draft_chain(h0, t0, K, swapped, shp).drafts, want)
    # (3) FFN without its residual add differs from torch's layers
    rdw, rshp, _ = _random_draft(dtype="f32")
    h = rng.standard_normal((8, rshp.H)).astype(np.float32)
    tok = rng.integers(0, rshp.V, 8)
    r = D.draft_block(h, tok, rdw, rshp)
    uh = O.rmsnorm(r.u, rdw["gamma_f"], rshp.eps, O.storage_round("f32"))
    g, up = uh @ rdw["w_gate"].T, uh @ rdw["w_up"].T
    no_res = (g / (1 + np.exp(-g)) * up) @ rdw["w_down"].T
    _, v_ref, _ = _torch_step(h, tok, rdw, rshp)
    assert np.abs(no_res - v_ref).max() > 1e-2
    # (4) the FFN normalised with the h gain instead of its own
    wrong = dict(rdw, gamma_f=rdw["gamma_h"])
    assert np.abs(D.draft_block(h, tok, wrong, rshp).v - v_ref).max() > 1e-3
