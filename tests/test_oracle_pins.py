"""Pins of the CPU oracle to things other than itself: library routines on the
CPU, closed forms, brute force on tiny inputs, invariants the pages state, and
the numbers the pages print.  No GPU needed.

Each pin is chosen so a plausible mistake in the oracle (a dropped term, a wrong
sign or index, a transposed operand, a missing rounding point) fails it; the
`test_sensitivity_*` cases plant such mistakes in copies of the oracle's
functions and check that the pin rejects them.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_oracle as O
from moe_decoder_speculative_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ---------------------------------------------------------------- bf16 ----

def _torch_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_bf16_round_matches_torch_all_high_halves():
    """Every high half (all signs, exponents, mantissas) with low halves that hit
    each rounding case: exact, below/at/above the tie, odd/even kept bit."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF], np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    got = O.bf16_round(x)
    ref = _torch_bf16(x)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_round_matches_torch_random_bits():
    bits = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    got, ref = O.bf16_round(x), _torch_bf16(x)
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_widen_is_exact():
    u = np.arange(1 << 16, dtype=np.uint16)
    f = O.bf16_bits_to_f32(u)
    back = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    ok = ~np.isnan(back)
    assert np.array_equal(f[ok].view(np.uint32), back[ok].view(np.uint32))


# ------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_matches_torch_rms_norm():
    x = rng.standard_normal((64, 1280)).astype(np.float32) * 3
    g = (1 + 0.1 * rng.standard_normal(1280)).astype(np.float32)
    ours = O.rmsnorm(x, g, 1e-6, O.storage_round("f32"))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (1280,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(ours, ref, rtol=2e-6, atol=1e-6)


def test_rmsnorm_closed_form_constant_row():
    # x = c * 1  ->  xh = sign(c) / sqrt(1 + eps / c^2)
    for c in (0.5, -2.0, 7.0):
        x = np.full((1, 256), c, np.float32)
        xh = O.rmsnorm(x, np.ones(256, np.float32), 1e-6, O.storage_round("f32"))
        np.testing.assert_allclose(xh, np.sign(c) / np.sqrt(1 + 1e-6 / (c * c)), rtol=1e-6)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    x = rng.standard_normal((16, 1280)).astype(np.float32)
    xh = O.rmsnorm(x, np.ones(1280, np.float32), 1e-6, O.storage_round("f32"))
    np.testing.assert_allclose(np.mean(xh.astype(np.float64) ** 2, axis=1), 1.0, rtol=1e-5)
    xh2 = O.rmsnorm(4 * x, np.ones(1280, np.float32), 1e-6, O.storage_round("f32"))
    np.testing.assert_allclose(xh, xh2, rtol=1e-5)


def test_rmsnorm_rounds_once_to_bf16():
    x = rng.standard_normal((8, 256)).astype(np.float32)
    xh = O.rmsnorm(x, np.ones(256, np.float32), 1e-6, O.storage_round("bf16"))
    exact = O.rmsnorm(x, np.ones(256, np.float32), 1e-6, O.storage_round("f32"))
    assert np.array_equal(xh, _torch_bf16(exact))


# --------------------------------------------------------------- top-k ----

def _brute_topk_set(z, k):
    best, best_set = -np.inf, None
    for sub in itertools.combinations(range(z.size), k):
        s = float(np.sum(z[list(sub)], dtype=np.float64))
        if s > best:
            best, best_set = s, set(sub)
    return best_set


def test_topk_brute_force_tiny():
    """All C(8,2) = 28 subsets: the selected pair is the one with the largest sum."""
    z = rng.standard_normal((200, 8)).astype(np.float32)
    idx, _ = O.topk_select(z, 2)
    for t in range(z.shape[0]):
        assert set(idx[t].tolist()) == _brute_topk_set(z[t], 2)


def test_topk_certificate_and_torch_topk():
    z = rng.standard_normal((500, 64)).astype(np.float32)
    idx, _ = O.topk_select(z, 6)
    for t in range(z.shape[0]):
        sel = np.zeros(64, bool)
        sel[idx[t]] = True
        assert z[t, sel].min() > z[t, ~sel].max()
        # descending order inside the selection
        assert np.all(np.diff(z[t, idx[t]]) <= 0)
    tv, ti = torch.topk(torch.from_numpy(z), 6, dim=1)
    assert np.array_equal(np.sort(ti.numpy(), 1), np.sort(idx, 1))


def test_topk_tie_break_lower_index_first():
    z = np.array([[1.0, 3.0, 3.0, 0.0, 3.0]], np.float32)
    idx, _ = O.topk_select(z, 2)
    assert idx.tolist() == [[1, 2]]


def test_gates_sum_to_one_and_ratio_closed_form():
    z = rng.standard_normal((300, 64)).astype(np.float32)
    idx, w = O.topk_select(z, 6)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)
    zs = np.take_along_axis(z, idx, 1).astype(np.float64)
    ratio = w[:, 1:] / w[:, :1]
    np.testing.assert_allclose(ratio, np.exp(zs[:, 1:] - zs[:, :1]), rtol=2e-6)
    ref = torch.softmax(torch.from_numpy(np.take_along_axis(z, idx, 1)), dim=1).numpy()
    np.testing.assert_allclose(w, ref, rtol=2e-6, atol=1e-7)


def test_gates_equal_renormalised_full_softmax():
    """Softmax over the selected logits equals softmax over all experts followed
    by renormalising the selected probabilities."""
    z = rng.standard_normal((100, 64)).astype(np.float32)
    idx, w = O.topk_select(z, 6)
    p = torch.softmax(torch.from_numpy(z).double(), 1).numpy()
    ps = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(w, ps / ps.sum(1, keepdims=True), rtol=3e-6)


# -------------------------------------------------------- permutation ----

def test_counting_sort_matches_stable_argsort():
    for E, P in ((8, 16), (64, 768), (64, 5000)):
        ids = rng.integers(0, E, P).astype(np.int32)
        cnt, off, perm = O.counting_sort(ids, E)
        assert np.array_equal(cnt, np.bincount(ids, minlength=E))
        assert off[0] == 0 and np.array_equal(np.diff(off), cnt)
        assert np.array_equal(perm, np.argsort(ids, kind="stable"))


def test_counting_sort_empty_experts():
    ids = np.array([3, 3, 0, 3], np.int32)
    cnt, off, perm = O.counting_sort(ids, 5)
    assert cnt.tolist() == [1, 0, 0, 3, 0]
    assert off.tolist() == [0, 1, 1, 1, 4, 4]
    assert perm.tolist() == [2, 0, 1, 3]


# ------------------------------------------------------------- experts ----

def _torch_swiglu(x, wg, wu, wd, bf16):
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float32)) for a in (x, wg, wu, wd))
    a = torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)
    if bf16:
        a = a.to(torch.bfloat16).to(torch.float32)
    return (a @ wd.T).numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_block_is_textbook_swiglu_mlp(dtype):
    """E = 1, k = 1, S = 0: the gate weight is exactly 1 and the block is
    x + SwiGLU(RMSNorm(x))."""
    H, I, T = 128, 96, 10
    g = np.random.default_rng(2024)  # its own stream: the draws do not depend on test order
    shp = O.Shape(H=H, E=1, k=1, S=0, I=I, V=16, dtype=dtype)
    lw = dict(gamma=np.ones(H, np.float32),
              router=g.standard_normal((1, H)).astype(np.float32) * 0.02,
              gate=g.standard_normal((1, I, H)).astype(np.float32) * 0.05,
              up=g.standard_normal((1, I, H)).astype(np.float32) * 0.05,
              down=g.standard_normal((1, H, I)).astype(np.float32) * 0.05,
              s_gate=np.zeros((0, I, H), np.float32), s_up=np.zeros((0, I, H), np.float32),
              s_down=np.zeros((0, H, I), np.float32))
    if dtype == "bf16":
        for key in ("router", "gate", "up", "down"):
            lw[key] = _torch_bf16(lw[key])
    x = g.standard_normal((T, H)).astype(np.float32)
    if dtype == "bf16":
        x = _torch_bf16(x)
    r = O.moe_block(x, lw, shp)
    assert np.all(r.w == 1.0)
    xn = torch.nn.functional.rms_norm(torch.from_numpy(x), (H,), eps=1e-6).numpy()
    if dtype == "bf16":
        xn = _torch_bf16(xn)
    ref = _torch_swiglu(xn, lw["gate"][0], lw["up"][0], lw["down"][0], dtype == "bf16")
    if dtype == "f32":
        np.testing.assert_allclose(r.m, ref, rtol=1e-4, atol=1e-6)
    else:
        # The oracle and torch add the projections' float32 products in
        # different orders, so an activation within an ulp of a bf16 rounding
        # boundary (the SwiGLU rounding point) can round the other way on one
        # side: that moves its token's row by ~2^-8 |a| |W_d| (1e-4 of the
        # row here), while a wrong operand or a missing norm moves it by O(1).
        row_rel = np.abs(r.m - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert row_rel.max() < 1e-3
        off = np.abs(r.m - ref) > 1e-6 + 1e-4 * np.abs(ref)
        assert off.mean() < 0.05


def _layer(H, E, S, I, scale=0.02, dtype="f32"):
    lw = dict(gamma=np.ones(H, np.float32),
              router=rng.standard_normal((E, H)).astype(np.float32) * scale,
              gate=rng.standard_normal((E, I, H)).astype(np.float32) * scale,
              up=rng.standard_normal((E, I, H)).astype(np.float32) * scale,
              down=rng.standard_normal((E, H, I)).astype(np.float32) * scale,
              s_gate=rng.standard_normal((S, I, H)).astype(np.float32) * scale,
              s_up=rng.standard_normal((S, I, H)).astype(np.float32) * scale,
              s_down=rng.standard_normal((S, H, I)).astype(np.float32) * scale)
    if dtype == "bf16":
        lw = {k: _torch_bf16(v) for k, v in lw.items()}
    return lw


@pytest.mark.parametrize("dtype,E,k,S", [("f32", 8, 2, 1), ("bf16", 16, 4, 2), ("bf16", 64, 6, 2)])
def test_sparse_dispatch_equals_dense_all_experts_times_mask(dtype, E, k, S):
    H, I, T = 128, 64, 40
    shp = O.Shape(H=H, E=E, k=k, S=S, I=I, V=16, dtype=dtype)
    lw = _layer(H, E, S, I, dtype=dtype)
    x = rng.standard_normal((T, H)).astype(np.float32)
    r = O.moe_block(x, lw, shp)
    xd, md = O.moe_block_dense(x, lw, shp)
    if dtype == "f32":
        np.testing.assert_allclose(r.m, md, rtol=2e-6, atol=2e-7)
    else:
        # The dense path runs each expert's products over all T rows, the
        # sparse one over the expert's own rows: BLAS blocks the two sums
        # differently, so an activation within an ulp of a bf16 rounding
        # boundary (the SwiGLU rounding point) can round the other way on one
        # side.  One such flip moves m by 2^-8 |a| |W_d| w (~1e-6 here); a
        # dropped expert or a wrong gate moves a row by a large fraction.
        off = np.abs(r.m - md) > 2e-7 + 2e-6 * np.abs(md)
        assert off.mean() < 1e-2
        row_rel = np.abs(r.m - md).max(axis=1) / np.abs(md).max(axis=1)
        assert row_rel.max() < 1e-3
    if dtype == "bf16":
        # R3 may land on the other side of a bf16 tie only if m moved by an ulp
        assert np.mean(r.x_out != xd) < 1e-3
    else:
        np.testing.assert_allclose(r.x_out, xd, rtol=2e-6, atol=2e-7)


def test_block_per_token_loop_reference():
    """The block row by row with explicit Python loops over experts."""
    H, E, k, S, I, T = 64, 8, 2, 1, 32, 6
    shp = O.Shape(H=H, E=E, k=k, S=S, I=I, V=16, dtype="f32")
    lw = _layer(H, E, S, I, scale=0.1)
    x = rng.standard_normal((T, H)).astype(np.float32)
    r = O.moe_block(x, lw, shp)
    for t in range(T):
        xt = x[t].astype(np.float64)
        xh = xt / np.sqrt(np.mean(xt * xt) + 1e-6)
        z = lw["router"].astype(np.float64) @ xh
        sel = sorted(range(E), key=lambda e: (-z[e], e))[:k]
        g = np.exp(z[sel] - z[sel].max())
        g /= g.sum()

        def mlp(wg, wu, wd):
            gg = wg.astype(np.float64) @ xh
            uu = wu.astype(np.float64) @ xh
            return wd.astype(np.float64) @ (gg / (1 + np.exp(-gg)) * uu)

        m = sum(mlp(lw["s_gate"][s], lw["s_up"][s], lw["s_down"][s]) for s in range(S))
        for e, ge in zip(sel, g):
            m = m + ge * mlp(lw["gate"][e], lw["up"][e], lw["down"][e])
        assert sorted(r.idx[t].tolist()) == sorted(sel)
        np.testing.assert_allclose(r.m[t], m, rtol=1e-4, atol=1e-6)
        np.testing.assert_allclose(r.x_out[t], xt + m, rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------- head ----

def test_lm_head_argmax_first_occurrence_and_loop():
    H, V, T = 64, 300, 12
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((V, H)) * 0.05).astype(np.float32)
    lg = O.lm_head_logits(x, np.ones(H, np.float32), W, 1e-6, O.storage_round("f32"))
    t = O.greedy_pick(lg)
    for i in range(T):
        best = 0
        for v in range(1, V):
            if lg[i, v] > lg[i, best]:
                best = v
        assert t[i] == best
    assert np.array_equal(t, torch.argmax(torch.from_numpy(lg), 1).numpy())
    tie = np.array([[0.0, 2.0, 2.0, 1.0]], np.float32)
    assert O.greedy_pick(tie)[0] == 1


def _torch_head_logits(x, gamma, W, eps, bf16):
    """Final norm and logits with torch's CPU routines: F.rms_norm in float32,
    the bf16 rounding of its output when the storage is bf16, then F.linear in
    float64 on those values."""
    import torch.nn.functional as F
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    xf = F.rms_norm(xt, (xt.shape[1],), weight=torch.from_numpy(np.asarray(gamma, np.float32)), eps=eps)
    if bf16:
        xf = xf.to(torch.bfloat16).to(torch.float32)
    return F.linear(xf.double(), torch.from_numpy(np.asarray(W, np.float64))).numpy()


def _head_mismatch(got, ref):
    """(fraction of logits off by more than 1e-5 of the logit scale, largest
    difference over that scale).  Summation order alone stays far below the
    first; a bf16 rounding that resolves the other way on one side moves a
    few logits by about |W| * 2^-8 * |xf|, which stays below the second."""
    scale = np.abs(ref).max()
    d = np.abs(np.asarray(got, np.float64) - ref) / scale
    return float(np.mean(d > 1e-5)), float(d.max())


def _head_case(H, V, T, dtype, seed):
    g = np.random.default_rng(seed)
    # rows of very different scale (the norm matters) and a non-unit gain
    x = (g.standard_normal((T, H)) * g.uniform(0.2, 5.0, (T, 1))).astype(np.float32)
    gamma = g.uniform(0.5, 1.5, H).astype(np.float32)
    W = (g.standard_normal((V, H)) * 0.02).astype(np.float32)
    if dtype == "bf16":
        x, gamma, W = _torch_bf16(x), _torch_bf16(gamma), _torch_bf16(W)
    return x, gamma, W


@pytest.mark.parametrize("H,V,T,dtype", [(256, 1024, 8, "f32"), (256, 1024, 8, "bf16"), (384, 777, 33, "bf16"),
                                         (128, 300, 5, "f32")])
def test_lm_head_logits_match_torch_rms_norm_and_linear(H, V, T, dtype):
    """lm_head_logits (final RMSNorm with its gain, the R1 rounding for bf16,
    then the vocabulary product) against torch's rms_norm and linear, at the
    tiny workload's head shape and small bf16 shapes with ragged sizes."""
    x, gamma, W = _head_case(H, V, T, dtype, seed=H + V + T)
    eps = 1e-6
    got = O.lm_head_logits(x, gamma, W, eps, O.storage_round(dtype))
    ref = _torch_head_logits(x, gamma, W, eps, dtype == "bf16")
    frac, worst = _head_mismatch(got, ref)
    assert frac <= 0.01 and worst <= 2e-3, (frac, worst)
    if dtype == "f32":
        assert worst <= 1e-5
    decided = O.argmax_margin(ref.astype(np.float32)) >= 1e-3 * np.abs(ref).max()
    assert np.array_equal(O.greedy_pick(got)[decided], np.argmax(ref, 1)[decided])


def test_lm_head_logits_pin_rejects_planted_mistakes():
    """The head pin fails for a dropped final norm, a skipped R1 rounding and
    an ignored gain, each planted in a copy of lm_head_logits."""
    H, V, T, eps = 256, 1024, 16, 1e-6
    x, gamma, W = _head_case(H, V, T, "bf16", seed=99)
    ref = _torch_head_logits(x, gamma, W, eps, True)
    bf = O.storage_round("bf16")

    def no_norm(x, gamma_f, w_lm, eps, store):
        return (store(O.as_f32(x) * gamma_f) @ O.as_f32(w_lm).T).astype(np.float32)

    def no_r1(x, gamma_f, w_lm, eps, store):
        return O.lm_head_logits(x, gamma_f, w_lm, eps, O.storage_round("f32"))

    def no_gain(x, gamma_f, w_lm, eps, store):
        return O.lm_head_logits(x, np.ones_like(gamma_f), w_lm, eps, store)

    frac, worst = _head_mismatch(O.lm_head_logits(x, gamma, W, eps, bf), ref)
    assert frac <= 0.01 and worst <= 2e-3
    for bad in (no_norm, no_r1, no_gain):
        frac, worst = _head_mismatch(bad(x, gamma, W, eps, bf), ref)
        assert frac > 0.01 or worst > 2e-3, bad.__name__


# ---------------------------------------------------------- acceptance ----

@pytest.mark.parametrize("K", [0, 1, 2, 3, 4])
def test_acceptance_exhaustive_patterns(K):
    """All 2^K draft-correctness patterns: counts = 1 + index of the first wrong
    draft; all correct -> K + 1 with the bonus token."""
    V = 50
    pats = list(itertools.product([True, False], repeat=K))
    B = len(pats)
    tstar = rng.integers(0, V, (B, K + 1)).astype(np.int32)
    drafts = np.empty((B, K), np.int32)
    for b, pat in enumerate(pats):
        for j, ok in enumerate(pat):
            drafts[b, j] = tstar[b, j] if ok else (tstar[b, j] + 1 + rng.integers(0, V - 1)) % V
    committed, counts = O.accept_prefix(tstar, drafts)
    for b, pat in enumerate(pats):
        first_bad = next((j for j, ok in enumerate(pat) if not ok), K)
        assert counts[b] == first_bad + 1
        assert 1 <= counts[b] <= K + 1
        assert committed[b, :counts[b]].tolist() == tstar[b, :counts[b]].tolist()
        assert np.all(committed[b, counts[b]:] == -1)
    if K > 0:
        assert counts[0] == K + 1 and committed[0, K] == tstar[0, K]   # bonus


def test_k0_is_one_greedy_step():
    tstar = rng.integers(0, 100, (7, 1)).astype(np.int32)
    committed, counts = O.accept_prefix(tstar, np.zeros((7, 0), np.int32))
    assert np.all(counts == 1) and np.array_equal(committed[:, 0], tstar[:, 0])


def test_correct_draft_after_a_wrong_one_is_not_accepted():
    tstar = np.array([[5, 6, 7, 8]], np.int32)
    committed, counts = O.accept_prefix(tstar, np.array([[5, 9, 7]], np.int32))
    assert counts[0] == 2 and committed[0].tolist() == [5, 6, -1, -1]


# -------------------------------------------------- greedy equivalence ----

class _ToyLM:
    """h(token, pos) = Emb[token] + Pos[pos] -> tiny fp32 MoE block -> head.
    No attention, so the next token depends on (token, position) only."""

    def __init__(self):
        w = synth.WORKLOADS["tiny_fp32"]
        self.shp = O.Shape(H=w.H, E=w.E, k=w.k, S=w.S, I=w.I, V=w.V, dtype="f32")
        self.wt = synth.gen_weights(w)
        g = np.random.default_rng(777)
        self.emb = g.standard_normal((w.V, w.H)).astype(np.float32)
        self.pos = g.standard_normal((512, w.H)).astype(np.float32)

    def picks(self, tokens, start_pos):
        h = self.emb[np.asarray(tokens)] + self.pos[start_pos + np.arange(len(tokens))]
        x = O.moe_block(h, self.wt["layers"][0], self.shp).x_out
        lg = O.lm_head_logits(x, self.wt["final_gamma"], self.wt["lm_head"], 1e-6, O.storage_round("f32"))
        return O.greedy_pick(lg)


@pytest.fixture(scope="module")
def toy():
    return _ToyLM()


def _greedy_stream(toy, first, n):
    out = [first]
    while len(out) < n:
        out.append(int(toy.picks([out[-1]], len(out) - 1)[0]))
    return out


def _spec_stream(toy, first, n, K, draft_fn):
    out, steps = [first], 0
    while len(out) < n:
        p = len(out) - 1
        d = [int(v) for v in draft_fn(out, K)]
        ts = toy.picks([out[-1]] + d, p)
        committed, counts = O.accept_prefix(ts.reshape(1, K + 1), np.array([d], np.int32).reshape(1, K))
        out.extend(int(v) for v in committed[0, :counts[0]])
        steps += 1
    return out[:n], steps


@pytest.mark.parametrize("K", [0, 1, 2, 3])
def test_speculative_stream_equals_greedy_stream(toy, K):
    """The committed stream equals one-token-at-a-time greedy decoding for any
    draft source ([CLAWPIT] 'Speculative decoding without accuracy loss')."""
    n = 160
    ref = _greedy_stream(toy, 3, n + 8)
    g = np.random.default_rng(K)

    def random_drafts(out, K):
        return g.integers(0, 1024, K)

    def oracle_drafts(out, K):
        p = len(out)
        return ref[p:p + K] if p + K <= len(ref) else g.integers(0, 1024, K)

    def noisy_drafts(out, K):
        d = list(oracle_drafts(out, K))
        return [v if g.random() < 0.7 else int(g.integers(0, 1024)) for v in d]

    for fn in (random_drafts, oracle_drafts, noisy_drafts):
        got, steps = _spec_stream(toy, 3, n, K, fn)
        assert got == ref[:n]
        if fn is oracle_drafts:
            assert steps <= -(-n // (K + 1)) + 1


# ----------------------------------------------- statistics of drafts ----

def test_independent_draft_acceptance_mean_counts():
    """Each draft correct independently with p = 0.576: E[counts] = 1+p+p^2+p^3."""
    w = synth.WORKLOADS["decode_b32_zipf"]
    B = 40000
    tstar = rng.integers(0, w.V, (B, 4)).astype(np.int32)
    g = np.random.default_rng(99)
    u, r = g.random((B, 3)), g.integers(0, w.V - 1, (B, 3))
    d = synth.make_drafts(w, tstar, u, r)
    _, counts = O.accept_prefix(tstar, d)
    exp = O.expected_counts_independent(0.576, 3)
    assert abs(exp - 2.0990) < 1e-3
    sd = counts.std() / np.sqrt(B)
    assert abs(counts.mean() - exp) < 4 * sd


# ------------------------------------------- the pages' printed numbers ----

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_pages_decode_measures_definitions():
    g = _golden("l4_speculative_decoding.json")
    K = g["K"]
    # tau is printed to 2 decimals: the acceptance rate must fall in the interval it allows
    lo = O.acceptance_rate(g["tau_eager"] - 0.005, K)
    hi = O.acceptance_rate(g["tau_eager"] + 0.005, K)
    assert lo <= g["acceptance_rate"] <= hi
    S = g["spec_eager_tok_s"] / g["ar_eager_tok_s"]
    assert abs(S - g["speedup_eager"]) < 0.005
    assert abs(O.step_cost(g["tau_eager"], S) - g["c_eager"]) < 0.005
    # with graphs: c = 2.51 AR steps at 158.3 tok/s; speculative step minus AR step ~ 9 ms
    step_graphs = g["c_graphs"] / g["ar_graphs_tok_s"]
    step_eager = g["c_eager"] / g["ar_eager_tok_s"]
    assert abs((step_graphs - 1 / g["ar_graphs_tok_s"]) * 1e3 - g["overhead_ms"]) < 1.0
    assert abs((step_eager - 1 / g["ar_eager_tok_s"]) * 1e3 - g["overhead_ms"]) < 1.0
    assert abs(g["k1_graphs_tok_s"] / g["ar_graphs_tok_s"] - g["k1_speedup_graphs"]) < 0.005


def test_pages_shape_constants():
    g = _golden("decoder_shape.json")
    assert g["global_tokens"] + g["max_tiles"] * g["tokens_per_tile"] == g["max_visual_tokens"]
    w = synth.WORKLOADS
    assert w["prefill_8pages"].T == 8 * (g["max_visual_tokens"] + 64)
    for name in ("decode_b1", "decode_b32_zipf", "stack12_b32_zipf", "prefill_8pages"):
        assert (w[name].E, w[name].S, w[name].k) == (g["routed_experts"], g["shared_experts"], g["top_k"])
    assert w["stack12_b32_zipf"].L == g["layers"]
    assert w["decode_b32_zipf"].B == g["concurrency"]


# --------------------------------------------------------- sensitivity ----

def test_sensitivity_pins_reject_planted_mistakes():
    """Plant plausible mistakes in copies of oracle steps and check the pins
    above would reject them."""
    z = rng.standard_normal((50, 8)).astype(np.float32)
    # (1) top-k picking the smallest logits
    wrong_idx = np.argsort(z, axis=1, kind="stable")[:, :2]
    assert any(set(wrong_idx[t].tolist()) != _brute_topk_set(z[t], 2) for t in range(50))
    # (2) gates = softmax over all experts, not renormalised
    p = torch.softmax(torch.from_numpy(z), 1).numpy()
    idx, _ = O.topk_select(z, 2)
    assert not np.allclose(np.take_along_axis(p, idx, 1).sum(1), 1.0, atol=1e-6)
    # (3) acceptance counting all matches instead of the leading ones
    tstar = np.array([[1, 2, 3, 4]], np.int32)
    drafts = np.array([[1, 9, 3]], np.int32)
    wrong_count = 1 + int(np.sum(drafts[0] == tstar[0, :3]))
    assert wrong_count != O.accept_prefix(tstar, drafts)[1][0]
    # (4) draft j compared with the pick one position later (off-by-one)
    d = tstar[:, 1:]
    assert O.accept_prefix(tstar, d)[1][0] != 4
    # (5) SwiGLU without the R2 rounding differs from the bf16 textbook MLP
    H, I = 128, 96
    x = _torch_bf16(rng.standard_normal((64, H)).astype(np.float32))
    wg, wu, wd = (_torch_bf16(rng.standard_normal(s).astype(np.float32) * 0.1)
                  for s in ((I, H), (I, H), (H, I)))
    ref = _torch_swiglu(x, wg, wu, wd, True)
    no_r2 = O.swiglu_expert(x, wg, wu, wd, O.storage_round("f32"))
    with_r2 = O.swiglu_expert(x, wg, wu, wd, O.storage_round("bf16"))
    assert np.abs(with_r2 - ref).max() < np.abs(no_r2 - ref).max()
    # (6) a dropped shared expert changes m by far more than rounding
    shp = O.Shape(H=64, E=8, k=2, S=1, I=32, V=16, dtype="f32")
    lw = _layer(64, 8, 1, 32, scale=0.1)
    xx = rng.standard_normal((5, 64)).astype(np.float32)
    full = O.moe_block(xx, lw, shp).m
    lw0 = dict(lw, s_down=np.zeros_like(lw["s_down"]))
    assert np.abs(O.moe_block(xx, lw0, shp).m - full).max() > 1e-3
