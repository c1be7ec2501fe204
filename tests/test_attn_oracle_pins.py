"""Pins of the attention oracle (oracle/attn_oracle.py) to things other than
itself: the complex-number form of the rotary embedding and its relative-
position property, torch's scaled_dot_product_attention and complex RoPE in a
textbook torch layer, the KV cache against one full causal pass, and the
lossless decode loop with a cache whose rejected entries are overwritten.
No GPU needed."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import attn_oracle as A

rng = np.random.default_rng(777)
F = torch.nn.functional


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


# ------------------------------------------------------------------ rope ----

def test_rope_is_complex_rotation():
    """Pair (2i, 2i+1) as the complex number x_2i + j x_2i+1, multiplied by
    exp(j * pos * theta^(-2i/d))."""
    T, nh, d = 20, 3, 128
    x = rng.standard_normal((T, nh, d)).astype(np.float32)
    pos = rng.integers(0, 32768, T)
    got = A.rope(x, pos, 10000.0)
    z = x[..., 0::2].astype(np.float64) + 1j * x[..., 1::2].astype(np.float64)
    inv = 10000.0 ** (-np.arange(d // 2) * 2.0 / d)
    ang = pos[:, None].astype(np.float64) * inv[None, :]
    ref = z * np.exp(1j * ang)[:, None, :]
    # the float32 angle differs from the exact one by up to pos * 2^-24 rad
    tol = 32768 * 2.0 ** -23 * np.abs(z).max() + 1e-5
    assert np.abs(got[..., 0::2] - ref.real).max() < tol
    assert np.abs(got[..., 1::2] - ref.imag).max() < tol
    # small positions are accurate to float32 rounding
    p0 = np.arange(T)
    z0 = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * p0[:, None] * inv[None, :])[:, None, :]
    g0 = A.rope(x, p0, 10000.0)
    np.testing.assert_allclose(g0[..., 0::2], z0.real, atol=2e-5)
    np.testing.assert_allclose(g0[..., 1::2], z0.imag, atol=2e-5)


def test_rope_relative_position_and_identity():
    d = 128
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    assert np.array_equal(A.rope(q, [0], 10000.0), q)
    dots = [float((A.rope(q, [m + s], 1e4) * A.rope(k, [n + s], 1e4)).sum()) for (m, n, s) in
            [(7, 3, 0), (7, 3, 100), (7, 3, 1000)]]
    np.testing.assert_allclose(dots, dots[0], rtol=2e-4)
    np.testing.assert_allclose(np.linalg.norm(A.rope(q, [12345], 1e4)), np.linalg.norm(q), rtol=1e-6)


# ------------------------------------------------------------- attention ----

def _attn_layer(H, nh, dtype="f32", scale=0.05):
    lw = dict(attn_gamma=(1 + 0.1 * rng.uniform(-1, 1, H)).astype(np.float32),
              w_q=(rng.standard_normal((H, H)) * scale).astype(np.float32),
              w_k=(rng.standard_normal((H, H)) * scale).astype(np.float32),
              w_v=(rng.standard_normal((H, H)) * scale).astype(np.float32),
              w_o=(rng.standard_normal((H, H)) * scale).astype(np.float32))
    if dtype == "bf16":
        lw = {k: _bf16(v) for k, v in lw.items()}
    return lw


def _cache(B, nh, P, d, fill, dtype):
    kc = np.zeros((B, nh, P, d), np.float32)
    vc = np.zeros((B, nh, P, d), np.float32)
    for b in range(B):
        kc[b, :, :fill[b]] = rng.standard_normal((nh, fill[b], d))
        vc[b, :, :fill[b]] = rng.standard_normal((nh, fill[b], d))
    if dtype == "bf16":
        kc, vc = _bf16(kc), _bf16(vc)
    return kc, vc


@pytest.mark.parametrize("K", [0, 3])
def test_attention_matches_torch_sdpa(K):
    """Each query against the cache prefix plus the step's own keys, with the
    causal mask, through torch's scaled_dot_product_attention (float64)."""
    H, nh, d, P, B = 256, 2, 128, 64, 3
    ash = A.AttnShape(H=H, n_heads=nh, d_head=d, P=P, dtype="f32")
    lw = _attn_layer(H, nh)
    positions = np.array([0, 5, 40])
    kc, vc = _cache(B, nh, P, d, positions, "f32")
    x = rng.standard_normal((B * (K + 1), H)).astype(np.float32)
    r = A.attn_sublayer(x, positions, B, K, kc, vc, lw, ash)
    ctx = r.ctx.reshape(B, K + 1, nh, d)
    for b in range(B):
        n = positions[b] + K + 1
        qb = torch.from_numpy(r.q.reshape(B, K + 1, nh, d)[b].transpose(1, 0, 2).astype(np.float64))
        kb = torch.from_numpy(kc[b, :, :n].astype(np.float64))
        vb = torch.from_numpy(vc[b, :, :n].astype(np.float64))
        mask = torch.from_numpy(np.arange(n)[None, :] <= positions[b] + np.arange(K + 1)[:, None])
        ref = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask).numpy()   # [nh, K+1, d]
        np.testing.assert_allclose(ctx[b].transpose(1, 0, 2), ref, rtol=1e-4, atol=1e-5)
    # the cache now holds this step's keys and values
    kk = r.k.reshape(B, K + 1, nh, d)
    for b in range(B):
        for j in range(K + 1):
            assert np.array_equal(kc[b, :, positions[b] + j], kk[b, j])


def _torch_layer(x, lw, nh, d, theta, eps):
    """A textbook pre-norm attention sublayer over one whole sequence in torch:
    rms_norm, linear projections, complex rotary embedding, causal SDPA."""
    T, H = x.shape
    X = torch.from_numpy(x.astype(np.float64))
    W = {k: torch.from_numpy(v.astype(np.float64)) for k, v in lw.items()}
    xh = F.rms_norm(X, (H,), W["attn_gamma"], eps)
    q, k, v = (F.linear(xh, W[n]).view(T, nh, d) for n in ("w_q", "w_k", "w_v"))
    freqs = torch.outer(torch.arange(T, dtype=torch.float64),
                        theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d))
    rot = torch.polar(torch.ones_like(freqs), freqs)[:, None, :]
    q = torch.view_as_real(torch.view_as_complex(q.reshape(T, nh, d // 2, 2)) * rot).reshape(T, nh, d)
    k = torch.view_as_real(torch.view_as_complex(k.reshape(T, nh, d // 2, 2)) * rot).reshape(T, nh, d)
    ctx = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True)
    return (X + F.linear(ctx.transpose(0, 1).reshape(T, H), W["w_o"])).numpy()


def test_sublayer_over_a_sequence_matches_textbook_torch_layer():
    H, nh, d, T = 256, 2, 128, 24
    ash = A.AttnShape(H=H, n_heads=nh, d_head=d, P=32, dtype="f32")
    lw = _attn_layer(H, nh)
    x = rng.standard_normal((T, H)).astype(np.float32)
    kc, vc = _cache(1, nh, 32, d, [0], "f32")
    r = A.attn_sublayer(x, [0], 1, T - 1, kc, vc, lw, ash)
    ref = _torch_layer(x, lw, nh, d, 1e4, 1e-6)
    np.testing.assert_allclose(r.x_out, ref, rtol=1e-4, atol=1e-4)


def _stack_weights(H, nh, E, k, S, I, V, L, dtype):
    layers = []
    for _ in range(L):
        lw = _attn_layer(H, nh, dtype)
        moe = dict(gamma=np.ones(H, np.float32),
                   router=rng.standard_normal((E, H)).astype(np.float32) * 0.1,
                   gate=rng.standard_normal((E, I, H)).astype(np.float32) * 0.05,
                   up=rng.standard_normal((E, I, H)).astype(np.float32) * 0.05,
                   down=rng.standard_normal((E, H, I)).astype(np.float32) * 0.05,
                   s_gate=rng.standard_normal((S, I, H)).astype(np.float32) * 0.05,
                   s_up=rng.standard_normal((S, I, H)).astype(np.float32) * 0.05,
                   s_down=rng.standard_normal((S, H, I)).astype(np.float32) * 0.05)
        if dtype == "bf16":
            moe = {kk: _bf16(vv) for kk, vv in moe.items()}
        lw.update(moe)
        layers.append(lw)
    return dict(layers=layers, final_gamma=np.ones(H, np.float32),
                lm_head=(rng.standard_normal((V, H)) * (1.0 if dtype == "f32" else 1.0)).astype(np.float32))


def test_cache_in_chunks_equals_one_causal_pass():
    """A sequence through two layers in one step equals the same rows in three
    steps of different sizes, each continuing the cache where the last stopped."""
    H, nh, d, P = 256, 2, 128, 32
    shp = O.Shape(H=H, E=4, k=2, S=1, I=64, V=50, L=2, dtype="f32")
    ash = A.AttnShape(H=H, n_heads=nh, d_head=d, P=P, dtype="f32")
    w = _stack_weights(H, nh, 4, 2, 1, 64, 50, 2, "f32")
    x = rng.standard_normal((12, H)).astype(np.float32)

    def fresh():
        return [(np.zeros((1, nh, P, d), np.float32), np.zeros((1, nh, P, d), np.float32)) for _ in range(2)]

    full = A.verify_step_attn(shp, ash, w, x, np.zeros((1, 11), np.int32), [0], fresh(), 1, 11)
    caches = fresh()
    outs = []
    for start, n in [(0, 4), (4, 2), (6, 6)]:
        r = A.verify_step_attn(shp, ash, w, x[start:start + n], np.zeros((1, n - 1), np.int32), [start], caches,
                               1, n - 1)
        outs.append(r.hidden_out)
    np.testing.assert_allclose(np.concatenate(outs), full.hidden_out, rtol=2e-5, atol=2e-5)


class _ToyAttnLM:
    """Token embedding -> verify_step_attn layers -> head; greedy next tokens."""

    def __init__(self, seed=5, V=40, H=256, nh=2, L=2, P=64):
        global rng
        rng = np.random.default_rng(seed)
        self.V, self.H, self.nh, self.P = V, H, nh, P
        self.shp = O.Shape(H=H, E=4, k=2, S=1, I=64, V=V, L=L, dtype="f32")
        self.ash = A.AttnShape(H=H, n_heads=nh, d_head=128, P=P, dtype="f32")
        self.w = _stack_weights(H, nh, 4, 2, 1, 64, V, L, "f32")
        self.emb = rng.standard_normal((V, H)).astype(np.float32)

    def caches(self):
        return [(np.zeros((1, self.nh, self.P, 128), np.float32), np.zeros((1, self.nh, self.P, 128), np.float32))
                for _ in range(self.shp.L)]

    def step(self, caches, pos, tokens, drafts):
        K = len(tokens) - 1
        return A.verify_step_attn(self.shp, self.ash, self.w, self.emb[tokens], np.asarray(drafts).reshape(1, K),
                                  [pos], caches, 1, K)


@pytest.mark.parametrize("K", [1, 3])
def test_speculative_decoding_with_cache_equals_greedy(K):
    """Greedy one token at a time against speculative steps whose drafts are
    partly right: rejected drafts leave stale cache entries that the next step
    overwrites, and the committed stream is the greedy one."""
    m = _ToyAttnLM()
    g = np.random.default_rng(9)
    prompt = [3, 17, 8]
    n_new = 14
    # greedy
    c = m.caches()
    stream = list(prompt)
    for p in range(len(prompt) - 1):
        m.step(c, p, [prompt[p]], [])
    pos = len(prompt) - 1
    while len(stream) < len(prompt) + n_new:
        r = m.step(c, pos, [stream[-1]], [])
        stream.append(int(r.committed[0, 0]))
        pos += 1
    greedy = stream
    # speculative
    c = m.caches()
    for p in range(len(prompt) - 1):
        m.step(c, p, [prompt[p]], [])
    pos = len(prompt) - 1
    out = list(prompt)
    steps = 0
    while len(out) < len(prompt) + n_new:
        future = greedy[len(out):len(out) + K]
        future += [0] * (K - len(future))
        drafts = [t if g.random() < 0.6 else (t + 1 + g.integers(0, m.V - 1)) % m.V for t in future]
        r = m.step(c, pos, [out[-1]] + drafts, drafts)
        n = int(r.counts[0])
        out.extend(int(t) for t in r.committed[0, :n])
        pos += n
        steps += 1
    assert out[:len(greedy)] == greedy
    assert steps < n_new   # some drafts were accepted


# ---------------------------------------------------------- sensitivity ----

def test_sensitivity_pins_reject_planted_mistakes():
    H, nh, d, P, B, K = 256, 2, 128, 64, 2, 3
    positions = np.array([4, 20])
    kc, vc = _cache(B, nh, P, d, positions, "f32")
    q = rng.standard_normal((nh, d)).astype(np.float32)
    n = positions[0] + 1
    good = np.stack([A.attend(q[h], kc[0, h], vc[0, h], n, d) for h in range(nh)])
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]
    ref = F.scaled_dot_product_attention(qt, torch.from_numpy(kc[0, :, :n].astype(np.float64)),
                                         torch.from_numpy(vc[0, :, :n].astype(np.float64)))[:, 0].numpy()
    np.testing.assert_allclose(good, ref, rtol=1e-4, atol=1e-5)
    # (1) scores scaled by 1/d
    bad = np.stack([A.attend(q[h] / np.sqrt(d), kc[0, h], vc[0, h], n, d) for h in range(nh)])
    assert np.abs(bad - ref).max() > 1e-3
    # (2) one position too many (the causal mask off by one)
    bad = np.stack([A.attend(q[h], kc[0, h], vc[0, h], n + 1, d) for h in range(nh)])
    assert np.abs(bad - ref).max() > 1e-3
    # (3) rotate-half pairing (i, i + d/2) instead of (2i, 2i+1)
    x = rng.standard_normal((3, 1, d)).astype(np.float32)
    pos = np.array([1, 50, 900])
    half = np.concatenate([x[..., :d // 2], x[..., d // 2:]], -1)
    ang = A.rope_angles(pos, d, 1e4)[:, None, :]
    rh = np.concatenate([half[..., :d // 2] * np.cos(ang) - half[..., d // 2:] * np.sin(ang),
                         half[..., :d // 2] * np.sin(ang) + half[..., d // 2:] * np.cos(ang)], -1)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None, None] * 1e4 ** (-np.arange(d // 2) * 2 / d))
    assert np.abs(rh[..., 0::2] - z.real).max() > 1e-2
    # (4) the sublayer without its residual differs from the textbook layer
    lw = _attn_layer(H, nh)
    xs = rng.standard_normal((8, H)).astype(np.float32)
    kc1, vc1 = _cache(1, nh, 16, d, [0], "f32")
    r = A.attn_sublayer(xs, [0], 1, 7, kc1, vc1, lw, A.AttnShape(H=H, n_heads=nh, d_head=d, P=16, dtype="f32"))
    assert np.abs(r.o - _torch_layer(xs, lw, nh, d, 1e4, 1e-6)).max() > 1e-1
