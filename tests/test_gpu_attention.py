"""Parity of the verify step with attention and a KV cache (moe_verify_step_kv)
with the CPU oracle, through the C ABI.

Small shapes (two heads of 128) over several layers with ragged batches,
K = 0, 3 and 7, cache positions from empty to the last that fits, two steps
in a row continuing the cache (positions advanced by the committed counts);
the full-size one-layer workloads; a cache of 32,768 positions (the largest
accepted) at full width; and sampled sequences of the 12-layer batch-32 step
with attention (a complete verify forward of the pages' decoder shape).  Bar: tests/parity.py, check_attn_step_teacher_forced.
"""
import functools

import numpy as np
import pytest

from oracle import attn_oracle as A
from oracle import moe_oracle as O
from moe_decoder_speculative_amd import synth
from moe_decoder_speculative_amd.model import VerifyModel, to_device
import parity
import workloads

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _prefix(w, positions, seqs=None):
    """kv0[l] = (k, v) float32 [B', nh, P, 128] for sequences `seqs`, and the
    bf16 bits of every (l, b) prefix for the upload."""
    seqs = range(len(positions)) if seqs is None else seqs
    bits = {}
    kv0 = []
    for l in range(w.L):
        kc = np.zeros((len(seqs), w.n_heads, w.P, 128), np.float32)
        vc = np.zeros_like(kc)
        for i, b in enumerate(seqs):
            k, v = synth.kv_prefix(w, l, b, int(positions[b]))
            bits[(l, b)] = (k, v)
            kc[i, :, :positions[b]] = O.as_f32(k)
            vc[i, :, :positions[b]] = O.as_f32(v)
        kv0.append((kc, vc))
    return kv0, bits


@functools.lru_cache(maxsize=1)
def _stack_weights(w):
    """Weights of a workload, kept for the next test of the same workload (the
    12-layer ones take a minute or two to generate)."""
    return synth.gen_weights(w)


def _ash(w):
    return A.AttnShape(H=w.H, n_heads=w.n_heads, d_head=128, P=w.P, theta=w.rope_theta, eps=w.eps, dtype=w.dtype)


def _drafts(w, weights, hidden, positions, kv0):
    """Drafts from the oracle's own greedy picks (kept with probability p)."""
    caches = [(k.copy(), v.copy()) for k, v in kv0]
    r = A.verify_step_attn(workloads.shape_of(w), _ash(w), weights, hidden, np.zeros((w.B, w.K), np.int32),
                           positions, caches, w.B, w.K)
    return synth.make_drafts(w, r.tstar.reshape(w.B, w.K + 1))


def _gpu_step(vm, w, hidden, drafts, positions, B, K):
    torch = _torch()
    T = B * (K + 1)
    aux = vm.alloc_aux(T)
    committed, counts = vm.alloc_outputs(B, K)
    vm.step_kv(to_device(hidden), to_device(np.asarray(drafts, np.int32)) if K else None,
               to_device(np.asarray(positions, np.int32)), B, K, committed, counts, aux)
    torch.cuda.synchronize()
    out = {k: (parity.storage_to_f32(t) if k in ("hidden_out", "attn_out") else t.cpu().numpy())
           for k, t in aux.items()}
    out["committed"], out["counts"] = committed.cpu().numpy(), counts.cpu().numpy()
    return out


def _gpu_kv(vm, w, seqs):
    kv = []
    for l in range(w.L):
        ks, vs = zip(*(vm.kv_read(l, b) for b in seqs))
        kv.append((O.as_f32(np.stack(ks)), O.as_f32(np.stack(vs))))
    return kv


def _rows(out, seqs, K1):
    """The rows of sequences `seqs` from a whole step's outputs."""
    rows = np.concatenate([np.arange(b * K1, (b + 1) * K1) for b in seqs])
    sub = {k: out[k][:, rows] for k in ("attn_out", "moe_out", "topk_idx", "topk_w")}
    sub.update(hidden_out=out["hidden_out"][rows], tstar=out["tstar"][rows], counts=out["counts"][list(seqs)],
               committed=out["committed"][list(seqs)])
    return sub


def _small_case(B, K, L, P, seed, edge=True):
    w = workloads.small_bf16(name="attn_small", B=B, K=K, L=L, seed_id=seed).with_(n_heads=2, P=P)
    positions = synth.kv_positions(w)
    if edge and B >= 2:
        positions[0], positions[-1] = 0, P - (K + 1)     # an empty cache and a full one
    return w, positions


@pytest.mark.parametrize("B,K,L,P", [(5, 3, 2, 64), (3, 0, 1, 64), (2, 7, 1, 80), (33, 3, 1, 128), (1, 3, 3, 256)])
def test_attention_step_small(B, K, L, P):
    w, positions = _small_case(B, K, L, P, seed=500 + B + 10 * K + 100 * L)
    parity.say(f"[attn small] B={B} K={K} L={L} P={P} H={w.H} heads={w.n_heads} positions={positions.tolist()[:6]} "
               f"entry=moe_verify_step_kv")
    weights = synth.gen_weights(w)
    hidden = synth.to_storage(synth.HiddenNoise(w).draw(w.T), w.dtype)
    kv0, bits = _prefix(w, positions)
    drafts = _drafts(w, weights, hidden, positions, kv0) if K else np.zeros((B, 0), np.int32)
    vm = VerifyModel(w, weights, max_tokens=w.T, max_seqs=B)
    try:
        for (l, b), (k, v) in bits.items():
            vm.kv_write(l, b, k, v)
        out = _gpu_step(vm, w, hidden, drafts, positions, B, K)
        msg = parity.check_attn_step_teacher_forced(out, _gpu_kv(vm, w, range(B)), hidden, drafts, positions, kv0,
                                                    weights, workloads.shape_of(w), _ash(w))
        parity.say(f"[attn small] ok: {msg}")
    finally:
        vm.close()


def test_attention_two_steps_continue_the_cache():
    """Step 1, then step 2 at positions + counts on the same cache (rejected
    drafts' rows are overwritten); the oracle checks step 2 from the GPU's
    cache after step 1."""
    B, K, L, P = 4, 3, 2, 96
    w, positions = _small_case(B, K, L, P, seed=611, edge=False)
    positions = np.minimum(positions, P - 2 * (K + 1))
    weights = synth.gen_weights(w)
    noise = synth.HiddenNoise(w)
    kv0, bits = _prefix(w, positions)
    vm = VerifyModel(w, weights, max_tokens=w.T, max_seqs=B)
    try:
        for (l, b), (k, v) in bits.items():
            vm.kv_write(l, b, k, v)
        for step in range(2):
            hidden = synth.to_storage(noise.draw(w.T), w.dtype)
            drafts = _drafts(w, weights, hidden, positions, kv0)
            parity.say(f"[attn two steps] step {step} positions {positions.tolist()}")
            out = _gpu_step(vm, w, hidden, drafts, positions, B, K)
            kv_after = _gpu_kv(vm, w, range(B))
            msg = parity.check_attn_step_teacher_forced(out, kv_after, hidden, drafts, positions, kv0, weights,
                                                        workloads.shape_of(w), _ash(w))
            parity.say(f"[attn two steps] ok: {msg}")
            positions = positions + out["counts"]
            kv0 = kv_after
    finally:
        vm.close()


@pytest.mark.parametrize("pos_in,pos_out", [(60, 200), (0, -9)])
def test_attention_positions_outside_the_cache_are_clamped(pos_in, pos_out):
    """Two sequences with identical rows, drafts and cache contents, one at a
    position at the edge of the range (0 or P - K - 1) and one beyond it on
    the same side: the second is clamped to the first in every kernel, so
    both give the same picks, counts, committed tokens, residual rows and
    cache rows, bit for bit; the first is also checked against the oracle."""
    B, K, L, P = 2, 3, 2, 64
    w, _ = _small_case(B, K, L, P, seed=733, edge=False)
    positions = np.array([pos_in, pos_out], np.int32)
    clamped = np.array([pos_in, pos_in], np.int32)
    parity.say(f"[attn clamp] positions {positions.tolist()} (both at {pos_in}) K={K} L={L} P={P} entry=moe_verify_step_kv")
    weights = synth.gen_weights(w)
    K1 = K + 1
    one = synth.to_storage(synth.HiddenNoise(w).draw(K1), w.dtype)
    hidden = np.concatenate([one, one])
    kv0, bits = _prefix(w, clamped, seqs=[0])
    kv0 = [(np.concatenate([k, k]), np.concatenate([v, v])) for k, v in kv0]
    d1 = _drafts(w.with_(B=1, T=K1), weights, one, clamped[:1], [(k[:1], v[:1]) for k, v in kv0])
    drafts = np.concatenate([d1, d1])
    vm = VerifyModel(w, weights, max_tokens=w.T, max_seqs=B)
    try:
        for (l, b), (k, v) in bits.items():
            vm.kv_write(l, 0, k, v)
            vm.kv_write(l, 1, k, v)
        out = _gpu_step(vm, w, hidden, drafts, positions, B, K)
        kv = _gpu_kv(vm, w, range(B))
        for name in ("hidden_out", "tstar"):
            assert np.array_equal(out[name][:K1], out[name][K1:]), name
        for name in ("attn_out", "moe_out", "topk_idx", "topk_w"):
            assert np.array_equal(out[name][:, :K1], out[name][:, K1:]), name
        assert out["counts"][0] == out["counts"][1] and np.array_equal(out["committed"][0], out["committed"][1])
        for l in range(L):
            assert np.array_equal(kv[l][0][0], kv[l][0][1]) and np.array_equal(kv[l][1][0], kv[l][1][1]), l
        msg = parity.check_attn_step_teacher_forced(_rows(out, [0], K1), [(k[:1], v[:1]) for k, v in kv], one, d1,
                                                    clamped[:1], [(k[:1], v[:1]) for k, v in kv0], weights,
                                                    workloads.shape_of(w), _ash(w))
        parity.say(f"[attn clamp] ok: the clamped sequence equals the in-range one; {msg}")
    finally:
        vm.close()


@pytest.mark.parametrize("name,sample", [("attn_b1", None), ("attn_b32_zipf", [0, 7, 19, 31])])
def test_attention_full_size_one_layer(name, sample):
    w = synth.WORKLOADS[name]
    _full(w, sample)


@pytest.mark.slow
def test_attention_stack12_b32_sampled():
    """The 12-layer batch-32 step with attention as the benchmark runs it;
    sequences 0 and 21 followed by the oracle layer by layer."""
    _full(synth.WORKLOADS["attn_stack12_b32_zipf"], [0, 21])


@pytest.mark.slow
def test_attn_stack12_margin_sequences_end_to_end():
    """The 12-layer step with attention, end to end against the oracle's own
    step: single-row sequences (K = 0, greedy decoding through the whole
    stack) whose every layer's top-k gap and head gap exceed 1.5 times the
    MoE-only stack's drift schedule along the oracle's trajectory
    (tests/golden/attn_stack12_b32_zipf_seqs.json, written from the oracle
    and the seeded generators only), each with its own cache part-way
    through a page.  Every layer's expert sets and the picks bit for bit."""
    _torch()
    case = workloads.attn_margin_seqs_case(_stack_weights)  # asserts the schedule along the oracle's trajectory
    w, base, weights, hidden, positions, cands, ref = (case.w, case.base, case.weights, case.hidden,
                                                       case.positions, case.cands, case.ref)
    n = len(cands)
    parity.say(f"[attn margin] {w.name}: B={n} K=0 L={w.L} P={w.P} candidates {cands} positions "
               f"{positions.tolist()} entry=moe_verify_step_kv")
    vm = VerifyModel(w, weights, max_tokens=n, max_seqs=n)
    try:
        for l in range(w.L):
            for i, c in enumerate(cands):
                k, v = synth.kv_prefix(base, l, c, int(positions[i]))
                vm.kv_write(l, i, k, v)
        out = _gpu_step(vm, w, hidden, None, positions, n, 0)
    finally:
        vm.close()
    for l, blk in enumerate(ref.blocks):
        assert np.array_equal(np.sort(out["topk_idx"][l], 1), np.sort(blk.idx, 1)), f"layer {l}: expert sets differ"
    assert np.array_equal(out["tstar"], ref.tstar), f"picks differ: {out['tstar']} vs {ref.tstar}"
    assert np.array_equal(out["counts"], ref.counts) and np.array_equal(out["committed"].reshape(-1),
                                                                       ref.committed.reshape(-1))
    parity.say(f"[attn margin] ok: {n} sequences x {w.L} layers, expert sets and picks equal to the oracle's "
               f"own step ({n}/{n})")


@pytest.mark.slow
def test_attention_near_max_positions():
    """The largest cache the library accepts -- 32,768 positions, the pages'
    position limit -- at full width (10 heads of 128): one sequence whose
    step ends on the last cache row and one in the middle (rotary angles up
    to ~32,767 rad, 512 position tiles in 52 groups)."""
    w = synth.WORKLOADS["attn_b1"].with_(name="attn_maxpos", B=2, T=8, P=32768)
    _full(w, None, positions=np.array([w.P - (w.K + 1), 17001], np.int32))


def _full(w, sample, positions=None):
    positions = synth.kv_positions(w) if positions is None else positions
    seqs = list(range(w.B)) if sample is None else sample
    parity.say(f"[attn full] {w.name}: B={w.B} K={w.K} L={w.L} P={w.P} sampled sequences {seqs} "
               f"positions {positions[seqs].tolist()}")
    weights = _stack_weights(w)
    noise = synth.HiddenNoise(w)
    hidden = synth.to_storage(noise.draw(w.T) + synth.hidden_offset(w, weights, noise), w.dtype)
    K1 = w.K + 1
    rows = np.concatenate([np.arange(b * K1, (b + 1) * K1) for b in seqs])
    # drafts: the sampled sequences' from the oracle's picks, the rest random
    kv0, _ = _prefix(w, positions, seqs)
    sub_w = w.with_(B=len(seqs), T=len(seqs) * K1)
    d_sub = _drafts(sub_w, weights, hidden[rows], positions[seqs], kv0)
    drafts = np.random.default_rng(5).integers(0, w.V, size=(w.B, w.K)).astype(np.int32)
    drafts[seqs] = d_sub
    vm = VerifyModel(w, weights, max_tokens=w.T, max_seqs=w.B)
    try:
        for l in range(w.L):
            for b in range(w.B):
                k, v = synth.kv_prefix(w, l, b, int(positions[b]))
                vm.kv_write(l, b, k, v)
        out = _gpu_step(vm, w, hidden, drafts, positions, w.B, w.K)
        msg = parity.check_attn_step_teacher_forced(_rows(out, seqs, K1), _gpu_kv(vm, w, seqs), hidden[rows],
                                                    drafts[seqs], positions[seqs], kv0, weights,
                                                    workloads.shape_of(w), _ash(w))
        parity.say(f"[attn full] {w.name} ok: {msg}")
    finally:
        vm.close()


def test_attention_graph_replay_matches_eager():
    """moe_verify_graph_create_kv: a captured step with attention replayed four
    times, eager steps of the same context between the replays; committed
    tokens, counts and every cache row equal the eager step's, bit for bit."""
    torch = _torch()
    from moe_decoder_speculative_amd import binding
    B, K, L, P = 4, 3, 2, 64
    w, positions = _small_case(B, K, L, P, seed=707)
    parity.say(f"[attn graph] B={B} K={K} L={L} P={P} entry=moe_verify_graph_create_kv/moe_verify_graph_launch")
    weights = synth.gen_weights(w)
    hidden_np = synth.to_storage(synth.HiddenNoise(w).draw(w.T), w.dtype)
    kv0, bits = _prefix(w, positions)
    drafts_np = _drafts(w, weights, hidden_np, positions, kv0)
    vm = VerifyModel(w, weights, max_tokens=w.T, max_seqs=B)
    g = None
    try:
        for (l, b), (k, v) in bits.items():
            vm.kv_write(l, b, k, v)
        hidden, drafts, pos = to_device(hidden_np), to_device(drafts_np), to_device(np.asarray(positions, np.int32))
        c_ref, n_ref = vm.alloc_outputs(B, K)
        vm.step_kv(hidden, drafts, pos, B, K, c_ref, n_ref)
        torch.cuda.synchronize()
        kv_ref = _gpu_kv(vm, w, range(B))
        stream = torch.cuda.Stream()
        c_g, n_g = vm.alloc_outputs(B, K)
        torch.cuda.synchronize()
        g = binding.moe_verify_graph_create_kv(vm.ctx, hidden, drafts, pos, B, K, c_g, n_g, stream)
        c_e, n_e = vm.alloc_outputs(B, K)
        for rep in range(4):
            c_g.fill_(-5)
            n_g.fill_(-5)
            torch.cuda.synchronize()
            binding.moe_verify_graph_launch(g, stream)
            stream.synchronize()
            assert torch.equal(c_g, c_ref) and torch.equal(n_g, n_ref), f"replay {rep}: outputs differ"
            kv = _gpu_kv(vm, w, range(B))
            for l in range(L):
                assert np.array_equal(kv[l][0], kv_ref[l][0]) and np.array_equal(kv[l][1], kv_ref[l][1]), \
                    f"replay {rep}: layer {l} cache differs"
            vm.step_kv(hidden, drafts, pos, B, K, c_e, n_e)
            torch.cuda.synchronize()
            assert torch.equal(c_e, c_ref)
        parity.say(f"[attn graph] ok: 4 replays equal to eager, counts {n_ref.cpu().tolist()}")
    finally:
        if g:
            binding.moe_verify_graph_destroy(g)
        vm.close()
