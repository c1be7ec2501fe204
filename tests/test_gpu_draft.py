"""Parity of the HIP draft head with the CPU oracle, through the C ABI.

Small shapes that span several kernel tiles, ragged batches (1, 5, 33, 130:
the three LM-head paths), K from 1 to 7, R from 1 to 8, dense widths that
split into one, two or seven expert slots and a draft head restricted to a
subset of the vocabulary; inputs that hold invalid token ids and counts out
of range; repeated calls with a smaller batch (the arg-max keys must be left
at zero); the hand-off from a verify step; and the full-size draft workloads.
Bar: tests/parity.py, check_draft_teacher_forced.
"""
import numpy as np
import pytest

from oracle import draft_oracle as D
from moe_decoder_speculative_amd import synth
from moe_decoder_speculative_amd.model import DraftModel, VerifyModel, to_device
import parity
import workloads

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _run(dm: DraftModel, hidden, committed, counts, R, B, K, H):
    torch = _torch()
    h = to_device(hidden)
    c = to_device(np.ascontiguousarray(committed, np.int32))
    n = to_device(np.ascontiguousarray(counts, np.int32)) if counts is not None else None
    drafts = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    states = torch.empty((K, B, H), dtype=torch.bfloat16, device="cuda")
    dm.step(h, c, n, R, B, K, drafts, states)
    torch.cuda.synchronize()
    return drafts.cpu().numpy(), parity.storage_to_f32(states)


class _Setup:
    def __init__(self, base, dwl, max_batch, k_max=7):
        self.base, self.dwl = base, dwl
        self.weights = synth.gen_weights(base)
        self.dw = synth.gen_draft_weights(dwl, base, self.weights["lm_head"])
        self.dshp = D.DraftShape(H=base.H, Id=dwl.Id, V=base.V, Vd=dwl.head_rows or base.V, dtype=base.dtype)
        self.vm = VerifyModel(base, self.weights, max_tokens=max(base.T, 8))
        self.dm = DraftModel(self.vm, dwl.Id, self.dw, max_batch=max_batch, k_max=k_max)

    def close(self):
        self.dm.close()
        self.vm.close()


def _small(Id, head_rows, seed):
    base = workloads.small_bf16(name="draft_base", B=4, K=3, L=1, seed_id=300 + seed)
    dwl = synth.DraftWorkload("draft_small", base.name, Id=Id, head_rows=head_rows, B=1, K=1, R=1, seed_id=seed)
    return base, dwl


def _inputs(setup, B, R, seed, with_counts=True, invalid=True):
    g = np.random.default_rng(seed)
    base = setup.base
    hidden = synth.to_storage(g.standard_normal((B * R, base.H), dtype=np.float32), base.dtype)
    committed = g.integers(0, base.V, size=(B, R)).astype(np.int32)
    counts = g.integers(1, R + 1, size=B).astype(np.int32) if with_counts else None
    if invalid and B >= 3:
        committed.flat[0], committed.flat[-1] = -1, base.V          # zero embeddings
        if with_counts:
            counts[1], counts[2] = 0, R + 3                          # clamped into [1, R]
    return hidden, committed, counts


@pytest.mark.parametrize("B,K,R,Id,head_rows,with_counts", [
    (1, 3, 4, 384, 0, True),
    (5, 3, 4, 1280, 0, True),
    (33, 7, 1, 384, 0, False),
    (9, 1, 8, 7168, 200, True),
    (130, 2, 4, 256, 0, True),
])
def test_draft_small(B, K, R, Id, head_rows, with_counts):
    base, dwl = _small(Id, head_rows, seed=B + 10 * K)
    parity.say(f"[draft small] B={B} K={K} R={R} Id={Id} head_rows={head_rows} counts={with_counts} "
               f"H={base.H} V={base.V} entry=moe_draft_step")
    s = _Setup(base, dwl, max_batch=max(B, 8))
    try:
        hidden, committed, counts = _inputs(s, B, R, seed=B * 7 + K)
        drafts, states = _run(s.dm, hidden, committed, counts, R, B, K, base.H)
        msg = parity.check_draft_teacher_forced(drafts, states, hidden, committed, counts, R, s.dw, s.dshp)
        parity.say(f"[draft small] ok: {msg}")
    finally:
        s.close()


def test_draft_repeated_calls_smaller_batch():
    """Two calls in a row, the second with fewer sequences and steps: the
    arg-max keys and the workspace carry nothing from one call to the next."""
    base, dwl = _small(512, 0, seed=77)
    s = _Setup(base, dwl, max_batch=40)
    try:
        for B, K, R in [(40, 3, 4), (6, 2, 2), (40, 3, 4)]:
            parity.say(f"[draft repeat] B={B} K={K} R={R}")
            hidden, committed, counts = _inputs(s, B, R, seed=1000 + B + K)
            drafts, states = _run(s.dm, hidden, committed, counts, R, B, K, base.H)
            parity.say("[draft repeat] ok: " + parity.check_draft_teacher_forced(
                drafts, states, hidden, committed, counts, R, s.dw, s.dshp))
    finally:
        s.close()


def test_draft_continues_from_verify_step():
    """A verify step's hidden_out, committed and counts handed straight to the
    draft call (R = K + 1 rows per sequence)."""
    torch = _torch()
    w = workloads.small_bf16(name="draft_chain", B=6, K=3, L=1, seed_id=88)
    case = workloads.build_case(w)
    dwl = synth.DraftWorkload("draft_chain", w.name, Id=384, head_rows=0, B=w.B, K=3, R=w.K + 1, seed_id=88)
    dw = synth.gen_draft_weights(dwl, w, case.weights["lm_head"])
    dshp = D.DraftShape(H=w.H, Id=dwl.Id, V=w.V, Vd=w.V, dtype=w.dtype)
    parity.say(f"[draft chain] B={w.B} K={w.K} entry=moe_verify_step_ex -> moe_draft_step")
    vm = VerifyModel(w, case.weights, max_tokens=w.T)
    dm = DraftModel(vm, dwl.Id, dw, max_batch=w.B)
    try:
        hidden = to_device(case.hidden)
        drafts_in = to_device(case.drafts.astype(np.int32))
        committed, counts = vm.alloc_outputs(w.B, w.K)
        aux = vm.alloc_aux(w.T)
        vm.step(hidden, drafts_in, w.B, w.K, committed, counts, aux)
        new_drafts = torch.full((w.B, 3), -7, dtype=torch.int32, device="cuda")
        states = torch.empty((3, w.B, w.H), dtype=torch.bfloat16, device="cuda")
        dm.step(aux["hidden_out"], committed, counts, w.K + 1, w.B, 3, new_drafts, states)
        torch.cuda.synchronize()
        out_h = parity.storage_to_f32(aux["hidden_out"])
        out_c, out_n = committed.cpu().numpy(), counts.cpu().numpy()
        parity.check_step(dict(committed=out_c, counts=out_n, hidden_out=out_h, tstar=aux["tstar"].cpu().numpy(),
                               **{k: aux[k].cpu().numpy() for k in ("topk_idx", "topk_w", "expert_count",
                                                                   "expert_offset", "perm", "moe_out")}),
                          case, w.B, w.K, "draft chain verify")
        hid_bits = synth.to_storage(out_h, "bf16")
        msg = parity.check_draft_teacher_forced(new_drafts.cpu().numpy(), parity.storage_to_f32(states), hid_bits,
                                                out_c, out_n, w.K + 1, dw, dshp)
        parity.say(f"[draft chain] ok: counts {out_n.tolist()}; {msg}")
    finally:
        dm.close()
        vm.close()


@pytest.mark.parametrize("name", ["draft_b1", "draft_b32", "draft_b1_head32k"])
def test_draft_full_size(name):
    """The full-size draft workloads in the launch configuration the benchmark
    times (H 1280, V 129,280, dense width 7,168, K = 3)."""
    dwl = synth.DRAFT_WORKLOADS[name]
    base = synth.WORKLOADS[dwl.base].with_(L=1)
    parity.say(f"[draft full] {name}: B={dwl.B} K={dwl.K} R={dwl.R} Id={dwl.Id} head_rows={dwl.head_rows}")
    s = _Setup(base, dwl, max_batch=dwl.B, k_max=dwl.K)
    try:
        hidden, committed, counts = synth.draft_inputs(dwl, base)
        drafts, states = _run(s.dm, hidden, committed, counts, dwl.R, dwl.B, dwl.K, base.H)
        msg = parity.check_draft_teacher_forced(drafts, states, hidden, committed, counts, dwl.R, s.dw, s.dshp)
        parity.say(f"[draft full] {name} ok: {msg}")
    finally:
        s.close()


def test_draft_graph_replay_matches_eager():
    """A captured draft call replayed four times, with eager calls of the same
    context between the replays: every replay equals the eager result bit for
    bit."""
    torch = _torch()
    from moe_decoder_speculative_amd import binding
    base, dwl = _small(1280, 0, seed=55)
    B, K, R = 12, 3, 4
    parity.say(f"[draft graph] B={B} K={K} R={R} entry=moe_draft_graph_create/moe_verify_graph_launch")
    s = _Setup(base, dwl, max_batch=B)
    g = None
    try:
        hidden, committed, counts = _inputs(s, B, R, seed=5)
        h = to_device(hidden)
        c = to_device(committed)
        n = to_device(counts)
        ref_d = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
        ref_s = torch.empty((K, B, base.H), dtype=torch.bfloat16, device="cuda")
        s.dm.step(h, c, n, R, B, K, ref_d, ref_s)
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        gd = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
        gs = torch.zeros((K, B, base.H), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        g = binding.moe_draft_graph_create(s.dm.ctx, h, c, n, R, B, K, gd, gs, stream)
        other_d = torch.empty_like(ref_d)
        for rep in range(4):
            gd.fill_(-7)
            gs.zero_()
            torch.cuda.synchronize()
            binding.moe_verify_graph_launch(g, stream)
            stream.synchronize()
            assert torch.equal(gd, ref_d), f"replay {rep}: drafts differ"
            assert torch.equal(gs, ref_s), f"replay {rep}: states differ"
            s.dm.step(h, c, n, R, B, K, other_d)
            torch.cuda.synchronize()
            assert torch.equal(other_d, ref_d)
        parity.say(f"[draft graph] ok: 4 replays equal to eager, drafts[0] {ref_d[0].tolist()}")
    finally:
        if g:
            binding.moe_verify_graph_destroy(g)
        s.close()
