"""The margin-selected rows of the 12-block workload, on the CPU: the stored
stream positions reproduce rows that meet the stored gap schedule along the
oracle's own trajectory, and a second float32 evaluation of the same stack --
every sum accumulated in float64 and rounded once, with the same bf16
rounding points -- takes the same expert set at every block and the same
greedy pick for every row.  The GPU test of the stack holds the kernels to the
oracle on exactly these rows."""
import numpy as np
import pytest

from oracle import moe_oracle as O
import parity
import workloads


def _second_evaluation_block(x, lw, shp):
    """One block with float64 accumulation of every sum (RMS, router logits,
    gate/up/down products), each result rounded once to float32, then the
    same R1/R2/R3 roundings and combine order as the oracle."""
    F32 = np.float32
    store = O.storage_round(shp.dtype)
    x = O.as_f32(x)
    ms = np.mean(x.astype(np.float64) ** 2, axis=-1, keepdims=True).astype(F32)
    xh = store((x / np.sqrt(ms + F32(shp.eps)) * O.as_f32(lw["gamma"])).astype(F32))
    z = (xh.astype(np.float64) @ O.as_f32(lw["router"]).astype(np.float64).T).astype(F32)
    idx, wt = O.topk_select(z, shp.k)

    def expert(rows, g, u, d):
        rows = rows.astype(np.float64)
        gg = (rows @ O.as_f32(g).astype(np.float64).T).astype(F32)
        uu = (rows @ O.as_f32(u).astype(np.float64).T).astype(F32)
        a = store((gg / (F32(1) + np.exp(-gg)) * uu).astype(F32))
        return (a.astype(np.float64) @ O.as_f32(d).astype(np.float64).T).astype(F32)

    m = np.zeros(x.shape, F32)
    for s in range(shp.S):
        m = m + expert(xh, lw["s_gate"][s], lw["s_up"][s], lw["s_down"][s])
    y = {}
    for e in np.unique(idx):
        rows = np.where((idx == e).any(1))[0]
        for r, v in zip(rows, expert(xh[rows], lw["gate"][e], lw["up"][e], lw["down"][e])):
            y[(int(r), int(e))] = v
    for t in range(x.shape[0]):
        for j in np.argsort(idx[t], kind="stable"):
            m[t] = m[t] + wt[t, j] * y[(t, int(idx[t, j]))]
    return store((x + m).astype(F32)), idx


@pytest.mark.slow
def test_stack12_margin_rows_survive_a_second_float32_evaluation():
    case = workloads.margin_rows_case("stack12_b32_zipf")   # asserts the schedule on the oracle's trajectory
    shp = case.shp
    x = O.as_f32(case.hidden)
    for l in range(shp.L):
        x, idx = _second_evaluation_block(x, case.weights["layers"][l], shp)
        assert np.array_equal(np.sort(idx, 1), np.sort(case.ref.blocks[l].idx, 1)), f"block {l}"
    lg = O.lm_head_logits(x, case.weights["final_gamma"], case.weights["lm_head"], shp.eps,
                          O.storage_round(shp.dtype))
    assert np.array_equal(O.greedy_pick(lg), case.ref.tstar)
    # the two evaluations' residual streams after the twelfth block differ by
    # about 2e-2 of a row's scale (the trajectories drift); the GPU test's
    # end-to-end bar for that residual sits above this spread
    spread = parity.rowwise_rel_err(x, case.ref.hidden_out).max()
    assert spread <= 3e-2 < parity.STACK12_HIDDEN_TOL, spread


@pytest.mark.slow
def test_attn_stack12_margin_sequences_meet_their_schedule():
    """The stored single-row sequences of the 12-layer step with attention
    reproduce, from their stream positions and cache seeds, rows whose every
    layer's top-k gap and the head's arg-max gap meet the stored schedule
    along the oracle's own trajectory; the schedule is 1.5 times the MoE-only
    stack's at every layer and at the head."""
    import json
    import os
    with open(os.path.join(workloads.GOLDEN, "attn_stack12_b32_zipf_seqs.json")) as f:
        spec = json.load(f)
    moe = json.load(open(os.path.join(workloads.GOLDEN, "stack12_b32_zipf_rows.json")))
    assert np.allclose(spec["router_margin"], 1.5 * np.asarray(moe["router_margin"]))
    assert np.isclose(spec["head_margin"], 1.5 * moe["head_margin"])
    case = workloads.attn_margin_seqs_case()      # asserts the schedule
    assert len(case.cands) == len(set(case.cands)) >= 6
    assert np.all(case.positions + 1 <= case.w.P)
