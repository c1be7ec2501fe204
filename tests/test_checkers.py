"""The GPU-parity checkers themselves, on the CPU: fed the oracle's own
per-block results they pass, and each planted mistake makes them fail."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from moe_decoder_speculative_amd import synth
import parity
import workloads

W = workloads.small_bf16(B=16, K=0, L=3, seed_id=90).with_(has_lm_head=False, drafts="none")


def _per_layer(w):
    """The oracle's own per-block outputs, shaped as the GPU tests collect them."""
    shp = workloads.shape_of(w)
    weights = synth.gen_weights(w)
    noise = synth.HiddenNoise(w)
    offset = synth.hidden_offset(w, weights, noise)
    x0 = synth.to_storage(noise.draw(w.T) + offset, w.dtype)
    per = []
    x = O.as_f32(x0)
    for l in range(w.L):
        r = O.moe_block(x, weights["layers"][l], shp)
        per.append({"topk_idx": r.idx.copy(), "topk_w": r.w.copy(), "moe_out": r.m.copy(),
                    "x_out": r.x_out.copy(), "z": r.z})
        x = r.x_out
    return shp, weights, x0, per


def test_rows_teacher_forced_accepts_the_oracle():
    shp, weights, x0, per = _per_layer(W)
    parity.check_rows_teacher_forced(per, x0, weights, shp)


@pytest.mark.parametrize("plant", ["x_out_ulp", "moe_out", "gate_weight", "expert"])
def test_rows_teacher_forced_rejects(plant):
    shp, weights, x0, per = _per_layer(W)
    g = per[1]
    if plant == "x_out_ulp":
        # one element of the block output one bf16 ulp off
        bits = g["x_out"].view(np.uint32)
        bits[5, 7] += np.uint32(1 << 16)
    elif plant == "moe_out":
        g["moe_out"][3] *= 1.05
    elif plant == "gate_weight":
        g["topk_w"][2, 0] += 5e-3
    else:
        # the best-separated row gets one selected expert swapped for an unselected one
        t = int(np.argmax(O.topk_margin(g["z"], shp.k)))
        unused = np.setdiff1d(np.arange(shp.E), g["topk_idx"][t])[0]
        g["topk_idx"][t, -1] = unused
    with pytest.raises(AssertionError):
        parity.check_rows_teacher_forced(per, x0, weights, shp)
