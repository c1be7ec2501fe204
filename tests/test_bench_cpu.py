"""bench.py on the CPU: its byte and flop models against hand-computed values,
its workload list against the generators', and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from moe_decoder_speculative_amd import synth  # noqa: E402


def test_lmhead_bytes_decode_b1():
    # V*H*2 + T*H*2 + T*8 at V = 129,280, H = 1,280, T = 4
    assert bench.lmhead_bytes(synth.WORKLOADS["decode_b1"]) == 129280 * 1280 * 2 + 4 * 1280 * 2 + 4 * 8
    assert bench.lmhead_bytes(synth.WORKLOADS["decode_b1"]) == 330_967_072


def test_expert_and_step_bytes():
    w = synth.WORKLOADS["decode_b1"]
    assert bench.expert_bytes(w) == 6_881_280
    # one layer, 22 touched experts
    want = 22 * 6_881_280 + 2 * 6_881_280 + 64 * 1280 * 2 + 2 * 4 * 1280 * 2 + 129280 * 1280 * 2
    assert bench.step_bytes(w, [22]) == want


def test_draft_bytes():
    H, Id, V, B, K = 1280, 7168, 129280, 1, 3
    head = V * H * 2 + B * H * 2 + 8 * B
    assert bench.draft_head_bytes(H, V, B) == head
    per = 2 * H * H * 2 + 3 * Id * H * 2 + head + 2 * B * H * 2
    assert bench.draft_call_bytes(H, Id, V, B, K) == K * per + B * H * 2 + B * K * 4


def test_attention_bytes():
    w = synth.WORKLOADS["attn_b32_zipf"]
    pos = np.array([100, 2000] + [1220] * (w.B - 2))
    assert bench.attn_kv_bytes(w, pos) == sum(10 * (p + 4) * 512 for p in pos)
    assert bench.attn_step_bytes(w, pos) == 4 * 1280 * 1280 * 2 + bench.attn_kv_bytes(w, pos) + w.T * 10 * 512
    assert bench.attn_step_bytes(synth.WORKLOADS["decode_b1"], None) == 0


def _workload_choices():
    src = open(os.path.join(ROOT, "bench.py")).read()
    start = src.index('ap.add_argument("--workload"')
    block = src[start:src.index("])", start)]
    return set(eval("[" + block.split("choices=[", 1)[1] + "]"))


def test_every_workload_is_a_bench_choice():
    choices = _workload_choices()
    for name in list(synth.WORKLOADS) + list(synth.DRAFT_WORKLOADS):
        if name == "tiny_fp32":
            continue
        assert name in choices, name


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
