"""The C ABI library loads, exports every function include/*.h declares,
and rejects bad arguments before any HIP runtime call (so these run without a
GPU)."""
import ctypes
import os
import re

import pytest

from moe_decoder_speculative_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared():
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names.update(re.findall(r"\b(moe_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_binding_names():
    assert _declared() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(hidden=256, n_routed=8, top_k=2, n_shared=1, inter=128, vocab=1024, n_layers=1,
                max_tokens=64, max_prefill_tokens=0, k_max=3, rms_eps=1e-6, dtype=B.MOE_DTYPE_BF16,
                has_lm_head=1)
    base.update(kw)
    return B.MoeVerifyConfig(**base)


FAKE = 0x10000  # aligned, never dereferenced: validation fails first


def _weights(**kw):
    base = {n: FAKE for n, _ in B.MoeVerifyWeights._fields_}
    base.update(kw)
    return B.MoeVerifyWeights(**base)


def _init_rc(cfg, w):
    lib = B.load_library()
    out = ctypes.c_void_p(1234)
    rc = lib.moe_verify_init(ctypes.byref(cfg) if cfg is not None else None,
                             ctypes.byref(w) if w is not None else None, None, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("bad", [
    dict(hidden=100), dict(hidden=0), dict(hidden=1664), dict(hidden=896, dtype=0), dict(inter=96), dict(n_routed=0),
    dict(n_routed=65), dict(top_k=0), dict(top_k=9), dict(n_routed=4, top_k=5), dict(n_shared=-1),
    dict(n_shared=5), dict(n_layers=0), dict(max_tokens=0), dict(max_tokens=70000),
    dict(max_prefill_tokens=-1), dict(k_max=-1), dict(k_max=8), dict(rms_eps=0.0),
    dict(rms_eps=float("nan")), dict(dtype=2), dict(has_lm_head=2), dict(vocab=0),
])
def test_init_rejects_bad_config(bad):
    rc, out = _init_rc(_cfg(**bad), _weights())
    assert rc == B.MOE_EINVAL
    assert out is None
    assert B.moe_verify_last_error().startswith("config:")


@pytest.mark.parametrize("field", ["router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                   "norm_gamma", "final_gamma", "lm_head"])
def test_init_rejects_null_or_misaligned_weight(field):
    rc, _ = _init_rc(_cfg(), _weights(**{field: None}))
    assert rc == B.MOE_EINVAL and field in B.moe_verify_last_error()
    rc, _ = _init_rc(_cfg(), _weights(**{field: FAKE + 8}))
    assert rc == B.MOE_EINVAL and "aligned" in B.moe_verify_last_error()


def test_optional_weights_may_be_null():
    # S = 0 and no LM head: shared and head pointers are not required.  The
    # injected allocation failure stops init right after validation.
    os.environ["MOE_VERIFY_FAULT"] = "alloc"
    try:
        rc, out = _init_rc(_cfg(n_shared=0, has_lm_head=0),
                           _weights(s_gate=None, s_up=None, s_down=None, final_gamma=None, lm_head=None))
    finally:
        del os.environ["MOE_VERIFY_FAULT"]
    assert rc in (B.MOE_ENOMEM, B.MOE_EHIP) and out is None


def test_init_null_arguments():
    assert _init_rc(None, _weights())[0] == B.MOE_EINVAL
    assert _init_rc(_cfg(), None)[0] == B.MOE_EINVAL


def test_step_and_block_reject_null_context():
    lib = B.load_library()
    rc = lib.moe_verify_step(None, FAKE, FAKE, 1, 3, FAKE, FAKE, None)
    assert rc == B.MOE_EINVAL and "ctx" in B.moe_verify_last_error()
    rc = lib.moe_verify_step_ex(None, FAKE, FAKE, 1, 3, FAKE, FAKE, None, None)
    assert rc == B.MOE_EINVAL
    rc = lib.moe_block_forward(None, 0, FAKE, 4, FAKE, None, None)
    assert rc == B.MOE_EINVAL
    rc = lib.moe_verify_step_static(None, FAKE, FAKE, 1, 3, FAKE, FAKE, None)
    assert rc == B.MOE_EINVAL and "ctx" in B.moe_verify_last_error()


def test_destroy_null_is_a_no_op():
    B.moe_verify_destroy(None)


def test_binding_raises_with_message():
    with pytest.raises(B.MoeVerifyError) as ei:
        B.moe_verify_init(_cfg(hidden=3), _weights())
    assert ei.value.code == B.MOE_EINVAL and "hidden" in ei.value.message


def test_graph_calls_reject_null_arguments():
    lib = B.load_library()
    out = ctypes.c_void_p(1)
    rc = lib.moe_verify_graph_create(None, None, None, 1, 3, None, None, ctypes.c_void_p(1), ctypes.byref(out))
    assert rc == B.MOE_EINVAL and "ctx" in B.moe_verify_last_error() and out.value is None
    rc = lib.moe_verify_graph_create(ctypes.c_void_p(8), None, None, 1, 3, None, None, ctypes.c_void_p(1), None)
    assert rc == B.MOE_EINVAL and "out" in B.moe_verify_last_error()
    rc = lib.moe_verify_graph_launch(None, None)
    assert rc == B.MOE_EINVAL and "graph" in B.moe_verify_last_error()
    lib.moe_verify_graph_destroy(None)


def test_draft_calls_reject_null_arguments():
    lib = B.load_library()
    out = ctypes.c_void_p(99)
    cfg = B.MoeDraftConfig(inter=256, head_rows=0, max_batch=4, k_max=3)
    w = B.MoeDraftWeights(**{n: FAKE for n, _ in B.MoeDraftWeights._fields_})
    assert lib.moe_draft_init(None, ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == B.MOE_EINVAL
    assert out.value is None
    assert lib.moe_draft_step(None, FAKE, FAKE, None, 4, 1, 3, FAKE, None, None) == B.MOE_EINVAL
    assert "NULL" in B.moe_verify_last_error()
    assert lib.moe_draft_graph_create(None, FAKE, FAKE, None, 4, 1, 3, FAKE, None, FAKE, None) == B.MOE_EINVAL
    g = ctypes.c_void_p(5)
    assert lib.moe_draft_graph_create(None, FAKE, FAKE, None, 4, 1, 3, FAKE, None, FAKE, ctypes.byref(g)) == \
        B.MOE_EINVAL
    assert g.value is None
    assert lib.moe_draft_set_stage_events(None, 0, None, None) == B.MOE_EINVAL
    lib.moe_draft_destroy(None)


def _attn_cfg(**kw):
    base = dict(n_heads=2, max_positions=64, max_seqs=4, rope_theta=10000.0)
    base.update(kw)
    return _cfg(**base)


@pytest.mark.parametrize("bad", [
    dict(n_heads=-1), dict(n_heads=3), dict(max_positions=4), dict(max_positions=40000), dict(max_seqs=0),
    dict(max_seqs=2000), dict(rope_theta=0.0), dict(rope_theta=float("inf")),
])
def test_init_rejects_bad_attention_config(bad):
    rc, out = _init_rc(_attn_cfg(**bad), _weights())
    assert rc == B.MOE_EINVAL and out is None
    assert B.moe_verify_last_error().startswith("config:")


def test_attention_needs_bf16():
    rc, out = _init_rc(_attn_cfg(dtype=B.MOE_DTYPE_F32), _weights())
    assert rc == B.MOE_EUNSUPPORTED and out is None


@pytest.mark.parametrize("field", ["attn_gamma", "w_q", "w_k", "w_v", "w_o"])
def test_attention_weights_required(field):
    rc, _ = _init_rc(_attn_cfg(), _weights(**{field: None}))
    assert rc == B.MOE_EINVAL and field in B.moe_verify_last_error()
    # without attention they may be NULL (init then stops at the injected allocation failure)
    os.environ["MOE_VERIFY_FAULT"] = "alloc"
    try:
        rc, _ = _init_rc(_cfg(), _weights(**{field: None}))
    finally:
        del os.environ["MOE_VERIFY_FAULT"]
    assert rc in (B.MOE_ENOMEM, B.MOE_EHIP)


def test_step_kv_and_cache_reject_null_arguments():
    lib = B.load_library()
    rc = lib.moe_verify_step_kv(None, FAKE, FAKE, FAKE, 1, 3, FAKE, FAKE, None, None)
    assert rc == B.MOE_EINVAL and "ctx" in B.moe_verify_last_error()
    rc = lib.moe_verify_step_kv(None, FAKE, FAKE, None, 1, 3, FAKE, FAKE, None, None)
    assert rc == B.MOE_EINVAL and "positions" in B.moe_verify_last_error()
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.moe_verify_kv_cache(None, ctypes.byref(k), ctypes.byref(v)) == B.MOE_EINVAL


def test_graph_kv_rejects_null_arguments():
    lib = B.load_library()
    out = ctypes.c_void_p(1)
    rc = lib.moe_verify_graph_create_kv(None, FAKE, FAKE, FAKE, 1, 3, FAKE, FAKE, FAKE, ctypes.byref(out))
    assert rc == B.MOE_EINVAL and out.value is None
    rc = lib.moe_verify_graph_create_kv(ctypes.c_void_p(8), FAKE, FAKE, None, 1, 3, FAKE, FAKE, FAKE,
                                        ctypes.byref(out))
    assert rc == B.MOE_EINVAL and "positions" in B.moe_verify_last_error()
