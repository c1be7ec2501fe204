"""Thin ctypes binding of libmoeverify.so (C ABI in include/moe_verify.h and
include/moe_draft.h).

The functions keep the C names.  They only marshal arguments: torch tensors
supply device memory (data_ptr) and the HIP stream (the current torch stream
by default); every step of the computation runs in the library's HIP kernels.
If the library has not been built the import of any entry point raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoeverify.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOMEM, MOE_EHIP = 0, -1, -2, -3, -4
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
EXPORTED = ("moe_verify_init", "moe_verify_step", "moe_verify_step_ex", "moe_verify_step_kv",
            "moe_verify_step_static",
            "moe_verify_kv_cache", "moe_block_forward",
            "moe_verify_graph_create", "moe_verify_graph_create_kv", "moe_verify_graph_launch",
            "moe_verify_graph_destroy",
            "moe_verify_set_stage_events", "moe_verify_destroy", "moe_verify_last_error",
            "moe_draft_init", "moe_draft_step", "moe_draft_graph_create", "moe_draft_set_stage_events",
            "moe_draft_destroy")
MOE_STAGE_LMHEAD, MOE_STAGE_EXPERT_UP, MOE_STAGE_EXPERT_DOWN, MOE_STAGE_ALL, MOE_STAGE_ATTENTION = 0, 1, 2, 3, 4


class MoeVerifyError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


class MoeVerifyConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("inter", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("max_prefill_tokens", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("has_lm_head", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("max_positions", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
                ("rope_theta", ctypes.c_float)]


class MoeVerifyWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("router", "w_gate", "w_up", "w_down", "s_gate", "s_up",
                                                "s_down", "norm_gamma", "final_gamma", "lm_head", "attn_gamma",
                                                "w_q", "w_k", "w_v", "w_o")]


class MoeVerifyAux(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_w", "expert_count", "expert_offset",
                                                "perm", "moe_out", "hidden_out", "tstar", "attn_out")]


class MoeDraftConfig(ctypes.Structure):
    _fields_ = [("inter", ctypes.c_int32), ("head_rows", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("k_max", ctypes.c_int32)]


class MoeDraftWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("embed", "gamma_h", "gamma_e", "w_proj", "gamma_f", "w_gate",
                                                "w_up", "w_down", "gamma_o", "head", "head_ids")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.moe_verify_init.argtypes = [ctypes.POINTER(MoeVerifyConfig), ctypes.POINTER(MoeVerifyWeights), vp,
                                    ctypes.POINTER(vp)]
    lib.moe_verify_init.restype = ctypes.c_int
    lib.moe_verify_step.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp]
    lib.moe_verify_step.restype = ctypes.c_int
    lib.moe_verify_step_static.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp]
    lib.moe_verify_step_static.restype = ctypes.c_int
    lib.moe_verify_step_ex.argtypes = [vp, vp, vp, i32, i32, vp, vp, ctypes.POINTER(MoeVerifyAux), vp]
    lib.moe_verify_step_ex.restype = ctypes.c_int
    lib.moe_verify_step_kv.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, ctypes.POINTER(MoeVerifyAux), vp]
    lib.moe_verify_step_kv.restype = ctypes.c_int
    lib.moe_verify_kv_cache.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.moe_verify_kv_cache.restype = ctypes.c_int
    lib.moe_block_forward.argtypes = [vp, i32, vp, i32, vp, ctypes.POINTER(MoeVerifyAux), vp]
    lib.moe_block_forward.restype = ctypes.c_int
    lib.moe_verify_graph_create.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, ctypes.POINTER(vp)]
    lib.moe_verify_graph_create.restype = ctypes.c_int
    lib.moe_verify_graph_create_kv.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, ctypes.POINTER(vp)]
    lib.moe_verify_graph_create_kv.restype = ctypes.c_int
    lib.moe_verify_graph_launch.argtypes = [vp, vp]
    lib.moe_verify_graph_launch.restype = ctypes.c_int
    lib.moe_verify_graph_destroy.argtypes = [vp]
    lib.moe_verify_graph_destroy.restype = None
    lib.moe_verify_set_stage_events.argtypes = [vp, i32, vp, vp]
    lib.moe_verify_set_stage_events.restype = ctypes.c_int
    lib.moe_verify_destroy.argtypes = [vp]
    lib.moe_verify_destroy.restype = None
    lib.moe_verify_last_error.argtypes = []
    lib.moe_verify_last_error.restype = ctypes.c_char_p
    lib.moe_draft_init.argtypes = [vp, ctypes.POINTER(MoeDraftConfig), ctypes.POINTER(MoeDraftWeights), vp,
                                   ctypes.POINTER(vp)]
    lib.moe_draft_init.restype = ctypes.c_int
    lib.moe_draft_step.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.moe_draft_step.restype = ctypes.c_int
    lib.moe_draft_graph_create.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, ctypes.POINTER(vp)]
    lib.moe_draft_graph_create.restype = ctypes.c_int
    lib.moe_draft_set_stage_events.argtypes = [vp, i32, vp, vp]
    lib.moe_draft_set_stage_events.restype = ctypes.c_int
    lib.moe_draft_destroy.argtypes = [vp]
    lib.moe_draft_destroy.restype = None
    _lib = lib
    return lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeVerifyError(rc, moe_verify_last_error())


def _ptr(t) -> int | None:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None  # the default stream; calls without a GPU fail in validation or in HIP
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def moe_verify_last_error() -> str:
    return load_library().moe_verify_last_error().decode()


def moe_verify_init(cfg: MoeVerifyConfig, weights: MoeVerifyWeights, stream=None) -> int:
    """Create a context (weights are repacked into it); returns its handle."""
    out = ctypes.c_void_p()
    _check(load_library().moe_verify_init(ctypes.byref(cfg), ctypes.byref(weights), _stream(stream),
                                          ctypes.byref(out)))
    return out.value


def moe_verify_step(ctx: int, hidden, drafts, B: int, K: int, committed, counts, stream=None) -> None:
    _check(load_library().moe_verify_step(ctx, _ptr(hidden), _ptr(drafts), B, K, _ptr(committed),
                                          _ptr(counts), _stream(stream)))


def moe_verify_step_static(ctx: int, hidden, drafts, B: int, K: int, committed, counts, stream=None) -> None:
    """moe_verify_step with the workspace in the library's static device scratch (allocates nothing)."""
    _check(load_library().moe_verify_step_static(ctx, _ptr(hidden), _ptr(drafts), B, K, _ptr(committed),
                                                 _ptr(counts), _stream(stream)))


def make_aux(**tensors) -> MoeVerifyAux:
    """An aux struct from tensors keyed by field name (missing fields NULL)."""
    aux = MoeVerifyAux()
    for name, _ in MoeVerifyAux._fields_:
        setattr(aux, name, _ptr(tensors.get(name)))
    return aux


def moe_verify_step_ex(ctx: int, hidden, drafts, B: int, K: int, committed, counts, aux: MoeVerifyAux | None,
                       stream=None) -> None:
    _check(load_library().moe_verify_step_ex(ctx, _ptr(hidden), _ptr(drafts), B, K, _ptr(committed),
                                             _ptr(counts), ctypes.byref(aux) if aux is not None else None,
                                             _stream(stream)))


def moe_verify_step_kv(ctx: int, hidden, drafts, positions, B: int, K: int, committed, counts,
                       aux: MoeVerifyAux | None = None, stream=None) -> None:
    _check(load_library().moe_verify_step_kv(ctx, _ptr(hidden), _ptr(drafts), _ptr(positions), B, K,
                                             _ptr(committed), _ptr(counts),
                                             ctypes.byref(aux) if aux is not None else None, _stream(stream)))


def moe_verify_kv_cache(ctx: int) -> tuple[int, int]:
    """Device addresses of the key and value caches ([L][seqs][heads][P][128] bf16)."""
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    _check(load_library().moe_verify_kv_cache(ctx, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def moe_block_forward(ctx: int, layer: int, x, T: int, y, aux: MoeVerifyAux | None = None, stream=None) -> None:
    _check(load_library().moe_block_forward(ctx, layer, _ptr(x), T, _ptr(y),
                                            ctypes.byref(aux) if aux is not None else None, _stream(stream)))


def moe_verify_graph_create(ctx: int, hidden, drafts, B: int, K: int, committed, counts, stream) -> int:
    """Capture one verify step on `stream` (not the default stream) into a graph handle."""
    out = ctypes.c_void_p()
    _check(load_library().moe_verify_graph_create(ctx, _ptr(hidden), _ptr(drafts), B, K, _ptr(committed),
                                                  _ptr(counts), _stream(stream), ctypes.byref(out)))
    return out.value


def moe_verify_graph_create_kv(ctx: int, hidden, drafts, positions, B: int, K: int, committed, counts,
                               stream) -> int:
    """Capture one moe_verify_step_kv on `stream` into a graph handle."""
    out = ctypes.c_void_p()
    _check(load_library().moe_verify_graph_create_kv(ctx, _ptr(hidden), _ptr(drafts), _ptr(positions), B, K,
                                                     _ptr(committed), _ptr(counts), _stream(stream),
                                                     ctypes.byref(out)))
    return out.value


def moe_verify_graph_launch(graph: int, stream=None) -> None:
    _check(load_library().moe_verify_graph_launch(graph, _stream(stream)))


def moe_verify_graph_destroy(graph: int | None) -> None:
    load_library().moe_verify_graph_destroy(graph)


def moe_verify_set_stage_events(ctx: int, stage: int, before: int | None, after: int | None) -> None:
    """Bracket `stage` of the next call on ctx with two hipEvent_t handles."""
    _check(load_library().moe_verify_set_stage_events(ctx, stage, before, after))


def moe_verify_destroy(ctx: int | None) -> None:
    load_library().moe_verify_destroy(ctx)


def moe_draft_init(verifier: int, cfg: MoeDraftConfig, weights: MoeDraftWeights, stream=None) -> int:
    """Create a draft context bound to a verifier context; returns its handle."""
    out = ctypes.c_void_p()
    _check(load_library().moe_draft_init(verifier, ctypes.byref(cfg), ctypes.byref(weights), _stream(stream),
                                         ctypes.byref(out)))
    return out.value


def moe_draft_step(ctx: int, hidden, committed, counts, R: int, B: int, K: int, drafts, states=None,
                   stream=None) -> None:
    _check(load_library().moe_draft_step(ctx, _ptr(hidden), _ptr(committed), _ptr(counts), R, B, K, _ptr(drafts),
                                         _ptr(states), _stream(stream)))


def moe_draft_graph_create(ctx: int, hidden, committed, counts, R: int, B: int, K: int, drafts, states,
                           stream) -> int:
    """Capture one draft call on `stream` into a graph handle (launch / destroy
    with moe_verify_graph_launch / moe_verify_graph_destroy)."""
    out = ctypes.c_void_p()
    _check(load_library().moe_draft_graph_create(ctx, _ptr(hidden), _ptr(committed), _ptr(counts), R, B, K,
                                                 _ptr(drafts), _ptr(states), _stream(stream), ctypes.byref(out)))
    return out.value


def moe_draft_set_stage_events(ctx: int, stage: int, before: int | None, after: int | None) -> None:
    _check(load_library().moe_draft_set_stage_events(ctx, stage, before, after))


def moe_draft_destroy(ctx: int | None) -> None:
    load_library().moe_draft_destroy(ctx)
