"""Device-side setup around the C ABI: upload seeded weights, create a
context, allocate step buffers.  Torch provides device memory and streams only.
"""
from __future__ import annotations

import numpy as np

from . import binding as B_
from .synth import Workload


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray, device="cuda"):
    """numpy float32 / uint16 (bfloat16 bits) / int32 array -> device tensor."""
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


_hip = None


def hip_memcpy(dst: int, src: int, nbytes: int, kind: int):
    """Synchronous hipMemcpy between raw addresses (kind 1: host to device,
    2: device to host), for filling or reading a context's KV cache."""
    import ctypes
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    rc = _hip.hipMemcpy(dst, src, nbytes, kind)
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")


def _stacked(weights: dict, key: str, device):
    """Per-layer arrays stacked into one [L, ...] device tensor, one layer at a time."""
    torch = _torch()
    layers = weights["layers"]
    first = layers[0][key]
    dtype = torch.bfloat16 if first.dtype == np.uint16 else torch.float32
    out = torch.empty((len(layers),) + first.shape, dtype=dtype, device=device)
    for l, lw in enumerate(layers):
        out[l].copy_(to_device(lw[key], device))
    return out


class VerifyModel:
    """A library context for a workload's shapes and weights.

    Weights are uploaded, handed to moe_verify_init (which repacks them into
    the context) and released again.
    """

    def __init__(self, w: Workload, weights: dict, max_tokens: int | None = None,
                 max_prefill_tokens: int = 0, k_max: int = 7, device="cuda", stream=None, copies: int = 1,
                 max_seqs: int | None = None):
        torch = _torch()
        self.w = w
        self.device = device
        self.max_tokens = max_tokens or max(w.T, 1)
        cfg = B_.MoeVerifyConfig(
            hidden=w.H, n_routed=w.E, top_k=w.k, n_shared=w.S, inter=w.I, vocab=w.V if w.has_lm_head else 0,
            n_layers=len(weights["layers"]), max_tokens=self.max_tokens, max_prefill_tokens=max_prefill_tokens,
            k_max=k_max, rms_eps=w.eps, dtype=B_.MOE_DTYPE_BF16 if w.dtype == "bf16" else B_.MOE_DTYPE_F32,
            has_lm_head=1 if w.has_lm_head else 0, n_heads=w.n_heads,
            max_positions=w.P if w.n_heads else 0, max_seqs=(max_seqs or max(w.B, 1)) if w.n_heads else 0,
            rope_theta=w.rope_theta if w.n_heads else 0.0)
        self.cfg = cfg
        names = ["router", "gate", "up", "down", "s_gate", "s_up", "s_down", "gamma"]
        if w.n_heads:
            names += ["attn_gamma", "w_q", "w_k", "w_v", "w_o"]
        t = {k: _stacked(weights, k, device) for k in names}
        fg = to_device(weights["final_gamma"], device) if w.has_lm_head else None
        lm = to_device(weights["lm_head"], device) if w.has_lm_head else None
        wts = B_.MoeVerifyWeights(
            router=t["router"].data_ptr(), w_gate=t["gate"].data_ptr(), w_up=t["up"].data_ptr(),
            w_down=t["down"].data_ptr(),
            s_gate=t["s_gate"].data_ptr() if w.S else None, s_up=t["s_up"].data_ptr() if w.S else None,
            s_down=t["s_down"].data_ptr() if w.S else None, norm_gamma=t["gamma"].data_ptr(),
            final_gamma=fg.data_ptr() if fg is not None else None, lm_head=lm.data_ptr() if lm is not None else None,
            **({k: t[k].data_ptr() for k in ("attn_gamma", "w_q", "w_k", "w_v", "w_o")} if w.n_heads else {}))
        torch.cuda.synchronize()
        # `copies` independent contexts (separate repacked weights) let a
        # benchmark rotate among them so no weight byte is served from the
        # last-level cache of a previous step
        self.ctxs = []
        try:
            for _ in range(copies):
                self.ctxs.append(B_.moe_verify_init(cfg, wts, stream))
        except Exception:
            self.close()
            raise
        self.ctx = self.ctxs[0]
        del t, fg, lm
        torch.cuda.synchronize()
        self.store_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    # ------------------------------------------------------------------
    def kv_slab_elems(self) -> int:
        """bf16 elements of one (layer, sequence) slab of the cache: [heads][P][128]."""
        return self.cfg.n_heads * self.cfg.max_positions * 128

    def kv_write(self, l: int, b: int, k: np.ndarray, v: np.ndarray, copy: int = 0):
        """Cache entries 0..n-1 of layer l, sequence b from uint16 (bf16 bits)
        arrays [heads, n, 128]; the rest of the slab is zeroed."""
        P = self.cfg.max_positions
        kptr, vptr = B_.moe_verify_kv_cache(self.ctxs[copy])
        off = (l * self.cfg.max_seqs + b) * self.kv_slab_elems() * 2
        for src, base in ((k, kptr), (v, vptr)):
            slab = np.zeros((self.cfg.n_heads, P, 128), np.uint16)
            slab[:, :src.shape[1]] = src
            hip_memcpy(base + off, slab.ctypes.data, slab.nbytes, 1)

    def kv_read(self, l: int, b: int, copy: int = 0):
        """(k, v) slabs of layer l, sequence b as uint16 arrays [heads, P, 128]."""
        _torch().cuda.synchronize()
        P = self.cfg.max_positions
        kptr, vptr = B_.moe_verify_kv_cache(self.ctxs[copy])
        off = (l * self.cfg.max_seqs + b) * self.kv_slab_elems() * 2
        out = []
        for base in (kptr, vptr):
            slab = np.empty((self.cfg.n_heads, P, 128), np.uint16)
            hip_memcpy(slab.ctypes.data, base + off, slab.nbytes, 2)
            out.append(slab)
        return out

    def step_kv(self, hidden, drafts, positions, B: int, K: int, committed, counts, aux: dict | None = None,
                stream=None, copy: int = 0):
        B_.moe_verify_step_kv(self.ctxs[copy], hidden, drafts if K > 0 else None, positions, B, K, committed, counts,
                              B_.make_aux(**aux) if aux else None, stream)

    def alloc_outputs(self, B: int, K: int):
        torch = _torch()
        committed = torch.empty((B, K + 1), dtype=torch.int32, device=self.device)
        counts = torch.empty((B,), dtype=torch.int32, device=self.device)
        return committed, counts

    def alloc_aux(self, T: int, layers: int | None = None, with_hidden=True):
        torch = _torch()
        L = layers or self.cfg.n_layers
        w = self.w
        aux = dict(
            topk_idx=torch.empty((L, T, w.k), dtype=torch.int32, device=self.device),
            topk_w=torch.empty((L, T, w.k), dtype=torch.float32, device=self.device),
            expert_count=torch.empty((L, w.E), dtype=torch.int32, device=self.device),
            expert_offset=torch.empty((L, w.E + 1), dtype=torch.int32, device=self.device),
            perm=torch.empty((L, T * w.k), dtype=torch.int32, device=self.device),
            moe_out=torch.empty((L, T, w.H), dtype=torch.float32, device=self.device),
            tstar=torch.empty((T,), dtype=torch.int32, device=self.device),
        )
        if with_hidden:
            aux["hidden_out"] = torch.empty((T, w.H), dtype=self.store_dtype, device=self.device)
        if w.n_heads:
            aux["attn_out"] = torch.empty((L, T, w.H), dtype=self.store_dtype, device=self.device)
        return aux

    def step(self, hidden, drafts, B: int, K: int, committed, counts, aux: dict | None = None, stream=None,
             copy: int = 0):
        ctx = self.ctxs[copy]
        if aux is None:
            B_.moe_verify_step(ctx, hidden, drafts if K > 0 else None, B, K, committed, counts, stream)
        else:
            B_.moe_verify_step_ex(ctx, hidden, drafts if K > 0 else None, B, K, committed, counts,
                                  B_.make_aux(**aux), stream)

    def block_forward(self, layer: int, x, T: int, y, aux: dict | None = None, stream=None, copy: int = 0):
        B_.moe_block_forward(self.ctxs[copy], layer, x, T, y, B_.make_aux(**aux) if aux else None, stream)

    def close(self):
        for c in getattr(self, "ctxs", []):
            B_.moe_verify_destroy(c)
        self.ctxs = []
        self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DraftModel:
    """A draft-head context bound to a VerifyModel's context (sharing its LM
    head when the draft head has no rows of its own)."""

    def __init__(self, verifier: VerifyModel, Id: int, dweights: dict, max_batch: int, k_max: int = 7,
                 device="cuda", stream=None, copy: int = 0):
        torch = _torch()
        self.verifier = verifier
        self.device = device
        self.H = verifier.w.H
        names = ("embed", "gamma_h", "gamma_e", "w_proj", "gamma_f", "w_gate", "w_up", "w_down", "gamma_o")
        t = {k: to_device(dweights[k], device) for k in names}
        own_head = "head_ids" in dweights
        head = to_device(dweights["head"], device) if own_head else None
        ids = to_device(np.asarray(dweights["head_ids"], np.int32), device) if own_head else None
        cfg = B_.MoeDraftConfig(inter=Id, head_rows=len(dweights["head_ids"]) if own_head else 0,
                                max_batch=max_batch, k_max=k_max)
        wts = B_.MoeDraftWeights(**{k: t[k].data_ptr() for k in names},
                                 head=head.data_ptr() if own_head else None,
                                 head_ids=ids.data_ptr() if own_head else None)
        torch.cuda.synchronize()
        self.ctx = B_.moe_draft_init(verifier.ctxs[copy], cfg, wts, stream)
        del t, head, ids
        torch.cuda.synchronize()

    def step(self, hidden, committed, counts, R: int, B: int, K: int, drafts, states=None, stream=None):
        B_.moe_draft_step(self.ctx, hidden, committed, counts, R, B, K, drafts, states, stream)

    def close(self):
        if getattr(self, "ctx", None):
            B_.moe_draft_destroy(self.ctx)
        self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
