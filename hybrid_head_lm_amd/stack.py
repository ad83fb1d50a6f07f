"""A stack of prefill mixer layers with cross-layer KV sharing.

Hymba keeps full attention in the first, middle and last layer and a sliding
window elsewhere, and adjacent sliding-window layers share one KV cache
instead of keeping their own (Hymba blog, juejin.cn "NVIDIA提出Hymba网络",
"Hymba 的整体架构").  In prefill the shared object is the prepared K/V (rotated
K and laid-out V): the producer layer prepares it, the consumer layer attends
over it with its own queries and never reads its own K/V.

StackPlan chains mixer cores, each over its own already-projected inputs.
BlockStack chains whole blocks (norm, projections, mixer, norm, FFN) over one
hidden-state tensor, as the model does: a block that reuses its neighbour's
K/V has no K, V projection of its own.
"""
from __future__ import annotations

import torch

from .api import BlockPlan, PrefillPlan


class StackPlan:
    """``layers[i]`` holds layer i's device tensors (see PrefillPlan);
    ``roles[i] = (window, kv_source)``: a layer whose kv_source is an earlier
    layer reuses that layer's prepared K/V (its own k, v may be absent).
    Outputs go to shared buffers unless ``keep_outputs``."""

    def __init__(self, layers, roles, n_meta: int, rope_base: float = 10000.0,
                 eps: float = 1e-6, keep_outputs: bool = False, stream2=None):
        if len(layers) != len(roles):
            raise ValueError("one role per layer")
        q0 = layers[0]["q"]
        B, T = q0.shape[0], q0.shape[1]
        Di = layers[0]["x"].shape[2]
        shared = None
        if not keep_outputs:
            shared = [torch.empty((B, T, Di), dtype=q0.dtype, device=q0.device) for _ in range(3)]
        self.plans = []
        kvs = {}
        ws = None
        for i, ((window, src), t) in enumerate(zip(roles, layers)):
            if src > i:
                raise ValueError("a layer can only reuse the K/V of an earlier layer")
            reuse = src != i
            if reuse and src not in kvs:
                raise ValueError(f"layer {i} reuses K/V of layer {src}, which prepares none")
            if reuse and "Hkv" not in t:
                t = dict(t, Hkv=layers[src]["k"].shape[2])
            o, ya, ys = shared if shared is not None else (None, None, None)
            p = PrefillPlan(t, n_meta, window, rope_base=rope_base, eps=eps,
                            want_states=keep_outputs, out=o, ya=ya, ys=ys, workspace=ws,
                            kv=kvs[src] if reuse else None, kv_reuse=reuse, stream2=stream2)
            ws = p.ws if shared is not None else None
            if not reuse:
                kvs[i] = p.kv
            self.plans.append(p)

    def run(self, events=None):
        """events: optional per-layer lists of 4 timing events (see
        PrefillPlan.run)."""
        if events is None:
            for p in self.plans:
                p.run()
        else:
            for p, ev in zip(self.plans, events):
                p.run(events=ev)


class BlockStack:
    """Whole blocks over ``hidden`` [B, T, d_model] (bf16, updated in place).
    ``layers[i]`` holds block i's weights (see BlockPlan); ``roles[i] =
    (window, kv_source)`` as for StackPlan.  All blocks share one workspace;
    every producer block keeps its own prepared K/V buffer."""

    def __init__(self, layers, roles, hidden, Hq: int, Hkv: int, n_meta: int,
                 rope_base: float = 10000.0, eps: float = 1e-6):
        if len(layers) != len(roles):
            raise ValueError("one role per layer")
        self.hidden = hidden
        self.plans = []
        kvs = {}
        ws = None
        for i, ((window, src), w) in enumerate(zip(roles, layers)):
            if src > i:
                raise ValueError("a block can only reuse the K/V of an earlier block")
            reuse = src != i
            if reuse and src not in kvs:
                raise ValueError(f"block {i} reuses K/V of block {src}, which prepares none")
            p = BlockPlan(w, hidden, Hq, Hkv, n_meta, window, rope_base=rope_base, eps=eps,
                          kv=kvs[src] if reuse else None, kv_reuse=reuse, workspace=ws)
            ws = p.ws
            if not reuse:
                kvs[i] = p.kv
            self.plans.append(p)

    def run(self):
        for p in self.plans:
            p.run()
        return self.hidden
