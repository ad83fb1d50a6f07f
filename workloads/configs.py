"""Workload shapes for the hybrid-head mixer core.

The Hymba-1.5B layer shape (width 1600, 25 attention heads, GQA, RoPE, 16 SSM
states, 32 layers with full attention in the first, middle and last layer and
sliding-window attention elsewhere) is taken from the Hymba-1.5B-Base model card
("Model architecture") and the juejin.cn Hymba blog ("Hymba 的整体架构").
The remaining sizes (128 meta tokens, 5 KV heads, window 1024, conv width 4,
batch and sequence lengths) are the five synthetic workloads this library is
measured and checked on; none of them is printed on those pages.

This module holds shapes only: no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class MixerShape:
    name: str
    B: int            # batch
    M: int            # meta tokens prepended to every sequence
    N: int            # real tokens
    Hq: int           # query heads
    Hkv: int          # key/value heads (GQA groups)
    Dh: int           # head dim
    W: int            # sliding window (<= 0: global causal attention)
    Di: int           # SSM inner width (== Hq * Dh)
    Ns: int = 16      # SSM states per channel
    K: int = 4        # causal conv width
    dtype: str = "bf16"   # activation dtype: "f32" or "bf16"
    rope_base: float = 10000.0
    eps: float = 1e-6
    # decode-only
    n_prev: int = 0       # tokens already in the sequence (after the meta prefix)
    cache_slots: int = 0  # ring slots after the meta prefix
    # stack-only
    layers: int = 1
    global_layers: Tuple[int, ...] = field(default_factory=tuple)
    # whole blocks only: model width (the in-projection's input) and FFN width
    d_model: int = 0
    d_ffn: int = 0

    @property
    def T(self) -> int:
        return self.M + self.N


TINY = MixerShape("tiny-f32", B=1, M=4, N=60, Hq=2, Hkv=1, Dh=16, W=16, Di=32,
                  dtype="f32")
SWA_PREFILL = MixerShape("swa-prefill-b1-t2176", B=1, M=128, N=2048, Hq=25, Hkv=5,
                         Dh=64, W=1024, Di=1600)
GLOBAL_PREFILL = MixerShape("global-prefill-b4-t8320", B=4, M=128, N=8192, Hq=25,
                            Hkv=5, Dh=64, W=0, Di=1600)
DECODE_PAIR = MixerShape("decode-pair-b64-cache1152", B=64, M=128, N=1, Hq=25, Hkv=5,
                         Dh=64, W=1024, Di=1600, n_prev=2048, cache_slots=1024)
STACK = MixerShape("stack32-b2-t16512", B=2, M=128, N=16384, Hq=25, Hkv=5, Dh=64,
                   W=1024, Di=1600, layers=32, global_layers=(0, 15, 31))

# Whole blocks (norm, mixer, norm, FFN) at the model card's widths 1600 / 5504.
BLOCK_SWA = replace(SWA_PREFILL, name="block-swa-prefill-b1-t2176", d_model=1600, d_ffn=5504)
BLOCK_STACK = replace(STACK, name="block-stack32-b2-t16512", d_model=1600, d_ffn=5504)

ALL = (TINY, SWA_PREFILL, GLOBAL_PREFILL, DECODE_PAIR, STACK)


def stack_layer_roles(shape: MixerShape):
    """Per layer: (window, kv_source_layer).

    Global layers keep their own K/V with no window. Between global layers the
    sliding-window layers are paired (first of a pair produces K/V, the second
    reuses it); a leftover unpaired SWA layer keeps its own K/V. This is the
    reading of "adjacent blocks share their KV cache" (juejin.cn Hymba blog,
    "Hymba 的整体架构").
    """
    roles = []
    pending_producer = None
    for layer in range(shape.layers):
        if layer in shape.global_layers:
            roles.append((0, layer))
            pending_producer = None
            continue
        nxt_is_swa = (layer + 1 < shape.layers) and (layer + 1 not in shape.global_layers)
        if pending_producer is None:
            roles.append((shape.W, layer))
            pending_producer = layer if nxt_is_swa else None
        else:
            roles.append((shape.W, pending_producer))
            pending_producer = None
    return roles


def with_(shape: MixerShape, **kw) -> MixerShape:
    return replace(shape, **kw)
