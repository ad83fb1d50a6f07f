"""CPU oracle of the Hymba hybrid-head mixer core.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The GPU library never calls it, and it never calls the GPU library:
the two share no code.  The oracle is plain NumPy in float64, written from the
pages' description of the method:

* attention heads, Eq. (1), and sliding-window + meta-token visibility —
  juejin.cn blog "NVIDIA提出Hymba网络，Mamba+Attenation解决transformer的长序列
  低效难题" (below: "Hymba blog"), sections "Hymba简介", "Hymba 的整体架构" and
  "数学表示" §1–§3;
* SSM heads, Eq. (2) — Hymba blog, "数学表示" §4;
* branch normalisation and averaging — Hymba blog, "深入理解混合头模块" and
  "数学表示" §5; Telegram post "Mamba, Jamba, Ху...Hymba!" (outputs averaged);
* GQA and RoPE — Hymba-1.5B-Base model card, "模型架构" (model architecture);
* cross-layer KV sharing — Hymba blog, "Hymba 的整体架构";
* whole blocks (norm, mixer, norm, FFN) and their stack — Hymba blog,
  "Hymba 的整体架构" and "数学表示" §2, §5; model card, "模型架构".

Readings of silent or garbled points (softmax scale, window off-by-one, RoPE
variant, conv, D term, SiLU gate, RMS norm, epsilon, sum vs average) are stated
in the docstring of the function that takes them.

Every function here is pinned by CPU tests against something other than
itself (closed forms, library routines, a second formulation, brute force);
none is "parity unpinned".
"""
from .mask import visible, mask, mask_rows, visible_count, tile_kinds, cache_slot
from .rope import rope_angles, rope, rope_at
from .attention import attention
from .conv import causal_conv1d, conv_step
from .scan import selective_scan, scan_step
from .norm import rms_normalize, branch_norm_mean
from .mixer import mixer_prefill, meta_cache, mixer_prefill_cached_meta
from .step import build_cache, valid_slots, mixer_step, mixer_step_ragged
from .linear import linear, split_columns
from .block import rms_norm, silu, softplus, ffn, block_prefill, stack_prefill

__all__ = [
    "visible", "mask", "mask_rows", "visible_count", "tile_kinds", "cache_slot",
    "rope_angles", "rope", "rope_at", "attention", "causal_conv1d", "conv_step",
    "selective_scan", "scan_step", "rms_normalize", "branch_norm_mean",
    "mixer_prefill", "meta_cache", "mixer_prefill_cached_meta", "build_cache", "valid_slots", "mixer_step", "mixer_step_ragged", "linear", "split_columns",
    "rms_norm", "silu", "softplus", "ffn", "block_prefill", "stack_prefill",
]
