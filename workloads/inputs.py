"""Seeded synthetic inputs for the mixer core.

Both the GPU path and the CPU oracle consume exactly these arrays, so this
module is the only code the two share. It holds the input distributions and
nothing of the method's arithmetic:

  q, k, v, x, B, C, z, D ~ N(0, 1)
  delta = softplus(N(-2, 0.5))          (already >= 0; no dt bias downstream)
  A     = -exp(N(0, 0.5))               (real, negative, per channel and state)
  conv_w ~ N(0, 1) / sqrt(K), conv_b ~ 0.1 N(0, 1)
  beta_a, beta_s ~ 1 + 0.1 N(0, 1)

The second argument of N(.,.) is a standard deviation. Draws are float64 from
numpy's PCG64 in a fixed order, then cast: activations to bfloat16 (round to
nearest even) for bf16 workloads or to float32 for f32 workloads; parameters
and recurrent states always to float32.  Arrays are returned as float32 whose
values are exactly representable in the workload dtype, plus helpers that give
the bf16 bit pattern for upload.
"""
from __future__ import annotations

import numpy as np

from .configs import MixerShape


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit pattern of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _act(a: np.ndarray, dtype: str) -> np.ndarray:
    a = a.astype(np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def _softplus(a: np.ndarray) -> np.ndarray:
    return np.log1p(np.exp(a))


def _params(rng: np.random.Generator, Di: int, Ns: int, K: int) -> dict:
    A = (-np.exp(rng.normal(0.0, 0.5, size=(Di, Ns)))).astype(np.float32)
    D = rng.standard_normal(Di).astype(np.float32)
    conv_w = (rng.standard_normal((Di, K)) / np.sqrt(K)).astype(np.float32)
    conv_b = (0.1 * rng.standard_normal(Di)).astype(np.float32)
    beta_a = (1.0 + 0.1 * rng.standard_normal(Di)).astype(np.float32)
    beta_s = (1.0 + 0.1 * rng.standard_normal(Di)).astype(np.float32)
    return dict(A=A, D=D, conv_w=conv_w, conv_b=conv_b, beta_a=beta_a, beta_s=beta_s)


def prefill_inputs(shape: MixerShape, seed=0, layer: int | None = None) -> dict:
    """One layer's prefill inputs over X~ = [meta; tokens] (length T = M + N).

    Draw order: q, k, v, x, delta, B, C, z, then the parameters A, D, conv_w,
    conv_b, beta_a, beta_s. A stack layer uses the seed sequence [seed, layer].
    """
    rng = np.random.default_rng(seed if layer is None else [seed, layer])
    B, T, dt = shape.B, shape.T, shape.dtype
    out = {}
    out["q"] = _act(rng.standard_normal((B, T, shape.Hq, shape.Dh)), dt)
    out["k"] = _act(rng.standard_normal((B, T, shape.Hkv, shape.Dh)), dt)
    out["v"] = _act(rng.standard_normal((B, T, shape.Hkv, shape.Dh)), dt)
    out["x"] = _act(rng.standard_normal((B, T, shape.Di)), dt)
    out["delta"] = _act(_softplus(rng.normal(-2.0, 0.5, size=(B, T, shape.Di))), dt)
    out["Bm"] = _act(rng.standard_normal((B, T, shape.Ns)), dt)
    out["Cm"] = _act(rng.standard_normal((B, T, shape.Ns)), dt)
    out["z"] = _act(rng.standard_normal((B, T, shape.Di)), dt)
    out.update(_params(rng, shape.Di, shape.Ns, shape.K))
    return out


_ROW_KEYS = ("q", "k", "v", "x", "delta", "Bm", "Cm", "z")
_PARAM_KEYS = ("A", "D", "conv_w", "conv_b", "beta_a", "beta_s")


def cached_meta_inputs(shape: MixerShape, seed=0):
    """Inputs for a prefill whose meta rows are cached.  The meta rows are the
    same for every sequence (batch 0's first M rows of ``prefill_inputs``).

    Returns (full, tokens, meta): ``full`` is the whole [B, M + N] input with
    those shared meta rows, ``tokens`` its last N rows (plus the parameters),
    ``meta`` the M meta rows of one sequence ([M, ...], plus the parameters).
    """
    full = prefill_inputs(shape, seed)
    M = shape.M
    for key in _ROW_KEYS:
        full[key] = np.ascontiguousarray(full[key])
        full[key][:, :M] = full[key][0:1, :M]
    tokens = {key: np.ascontiguousarray(full[key][:, M:]) for key in _ROW_KEYS}
    meta = {key: np.ascontiguousarray(full[key][0, :M]) for key in _ROW_KEYS}
    for key in _PARAM_KEYS:
        tokens[key] = full[key]
        meta[key] = full[key]
    return full, tokens, meta


def decode_inputs(shape: MixerShape, seed=0) -> dict:
    """Inputs of one decode token through an adjacent pair of layers.

    Draw order: the shared cache (K already rotated, then V), then for layer
    "a" (producer) and layer "b" (consumer) in turn: q, [k_new, v_new for the
    producer only], x, delta, B, C, z, conv_state, ssm_state, then parameters.
    The cache holds n_meta + cache_slots rows per sequence.
    """
    rng = np.random.default_rng(seed)
    B, dt = shape.B, shape.dtype
    S = shape.M + shape.cache_slots
    out = {
        "k_cache": _act(rng.standard_normal((B, S, shape.Hkv, shape.Dh)), dt),
        "v_cache": _act(rng.standard_normal((B, S, shape.Hkv, shape.Dh)), dt),
    }
    for name in ("a", "b"):
        d = {"q": _act(rng.standard_normal((B, shape.Hq, shape.Dh)), dt)}
        if name == "a":
            d["k_new"] = _act(rng.standard_normal((B, shape.Hkv, shape.Dh)), dt)
            d["v_new"] = _act(rng.standard_normal((B, shape.Hkv, shape.Dh)), dt)
        d["x"] = _act(rng.standard_normal((B, shape.Di)), dt)
        d["delta"] = _act(_softplus(rng.normal(-2.0, 0.5, size=(B, shape.Di))), dt)
        d["Bm"] = _act(rng.standard_normal((B, shape.Ns)), dt)
        d["Cm"] = _act(rng.standard_normal((B, shape.Ns)), dt)
        d["z"] = _act(rng.standard_normal((B, shape.Di)), dt)
        d["conv_state"] = rng.standard_normal((B, shape.Di, shape.K - 1)).astype(np.float32)
        d["ssm_state"] = rng.standard_normal((B, shape.Di, shape.Ns)).astype(np.float32)
        d.update(_params(rng, shape.Di, shape.Ns, shape.K))
        out[name] = d
    return out


def block_weight_rows(shape: MixerShape, producer: bool) -> int:
    """Rows of a block's in-projection: Q, [K, V,] x, z."""
    return shape.Hq * shape.Dh + (2 * shape.Hkv * shape.Dh if producer else 0) + 2 * shape.Di


def block_inputs(shape: MixerShape, seed=0, layer: int = 0, producer: bool = True) -> dict:
    """Hidden states and weights of one whole block (model width d = d_model,
    FFN width F = d_ffn).  Distributions:

      hidden ~ N(0, 1) [B, T, d]
      ln1, ln2 ~ 1 + 0.1 N(0, 1) [d]
      w_in ~ N(0, 1) / sqrt(d)    [block_weight_rows, d]
      w_dbc: the first Di rows 0.5 N(0, 1) / sqrt(Di), the last 2 Ns rows
             N(0, 1) / sqrt(Di)   [Di + 2 Ns, Di]
      dt_bias ~ -2 + 0.1 N(0, 1) [Di]
      A, D, conv_w, conv_b, beta_a, beta_s as for the mixer core
      w_out ~ N(0, 1) / sqrt(Di) [d, Di]; w_up ~ N(0, 1) / sqrt(d) [F, d];
      w_down ~ N(0, 1) / sqrt(F) [d, F]

    Draw order: hidden, ln1, w_in, w_dbc, dt_bias, the mixer parameters, w_out,
    ln2, w_up, w_down; seed sequence [seed, layer].  Matrices and hidden states
    are activations (bf16-rounded for bf16 workloads); vectors are float32.
    """
    rng = np.random.default_rng([seed, layer])
    B, T, dt = shape.B, shape.T, shape.dtype
    d, F, Di, Ns = shape.d_model, shape.d_ffn, shape.Di, shape.Ns
    out = {"hidden": _act(rng.standard_normal((B, T, d)), dt)}
    out["ln1"] = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    out["w_in"] = _act(rng.standard_normal((block_weight_rows(shape, producer), d)) / np.sqrt(d), dt)
    wd = rng.standard_normal((Di + 2 * Ns, Di)) / np.sqrt(Di)
    wd[:Di] *= 0.5
    out["w_dbc"] = _act(wd, dt)
    out["dt_bias"] = (-2.0 + 0.1 * rng.standard_normal(Di)).astype(np.float32)
    out.update(_params(rng, Di, Ns, shape.K))
    out["w_out"] = _act(rng.standard_normal((d, Di)) / np.sqrt(Di), dt)
    out["ln2"] = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    out["w_up"] = _act(rng.standard_normal((F, d)) / np.sqrt(d), dt)
    out["w_down"] = _act(rng.standard_normal((d, F)) / np.sqrt(F), dt)
    return out


def block_inputs_torch(shape: MixerShape, seed: int, layer: int, producer: bool, device,
                       hidden: bool = False) -> dict:
    """Device-side generator of one block's weights (and, with ``hidden``, its
    input hidden states) for the large stack workload: the distributions of
    ``block_inputs``, torch's Philox stream instead of PCG64."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 7919 * int(layer) + 17)
    act = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    d, F, Di, Ns, K = shape.d_model, shape.d_ffn, shape.Di, shape.Ns, shape.K

    def n(*s):
        return torch.randn(*s, generator=g, device=device, dtype=torch.float32)

    out = {}
    if hidden:
        out["hidden"] = n(shape.B, shape.T, d).to(act)
    out["ln1"] = 1.0 + 0.1 * n(d)
    out["w_in"] = (n(block_weight_rows(shape, producer), d) / float(np.sqrt(d))).to(act)
    wd = n(Di + 2 * Ns, Di) / float(np.sqrt(Di))
    wd[:Di] *= 0.5
    out["w_dbc"] = wd.to(act)
    out["dt_bias"] = -2.0 + 0.1 * n(Di)
    out["A"] = -torch.exp(n(Di, Ns) * 0.5)
    out["D"] = n(Di)
    out["conv_w"] = n(Di, K) / float(np.sqrt(K))
    out["conv_b"] = 0.1 * n(Di)
    out["beta_a"] = 1.0 + 0.1 * n(Di)
    out["beta_s"] = 1.0 + 0.1 * n(Di)
    out["w_out"] = (n(d, Di) / float(np.sqrt(Di))).to(act)
    out["ln2"] = 1.0 + 0.1 * n(d)
    out["w_up"] = (n(F, d) / float(np.sqrt(d))).to(act)
    out["w_down"] = (n(d, F) / float(np.sqrt(F))).to(act)
    return out


def prefill_inputs_torch(shape: MixerShape, seed: int, layer: int, device):
    """Device-side generator for the large stack workload (same distributions,
    torch's Philox stream instead of PCG64; activations rounded to bf16).

    Returns torch tensors on `device`. The oracle checks sampled outputs of
    these by copying them to the host, so both sides still see the same bytes.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(layer))
    B, T = shape.B, shape.T
    act = torch.bfloat16 if shape.dtype == "bf16" else torch.float32

    def n(*s):
        return torch.randn(*s, generator=g, device=device, dtype=torch.float32)

    out = {}
    out["q"] = n(B, T, shape.Hq, shape.Dh).to(act)
    out["k"] = n(B, T, shape.Hkv, shape.Dh).to(act)
    out["v"] = n(B, T, shape.Hkv, shape.Dh).to(act)
    out["x"] = n(B, T, shape.Di).to(act)
    out["delta"] = torch.nn.functional.softplus(n(B, T, shape.Di) * 0.5 - 2.0).to(act)
    out["Bm"] = n(B, T, shape.Ns).to(act)
    out["Cm"] = n(B, T, shape.Ns).to(act)
    out["z"] = n(B, T, shape.Di).to(act)
    Di, Ns, K = shape.Di, shape.Ns, shape.K
    out["A"] = -torch.exp(n(Di, Ns) * 0.5)
    out["D"] = n(Di)
    out["conv_w"] = n(Di, K) / float(np.sqrt(K))
    out["conv_b"] = 0.1 * n(Di)
    out["beta_a"] = 1.0 + 0.1 * n(Di)
    out["beta_s"] = 1.0 + 0.1 * n(Di)
    return out


ACT_KEYS = ("q", "k", "v", "x", "delta", "Bm", "Cm", "z", "k_new", "v_new", "k_cache", "v_cache",
            "hidden", "w_in", "w_dbc", "w_out", "w_up", "w_down")


def to_device(d: dict, dtype: str, device="cuda") -> dict:
    """Upload generator output: activations in the workload dtype (exact bf16
    bit patterns), parameters and states as float32.  Nested dicts recurse."""
    import torch

    out = {}
    for k, v in d.items():
        if isinstance(v, dict):
            out[k] = to_device(v, dtype, device)
        elif k in ACT_KEYS and dtype == "bf16":
            out[k] = torch.from_numpy(bf16_bits(v).view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device)
    return out
