"""torch-facing wrappers of the libhm C ABI (argument marshalling only).

Every function takes contiguous CUDA (HIP) tensors on one device, passes
their device pointers and the current stream to the library, and raises
HmError with the library's message on any non-zero status.  The library sees
plain pointers and cannot know a buffer's size, so every tensor is checked
here against the element count and dtype the call implies (ValueError before
any launch; a view of another shape over the same elements is accepted).  Workspaces are allocated here with torch (the library
itself never allocates).
"""
from __future__ import annotations

import ctypes

import torch

from . import (HM_ACT_NONE, HM_ACT_SILU, HM_ACT_SOFTPLUS, HM_BF16, HM_F32, BlockArgs, HmError,
               LinearEpilogue, PrefillArgs, StepArgs, lib)

__all__ = [
    "swa_meta_attn", "attn_kv_bytes", "attn_kv_prepare", "attn_with_kv", "causal_conv1d", "selective_scan", "conv_selective_scan",
    "branch_norm_mean", "linear", "rms_norm", "BlockPlan", "mixer_prefill", "PrefillPlan", "mixer_step", "StepPlan",
    "debug_attn_mask", "debug_tile_plan", "debug_attn_tiles", "debug_cache_slot",
    "debug_step_positions", "dtype_code",
]


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HM_BF16
    if t.dtype == torch.float32:
        return HM_F32
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int):
    if status != 0:
        raise HmError(status, lib.hm_last_error().decode())


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libhm takes device tensors")
        if not t.is_contiguous():
            raise ValueError("libhm takes contiguous tensors")
        if dev is not None and t.device != dev:
            raise ValueError("libhm takes tensors on one device")
        dev = t.device
    return dev


def _expect(name, t, shape, dtype=None):
    """Raise unless t (when given) holds as many elements as `shape` (any view
    of the same contiguous buffer will do) and has this dtype."""
    if t is None:
        return
    n = 1
    for d in shape:
        n *= int(d)
    if t.numel() != n or (dtype is not None and t.dtype != dtype):
        want = str(tuple(shape)) + ("" if dtype is None else f" {dtype}")
        raise ValueError(f"{name}: expected {want}, got {tuple(t.shape)} {t.dtype}")


def _rank(name, t, n):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got {tuple(t.shape)}")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _f32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise TypeError("parameters and states must be float32")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ attention
def swa_meta_attn(q, k, v, n_meta: int, window: int, rope_base: float = 10000.0,
                  pos0: int = 0, scale: float = 0.0, out=None, workspace=None):
    """O = attention over X~ (meta prefix + causal sliding window), GQA, RoPE."""
    dev = _dev(q, k, v, out, workspace)
    _rank("q", q, 4)
    _rank("k", k, 4)
    B, T, Hq, Dh = q.shape
    Hkv = k.shape[2]
    _expect("k", k, (B, T, Hkv, Dh), q.dtype)
    _expect("v", v, (B, T, Hkv, Dh), q.dtype)
    _expect("out", out, q.shape, q.dtype)
    dt = dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    nb = lib.hm_swa_meta_attn_workspace(B, T, Hkv, Dh, dt)
    ws = workspace if workspace is not None else _ws(nb, dev)
    _check(lib.hm_swa_meta_attn(_p(q), _p(k), _p(v), _p(out), B, T, Hq, Hkv, Dh, n_meta, window,
                                rope_base, pos0, scale, dt, _p(ws), _nbytes(ws), _stream()))
    return out


def attn_kv_bytes(B: int, T: int, Hkv: int, Dh: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (HM_BF16 if dtype == torch.bfloat16 else HM_F32)
    return lib.hm_attn_kv_bytes(B, T, Hkv, Dh, code)


def attn_kv_prepare(k, v, rope_base: float = 10000.0, pos0: int = 0, kv=None):
    """Rotate k and lay out k, v for the attention kernel; returns the kv buffer."""
    dev = _dev(k, v, kv)
    _rank("k", k, 4)
    _expect("v", v, k.shape, k.dtype)
    B, T, Hkv, Dh = k.shape
    dt = dtype_code(k)
    nb = lib.hm_attn_kv_bytes(B, T, Hkv, Dh, dt)
    if kv is None:
        kv = _ws(nb, dev)
    _check(lib.hm_attn_kv_prepare(_p(k), _p(v), _p(kv), _nbytes(kv), B, T,
                                  Hkv, Dh, rope_base, pos0, dt, _stream()))
    return kv


def attn_with_kv(q, kv, Hkv: int, n_meta: int, window: int, rope_base: float = 10000.0,
                 pos0: int = 0, scale: float = 0.0, out=None):
    """Attention of q over a buffer filled by attn_kv_prepare (same rope_base, pos0)."""
    _dev(q, kv, out)
    _rank("q", q, 4)
    B, T, Hq, Dh = q.shape
    _expect("out", out, q.shape, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    _check(lib.hm_attn_with_kv(_p(q), _p(kv), _nbytes(kv), _p(out), B, T, Hq,
                               Hkv, Dh, n_meta, window, rope_base, pos0, scale, dtype_code(q),
                               _stream()))
    return out


# ------------------------------------------------------------------ SSM branch
def causal_conv1d(x, w, bias=None, state_in=None, apply_silu=True, state_out=None, out=None):
    dev = _dev(x, w, bias, state_in, state_out, out)
    _f32(w, bias, state_in, state_out)
    _rank("x", x, 3)
    _rank("w", w, 2)
    B, T, Di = x.shape
    K = w.shape[1]
    _expect("w", w, (Di, K))
    _expect("bias", bias, (Di,))
    _expect("state_in", state_in, (B, Di, K - 1))
    _expect("state_out", state_out, (B, Di, K - 1))
    _expect("out", out, x.shape, x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _check(lib.hm_causal_conv1d(_p(x), _p(w), _p(bias), _p(state_in), _p(out), _p(state_out), B, T,
                                Di, K, int(bool(apply_silu)), dtype_code(x), _stream()))
    return out


def _scan_shapes(x, delta, A, Bm, Cm, D, z, h0, h_out, out):
    B, T, Di = x.shape
    N = A.shape[1]
    _expect("A", A, (Di, N))
    for name, t in (("delta", delta), ("z", z), ("out", out)):
        _expect(name, t, x.shape, x.dtype)
    _expect("Bm", Bm, (B, T, N), x.dtype)
    _expect("Cm", Cm, (B, T, N), x.dtype)
    _expect("D", D, (Di,))
    _expect("h0", h0, (B, Di, N))
    _expect("h_out", h_out, (B, Di, N))


def selective_scan(x, delta, A, Bm, Cm, D=None, z=None, h0=None, h_out=None, out=None,
                   workspace=None):
    dev = _dev(x, delta, A, Bm, Cm, D, z, h0, h_out, out, workspace)
    _f32(A, D, h0, h_out)
    _rank("x", x, 3)
    _rank("A", A, 2)
    B, T, Di = x.shape
    N = A.shape[1]
    _scan_shapes(x, delta, A, Bm, Cm, D, z, h0, h_out, out)
    if out is None:
        out = torch.empty_like(x)
    nb = lib.hm_selective_scan_workspace(B, T, Di, N)
    ws = workspace if workspace is not None else _ws(nb, dev)
    _check(lib.hm_selective_scan(_p(x), _p(delta), _p(A), _p(Bm), _p(Cm), _p(D), _p(z), _p(h0),
                                 _p(out), _p(h_out), B, T, Di, N, dtype_code(x), _p(ws),
                                 _nbytes(ws), _stream()))
    return out


def conv_selective_scan(x, conv_w, conv_b, delta, A, Bm, Cm, D=None, z=None, conv_state_in=None,
                        conv_state_out=None, h0=None, h_out=None, out=None, workspace=None):
    dev = _dev(x, conv_w, conv_b, delta, A, Bm, Cm, D, z, conv_state_in, conv_state_out, h0,
               h_out, out, workspace)
    _f32(conv_w, conv_b, A, D, conv_state_in, conv_state_out, h0, h_out)
    _rank("x", x, 3)
    _rank("A", A, 2)
    _rank("conv_w", conv_w, 2)
    B, T, Di = x.shape
    N, K = A.shape[1], conv_w.shape[1]
    _scan_shapes(x, delta, A, Bm, Cm, D, z, h0, h_out, out)
    _expect("conv_w", conv_w, (Di, K))
    _expect("conv_b", conv_b, (Di,))
    _expect("conv_state_in", conv_state_in, (B, Di, K - 1))
    _expect("conv_state_out", conv_state_out, (B, Di, K - 1))
    if out is None:
        out = torch.empty_like(x)
    nb = lib.hm_selective_scan_workspace(B, T, Di, N)
    ws = workspace if workspace is not None else _ws(nb, dev)
    _check(lib.hm_conv_selective_scan(_p(x), _p(conv_w), _p(conv_b), _p(conv_state_in),
                                      _p(conv_state_out), _p(delta), _p(A), _p(Bm), _p(Cm), _p(D),
                                      _p(z), _p(h0), _p(out), _p(h_out), B, T, Di, K, N,
                                      dtype_code(x), _p(ws), _nbytes(ws), _stream()))
    return out


# ------------------------------------------------------------------ fusion
def branch_norm_mean(ya, ys, beta_a, beta_s, eps: float = 1e-6, out=None):
    _dev(ya, ys, beta_a, beta_s, out)
    _f32(beta_a, beta_s)
    width = ya.shape[-1]
    rows = ya.numel() // width
    _expect("ys", ys, ya.shape, ya.dtype)
    _expect("beta_a", beta_a, (width,))
    _expect("beta_s", beta_s, (width,))
    _expect("out", out, ya.shape, ya.dtype)
    if out is None:
        out = torch.empty_like(ya)
    _check(lib.hm_branch_norm_mean(_p(ya), _p(ys), _p(beta_a), _p(beta_s), eps, _p(out), rows,
                                   width, dtype_code(ya), _stream()))
    return out


# ------------------------------------------------------------------ projections
_ACTS = {None: HM_ACT_NONE, "silu": HM_ACT_SILU, "softplus": HM_ACT_SOFTPLUS}


def linear(x, w, seg_cols=None, outs=None, epilogues=None):
    """y = x w^T (bf16; w in nn.Linear layout [N, K]) over the last dim of x.
    seg_cols splits the N output columns into tensors of those widths (a list
    is returned); default: one tensor [..., N].  epilogues: one dict per
    segment with optional "bias" (f32 [width]), "act" (None, "silu",
    "softplus") and "residual" (bf16 [..., width]; may be the output itself):
    y = act(x w^T + bias) + residual."""
    _dev(x, w)
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("linear takes bf16 x and w")
    _rank("w", w, 2)
    K = x.shape[-1]
    M = x.numel() // K
    N = w.shape[0]
    _expect("w", w, (N, K))
    cols = [N] if seg_cols is None else list(seg_cols)
    if sum(cols) != N:
        raise ValueError(f"seg_cols must add up to the {N} rows of w")
    if outs is None:
        outs = [torch.empty(x.shape[:-1] + (c,), dtype=x.dtype, device=x.device) for c in cols]
    if len(outs) != len(cols):
        raise ValueError("one output tensor per segment")
    _dev(x, *outs)
    for i, (o, c) in enumerate(zip(outs, cols)):
        _expect(f"outs[{i}]", o, x.shape[:-1] + (c,), torch.bfloat16)
    ptrs = (ctypes.c_void_p * len(cols))(*[o.data_ptr() for o in outs])
    widths = (ctypes.c_int * len(cols))(*cols)
    if epilogues is None:
        _check(lib.hm_linear_bf16(_p(x), _p(w), M, N, K, len(cols), ptrs, widths, _stream()))
    else:
        if len(epilogues) != len(cols):
            raise ValueError("one epilogue per segment")
        eps = (LinearEpilogue * len(cols))()
        for i, (e, d, c) in enumerate(zip(eps, epilogues, cols)):
            d = d or {}
            bias, res = d.get("bias"), d.get("residual")
            _dev(x, bias, res)
            _f32(bias)
            _expect(f"epilogues[{i}].bias", bias, (c,))
            _expect(f"epilogues[{i}].residual", res, x.shape[:-1] + (c,), torch.bfloat16)
            if d.get("act") not in _ACTS:
                raise ValueError(f"unknown activation {d.get('act')!r}")
            e.bias = None if bias is None else bias.data_ptr()
            e.residual = None if res is None else res.data_ptr()
            e.act = _ACTS[d.get("act")]
        _check(lib.hm_linear_bf16_ex(_p(x), _p(w), M, N, K, len(cols), ptrs, widths, eps,
                                     _stream()))
    return outs if seg_cols is not None else outs[0]


def rms_norm(x, w, eps: float = 1e-6, out=None):
    """x / sqrt(mean(x^2) + eps) * w over the last dim (w float32)."""
    _dev(x, w, out)
    _f32(w)
    width = x.shape[-1]
    _expect("w", w, (width,))
    _expect("out", out, x.shape, x.dtype)
    out = torch.empty_like(x) if out is None else out
    _check(lib.hm_rms_norm(_p(x), _p(w), eps, _p(out), x.numel() // width, width, dtype_code(x),
                           _stream()))
    return out


class BlockPlan:
    """One whole Hymba block (norm, in-projection, mixer, out-projection, norm,
    FFN) over ``hidden`` [B, T, d_model] (bf16, updated in place by ``run()``).

    ``w`` maps ln1, ln2, w_in, w_dbc, dt_bias, A, D, conv_w, conv_b, beta_a,
    beta_s, w_out, w_up, w_down to device tensors (matrices bf16 in nn.Linear
    layout, vectors float32).  kv: prepared K/V buffer (allocated when None);
    kv_reuse: attend over kv as an earlier block prepared it (w_in then has
    rows Q, x, z only).  ``run()`` allocates nothing."""

    def __init__(self, w: dict, hidden, Hq: int, Hkv: int, n_meta: int, window: int,
                 rope_base: float = 10000.0, eps: float = 1e-6, pos0: int = 0, scale: float = 0.0,
                 kv=None, kv_reuse=False, workspace=None):
        keys = ("ln1", "ln2", "w_in", "w_dbc", "dt_bias", "A", "D", "conv_w", "conv_b",
                "beta_a", "beta_s", "w_out", "w_up", "w_down")
        dev = _dev(hidden, *[w[k] for k in keys])
        _f32(*[w[k] for k in ("ln1", "ln2", "dt_bias", "A", "D", "conv_w", "conv_b", "beta_a",
                              "beta_s")])
        _rank("hidden", hidden, 3)
        for k in ("A", "conv_w", "w_up"):
            _rank(k, w[k], 2)
        B, T, d_model = hidden.shape
        Di, N = w["A"].shape
        Dh = Di // Hq
        d_ffn, K = w["w_up"].shape[0], w["conv_w"].shape[1]
        act = hidden.dtype
        n_in = Hq * Dh + (0 if kv_reuse else 2 * Hkv * Dh) + 2 * Di
        for k, shape, dt in (("ln1", (d_model,), None), ("ln2", (d_model,), None),
                             ("w_in", (n_in, d_model), act), ("w_dbc", (Di + 2 * N, Di), act),
                             ("dt_bias", (Di,), None), ("D", (Di,), None),
                             ("conv_w", (Di, K), None), ("conv_b", (Di,), None),
                             ("beta_a", (Di,), None), ("beta_s", (Di,), None),
                             ("w_out", (d_model, Di), act), ("w_up", (d_ffn, d_model), act),
                             ("w_down", (d_model, d_ffn), act)):
            _expect(k, w[k], shape, dt)
        a = BlockArgs()
        a.B, a.T, a.d_model, a.d_ffn = B, T, d_model, d_ffn
        a.Hq, a.Hkv, a.Dh, a.Di, a.N, a.K = Hq, Hkv, Dh, Di, N, K
        a.n_meta, a.window, a.pos0 = n_meta, window, pos0
        a.rope_base, a.scale, a.eps, a.dtype = rope_base, scale, eps, dtype_code(hidden)
        a.hidden = hidden.data_ptr()
        for k in keys:
            setattr(a, k, w[k].data_ptr())
        if kv is None:
            if kv_reuse:
                raise ValueError("kv_reuse needs the producer's kv buffer")
            kv = _ws(lib.hm_attn_kv_bytes(B, T, Hkv, Dh, dtype_code(hidden)), dev)
        self.kv = kv
        a.kv, a.kv_bytes, a.kv_reuse = kv.data_ptr(), _nbytes(kv), int(kv_reuse)
        nb = lib.hm_block_prefill_workspace(ctypes.byref(a))
        self.ws = workspace if workspace is not None else _ws(nb, dev)
        _dev(hidden, kv, self.ws)
        a.workspace, a.workspace_bytes = self.ws.data_ptr(), _nbytes(self.ws)
        self.args, self.w, self.hidden = a, w, hidden

    def run(self, stream=None):
        s = _stream() if stream is None else ctypes.c_void_p(stream.cuda_stream)
        _check(lib.hm_block_prefill(ctypes.byref(self.args), s))
        return self.hidden


# ------------------------------------------------------------------ whole layer
class PrefillPlan:
    """One prefill mixer layer with its outputs and workspace allocated once.

    ``t`` maps the input names (q, k, v, x, delta, Bm, Cm, z, A, D, conv_w,
    conv_b, beta_a, beta_s) to device tensors.  ``run()`` launches the layer on
    the current stream and allocates nothing.
    """

    def __init__(self, t: dict, n_meta: int, window: int, rope_base: float = 10000.0,
                 eps: float = 1e-6, pos0: int = 0, scale: float = 0.0, want_states=True,
                 out=None, ya=None, ys=None, workspace=None, kv=None, kv_reuse=False,
                 stream2=None, meta=None, conv_state_in=None, h0=None):
        """kv: prepared K/V buffer (allocated here when None).  kv_reuse: read
        kv as prepared by an earlier layer (t["k"], t["v"] are then unused).
        stream2: a torch stream on which the SSM branch runs concurrently.
        meta: cached meta tokens, {"k": [n_meta, Hkv, Dh], "v": ...}; t then
        holds the real-token rows only.  conv_state_in [B, Di, K-1], h0
        [B, Di, N]: SSM-branch states entering the rows (float32)."""
        q = t["q"]
        dev = _dev(*[t[k] for k in ("q", "x", "delta", "Bm", "Cm", "z", "A", "D",
                                     "conv_w", "conv_b", "beta_a", "beta_s")])
        if not kv_reuse:
            _dev(t["k"], t["v"])
        _f32(t["A"], t["D"], t["conv_w"], t["conv_b"], t["beta_a"], t["beta_s"])
        _rank("q", q, 4)
        for k in ("x", "A", "conv_w"):
            _rank(k, t[k], {"x": 3}.get(k, 2))
        B, T, Hq, Dh = q.shape
        Di = t["x"].shape[2]
        N, K = t["A"].shape[1], t["conv_w"].shape[1]
        Hkv = t["Hkv"] if "Hkv" in t else t["k"].shape[2]
        _expect("x", t["x"], (B, T, Di), q.dtype)
        _scan_shapes(t["x"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D"], t["z"], h0, None, None)
        if not kv_reuse:
            _expect("k", t["k"], (B, T, Hkv, Dh), q.dtype)
            _expect("v", t["v"], (B, T, Hkv, Dh), q.dtype)
        for k in ("conv_b", "beta_a", "beta_s"):
            _expect(k, t[k], (Di,))
        _expect("conv_w", t["conv_w"], (Di, K))
        for name, o in (("out", out), ("ya", ya), ("ys", ys)):
            _expect(name, o, (B, T, Di), q.dtype)
        if meta is not None:
            _expect("meta k", meta["k"], (n_meta, Hkv, Dh), q.dtype)
            _expect("meta v", meta["v"], (n_meta, Hkv, Dh), q.dtype)
        _expect("conv_state_in", conv_state_in, (B, Di, K - 1))
        _dev(q, out, ya, ys, kv, workspace)
        self.t = t
        self.ya = ya if ya is not None else torch.empty((B, T, Di), dtype=q.dtype, device=dev)
        self.ys = ys if ys is not None else torch.empty((B, T, Di), dtype=q.dtype, device=dev)
        self.out = out if out is not None else torch.empty((B, T, Di), dtype=q.dtype, device=dev)
        self.conv_state = self.h = None
        if want_states:
            self.conv_state = torch.empty((B, Di, t["conv_w"].shape[1] - 1), dtype=torch.float32,
                                          device=dev)
            self.h = torch.empty((B, Di, t["A"].shape[1]), dtype=torch.float32, device=dev)
        a = PrefillArgs()
        a.B, a.T, a.Hq, a.Hkv, a.Dh, a.Di = B, T, Hq, Hkv, Dh, Di
        a.N, a.K, a.n_meta, a.window = N, K, n_meta, window
        a.pos0, a.rope_base, a.scale, a.eps, a.dtype = pos0, rope_base, scale, eps, dtype_code(q)
        for k in ("q", "x", "delta", "Bm", "Cm", "z", "A", "D", "conv_w", "conv_b",
                  "beta_a", "beta_s"):
            setattr(a, k, t[k].data_ptr())
        if not kv_reuse:
            a.k, a.v = t["k"].data_ptr(), t["v"].data_ptr()
        if meta is not None:
            _dev(meta["k"], meta["v"])
            a.meta_k, a.meta_v = meta["k"].data_ptr(), meta["v"].data_ptr()
        _dev(conv_state_in, h0)
        if conv_state_in is not None:
            _f32(conv_state_in)
            a.conv_state_in = conv_state_in.data_ptr()
        if h0 is not None:
            _f32(h0)
            a.h0 = h0.data_ptr()
        self._keep = (meta, conv_state_in, h0)
        key_rows = T + (n_meta if meta is not None else 0)
        if kv is None:
            kv = _ws(lib.hm_attn_kv_bytes(B, key_rows, Hkv, Dh, dtype_code(q)), dev)
        self.kv = kv
        a.kv, a.kv_bytes, a.kv_reuse = kv.data_ptr(), _nbytes(kv), int(kv_reuse)
        self.stream2 = stream2
        a.stream2 = stream2.cuda_stream if stream2 is not None else None
        a.ya, a.ys, a.out = self.ya.data_ptr(), self.ys.data_ptr(), self.out.data_ptr()
        a.conv_state_out = self.conv_state.data_ptr() if want_states else None
        a.h_out = self.h.data_ptr() if want_states else None
        nb = lib.hm_mixer_prefill_workspace(ctypes.byref(a))
        self.ws = workspace if workspace is not None else _ws(nb, dev)
        a.workspace, a.workspace_bytes = self.ws.data_ptr(), _nbytes(self.ws)
        self.args = a

    def run(self, stream=None, events=None):
        """events: optional 4 torch.cuda.Event or None (timing enabled, already
        created by one record()) that the library records around its three
        launches (None entries are skipped)."""
        s = _stream() if stream is None else ctypes.c_void_p(stream.cuda_stream)
        if events is None:
            _check(lib.hm_mixer_prefill(ctypes.byref(self.args), s))
            return self.out
        if len(events) != 4:
            raise ValueError("events: four torch.cuda.Event")
        arr = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
        self.args.events = ctypes.cast(arr, ctypes.c_void_p)
        try:
            _check(lib.hm_mixer_prefill(ctypes.byref(self.args), s))
        finally:
            self.args.events = None
        return self.out


def mixer_prefill(t: dict, n_meta: int, window: int, **kw):
    plan = PrefillPlan(t, n_meta, window, **kw)
    plan.run()
    return {"ya": plan.ya, "ys": plan.ys, "out": plan.out, "conv_state": plan.conv_state,
            "ssm_state": plan.h}


class StepPlan:
    """One decode token through one layer of a KV-sharing pair (see hm_mixer_step).

    ``layer`` maps q, [k_new, v_new], x, delta, Bm, Cm, z, conv_state, ssm_state,
    A, D, conv_w, conv_b, beta_a, beta_s to device tensors; conv_state and
    ssm_state advance in place; the producer writes into k_cache / v_cache.
    """

    def __init__(self, layer: dict, k_cache, v_cache, n_prev: int, n_meta: int, window: int,
                 rope_base: float = 10000.0, eps: float = 1e-6, scale: float = 0.0,
                 want_branches=False, out=None, workspace=None, n_prev_seq=None):
        """n_prev_seq: optional int32 device tensor [B], one n_prev per sequence
        (ragged batch); n_prev must then be at least its largest entry."""
        q = layer["q"]
        producer = layer.get("k_new") is not None
        dev = _dev(q, k_cache, v_cache, layer.get("k_new"), layer.get("v_new"),
                   *[layer[k] for k in ("x", "delta", "Bm", "Cm", "z", "conv_state", "ssm_state",
                                        "A", "D", "conv_w", "conv_b", "beta_a", "beta_s")])
        _f32(layer["conv_state"], layer["ssm_state"], layer["A"], layer["D"], layer["conv_w"],
             layer["conv_b"], layer["beta_a"], layer["beta_s"])
        _rank("q", q, 3)
        _rank("k_cache", k_cache, 4)
        for k in ("x", "A", "conv_w"):
            _rank(k, layer[k], 2)
        B, Hq, Dh = q.shape
        S, Hkv = k_cache.shape[1], k_cache.shape[2]
        Di = layer["x"].shape[1]
        N, K = layer["A"].shape[1], layer["conv_w"].shape[1]
        act = q.dtype
        for k, shape, dt in (("k_cache", (B, S, Hkv, Dh), act), ("x", (B, Di), act),
                             ("delta", (B, Di), act), ("z", (B, Di), act), ("Bm", (B, N), act),
                             ("Cm", (B, N), act), ("A", (Di, N), None), ("D", (Di,), None),
                             ("conv_w", (Di, K), None), ("conv_b", (Di,), None),
                             ("conv_state", (B, Di, K - 1), None),
                             ("ssm_state", (B, Di, N), None), ("beta_a", (Di,), None),
                             ("beta_s", (Di,), None)):
            _expect(k, k_cache if k == "k_cache" else layer[k], shape, dt)
        _expect("v_cache", v_cache, k_cache.shape, act)
        if producer:
            _expect("k_new", layer["k_new"], (B, Hkv, Dh), act)
            _expect("v_new", layer.get("v_new"), (B, Hkv, Dh), act)
        _expect("out", out, (B, Di), act)
        _dev(q, out, workspace)
        a = StepArgs()
        a.B, a.Hq, a.Hkv, a.Dh, a.Di = B, Hq, Hkv, Dh, Di
        a.N, a.K, a.n_meta, a.window = N, K, n_meta, window
        a.cache_slots = S - n_meta
        a.n_prev, a.rope_base, a.scale, a.eps, a.dtype = n_prev, rope_base, scale, eps, dtype_code(q)
        a.q = q.data_ptr()
        a.k_new = layer["k_new"].data_ptr() if producer else None
        a.v_new = layer["v_new"].data_ptr() if producer else None
        a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
        for k in ("x", "delta", "Bm", "Cm", "z", "A", "D", "conv_w", "conv_b", "conv_state",
                  "ssm_state", "beta_a", "beta_s"):
            setattr(a, k, layer[k].data_ptr())
        self.out = out if out is not None else torch.empty((B, Di), dtype=q.dtype, device=dev)
        a.out = self.out.data_ptr()
        self.ya = self.ys = None
        if want_branches:
            self.ya = torch.empty((B, Di), dtype=torch.float32, device=dev)
            self.ys = torch.empty((B, Di), dtype=torch.float32, device=dev)
            a.ya_out, a.ys_out = self.ya.data_ptr(), self.ys.data_ptr()
        if n_prev_seq is not None:
            _dev(n_prev_seq)
            if n_prev_seq.dtype != torch.int32 or n_prev_seq.numel() != B:
                raise TypeError("n_prev_seq must be an int32 tensor with one entry per sequence")
            a.n_prev_seq = n_prev_seq.data_ptr()
        nb = lib.hm_mixer_step_workspace(ctypes.byref(a))
        self.ws = workspace if workspace is not None else _ws(nb, dev)
        a.workspace, a.workspace_bytes = self.ws.data_ptr(), _nbytes(self.ws)
        self.args = a
        self._keep = (layer, k_cache, v_cache, n_prev_seq)

    def run(self, stream=None):
        s = _stream() if stream is None else ctypes.c_void_p(stream.cuda_stream)
        _check(lib.hm_mixer_step(ctypes.byref(self.args), s))
        return self.out


def mixer_step(layer: dict, k_cache, v_cache, n_prev: int, n_meta: int, window: int, **kw):
    plan = StepPlan(layer, k_cache, v_cache, n_prev, n_meta, window, **kw)
    plan.run()
    return plan


# ------------------------------------------------------------------ index exports
def debug_attn_mask(T: int, n_meta: int, window: int, device="cuda"):
    out = torch.empty((T, T), dtype=torch.uint8, device=device)
    _check(lib.hm_debug_attn_mask(T, n_meta, window, _p(out), _stream()))
    return out


def debug_tile_plan(T: int, n_meta: int, window: int, bm: int, bn: int, device="cuda"):
    nq, nk = -(-T // bm), -(-T // bn)
    out = torch.empty((nq, nk), dtype=torch.int32, device=device)
    _check(lib.hm_debug_tile_plan(T, n_meta, window, bm, bn, _p(out), out.numel(), _stream()))
    return out


def debug_attn_tiles():
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.hm_debug_attn_tiles(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def debug_cache_slot(n_prev: int, n_meta: int, window: int) -> int:
    return lib.hm_debug_cache_slot(n_prev, n_meta, window)


def debug_step_positions(B: int, n_prev: int, n_meta: int, window: int, n_prev_seq=None,
                         device="cuda"):
    """[B, 3] int64 (slot, visible rows, position) per sequence, from the decode
    kernels' own device function."""
    _dev(n_prev_seq)
    if n_prev_seq is not None and (n_prev_seq.dtype != torch.int32 or n_prev_seq.numel() != B):
        raise TypeError("n_prev_seq must be an int32 tensor with one entry per sequence")
    out = torch.empty((B, 3), dtype=torch.int64, device=device)
    _check(lib.hm_debug_step_positions(B, n_prev, _p(n_prev_seq), n_meta, window, _p(out),
                                       _stream()))
    return out
