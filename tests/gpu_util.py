"""Helpers shared by the GPU parity tests: uploads, tolerances, error metrics."""
import numpy as np
import torch

from workloads import bf16_bits

DEV = "cuda"

ACT_KEYS = ("q", "k", "v", "x", "delta", "Bm", "Cm", "z", "k_new", "v_new",
            "k_cache", "v_cache")


def up(a: np.ndarray, dtype: str):
    """Upload a float32 array whose values are exact in `dtype`."""
    if dtype == "bf16":
        t = torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16)
        return t.to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def up_inputs(d: dict, dtype: str) -> dict:
    out = {}
    for k, v in d.items():
        if isinstance(v, dict):
            out[k] = up_inputs(v, dtype)
        elif k in ACT_KEYS:
            out[k] = up(v, dtype)
        else:
            out[k] = up(v, "f32")
    return out


def down(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over one output tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


TOL = {"f32": 1e-4, "bf16": 2e-2}


def assert_close(got, ref, dtype: str, what: str = ""):
    e = rel_err(got, ref)
    assert e <= TOL[dtype], f"{what}: max-rel error {e:.3e} > {TOL[dtype]:.0e}"
    return e
