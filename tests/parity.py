"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (taken from the project's stated bar; the pages fix no precision):
  fp32 I/O : max |o - o_ref| <= 1e-5, max |lse - lse_ref| <= 1e-5
  bf16 I/O : max |o - o_ref| <= 2e-2 and ||o - o_ref||_2 / ||o_ref||_2 <= 5e-3 over
             the whole output of one call; max |lse - lse_ref| <= 1e-3
The oracle always runs in fp64 on exactly the (bf16-rounded) inputs the GPU saw.
"""
import numpy as np
import torch

TOL = {
    torch.float32: dict(max_abs=1e-5, rel_l2=None, lse=1e-5),
    torch.bfloat16: dict(max_abs=2e-2, rel_l2=5e-3, lse=1e-3),
}


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(o_gpu, o_ref, lse_gpu=None, lse_ref=None) -> dict:
    o = to_np(o_gpu) if isinstance(o_gpu, torch.Tensor) else np.asarray(o_gpu, np.float64)
    r = np.asarray(o_ref, np.float64)
    diff = o - r
    out = {
        "max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / max(np.linalg.norm(r), 1e-300)) if diff.size else 0.0,
        "finite": bool(np.isfinite(o).all()),
    }
    if lse_gpu is not None:
        lg = to_np(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else np.asarray(lse_gpu)
        out["lse_max_abs"] = float(np.abs(lg - np.asarray(lse_ref)).max()) if lg.size else 0.0
        out["lse_finite"] = bool(np.isfinite(lg).all())
    return out


def assert_close(dtype, o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    e = errors(o_gpu, o_ref, lse_gpu, lse_ref)
    tol = TOL[dtype]
    msg = f"{what}: {e} vs {tol}"
    print(msg, flush=True)
    assert e["finite"], msg
    assert e["max_abs"] <= tol["max_abs"], msg
    if tol["rel_l2"] is not None:
        assert e["rel_l2"] <= tol["rel_l2"], msg
    if lse_gpu is not None:
        assert e["lse_finite"], msg
        assert e["lse_max_abs"] <= tol["lse"], msg
    return e
