"""libswasink: hybrid sliding-window attention forward for MI355X (gfx950).

Thin ctypes binding over the C ABI declared in include/swasink.h.  The functions
below only marshal arguments: they check that tensors are contiguous device
tensors of the right dtype, allocate the outputs with torch on the current
stream, and call the library entry point of the same name.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is not built, or the GPU is missing, calls raise.

    swa_sink_prefill(q, k, v, sinks, cu_seqlens, max_seqlen=None, window=128, scale=None)
    ga_causal_prefill(q, k, v, cu_seqlens, max_seqlen=None, scale=None)
    swa_sink_decode(q, k_new, v_new, k_cache, v_cache, ring_head, sinks, scale=None)

Each returns (out, lse): out like q (same dtype), lse fp32 [..., num_q_heads].
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["swa_sink_prefill", "ga_causal_prefill", "swa_sink_decode", "library", "library_path",
           "abi_version", "SwaError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libswasink.so"
_lib = None

DTYPE_F32 = 0
DTYPE_BF16 = 1

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float

_SIGNATURES = {
    "swa_sink_prefill": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P],
    "ga_causal_prefill": [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P],
    "swa_sink_decode": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P],
    "swa_sink_prefill_backward": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P,
                                  _P, _P, _P, _P, _P, ctypes.c_int64, _P],
    "swa_sink_prefill_backward_noalloc": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P,
                                          _P, _P, _P, _P, _P, _P],
    "swa_sink_decode_fp8kv": [_P, _P, _P, _P, _P, _F, _F, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                              _P, _P, _P],
    "swa_sink_prefill_fp8kv": [_P, _P, _P, _F, _F, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P,
                               _P],
    "swa_rope": [_P, _P, _I, _I, _I, _F, _I, _P],
    "swa_sink_decode_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I,
                             _P, _P, _P],
    "swa_sink_decode_rope_fp8kv": [_P, _P, _P, _P, _P, _F, _F, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                                   _F, _I, _P, _P, _P],
    "swa_sink_decode_rope_commit": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                    _I, _I, _F, _F, _I, _P, _P, _P],
    "swa_sink_decode_rope_commit_fp8kv": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _F, _F, _P, _P, _P, _I,
                                          _I, _I, _I, _I, _I, _F, _F, _I, _P, _P, _P],
    "swa_ring_append_rope": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P],
    "swa_ring_append_fp8kv": [_P, _P, _P, _P, _P, _P, _F, _F, _P, _I, _I, _I, _I, _I, _F, _I, _P],
    "swa_topk_select": [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P],
    "swa_sparse_decode": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P],
    "swa_sparse_decode_mtp": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P],
    "swa_sparse_decode_fp8kv": [_P, _P, _P, _F, _F, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                                _P, _P],
}

# HySparse2 selection sizes (MiMo-V3 / HySparse2 report): top 1024 plus the recent 128.
SPARSE_TOPK = 1024
SPARSE_RECENT = 128

# Rotary bases the pages give (technical report digest, section 3.1).
ROPE_BASE_SWA = 10000.0
ROPE_BASE_GA = 640000.0
ROPE_BASE_GA_256K = 5000000.0


class SwaError(RuntimeError):
    """A libswasink entry point returned a non-zero status."""

    def __init__(self, code: int, message: str):
        super().__init__(f"libswasink error {code}: {message}")
        self.code = code


def library_path() -> str:
    """The in-tree libswasink.so, or the build named by SWASINK_LIBRARY (used to run the
    ABI checks against a host-sanitizer build of the same sources)."""
    return os.environ.get("SWASINK_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def library() -> ctypes.CDLL:
    """Load the in-tree libswasink.so (built by sliding_window_attention_amd.build)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m sliding_window_attention_amd.build`")
        lib = ctypes.CDLL(path)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.swa_last_error.argtypes = []
        lib.swa_last_error.restype = ctypes.c_char_p
        lib.swa_sink_prefill_backward_workspace.argtypes = [_I, _I]
        lib.swa_sink_prefill_backward_workspace.restype = ctypes.c_int64
        lib.swa_abi_version.argtypes = []
        lib.swa_abi_version.restype = ctypes.c_int32
        _lib = lib
    return _lib


def abi_version() -> int:
    return int(library().swa_abi_version())


def _check(rc: int) -> None:
    if rc != 0:
        msg = library().swa_last_error().decode(errors="replace")
        raise SwaError(rc, msg)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _dev(t, name, dtype=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype} (got {t.dtype})")
    return t


def _stream(device) -> ctypes.c_void_p:
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale(scale) -> float:
    return 0.0 if scale is None else float(scale)


def swa_sink_prefill(q, k, v, sinks, cu_seqlens, max_seqlen=None, window=128, scale=None,
                     return_lse=True, out=None, lse=None):
    """Causal GQA sliding-window attention with per-head sinks over packed sequences.

    q [N, Hq, D], k/v [N, Hkv, D] (fp32 or bf16, one dtype), sinks [Hq] fp32,
    cu_seqlens [S+1] int32, all on one GPU.  max_seqlen defaults to N (an upper
    bound; the kernels do not need the exact value).
    """
    import torch

    _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [N, Hq, D] and k, v [N, Hkv, D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    n, hq, d = q.shape
    if k.shape[0] != n or k.shape[2] != d or sinks.numel() != hq:
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    ms = n if max_seqlen is None else int(max_seqlen)
    rc = library().swa_sink_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), sinks.data_ptr(), cu_seqlens.data_ptr(),
        cu_seqlens.numel() - 1, n, ms, hq, k.shape[1], d, int(window), _scale(scale),
        _dtype_code(q), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_prefill_fp8kv(q, k, v, k_scale, v_scale, sinks, cu_seqlens, max_seqlen=None, window=128,
                           scale=None, return_lse=True, out=None, lse=None):
    """swa_sink_prefill with k/v [N, Hkv, D] uint8 E4M3 codes, element value = code value *
    k_scale (K) or v_scale (V) (python floats).  sinks may be None (no sink); with
    window=None the window is unbounded (the GA layer)."""
    import torch

    _dev(q, "q")
    _dev(k, "k", torch.uint8)
    _dev(v, "v", torch.uint8)
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [N, Hq, D] and k, v [N, Hkv, D]")
    n, hq, d = q.shape
    if k.shape[0] != n or k.shape[2] != d or (sinks is not None and sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    ms = n if max_seqlen is None else int(max_seqlen)
    win = 0x7FFFFFFF if window is None else int(window)
    rc = library().swa_sink_prefill_fp8kv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), float(k_scale), float(v_scale),
        sinks.data_ptr() if sinks is not None else None, cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
        n, ms, hq, k.shape[1], d, win, _scale(scale), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def ga_causal_prefill(q, k, v, cu_seqlens, max_seqlen=None, scale=None, return_lse=True, out=None,
                      lse=None):
    """Global causal GQA attention (no window, no sink) over packed sequences."""
    import torch

    _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [N, Hq, D] and k, v [N, Hkv, D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    n, hq, d = q.shape
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((n, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    ms = n if max_seqlen is None else int(max_seqlen)
    rc = library().ga_causal_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, n,
        ms, hq, k.shape[1], d, _scale(scale), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_decode(q, k_new, v_new, k_cache, v_cache, ring_head, sinks, scale=None,
                    return_lse=True, out=None, lse=None):
    """Decode / MTP verify against a ring buffer.

    q [B, T, Hq, D]; k_new/v_new [B, T, Hkv, D]; k_cache/v_cache [B, Hkv, W, D]
    (W = window = ring slots); ring_head [B] int32; sinks [Hq] fp32.
    """
    import torch

    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _dev(t, nm, q.dtype)
    _dev(ring_head, "ring_head", torch.int32)
    _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, k_new must be [B, T, H, D] and caches [B, Hkv, W, D]")
    b, t, hq, d = q.shape
    hkv, w = k_cache.shape[1], k_cache.shape[2]
    if (k_new.shape != (b, t, hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape
            or k_cache.shape[0] != b or k_cache.shape[3] != d or ring_head.numel() != b
            or sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sink_decode(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        ring_head.data_ptr(), sinks.data_ptr(), b, t, hq, hkv, d, w, _scale(scale), _dtype_code(q),
        out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_decode_fp8kv(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, ring_head, sinks,
                          scale=None, return_lse=True, out=None, lse=None):
    """swa_sink_decode against an FP8 ring: k_cache/v_cache [B, Hkv, W, D] uint8 E4M3
    codes, element value = code value * k_scale (K) or v_scale (V) (python floats)."""
    import torch

    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _dev(t, nm, q.dtype)
    _dev(k_cache, "k_cache", torch.uint8)
    _dev(v_cache, "v_cache", torch.uint8)
    _dev(ring_head, "ring_head", torch.int32)
    _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, k_new must be [B, T, H, D] and caches [B, Hkv, W, D]")
    b, t, hq, d = q.shape
    hkv, w = k_cache.shape[1], k_cache.shape[2]
    if (k_new.shape != (b, t, hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape
            or k_cache.shape[0] != b or k_cache.shape[3] != d or ring_head.numel() != b
            or sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sink_decode_fp8kv(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        float(k_scale), float(v_scale), ring_head.data_ptr(), sinks.data_ptr(), b, t, hq, hkv, d, w,
        _scale(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream(q.device))
    _check(rc)
    return out, lse


def swa_rope(x, positions, rope_base=ROPE_BASE_SWA):
    """Rotary embedding of x [rows, heads, D] in place (row r at positions[r], int32).
    Returns x."""
    import torch

    _dev(x, "x")
    _dev(positions, "positions", torch.int32)
    if x.dim() != 3 or positions.numel() != x.shape[0]:
        raise ValueError("x must be [rows, heads, D] with one position per row")
    rc = library().swa_rope(x.data_ptr(), positions.data_ptr(), x.shape[0], x.shape[1], x.shape[2],
                            float(rope_base), _dtype_code(x), _stream(x.device))
    _check(rc)
    return x


def swa_sink_decode_rope(q, k_new, v_new, k_cache, v_cache, ring_head, positions, sinks,
                         rope_base=ROPE_BASE_SWA, scale=None, return_lse=True, out=None, lse=None):
    """swa_sink_decode with q and k_new unrotated: new token t of sequence b is rotated
    at positions[b] + t inside the kernel (positions [B] int32); the ring holds keys
    rotated at their own positions."""
    import torch

    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _dev(t, nm, q.dtype)
    _dev(ring_head, "ring_head", torch.int32)
    _dev(positions, "positions", torch.int32)
    _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, k_new must be [B, T, H, D] and caches [B, Hkv, W, D]")
    b, t, hq, d = q.shape
    hkv, w = k_cache.shape[1], k_cache.shape[2]
    if (k_new.shape != (b, t, hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape
            or k_cache.shape[0] != b or k_cache.shape[3] != d or ring_head.numel() != b
            or positions.numel() != b or sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sink_decode_rope(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        ring_head.data_ptr(), positions.data_ptr(), sinks.data_ptr(), b, t, hq, hkv, d, w,
        _scale(scale), float(rope_base), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_decode_rope_commit(q, k_new, v_new, positions, prev_k, prev_v, prev_accept, prev_positions,
                                k_cache, v_cache, ring_head, ring_head_out, sinks, rope_base=ROPE_BASE_SWA,
                                scale=None, return_lse=True, out=None, lse=None):
    """One MTP step: commit the previous step's first prev_accept[b] tokens (prev_k, prev_v
    [B, prev_T, Hkv, D], keys unrotated, token 0 at prev_positions[b]) to the ring, then
    verify the T new tokens against it as swa_sink_decode_rope does.  The caches are
    updated in place; ring_head is read and the new head written to ring_head_out."""
    import torch

    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (prev_k, "prev_k"), (prev_v, "prev_v"),
                  (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm, q.dtype)
    for t, nm in ((ring_head, "ring_head"), (ring_head_out, "ring_head_out"), (positions, "positions"),
                  (prev_accept, "prev_accept"), (prev_positions, "prev_positions")):
        _dev(t, nm, torch.int32)
    _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_new.dim() != 4 or prev_k.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, k_new, prev_k must be [B, T, H, D] and caches [B, Hkv, W, D]")
    b, t, hq, d = q.shape
    hkv, w = k_cache.shape[1], k_cache.shape[2]
    pt = prev_k.shape[1]
    if (k_new.shape != (b, t, hkv, d) or v_new.shape != k_new.shape or prev_k.shape != (b, pt, hkv, d)
            or prev_v.shape != prev_k.shape or v_cache.shape != k_cache.shape or k_cache.shape[0] != b
            or k_cache.shape[3] != d or ring_head.numel() != b or ring_head_out.numel() != b
            or positions.numel() != b or prev_accept.numel() != b or prev_positions.numel() != b
            or sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sink_decode_rope_commit(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(), prev_k.data_ptr(),
        prev_v.data_ptr(), prev_accept.data_ptr(), prev_positions.data_ptr(), pt, k_cache.data_ptr(),
        v_cache.data_ptr(), ring_head.data_ptr(), ring_head_out.data_ptr(), sinks.data_ptr(), b, t, hq,
        hkv, d, w, _scale(scale), float(rope_base), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_decode_rope_commit_fp8kv(q, k_new, v_new, positions, prev_k, prev_v, prev_accept, prev_positions,
                                      k_cache, v_cache, k_scale, v_scale, ring_head, ring_head_out, sinks,
                                      rope_base=ROPE_BASE_SWA, scale=None, return_lse=True, out=None, lse=None):
    """swa_sink_decode_rope_commit against an FP8 ring: k_cache/v_cache [B, Hkv, W, D] uint8
    E4M3 codes with per-tensor scales; the committed tokens enter the ring encoded as
    swa_ring_append_fp8kv encodes them."""
    import torch

    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (prev_k, "prev_k"), (prev_v, "prev_v")):
        _dev(t, nm, q.dtype)
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm, torch.uint8)
    for t, nm in ((ring_head, "ring_head"), (ring_head_out, "ring_head_out"), (positions, "positions"),
                  (prev_accept, "prev_accept"), (prev_positions, "prev_positions")):
        _dev(t, nm, torch.int32)
    _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_new.dim() != 4 or prev_k.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, k_new, prev_k must be [B, T, H, D] and caches [B, Hkv, W, D]")
    b, t, hq, d = q.shape
    hkv, w = k_cache.shape[1], k_cache.shape[2]
    pt = prev_k.shape[1]
    if (k_new.shape != (b, t, hkv, d) or v_new.shape != k_new.shape or prev_k.shape != (b, pt, hkv, d)
            or prev_v.shape != prev_k.shape or v_cache.shape != k_cache.shape or k_cache.shape[0] != b
            or k_cache.shape[3] != d or ring_head.numel() != b or ring_head_out.numel() != b
            or positions.numel() != b or prev_accept.numel() != b or prev_positions.numel() != b
            or sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sink_decode_rope_commit_fp8kv(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(), prev_k.data_ptr(),
        prev_v.data_ptr(), prev_accept.data_ptr(), prev_positions.data_ptr(), pt, k_cache.data_ptr(),
        v_cache.data_ptr(), float(k_scale), float(v_scale), ring_head.data_ptr(), ring_head_out.data_ptr(),
        sinks.data_ptr(), b, t, hq, hkv, d, w, _scale(scale), float(rope_base), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_decode_rope_fp8kv(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, ring_head, positions,
                               sinks, rope_base=ROPE_BASE_SWA, scale=None, return_lse=True, out=None,
                               lse=None):
    """swa_sink_decode_rope against an FP8 ring: q and k_new unrotated (rotated in the
    kernel at positions[b] + t); k_cache/v_cache [B, Hkv, W, D] uint8 E4M3 codes with
    per-tensor scales, keys rotated at their own positions before encoding."""
    import torch

    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _dev(t, nm, q.dtype)
    _dev(k_cache, "k_cache", torch.uint8)
    _dev(v_cache, "v_cache", torch.uint8)
    _dev(ring_head, "ring_head", torch.int32)
    _dev(positions, "positions", torch.int32)
    _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q, k_new must be [B, T, H, D] and caches [B, Hkv, W, D]")
    b, t, hq, d = q.shape
    hkv, w = k_cache.shape[1], k_cache.shape[2]
    if (k_new.shape != (b, t, hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape
            or k_cache.shape[0] != b or k_cache.shape[3] != d or ring_head.numel() != b
            or positions.numel() != b or sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sink_decode_rope_fp8kv(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        float(k_scale), float(v_scale), ring_head.data_ptr(), positions.data_ptr(), sinks.data_ptr(),
        b, t, hq, hkv, d, w, _scale(scale), float(rope_base), _dtype_code(q), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream(q.device))
    _check(rc)
    return out, lse


def _append_shapes(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head, cache_dtype):
    import torch

    _dev(k_new, "k_new")
    _dev(v_new, "v_new", k_new.dtype)
    _dev(k_cache, "k_cache", cache_dtype)
    _dev(v_cache, "v_cache", cache_dtype)
    _dev(n_accept, "n_accept", torch.int32)
    _dev(ring_head, "ring_head", torch.int32)
    if positions is not None:
        _dev(positions, "positions", torch.int32)
    if k_new.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("k_new must be [B, T, Hkv, D] and caches [B, Hkv, W, D]")
    b, t, hkv, d = k_new.shape
    w = k_cache.shape[2]
    if (v_new.shape != k_new.shape or v_cache.shape != k_cache.shape or k_cache.shape[0] != b
            or k_cache.shape[1] != hkv or k_cache.shape[3] != d or n_accept.numel() != b
            or ring_head.numel() != b or (positions is not None and positions.numel() != b)):
        raise ValueError("inconsistent shapes")
    return b, t, hkv, d, w


def swa_ring_append_rope(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head,
                         rope_base=ROPE_BASE_SWA):
    """Commit the first n_accept[b] new tokens of each sequence to its ring, keys rotated
    at positions[b] + t; k_cache, v_cache and ring_head are updated in place."""
    b, t, hkv, d, w = _append_shapes(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head,
                                     k_new.dtype)
    rc = library().swa_ring_append_rope(
        k_new.data_ptr(), v_new.data_ptr(), n_accept.data_ptr(),
        positions.data_ptr() if positions is not None else None, k_cache.data_ptr(),
        v_cache.data_ptr(), ring_head.data_ptr(), b, t, hkv, d, w, float(rope_base),
        _dtype_code(k_new), _stream(k_new.device))
    _check(rc)


def swa_ring_append_fp8kv(k_new, v_new, n_accept, positions, k_cache, v_cache, k_scale, v_scale,
                          ring_head, rope_base=ROPE_BASE_SWA):
    """swa_ring_append_rope into an FP8 ring: k_cache/v_cache [B, Hkv, W, D] uint8 receive
    the E4M3 codes of (rotated) key / k_scale and value / v_scale; updated in place."""
    import torch

    b, t, hkv, d, w = _append_shapes(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head,
                                     torch.uint8)
    rc = library().swa_ring_append_fp8kv(
        k_new.data_ptr(), v_new.data_ptr(), n_accept.data_ptr(),
        positions.data_ptr() if positions is not None else None, k_cache.data_ptr(),
        v_cache.data_ptr(), float(k_scale), float(v_scale), ring_head.data_ptr(), b, t, hkv, d, w,
        float(rope_base), _dtype_code(k_new), _stream(k_new.device))
    _check(rc)


def swa_topk_select(scores, lengths, k=SPARSE_TOPK, recent=SPARSE_RECENT, indices=None, counts=None):
    """Top-k positions older than the recent window per (sequence, KV head) row of
    scores [B, Hkv, Lmax] fp32 (lengths [B] int32).  Returns (indices [B, Hkv, k] int32
    increasing, -1 padded; counts [B, Hkv] int32)."""
    import torch

    _dev(scores, "scores", torch.float32)
    _dev(lengths, "lengths", torch.int32)
    if scores.dim() != 3 or lengths.numel() != scores.shape[0]:
        raise ValueError("scores must be [B, Hkv, Lmax] with one length per sequence")
    b, hkv, lmax = scores.shape
    if indices is None:
        indices = torch.empty((b, hkv, k), dtype=torch.int32, device=scores.device)
    if counts is None:
        counts = torch.empty((b, hkv), dtype=torch.int32, device=scores.device)
    _dev(indices, "indices", torch.int32)
    _dev(counts, "counts", torch.int32)
    rc = library().swa_topk_select(scores.data_ptr(), lengths.data_ptr(), b, hkv, lmax, k, recent,
                                   indices.data_ptr(), counts.data_ptr(), _stream(scores.device))
    _check(rc)
    return indices, counts


def swa_sparse_decode(q, k_cache, v_cache, lengths, indices, counts, sinks=None, recent=SPARSE_RECENT,
                      scale=None, return_lse=True, out=None, lse=None):
    """The newest token of each sequence (q [B, Hq, D]) over its selected positions plus
    the recent window of a [B, Hkv, Lmax, D] cache."""
    import torch

    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm, q.dtype)
    _dev(lengths, "lengths", torch.int32)
    _dev(indices, "indices", torch.int32)
    _dev(counts, "counts", torch.int32)
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32)
    if q.dim() != 3 or k_cache.dim() != 4 or indices.dim() != 3:
        raise ValueError("q must be [B, Hq, D], caches [B, Hkv, Lmax, D], indices [B, Hkv, k]")
    b, hq, d = q.shape
    hkv, lmax = k_cache.shape[1], k_cache.shape[2]
    k = indices.shape[2]
    if (k_cache.shape != (b, hkv, lmax, d) or v_cache.shape != k_cache.shape or lengths.numel() != b
            or indices.shape[:2] != (b, hkv) or counts.shape != (b, hkv)
            or (sinks is not None and sinks.numel() != hq)):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sparse_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lengths.data_ptr(), indices.data_ptr(),
        counts.data_ptr(), sinks.data_ptr() if sinks is not None else None, b, hq, hkv, d, lmax, k, recent,
        _scale(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream(q.device))
    _check(rc)
    return out, lse


def swa_sparse_decode_mtp(q, k_cache, v_cache, lengths, indices, counts, sinks=None, recent=SPARSE_RECENT,
                          scale=None, return_lse=True, out=None, lse=None):
    """MTP verify in a sparse layer: the newest T tokens of each sequence (q [B, T, Hq, D]),
    each over its own recent window and the selected positions below it."""
    import torch

    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm, q.dtype)
    _dev(lengths, "lengths", torch.int32)
    _dev(indices, "indices", torch.int32)
    _dev(counts, "counts", torch.int32)
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_cache.dim() != 4 or indices.dim() != 3:
        raise ValueError("q must be [B, T, Hq, D], caches [B, Hkv, Lmax, D], indices [B, Hkv, k]")
    b, t, hq, d = q.shape
    hkv, lmax = k_cache.shape[1], k_cache.shape[2]
    k = indices.shape[2]
    if (k_cache.shape != (b, hkv, lmax, d) or v_cache.shape != k_cache.shape or lengths.numel() != b
            or indices.shape[:2] != (b, hkv) or counts.shape != (b, hkv)
            or (sinks is not None and sinks.numel() != hq)):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sparse_decode_mtp(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lengths.data_ptr(), indices.data_ptr(),
        counts.data_ptr(), sinks.data_ptr() if sinks is not None else None, b, t, hq, hkv, d, lmax, k, recent,
        _scale(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream(q.device))
    _check(rc)
    return out, lse


def swa_sparse_decode_fp8kv(q, k_cache, v_cache, k_scale, v_scale, lengths, indices, counts, sinks=None,
                            recent=SPARSE_RECENT, scale=None, return_lse=True, out=None, lse=None):
    """swa_sparse_decode_mtp over an FP8 cache: k_cache/v_cache [B, Hkv, Lmax, D] uint8 E4M3
    codes, element value = code value * k_scale (K) or v_scale (V) (python floats);
    q [B, T, Hq, D] (T = 1: the single-token step)."""
    import torch

    _dev(q, "q")
    _dev(k_cache, "k_cache", torch.uint8)
    _dev(v_cache, "v_cache", torch.uint8)
    _dev(lengths, "lengths", torch.int32)
    _dev(indices, "indices", torch.int32)
    _dev(counts, "counts", torch.int32)
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32)
    if q.dim() != 4 or k_cache.dim() != 4 or indices.dim() != 3:
        raise ValueError("q must be [B, T, Hq, D], caches [B, Hkv, Lmax, D], indices [B, Hkv, k]")
    b, t, hq, d = q.shape
    hkv, lmax = k_cache.shape[1], k_cache.shape[2]
    k = indices.shape[2]
    if (k_cache.shape != (b, hkv, lmax, d) or v_cache.shape != k_cache.shape or lengths.numel() != b
            or indices.shape[:2] != (b, hkv) or counts.shape != (b, hkv)
            or (sinks is not None and sinks.numel() != hq)):
        raise ValueError("inconsistent shapes")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if return_lse and lse is None:
        lse = torch.empty((b, t, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    rc = library().swa_sparse_decode_fp8kv(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), float(k_scale), float(v_scale), lengths.data_ptr(),
        indices.data_ptr(), counts.data_ptr(), sinks.data_ptr() if sinks is not None else None, b, t, hq, hkv, d,
        lmax, k, recent, _scale(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream(q.device))
    _check(rc)
    return out, lse


def swa_sink_prefill_backward(q, k, v, sinks, cu_seqlens, out, lse, dout, max_seqlen=None,
                              window=128, scale=None, library_scratch=False, grads=None):
    """Gradients of swa_sink_prefill's output O: (dq, dk, dv, dsinks) for dout = dL/dO.

    q/out/dout [N, Hq, D], k/v [N, Hkv, D] in one dtype, lse [N, Hq] fp32 from the
    forward, sinks [Hq] fp32 or None (no sink; dsinks is then None).  The workspace
    the library needs is allocated here with torch; with library_scratch=True the call
    goes to swa_sink_prefill_backward_noalloc, which uses the library's own scratch
    array instead.  grads = (dq, dk, dv, dsinks) receives the gradients in caller
    buffers (then nothing at all is allocated here with library_scratch=True).
    """
    import torch

    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _dev(t, nm, q.dtype)
    _dev(lse, "lse", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, out, dout must be [N, Hq, D] and k, v [N, Hkv, D]")
    n, hq, d = q.shape
    if k.shape[0] != n or k.shape[2] != d or tuple(lse.shape) != (n, hq) or (
            sinks is not None and sinks.numel() != hq):
        raise ValueError("inconsistent shapes")
    lib = library()
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsinks = None if sinks is None else torch.empty(hq, dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, dsinks = grads
        for t, ref, nm in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
            _dev(t, nm, ref.dtype)
            if t.shape != ref.shape:
                raise ValueError(f"{nm} must have the shape of {nm[1:]}")
        if (dsinks is None) != (sinks is None) or (dsinks is not None and dsinks.numel() != hq):
            raise ValueError("dsinks must be given exactly when sinks is, with one value per head")
        if dsinks is not None:
            _dev(dsinks, "dsinks", torch.float32)
    ms = n if max_seqlen is None else int(max_seqlen)
    if library_scratch:
        rc = lib.swa_sink_prefill_backward_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), None if sinks is None else sinks.data_ptr(),
            cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, n, ms, hq, k.shape[1], d, int(window),
            _scale(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), None if dsinks is None else dsinks.data_ptr(), _stream(q.device))
        _check(rc)
        return dq, dk, dv, dsinks
    need = int(lib.swa_sink_prefill_backward_workspace(n, hq))
    if need < 0:
        raise ValueError("invalid sizes")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib.swa_sink_prefill_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), None if sinks is None else sinks.data_ptr(),
        cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, n, ms, hq, k.shape[1], d, int(window),
        _scale(scale), _dtype_code(q), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), None if dsinks is None else dsinks.data_ptr(), ws.data_ptr(),
        need, _stream(q.device))
    _check(rc)
    return dq, dk, dv, dsinks
