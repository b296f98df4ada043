"""Benchmark of the hybrid sliding-window attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

A step is one sliding-window-with-sink prefill of the 32K-token layer (32 query
heads / 4 KV heads, head_dim 128, window 128, bf16 in/out, fp32 LSE) with inputs
resident in HBM.  Input sets are rotated across steps (distinct buffers, 4 x 608
MB) so that no step finds its inputs in the 256 MB Infinity Cache.  Timing uses
HIP events on the stream the kernels are launched on.  The printed JSON line
reports the prefill TFLOP/s (unmasked (query, key) pairs only), the achieved
HBM GB/s of the kernel against the 8 TB/s peak, and, under "extra", the batched
decode / MTP-verify GB/s, the global-attention layer, the 5:1 hybrid block and the
262K-token varlen prefill, each timed the same way.  "cpu_baseline" times the fp64
oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
PRIMARY = "swa_prefill_32k"
METRIC = "SWA-sink prefill TFLOP/s (% MFMA peak); decode GB/s (% HBM peak)"


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _to(x, dev):
    return {k: (v.to(dev) if hasattr(v, "to") and hasattr(v, "dtype") else v) for k, v in x.items()}


def _clone_sets(x, n):
    sets = [x]
    for _ in range(n - 1):
        sets.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in x.items()})
    return sets


SETTLE_S = 0.3


def _time_calls(fn, sets, steps, warmup, per_call=True):
    """Warm up, then time `steps` calls (set rotated per call) with HIP events.

    Before the `warmup` counted calls the GPU is kept busy with untimed calls for
    at least SETTLE_S seconds, so that its clocks have left their idle state when
    the timed region opens (a few calls of a 0.15 ms kernel do not get there).
    Returns (per-call milliseconds list, milliseconds of the whole timed region).
    per_call=False records events only around the region (kernels of a few tens of
    microseconds: an event pair per launch would add its own dispatch overhead);
    the per-call list is then the region average repeated."""
    import torch

    for x in sets:  # marshal every input set once, outside the timed region
        fn(x)
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < SETTLE_S:
        fn(sets[n % len(sets)])
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    for s in range(warmup):
        fn(sets[s % len(sets)])
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    region0.record()
    for s in range(steps):
        if per_call:
            starts[s].record()
        fn(sets[s % len(sets)])
        if per_call:
            ends[s].record()
    region1.record()
    torch.cuda.synchronize()
    region = region0.elapsed_time(region1)
    if not per_call:
        return [region / steps] * steps, region
    return [a.elapsed_time(b) for a, b in zip(starts, ends)], region


def _prefill_fn(window, ga=False):
    """Timed call: the C entry point with arguments marshalled once per input set
    (the Python checks of the binding cost more than a decode kernel runs, which
    would let the GPU idle between launches)."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            swa.ga_causal_prefill(x["q"], x["k"], x["v"], x["cu_seqlens"], x["max_seqlen"],
                                  out=x["out"], lse=x["lse"]) if ga else \
                swa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], x["cu_seqlens"],
                                     x["max_seqlen"], window=window, out=x["out"], lse=x["lse"])
            n, hq, d = x["q"].shape
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            common = (x["cu_seqlens"].data_ptr(), x["cu_seqlens"].numel() - 1, n, int(x["max_seqlen"]),
                      hq, x["k"].shape[1], d)
            if ga:
                cache[key] = (lib.ga_causal_prefill,
                              (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), *common, 0.0, 1,
                               x["out"].data_ptr(), x["lse"].data_ptr(), stream))
            else:
                cache[key] = (lib.swa_sink_prefill,
                              (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["sinks"].data_ptr(),
                               *common, window, 0.0, 1, x["out"].data_ptr(), x["lse"].data_ptr(), stream))
        f, args = cache[key]
        rc = f(*args)
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _prefill_fp8_fn(window):
    """Timed call of swa_sink_prefill_fp8kv (E4M3 K/V), arguments marshalled once per input set."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            swa.swa_sink_prefill_fp8kv(x["q"], x["k"], x["v"], x["k_scale"], x["v_scale"], x["sinks"],
                                       x["cu_seqlens"], x["max_seqlen"], window=window, out=x["out"],
                                       lse=x["lse"])
            n, hq, d = x["q"].shape
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            cache[key] = (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), ctypes.c_float(x["k_scale"]),
                          ctypes.c_float(x["v_scale"]), x["sinks"].data_ptr(), x["cu_seqlens"].data_ptr(),
                          x["cu_seqlens"].numel() - 1, n, int(x["max_seqlen"]), hq, x["k"].shape[1], d,
                          window, 0.0, 1, x["out"].data_ptr(), x["lse"].data_ptr(), stream)
        rc = lib.swa_sink_prefill_fp8kv(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _decode_fn():
    """Timed call of swa_sink_decode, arguments marshalled once per input set."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            swa.swa_sink_decode(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                x["ring_head"], x["sinks"], out=x["out"], lse=x["lse"])
            b, t, hq, d = x["q"].shape
            hkv, w = x["k_cache"].shape[1], x["k_cache"].shape[2]
            cache[key] = (x["q"].data_ptr(), x["k_new"].data_ptr(), x["v_new"].data_ptr(),
                          x["k_cache"].data_ptr(), x["v_cache"].data_ptr(), x["ring_head"].data_ptr(),
                          x["sinks"].data_ptr(), b, t, hq, hkv, d, w, 0.0, 1, x["out"].data_ptr(),
                          x["lse"].data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sink_decode(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _decode_rope_fn():
    """Timed call of swa_sink_decode_rope (SWA base 10,000), arguments marshalled once per set."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            swa.swa_sink_decode_rope(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                     x["ring_head"], x["positions"], x["sinks"], swa.ROPE_BASE_SWA,
                                     out=x["out"], lse=x["lse"])
            b, t, hq, d = x["q"].shape
            hkv, w = x["k_cache"].shape[1], x["k_cache"].shape[2]
            cache[key] = (x["q"].data_ptr(), x["k_new"].data_ptr(), x["v_new"].data_ptr(),
                          x["k_cache"].data_ptr(), x["v_cache"].data_ptr(), x["ring_head"].data_ptr(),
                          x["positions"].data_ptr(), x["sinks"].data_ptr(), b, t, hq, hkv, d, w, 0.0,
                          swa.ROPE_BASE_SWA, 1, x["out"].data_ptr(), x["lse"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sink_decode_rope(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _decode_rope_fp8_fn():
    """Timed call of swa_sink_decode_rope_fp8kv (SWA base 10,000), arguments marshalled once
    per input set."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            swa.swa_sink_decode_rope_fp8kv(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                           x["k_scale"], x["v_scale"], x["ring_head"], x["positions"],
                                           x["sinks"], swa.ROPE_BASE_SWA, out=x["out"], lse=x["lse"])
            b, t, hq, d = x["q"].shape
            hkv, w = x["k_cache"].shape[1], x["k_cache"].shape[2]
            cache[key] = (x["q"].data_ptr(), x["k_new"].data_ptr(), x["v_new"].data_ptr(),
                          x["k_cache"].data_ptr(), x["v_cache"].data_ptr(), float(x["k_scale"]),
                          float(x["v_scale"]), x["ring_head"].data_ptr(), x["positions"].data_ptr(),
                          x["sinks"].data_ptr(), b, t, hq, hkv, d, w, 0.0, swa.ROPE_BASE_SWA, 1,
                          x["out"].data_ptr(), x["lse"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sink_decode_rope_fp8kv(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _rope_inputs(dev, nsets=1):
    """The 32K layer's Q (seeded like the prefill workload) and positions 0..32767, as
    `nsets` distinct copies of Q (268 MB each) sharing the positions."""
    import torch

    from sliding_window_attention_amd import workloads as wl

    x = _to(wl.make_workload(PRIMARY), dev)
    pos = torch.arange(32768, dtype=torch.int32, device=dev)
    return [{"q": x["q"] if i == 0 else x["q"].clone(), "positions": pos} for i in range(nsets)]


def _sparse_inputs(dev, set_index=0):
    """The sparse_b64 workload drawn on the GPU (64 sequences, [64, 4, 32768, 128] caches)
    with its selection, indices and counts allocated.  set_index > 0 draws another set of
    the same shape (seed offset), for rotation past the Infinity Cache."""
    import torch

    from sliding_window_attention_amd import workloads as wl

    w = wl.WORKLOADS["sparse_b64"]
    x = wl.make_sparse_device(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seq_len,
                              w.seed + 7919 * set_index, dev, min_len=w.extra["min_len"])
    x["lengths_host"] = x["lengths"]
    x["lengths"] = x["lengths"].to(dev)
    x["indices"] = torch.empty((w.batch, w.num_kv_heads, w.extra["topk"]), dtype=torch.int32, device=dev)
    x["counts"] = torch.empty((w.batch, w.num_kv_heads), dtype=torch.int32, device=dev)
    x["out"] = torch.empty_like(x["q"])
    x["lse"] = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    return x


def _topk_fn():
    """Timed call of swa_topk_select on the sparse workload's scores."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            b, hkv, lmax = x["scores"].shape
            cache[key] = (x["scores"].data_ptr(), x["lengths"].data_ptr(), b, hkv, lmax, x["indices"].shape[2],
                          swa.SPARSE_RECENT, x["indices"].data_ptr(), x["counts"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_topk_select(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _sparse_fn():
    """Timed call of swa_sparse_decode on the sparse workload (selection already made)."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            b, hq, d = x["q"].shape
            hkv, lmax = x["k_cache"].shape[1], x["k_cache"].shape[2]
            cache[key] = (x["q"].data_ptr(), x["k_cache"].data_ptr(), x["v_cache"].data_ptr(),
                          x["lengths"].data_ptr(), x["indices"].data_ptr(), x["counts"].data_ptr(),
                          None, b, hq, hkv, d, lmax, x["indices"].shape[2], swa.SPARSE_RECENT, 0.0, 1,
                          x["out"].data_ptr(), x["lse"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sparse_decode(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _sparse_mtp_fn():
    """Timed call of swa_sparse_decode_mtp (T = 2) on the sparse workload: the newest two
    tokens of each sequence as queries, the selection already made."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            if "q2" not in x:
                b, hq, d = x["q"].shape
                x["q2"] = torch.randn((b, 2, hq, d), generator=torch.Generator(device=x["q"].device).manual_seed(17),
                                      device=x["q"].device).to(x["q"].dtype)
                x["out2"] = torch.empty_like(x["q2"])
                x["lse2"] = torch.empty((b, 2, hq), dtype=torch.float32, device=x["q"].device)
            b, t, hq, d = x["q2"].shape
            hkv, lmax = x["k_cache"].shape[1], x["k_cache"].shape[2]
            cache[key] = (x["q2"].data_ptr(), x["k_cache"].data_ptr(), x["v_cache"].data_ptr(),
                          x["lengths"].data_ptr(), x["indices"].data_ptr(), x["counts"].data_ptr(),
                          None, b, t, hq, hkv, d, lmax, x["indices"].shape[2], swa.SPARSE_RECENT, 0.0, 1,
                          x["out2"].data_ptr(), x["lse2"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sparse_decode_mtp(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _sparse_fp8_fn(t_new):
    """Timed call of swa_sparse_decode_fp8kv (the newest t_new tokens as queries) on the
    sparse workload with its caches as E4M3 codes, the selection already made."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            qk, ok, lk = f"q{t_new}", f"out{t_new}", f"lse{t_new}"
            if qk not in x:
                b, hq, d = x["q"].shape
                x[qk] = torch.randn((b, t_new, hq, d), generator=torch.Generator(device=x["q"].device).manual_seed(17),
                                    device=x["q"].device).to(x["q"].dtype)
                x[ok] = torch.empty_like(x[qk])
                x[lk] = torch.empty((b, t_new, hq), dtype=torch.float32, device=x["q"].device)
            b, t, hq, d = x[qk].shape
            hkv, lmax = x["k_codes"].shape[1], x["k_codes"].shape[2]
            cache[key] = (x[qk].data_ptr(), x["k_codes"].data_ptr(), x["v_codes"].data_ptr(), ctypes.c_float(1 / 32),
                          ctypes.c_float(1 / 64), x["lengths"].data_ptr(), x["indices"].data_ptr(),
                          x["counts"].data_ptr(), None, b, t, hq, hkv, d, lmax, x["indices"].shape[2],
                          swa.SPARSE_RECENT, 0.0, 1, x[ok].data_ptr(), x[lk].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sparse_decode_fp8kv(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _with_fp8_caches(xs):
    """Replace each sparse set's bf16 caches by E4M3 codes of the same shape, drawn on the
    GPU per sequence (scales 1/32 and 1/64: values of about N(0, 1))."""
    import torch

    from sliding_window_attention_amd import workloads as wl

    for i, x in enumerate(xs):
        shape = tuple(x["k_cache"].shape)
        dev = x["k_cache"].device
        del x["k_cache"], x["v_cache"]
        gen = torch.Generator(device=dev).manual_seed(9001 + i)
        x["k_codes"] = torch.empty(shape, dtype=torch.uint8, device=dev)
        x["v_codes"] = torch.empty(shape, dtype=torch.uint8, device=dev)
        for b in range(shape[0]):
            x["k_codes"][b] = wl.e4m3_codes(shape[1:], gen)
            x["v_codes"][b] = wl.e4m3_codes(shape[1:], gen)
    torch.cuda.empty_cache()
    return xs


def _sparse_mtp_work(x, t_new=2, kv_elem_bytes=2):
    from sliding_window_attention_amd import workloads as wl

    w = wl.WORKLOADS["sparse_b64"]
    return wl.sparse_mtp_work(x["lengths_host"].tolist(), x["indices"].cpu().numpy(), x["counts"].cpu().numpy(),
                              w.num_q_heads, w.num_kv_heads, w.head_dim, w.extra["recent"], t_new, 2, kv_elem_bytes)


def _sparse_work(x):
    from sliding_window_attention_amd import workloads as wl

    w = wl.WORKLOADS["sparse_b64"]
    lens = x["lengths_host"].tolist()
    return (wl.topk_bytes(lens, w.num_kv_heads, w.extra["topk"], w.extra["recent"]),
            wl.sparse_bytes(lens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.extra["topk"], w.extra["recent"], 2),
            wl.sparse_flops(lens, w.num_q_heads, w.head_dim, w.extra["topk"], w.extra["recent"]))


def _append_inputs(dev, fp8=False):
    """Ring append after an MTP verify of the T = 4 decode workload (bf16 ring, or the FP8
    ring of the same shape): seeded accept counts ~ U{0..4} per sequence (keys rotated at
    base 10,000)."""
    import torch

    from sliding_window_attention_amd import workloads as wl

    x = _to(wl.make_workload("decode_rope_fp8_t4" if fp8 else "decode_rope_t4"), dev)
    gen = torch.Generator().manual_seed(3501)
    x["n_accept"] = torch.randint(0, 5, (x["q"].shape[0],), generator=gen,
                                  dtype=torch.int64).to(torch.int32).to(dev)
    return x


MTP_SETS = 8     # 8 x ~88 MB (decode T = 4 inputs + ring) per MTP-step rotation
SPARSE_SETS = 4  # 4 x 153 MB of gathered K/V rows (each set has its own 4 GB caches)
TOPK_SETS = 16   # 16 x 24.5 MB of candidate scores


def _mtp_sets(dev, fp8):
    """Distinct copies of the MTP-step inputs (each with its own ring, ring heads and
    outputs), rotated so that no step finds its ring in the Infinity Cache."""
    x = _with_outputs(_append_inputs(dev, fp8), "decode")
    sets = [x]
    for _ in range(MTP_SETS - 1):
        sets.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in x.items()})
    return sets


def _sparse_sets(dev, what):
    """Input sets for the sparse legs: the selection rotates over TOPK_SETS copies of the
    scores (sharing one workload's caches), the sparse decode over SPARSE_SETS workloads
    drawn with different seeds, each selected once beforehand."""
    import torch

    if what == "topk":
        x = _sparse_inputs(dev)
        sets = [x]
        for _ in range(TOPK_SETS - 1):
            y = dict(x)
            y["scores"] = x["scores"].clone()
            y["indices"] = torch.empty_like(x["indices"])
            y["counts"] = torch.empty_like(x["counts"])
            sets.append(y)
        return sets
    sets = []
    for i in range(SPARSE_SETS):
        x = _sparse_inputs(dev, i)
        _topk_fn()(x)
        sets.append(x)
    return sets


def _append_fn(fp8=False):
    """Timed call of swa_ring_append_rope (or swa_ring_append_fp8kv into an FP8 ring); each
    call commits the same accept counts again (the ring keeps rolling: the same work every
    call)."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            b, t, hkv, d = x["k_new"].shape
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            if fp8:
                cache[key] = (x["k_new"].data_ptr(), x["v_new"].data_ptr(), x["n_accept"].data_ptr(),
                              x["positions"].data_ptr(), x["k_cache"].data_ptr(), x["v_cache"].data_ptr(),
                              float(x["k_scale"]), float(x["v_scale"]), x["ring_head"].data_ptr(), b, t, hkv,
                              d, x["k_cache"].shape[2], swa.ROPE_BASE_SWA, 1, st)
            else:
                cache[key] = (x["k_new"].data_ptr(), x["v_new"].data_ptr(), x["n_accept"].data_ptr(),
                              x["positions"].data_ptr(), x["k_cache"].data_ptr(), x["v_cache"].data_ptr(),
                              x["ring_head"].data_ptr(), b, t, hkv, d, x["k_cache"].shape[2],
                              swa.ROPE_BASE_SWA, 1, st)
        rc = (lib.swa_ring_append_fp8kv if fp8 else lib.swa_ring_append_rope)(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _commit_fn(fp8=False):
    """Timed call of swa_sink_decode_rope_commit (or its FP8-ring form): the step's verify
    (T = 4) and the commit of the previous step's accepted tokens in one launch.  The set's
    own new tokens stand for the previous step's (prev_T = 4, its accept counts, its
    positions); the head is read from ring_head and written to ring_head_out, so every call
    does the same work."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            x["ring_head_out"] = torch.empty_like(x["ring_head"])
            b, t, hq, d = x["q"].shape
            hkv, w = x["k_cache"].shape[1], x["k_cache"].shape[2]
            scales = (float(x["k_scale"]), float(x["v_scale"])) if fp8 else ()
            cache[key] = (x["q"].data_ptr(), x["k_new"].data_ptr(), x["v_new"].data_ptr(),
                          x["positions"].data_ptr(), x["k_new"].data_ptr(), x["v_new"].data_ptr(),
                          x["n_accept"].data_ptr(), x["positions"].data_ptr(), t, x["k_cache"].data_ptr(),
                          x["v_cache"].data_ptr(), *scales, x["ring_head"].data_ptr(),
                          x["ring_head_out"].data_ptr(), x["sinks"].data_ptr(), b, t, hq, hkv, d, w, 0.0,
                          swa.ROPE_BASE_SWA, 1, x["out"].data_ptr(), x["lse"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = (lib.swa_sink_decode_rope_commit_fp8kv if fp8 else lib.swa_sink_decode_rope_commit)(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _rope_fn():
    """Timed call of swa_rope on the 32K layer's Q [32768, 32, 128] (positions 0..32767)."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()

    def fn(x):
        rc = lib.swa_rope(x["q"].data_ptr(), x["positions"].data_ptr(), x["q"].shape[0], x["q"].shape[1],
                          x["q"].shape[2], swa.ROPE_BASE_SWA, 1,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _decode_fp8_fn():
    """Timed call of swa_sink_decode_fp8kv, arguments marshalled once per input set."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            swa.swa_sink_decode_fp8kv(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                      x["k_scale"], x["v_scale"], x["ring_head"], x["sinks"],
                                      out=x["out"], lse=x["lse"])
            b, t, hq, d = x["q"].shape
            hkv, w = x["k_cache"].shape[1], x["k_cache"].shape[2]
            cache[key] = (x["q"].data_ptr(), x["k_new"].data_ptr(), x["v_new"].data_ptr(),
                          x["k_cache"].data_ptr(), x["v_cache"].data_ptr(), float(x["k_scale"]),
                          float(x["v_scale"]), x["ring_head"].data_ptr(), x["sinks"].data_ptr(),
                          b, t, hq, hkv, d, w, 0.0, 1, x["out"].data_ptr(), x["lse"].data_ptr(),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sink_decode_fp8kv(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _backward_fn():
    """Timed call of swa_sink_prefill_backward, arguments marshalled once per input set
    (x holds q, k, v, sinks, cu_seqlens, out, lse, dout and the gradient buffers)."""
    import ctypes

    import torch

    import sliding_window_attention_amd as swa

    lib = swa.library()
    cache = {}

    def fn(x):
        key = id(x)
        if key not in cache:
            n, hq, d = x["q"].shape
            need = int(lib.swa_sink_prefill_backward_workspace(n, hq))
            x["ws"] = torch.empty(need, dtype=torch.uint8, device=x["q"].device)
            for nm in ("dq", "dk", "dv"):
                x[nm] = torch.empty_like(x[nm[1]])
            x["dsinks"] = torch.empty(hq, dtype=torch.float32, device=x["q"].device)
            cache[key] = (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["sinks"].data_ptr(),
                          x["cu_seqlens"].data_ptr(), x["cu_seqlens"].numel() - 1, n, n, hq,
                          x["k"].shape[1], d, 128, 0.0, 1, x["out"].data_ptr(), x["lse"].data_ptr(),
                          x["dout"].data_ptr(), x["dq"].data_ptr(), x["dk"].data_ptr(), x["dv"].data_ptr(),
                          x["dsinks"].data_ptr(), x["ws"].data_ptr(), need,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        rc = lib.swa_sink_prefill_backward(*cache[key])
        if rc != 0:
            raise RuntimeError(lib.swa_last_error().decode())
    return fn


def _backward_inputs(dev):
    """The 32K layer's inputs, its forward output and LSE (from the library's forward,
    untimed) and a seeded dout: the backward's workload."""
    import torch

    import sliding_window_attention_amd as swa
    from sliding_window_attention_amd import workloads as wl

    x = _to(wl.make_workload(PRIMARY), dev)
    x["out"], x["lse"] = swa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], x["cu_seqlens"],
                                              x["max_seqlen"], window=128)
    gen = torch.Generator(device=dev).manual_seed(wl.WORKLOADS[PRIMARY].seed + 7)
    x["dout"] = torch.randn(x["q"].shape, generator=gen, device=dev).to(x["q"].dtype)
    return x


def _with_outputs(x, kind):
    import torch

    if kind == "decode":
        b, t, hq, _ = x["q"].shape
        x["out"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty((b, t, hq), dtype=torch.float32, device=x["q"].device)
    else:
        n, hq, _ = x["q"].shape
        x["out"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty((n, hq), dtype=torch.float32, device=x["q"].device)
    return x


def _stats(ms):
    s = sorted(ms)
    return {"mean_ms": sum(s) / len(s), "median_ms": s[len(s) // 2], "min_ms": s[0]}


# Sources each profiled kernel is built from: counters taken on a kernel stay valid
# while these files are unchanged.
KERNEL_SOURCES = {
    "swa_ring_kernel": ("prefill_mfma.hip", "mfma_tile.h", "common.h", "kernels.h"),
}


def kernel_source_digest(kernel: str = "swa_ring_kernel") -> str:
    """Hash of the HIP sources a kernel is built from; traffic counters are only
    reported for the kernel version they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sliding_window_attention_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, algorithmic_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the kernel's current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != kernel_source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(sample_tokens=32768):
    """The fp64 oracle on the first `sample_tokens` tokens of the 32K layer (by
    default the whole layer: a few seconds on a 16-core host)."""
    import numpy as np

    from oracle import swa_oracle as orc
    from sliding_window_attention_amd import workloads as wl

    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    x = wl.make_prefill([sample_tokens], 32, 4, 128, "bf16", seed=wl.WORKLOADS[PRIMARY].seed)
    t0 = time.perf_counter()
    orc.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], np.array([0, sample_tokens]), 128)
    dt = time.perf_counter() - t0
    flops = wl.prefill_flops([sample_tokens], 32, 128, 128)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{sample_tokens} of 32768 tokens of the layer (all 32 heads), fp64 numpy, {dt:.2f} s",
            "seconds": dt, "blas_threads": int(threads), "affinity_cores": len(os.sched_getaffinity(0))}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="time only the primary workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["prefill", "prefill_fp8", "decode", "decode1", "decode_fp8", "decode_fp8_1",
                                       "decode_rope", "decode_rope_1", "decode_rope_fp8", "append",
                                       "append_fp8", "mtp_step", "mtp_step_fp8", "mtp_fused", "mtp_fused_fp8", "rope",
                                       "topk", "sparse", "sparse_mtp", "sparse_fp8", "sparse_mtp_fp8",
                                       "ga", "varlen", "backward", "copy"],
                    default=None,
                    help="time a single workload (for profiling runs); prints no JSON line")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import torch

    import sliding_window_attention_amd as swa
    from sliding_window_attention_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    swa.library()
    steps, warmup = args.steps, args.warmup

    if args.only == "copy":
        # plain device copy of 512 MiB (read 512 MiB + write 512 MiB): the reference
        # kernel for scaling the HBM byte counters
        a = torch.empty(1 << 28, dtype=torch.bfloat16, device=dev).normal_()
        b = torch.empty_like(a)
        per, _ = _time_calls(lambda _: b.copy_(a), [None], steps, warmup)
        _log(f"copy 512 MiB: {_stats(per)}  {2 * a.numel() * 2 / (_stats(per)['mean_ms'] * 1e-3) / 1e9:.0f} GB/s")
        return 0
    if args.only == "backward":
        x = _backward_inputs(dev)
        per, _ = _time_calls(_backward_fn(), [x], max(20, steps), max(3, warmup), per_call=False)
        st = _stats(per)
        fl = wl.backward_flops([32768], 32, 128, 128)
        by = wl.backward_bytes(32768, 32, 4, 128, 2)
        _log(f"backward 32K: {st}  {fl / (st['mean_ms'] * 1e-3) / 1e12:.1f} TFLOP/s  "
             f"{by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s")
        return 0
    if args.only in ("mtp_fused", "mtp_fused_fp8"):
        fp8 = args.only.endswith("fp8")
        xs = _mtp_sets(dev, fp8)
        per, _ = _time_calls(_commit_fn(fp8), xs, max(steps, 200), warmup, per_call=False)
        st = _stats(per)
        by = (wl.workload_work("decode_rope_fp8_t4" if fp8 else "decode_rope_t4")[1]
              + wl.mtp_commit_bytes(256, int(xs[0]["n_accept"].sum()), 4, 128, 1 if fp8 else 2))
        _log(f"{args.only} B=256 T=4: {st}  {by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s ({by} bytes)")
        return 0
    if args.only in ("append", "mtp_step", "append_fp8", "mtp_step_fp8"):
        # append alone is launch-bound from this loop (a ~4 us kernel); in a decode loop it
        # is queued behind the verify kernel, which "mtp_step" times
        fp8 = args.only.endswith("fp8")
        xs = _mtp_sets(dev, fp8)
        x = xs[0]
        app_fn = _append_fn(fp8)
        if args.only.startswith("append"):
            fn = app_fn
        else:
            dec_fn = _decode_rope_fp8_fn() if fp8 else _decode_rope_fn()

            def fn(x_):
                dec_fn(x_)
                app_fn(x_)
        per, _ = _time_calls(fn, xs, max(steps, 200), warmup, per_call=False)
        st = _stats(per)
        by = wl.append_bytes(256, int(x["n_accept"].sum()), 4, 128, 2, cache_elem_bytes=1 if fp8 else None)
        _log(f"{args.only} B=256 T=4: {st}  (append bytes {by})")
        return 0
    if args.only in ("sparse_fp8", "sparse_mtp_fp8"):
        t_new = 1 if args.only == "sparse_fp8" else 2
        xs = _with_fp8_caches(_sparse_sets(dev, "sparse"))
        per, _ = _time_calls(_sparse_fp8_fn(t_new), xs, max(steps, 100), warmup, per_call=False)
        st = _stats(per)
        fl, by = _sparse_mtp_work(xs[0], t_new, 1)
        _log(f"{args.only} T={t_new} sparse_b64: {st}  {by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s ({by} bytes)")
        return 0
    if args.only == "sparse_mtp":
        xs = _sparse_sets(dev, "sparse")
        fn = _sparse_mtp_fn()
        per, _ = _time_calls(fn, xs, max(steps, 100), warmup, per_call=False)
        st = _stats(per)
        fl, by = _sparse_mtp_work(xs[0])
        _log(f"sparse_mtp T=2 sparse_b64: {st}  {by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s ({by} bytes)")
        return 0
    if args.only in ("topk", "sparse"):
        xs = _sparse_sets(dev, args.only)
        fn = _topk_fn() if args.only == "topk" else _sparse_fn()
        per, _ = _time_calls(fn, xs, max(steps, 100), warmup, per_call=False)
        st = _stats(per)
        tb, sb, sfl = _sparse_work(xs[0])
        by = tb if args.only == "topk" else sb
        _log(f"{args.only} sparse_b64: {st}  {by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s ({by} bytes)")
        return 0
    if args.only == "rope":
        per, _ = _time_calls(_rope_fn(), _rope_inputs(dev, 4), steps, warmup, per_call=False)
        st = _stats(per)
        by = wl.rope_bytes(32768, 32, 128, 2)
        _log(f"rope q 32K: {st}  {by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s")
        return 0
    if args.only is not None:
        name = {"prefill": PRIMARY, "prefill_fp8": "swa_prefill_fp8kv_32k", "decode": "decode_t4",
                "decode1": "decode_t1",
                "decode_fp8": "decode_fp8_t4", "decode_fp8_1": "decode_fp8_t1",
                "decode_rope": "decode_rope_t4", "decode_rope_1": "decode_rope_t1",
                "decode_rope_fp8": "decode_rope_fp8_t4",
                "ga": "hybrid_5to1_32k", "varlen": "varlen_262k"}[args.only]
        layer = 5 if args.only == "ga" else 0
        dec = args.only.startswith("decode")
        x = _with_outputs(_to(wl.make_workload(name, layer), dev), "decode" if dec else "p")
        if args.only.startswith("decode_fp8"):
            fn = _decode_fp8_fn()
        elif args.only == "decode_rope_fp8":
            fn = _decode_rope_fp8_fn()
        elif args.only == "prefill_fp8":
            fn = _prefill_fp8_fn(128)
        elif args.only.startswith("decode_rope"):
            fn = _decode_rope_fn()
        else:
            fn = _decode_fn() if dec else _prefill_fn(128, ga=args.only == "ga")
        nsets = 32 if dec else (1 if args.only in ("varlen", "ga") else 4)
        if args.only in ("varlen", "ga"):
            steps, warmup = max(steps, 20), max(warmup, 3)
        per, _ = _time_calls(fn, _clone_sets(x, nsets), steps, warmup, per_call=not dec)
        fl, by = wl.workload_work(name)
        if args.only == "ga":
            fl, by = wl.prefill_flops([32768], 32, 128, None), wl.prefill_bytes(32768, 32, 4, 128, 2)
        st = _stats(per)
        _log(f"{name}: {st}  {fl / (st['mean_ms'] * 1e-3) / 1e12:.1f} TFLOP/s  "
             f"{by / (st['mean_ms'] * 1e-3) / 1e9:.0f} GB/s")
        return 0

    # ---------------- primary: SWA-sink prefill, 32K tokens ----------------
    _log("generating swa_prefill_32k inputs")
    x = _with_outputs(_to(wl.make_workload(PRIMARY), dev), "prefill")
    sets = _clone_sets(x, 4)
    # K back-to-back launches between two HIP events on the launching stream: the
    # region over K is both the time per step and the kernel's average launch
    # duration (one launch per step); per-launch event pairs would add gaps
    per, region_ms = _time_calls(_prefill_fn(128), sets, steps, warmup, per_call=False)
    flops, nbytes = wl.workload_work(PRIMARY)
    st = _stats(per)
    ms_per_step = region_ms / steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    kernel_s = st["mean_ms"] * 1e-3
    achieved = nbytes / kernel_s / 1e9
    traffic = _traffic("swa_ring_kernel", nbytes)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": "swa_ring_kernel", "kernel_mean_ms": st["mean_ms"],
                "algorithmic_bytes_per_launch": nbytes,
                "mfma_frac": flops / kernel_s / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    _log(f"prefill 32K: {st}  {value:.1f} TFLOP/s  {achieved:.0f} GB/s")
    del sets, x
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        extra = run_extra(dev, max(steps, 20), warmup)

    cpu = None
    if not args.no_cpu:
        _log("timing the fp64 oracle on the host cores")
        cpu = cpu_baseline()

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16, N(0,1) fp32 sinks)",
        "config": {"workload": PRIMARY, "tokens": 32768, "q_heads": 32, "kv_heads": 4,
                   "head_dim": 128, "window": 128, "sink": True, "lse": True},
        "mfma_peak_frac": value / BF16_MFMA_PEAK_TFLOPS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


def run_extra(dev, steps, warmup):
    """Decode / MTP verify (bf16 and FP8 rings), the GA layer, the hybrid block, the
    varlen prefill and a plain device copy (achievable-bandwidth ceiling)."""
    import torch

    from sliding_window_attention_amd import workloads as wl

    extra = {}
    # plain copy: read + write of 1 GiB
    a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).normal_()
    b = torch.empty_like(a)
    per, _ = _time_calls(lambda _: b.copy_(a), [None], 20, 3)
    extra["copy_ceiling_gbps"] = 2 * a.numel() * 2 / (min(per) * 1e-3) / 1e9
    del a, b

    _log("swa_prefill_fp8kv_32k")
    x = _with_outputs(_to(wl.make_workload("swa_prefill_fp8kv_32k"), dev), "prefill")
    sets = _clone_sets(x, 4)
    per, _ = _time_calls(_prefill_fp8_fn(128), sets, steps, warmup, per_call=False)
    fl, by = wl.workload_work("swa_prefill_fp8kv_32k")
    st = _stats(per)
    extra["swa_prefill_fp8kv_32k"] = {**st, "gbps": by / (st["mean_ms"] * 1e-3) / 1e9,
                                      "hbm_frac": by / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                      "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12, "bytes": by}
    del sets, x
    torch.cuda.empty_cache()

    for name in ("decode_t1", "decode_t4", "decode_fp8_t1", "decode_fp8_t4", "decode_rope_t1",
                 "decode_rope_t4", "decode_rope_fp8_t4"):
        _log(f"{name}")
        x = _with_outputs(_to(wl.make_workload(name), dev), "decode")
        sets = _clone_sets(x, 32)  # 32 x 38-86 MB: more than the Infinity Cache
        fn = {"decode_fp8": _decode_fp8_fn, "decode_rope": _decode_rope_fn,
              "decode_rope_fp8": _decode_rope_fp8_fn}.get(wl.WORKLOADS[name].kind, _decode_fn)()
        per, _ = _time_calls(fn, sets, max(200, steps), warmup, per_call=False)
        fl, by = wl.workload_work(name)
        st = _stats(per)
        extra[name] = {**st, "gbps": by / (st["mean_ms"] * 1e-3) / 1e9,
                       "hbm_frac": by / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12, "bytes": by}
        del sets, x
        torch.cuda.empty_cache()

    for fp8 in (False, True):
        ring = "an FP8" if fp8 else "a bf16"
        _log(f"MTP step: verify T = 4 with RoPE against {ring} ring, then commit the accepted tokens (B = 256)")
        xs = _mtp_sets(dev, fp8)
        x = xs[0]
        dec_fn = _decode_rope_fp8_fn() if fp8 else _decode_rope_fn()
        app_fn = _append_fn(fp8)

        def step(x_):
            dec_fn(x_)
            app_fn(x_)
        per, _ = _time_calls(step, xs, max(200, steps), warmup, per_call=False)
        st = _stats(per)
        fl, by_dec = wl.workload_work("decode_rope_fp8_t4" if fp8 else "decode_rope_t4")
        by = by_dec + wl.append_bytes(256, int(x["n_accept"].sum()), 4, 128, 2,
                                      cache_elem_bytes=1 if fp8 else None)
        what = ("swa_sink_decode_rope_fp8kv (T=4) + swa_ring_append_fp8kv per step" if fp8
                else "swa_sink_decode_rope (T=4) + swa_ring_append_rope per step")
        extra["mtp_step_rope_fp8_t4" if fp8 else "mtp_step_rope_t4"] = {
            **st, "gbps": by / (st["mean_ms"] * 1e-3) / 1e9, "bytes": by,
            "accepted_tokens": int(x["n_accept"].sum()), "what": what, "sets": len(xs)}
        del x, xs
        torch.cuda.empty_cache()
    for fp8 in (False, True):
        ring = "an FP8" if fp8 else "a bf16"
        _log(f"MTP step in one launch against {ring} ring: commit the previous step's accepted tokens, "
             "verify T = 4 (B = 256)")
        xs = _mtp_sets(dev, fp8)
        per, _ = _time_calls(_commit_fn(fp8), xs, max(200, steps), warmup, per_call=False)
        st = _stats(per)
        n_acc = int(xs[0]["n_accept"].sum())
        by = (wl.workload_work("decode_rope_fp8_t4" if fp8 else "decode_rope_t4")[1]
              + wl.mtp_commit_bytes(256, n_acc, 4, 128, 1 if fp8 else 2))
        name = "swa_sink_decode_rope_commit_fp8kv" if fp8 else "swa_sink_decode_rope_commit"
        extra["mtp_step_fused_rope_fp8_t4" if fp8 else "mtp_step_fused_rope_t4"] = {
            **st, "gbps": by / (st["mean_ms"] * 1e-3) / 1e9,
            "hbm_frac": by / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": by,
            "accepted_tokens": n_acc, "sets": len(xs),
            "what": f"{name} (commit prev_T = 4 accepted, verify T = 4) per step"}
        del xs
        torch.cuda.empty_cache()
    _log("sparse attention: top-k selection and sparse decode, 64 sequences of 16K-32K tokens")
    xs = _sparse_sets(dev, "topk")
    tb, sb, sfl = _sparse_work(xs[0])
    per, _ = _time_calls(_topk_fn(), xs, max(100, steps), warmup, per_call=False)
    st = _stats(per)
    extra["topk_select_b64"] = {**st, "gbps": tb / (st["mean_ms"] * 1e-3) / 1e9, "bytes": tb, "sets": len(xs)}
    del xs
    torch.cuda.empty_cache()
    xs = _sparse_sets(dev, "sparse")
    per, _ = _time_calls(_sparse_fn(), xs, max(100, steps), warmup, per_call=False)
    st = _stats(per)
    extra["sparse_decode_b64"] = {**st, "gbps": sb / (st["mean_ms"] * 1e-3) / 1e9,
                                  "hbm_frac": sb / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": sb,
                                  "tflops": sfl / (st["mean_ms"] * 1e-3) / 1e12, "sets": len(xs)}
    _log("sparse MTP verify: the newest two tokens of the same 64 sequences")
    per, _ = _time_calls(_sparse_mtp_fn(), xs, max(100, steps), warmup, per_call=False)
    st = _stats(per)
    mfl, mby = _sparse_mtp_work(xs[0])
    extra["sparse_decode_mtp_t2_b64"] = {**st, "gbps": mby / (st["mean_ms"] * 1e-3) / 1e9,
                                         "hbm_frac": mby / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                         "bytes": mby, "tflops": mfl / (st["mean_ms"] * 1e-3) / 1e12,
                                         "sets": len(xs)}
    _log("sparse decode and MTP verify over an FP8 cache (E4M3 codes) of the same shape")
    xs = _with_fp8_caches(xs)
    for t_new, name in ((1, "sparse_decode_fp8_b64"), (2, "sparse_decode_mtp_fp8_t2_b64")):
        per, _ = _time_calls(_sparse_fp8_fn(t_new), xs, max(100, steps), warmup, per_call=False)
        st = _stats(per)
        ffl, fby = _sparse_mtp_work(xs[0], t_new, 1)
        extra[name] = {**st, "gbps": fby / (st["mean_ms"] * 1e-3) / 1e9,
                       "hbm_frac": fby / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": fby,
                       "tflops": ffl / (st["mean_ms"] * 1e-3) / 1e12, "sets": len(xs)}
    del xs
    torch.cuda.empty_cache()

    _log("rope in place, Q of the 32K layer")
    xs = _rope_inputs(dev, 4)
    per, _ = _time_calls(_rope_fn(), xs, steps, warmup, per_call=False)
    st = _stats(per)
    by = wl.rope_bytes(32768, 32, 128, 2)
    extra["rope_q_32k"] = {**st, "gbps": by / (st["mean_ms"] * 1e-3) / 1e9,
                           "hbm_frac": by / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": by,
                           "sets": len(xs)}
    del xs
    torch.cuda.empty_cache()

    _log("hybrid_5to1_32k (5 SWA + 1 GA layers)")
    layers = []
    for layer in range(6):
        layers.append(_with_outputs(_to(wl.make_workload("hybrid_5to1_32k", layer), dev), "prefill"))
    swa_fn, ga_fn = _prefill_fn(128), _prefill_fn(None, ga=True)
    ga_steps, ga_warmup = 20, 3
    per_ga, _ = _time_calls(ga_fn, [layers[5]], ga_steps, ga_warmup)
    fl_swa = wl.prefill_flops([32768], 32, 128, 128)
    fl_ga = wl.prefill_flops([32768], 32, 128, None)
    by = wl.prefill_bytes(32768, 32, 4, 128, 2)
    st_ga = _stats(per_ga)
    extra["ga_32k"] = {**st_ga, "tflops": fl_ga / (st_ga["mean_ms"] * 1e-3) / 1e12,
                       "mfma_frac": fl_ga / (st_ga["mean_ms"] * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}

    def block(_):
        for li in range(5):
            swa_fn(layers[li])
        ga_fn(layers[5])
    per_blk, _ = _time_calls(block, [None], ga_steps, ga_warmup)
    per_swa, _ = _time_calls(swa_fn, layers[:5], 20, 3)
    st_blk = _stats(per_blk)
    extra["hybrid_block"] = {**st_blk, "tflops": (5 * fl_swa + fl_ga) / (st_blk["mean_ms"] * 1e-3) / 1e12,
                             "swa_layer_mean_ms": _stats(per_swa)["mean_ms"],
                             "swa_layer_gbps": by / (_stats(per_swa)["mean_ms"] * 1e-3) / 1e9}
    del layers
    torch.cuda.empty_cache()

    _log("backward of the 32K layer")
    x = _backward_inputs(dev)
    per, _ = _time_calls(_backward_fn(), [x], 20, 3, per_call=False)
    st = _stats(per)
    fl = wl.backward_flops([32768], 32, 128, 128)
    by = wl.backward_bytes(32768, 32, 4, 128, 2)
    by_out = wl.backward_bytes(32768, 32, 4, 128, 2, with_out=True)  # with the forward output read too
    extra["backward_32k"] = {**st, "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12,
                             "gbps": by / (st["mean_ms"] * 1e-3) / 1e9, "flops": fl, "bytes": by,
                             "bytes_with_out": by_out}
    del x
    torch.cuda.empty_cache()

    _log("varlen_262k")
    x = _with_outputs(_to(wl.make_workload("varlen_262k"), dev), "prefill")
    per, _ = _time_calls(_prefill_fn(128), [x], 20, 3)
    fl, by = wl.workload_work("varlen_262k")
    st = _stats(per)
    extra["varlen_262k"] = {**st, "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12,
                            "gbps": by / (st["mean_ms"] * 1e-3) / 1e9,
                            "lengths": wl.lognormal_lengths(262144, 8, wl.WORKLOADS["varlen_262k"].seed)}
    del x
    torch.cuda.empty_cache()
    return extra


if __name__ == "__main__":
    sys.exit(main())
