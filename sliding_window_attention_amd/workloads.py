"""Seeded synthetic workloads and closed-form work counters.

This module holds no attention arithmetic: it draws the input tensors (shared by
the GPU path and the CPU oracle so both see identical values) and counts the
algorithmic FLOPs and bytes used for roofline reporting.

Input recipe: every tensor is drawn in fp32 on the CPU from
``torch.Generator().manual_seed(seed)`` in the order Q, K, V, sinks, then
extras (ring heads, sequence lengths), values ~ N(0, 1); tensors of bf16
workloads are then rounded to bf16 (round-to-nearest-even).  Sinks stay fp32.
There is no dataset: the pages describe no public benchmark for this operator.

Shapes follow the pages: window 128 (MiMo-V2-Flash Technical Report digest,
section 2.2.1), GQA with 4 KV heads in SWA layers (ICML 2026 keynote write-up,
section 02), a 5:1 SWA:GA interleave (digest, section 2.2.1) and 1 + 3 MTP draft
tokens verified together (digest, section 2.3).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "prefill_fp8" | "decode" | "decode_fp8" | "decode_rope" | "sparse" | "hybrid" | "varlen"
    dtype: str  # "f32" | "bf16"
    seq_len: int = 0  # total packed tokens for prefill kinds
    num_q_heads: int = 32
    num_kv_heads: int = 4
    head_dim: int = 128
    window: int = 128
    batch: int = 0  # decode sequences
    t_new: int = 0  # decode query tokens per sequence
    num_seqs: int = 1  # varlen sequence count
    seed: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # Tiny fp32 SWA-sink forward; the oracle finishes in well under a second.
    "tiny_fp32": Workload("tiny_fp32", "prefill", "f32", seq_len=512, num_q_heads=4,
                          num_kv_heads=1, head_dim=64, seed=1000),
    # One SWA layer prefill at 32K tokens, 32 q / 4 kv heads, head_dim 128.
    "swa_prefill_32k": Workload("swa_prefill_32k", "prefill", "bf16", seq_len=32768, seed=2000),
    # The same layer with K and V as E4M3 codes (per-tensor scales).
    "swa_prefill_fp8kv_32k": Workload("swa_prefill_fp8kv_32k", "prefill_fp8", "bf16", seq_len=32768,
                                      seed=2100),
    # Batched ring-buffer decode, one query token per sequence.
    "decode_t1": Workload("decode_t1", "decode", "bf16", batch=256, t_new=1, seed=3000),
    # MTP verify: 1 + 3 draft tokens per sequence, causal among themselves.
    "decode_t4": Workload("decode_t4", "decode", "bf16", batch=256, t_new=4, seed=3100),
    # The same two decode workloads against an FP8 (E4M3) ring with per-tensor scales.
    "decode_fp8_t1": Workload("decode_fp8_t1", "decode_fp8", "bf16", batch=256, t_new=1, seed=3200),
    "decode_fp8_t4": Workload("decode_fp8_t4", "decode_fp8", "bf16", batch=256, t_new=4, seed=3300),
    # The same two decode workloads with unrotated q / new keys and positions (RoPE in
    # the kernel, SWA base 10,000), and the commit of the accepted tokens to the ring.
    "decode_rope_t1": Workload("decode_rope_t1", "decode_rope", "bf16", batch=256, t_new=1, seed=3400),
    "decode_rope_t4": Workload("decode_rope_t4", "decode_rope", "bf16", batch=256, t_new=4, seed=3500),
    # The MTP verify with RoPE in the kernel against an FP8 ring, and its commit.
    "decode_rope_fp8_t4": Workload("decode_rope_fp8_t4", "decode_rope_fp8", "bf16", batch=256, t_new=4,
                                   seed=3550),
    # Sparse decode (HySparse2 selection: top 1024 + the recent 128) for 64 sequences of
    # 16K-32K cached tokens over a [64, 4, 32768, 128] cache; the scores stand for the
    # full-attention layer's (no sink in the sparse layers).
    "sparse_b64": Workload("sparse_b64", "sparse", "bf16", seq_len=32768, batch=64, t_new=1, seed=6000,
                           extra={"topk": 1024, "recent": 128, "min_len": 16384}),
    # Hybrid block: 5 SWA-sink layers (seeds 4000..4004) + 1 GA layer (seed 4005).
    "hybrid_5to1_32k": Workload("hybrid_5to1_32k", "hybrid", "bf16", seq_len=32768, seed=4000),
    # Packed varlen prefill: 8 log-normal sequence lengths summing to 262144.
    "varlen_262k": Workload("varlen_262k", "varlen", "bf16", seq_len=262144, num_seqs=8,
                            seed=5000),
}


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def lognormal_lengths(total: int, num_seqs: int, seed: int, sigma: float = 1.0) -> list[int]:
    """Sequence lengths x_s ~ LogNormal(0, sigma) rescaled to sum to `total`.

    floor(x_s / sum(x) * total), the remainder handed out by largest fractional
    part, every length at least 1.
    """
    rng = np.random.default_rng(seed)
    x = rng.lognormal(mean=0.0, sigma=sigma, size=num_seqs)
    raw = x / x.sum() * total
    lens = np.floor(raw).astype(np.int64)
    lens = np.maximum(lens, 1)
    rem = int(total - lens.sum())
    order = np.argsort(-(raw - np.floor(raw)), kind="stable")
    i = 0
    while rem != 0:
        j = order[i % num_seqs]
        if rem > 0:
            lens[j] += 1
            rem -= 1
        elif lens[j] > 1:
            lens[j] -= 1
            rem += 1
        i += 1
    return [int(v) for v in lens]


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_prefill(seq_lens, num_q_heads, num_kv_heads, head_dim, dtype, seed, with_sinks=True):
    """Packed prefill inputs: q [N, Hq, D], k/v [N, Hkv, D], sinks [Hq] fp32 (or None),
    cu_seqlens [S+1] int32.  All on the CPU."""
    lens = [int(x) for x in seq_lens]
    n = sum(lens)
    gen = torch.Generator().manual_seed(int(seed))
    td = _torch_dtype(dtype)
    q = torch.randn(n, num_q_heads, head_dim, generator=gen).to(td)
    k = torch.randn(n, num_kv_heads, head_dim, generator=gen).to(td)
    v = torch.randn(n, num_kv_heads, head_dim, generator=gen).to(td)
    sinks = torch.randn(num_q_heads, generator=gen) if with_sinks else None
    return {"q": q, "k": k, "v": v, "sinks": sinks, "cu_seqlens": cu_from_lengths(lens),
            "max_seqlen": max(lens) if lens else 0, "lengths": lens}


def make_decode(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed):
    """Decode inputs: q [B, T, Hq, D], k_new/v_new [B, T, Hkv, D], full caches
    [B, Hkv, W, D], ring_head [B] int32 ~ U[0, W), sinks [Hq] fp32.  CPU tensors."""
    gen = torch.Generator().manual_seed(int(seed))
    td = _torch_dtype(dtype)
    q = torch.randn(batch, t_new, num_q_heads, head_dim, generator=gen).to(td)
    k_new = torch.randn(batch, t_new, num_kv_heads, head_dim, generator=gen).to(td)
    v_new = torch.randn(batch, t_new, num_kv_heads, head_dim, generator=gen).to(td)
    sinks = torch.randn(num_q_heads, generator=gen)
    k_cache = torch.randn(batch, num_kv_heads, window, head_dim, generator=gen).to(td)
    v_cache = torch.randn(batch, num_kv_heads, window, head_dim, generator=gen).to(td)
    ring_head = torch.randint(0, window, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    return {"q": q, "k_new": k_new, "v_new": v_new, "k_cache": k_cache, "v_cache": v_cache,
            "ring_head": ring_head, "sinks": sinks}


def make_decode_rope(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed,
                     max_position=1 << 20):
    """make_decode plus positions [B] int32 ~ U[window, max_position): the position of
    each sequence's new token 0 (q and k_new are then read as unrotated; the ring's
    values stand for keys rotated at their own positions).  Drawn after the decode
    tensors from the same generator."""
    x = make_decode(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed)
    gen = torch.Generator().manual_seed(int(seed) + 1)
    x["positions"] = torch.randint(window, max_position, (batch,), generator=gen,
                                   dtype=torch.int64).to(torch.int32)
    return x


def make_sparse(batch, num_q_heads, num_kv_heads, head_dim, max_len, dtype, seed, min_len=1,
                with_sinks=True):
    """Sparse-decode inputs: q [B, Hq, D] (the newest token of each sequence), caches
    [B, Hkv, Lmax, D], lengths [B] int32 ~ U[min_len, max_len], sinks [Hq] fp32 (or None)
    and the full-attention layer's scores [B, Hkv, Lmax] fp32 ~ N(0, 1).  CPU tensors."""
    gen = torch.Generator().manual_seed(int(seed))
    td = _torch_dtype(dtype)
    q = torch.randn(batch, num_q_heads, head_dim, generator=gen).to(td)
    k_cache = torch.randn(batch, num_kv_heads, max_len, head_dim, generator=gen).to(td)
    v_cache = torch.randn(batch, num_kv_heads, max_len, head_dim, generator=gen).to(td)
    sinks = torch.randn(num_q_heads, generator=gen)
    scores = torch.randn(batch, num_kv_heads, max_len, generator=gen)
    lengths = torch.randint(min_len, max_len + 1, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    return {"q": q, "k_cache": k_cache, "v_cache": v_cache, "lengths": lengths,
            "sinks": sinks if with_sinks else None, "scores": scores}


def make_sparse_fp8(batch, num_q_heads, num_kv_heads, head_dim, max_len, dtype, seed, min_len=1,
                    with_sinks=True):
    """make_sparse with the caches as E4M3 codes [B, Hkv, Lmax, D] uint8 and per-tensor
    scales k_scale = 1/32, v_scale = 1/64 (values of about N(0, 1))."""
    x = make_sparse(batch, num_q_heads, num_kv_heads, head_dim, max_len, dtype, seed, min_len, with_sinks)
    gen = torch.Generator().manual_seed(int(seed) + 17)
    shape = tuple(x["k_cache"].shape)
    x["k_cache"] = e4m3_codes(shape, gen)
    x["v_cache"] = e4m3_codes(shape, gen)
    x["k_scale"], x["v_scale"] = 1.0 / 32, 1.0 / 64
    return x


def make_sparse_device(batch, num_q_heads, num_kv_heads, head_dim, max_len, seed, device, min_len=1):
    """make_sparse for caches too large to draw on the host (bf16, no sinks): q, caches
    and scores drawn on `device` by a seeded device generator, lengths on the host."""
    gen = torch.Generator(device=device).manual_seed(int(seed))
    hgen = torch.Generator().manual_seed(int(seed) + 1)
    q = _randn_device((batch, num_q_heads, head_dim), gen, device, torch.bfloat16)
    kc = _randn_device((batch * num_kv_heads * max_len, head_dim), gen, device, torch.bfloat16)
    vc = _randn_device((batch * num_kv_heads * max_len, head_dim), gen, device, torch.bfloat16)
    scores = torch.randn((batch, num_kv_heads, max_len), generator=gen, device=device)
    lengths = torch.randint(min_len, max_len + 1, (batch,), generator=hgen, dtype=torch.int64).to(torch.int32)
    return {"q": q, "k_cache": kc.view(batch, num_kv_heads, max_len, head_dim),
            "v_cache": vc.view(batch, num_kv_heads, max_len, head_dim), "lengths": lengths,
            "sinks": None, "scores": scores}


def sparse_bytes(lengths, num_q_heads, num_kv_heads, head_dim, topk, recent, elem_bytes, kv_elem_bytes=None):
    """Sparse decode: per (sequence, KV head) the selected and recent K and V rows read
    once, the query read and the output written, the selection (indices, counts) and
    the LSE.  kv_elem_bytes: bytes per cache element (1 for E4M3 codes; default
    elem_bytes)."""
    keys = sum(min(topk, max(0, int(n) - recent)) + min(recent, int(n)) for n in lengths)
    b = len(lengths)
    kvb = elem_bytes if kv_elem_bytes is None else kv_elem_bytes
    return (2 * keys * num_kv_heads * head_dim * kvb + 2 * b * num_q_heads * head_dim * elem_bytes
            + b * num_kv_heads * (topk + 1) * 4 + 4 * b * num_q_heads)


def sparse_mtp_work(lengths, indices, counts, num_q_heads, num_kv_heads, head_dim, recent, t_new, elem_bytes,
                    kv_elem_bytes=None):
    """(flops, bytes) of the sparse MTP verify of the newest t_new tokens: 4 D FLOPs per
    (query head, visible key) -- query t sees the selected positions below its window and
    the window -- and per (sequence, KV head) the selection plus the windows' union read
    once as K and V rows, the queries read, the outputs and LSE written, the selection.
    kv_elem_bytes: bytes per cache element (1 for E4M3 codes; default elem_bytes)."""
    import numpy as np

    idx = np.asarray(indices)
    cnt = np.asarray(counts)
    grp = num_q_heads // num_kv_heads
    visible = rows = 0
    for b, n in enumerate(lengths):
        n = max(int(n), t_new)
        for g in range(num_kv_heads):
            sel = idx[b, g, :cnt[b, g]]
            rows += len(sel) + min(recent + t_new - 1, n)
            for t in range(t_new):
                p = n - t_new + t
                lo = max(0, p - recent + 1)
                visible += grp * (int((sel < lo).sum()) + p - lo + 1)
    bsz = len(lengths)
    kvb = elem_bytes if kv_elem_bytes is None else kv_elem_bytes
    by = (2 * rows * head_dim * kvb + 2 * bsz * t_new * num_q_heads * head_dim * elem_bytes
          + 4 * int(cnt.size) + 4 * int(cnt.sum()) + 4 * bsz * t_new * num_q_heads)
    return 4 * head_dim * visible, by


def sparse_flops(lengths, num_q_heads, head_dim, topk, recent):
    """4 D FLOPs per (query head, key) over the selected and recent keys."""
    keys = sum(min(topk, max(0, int(n) - recent)) + min(recent, int(n)) for n in lengths)
    return 4 * head_dim * num_q_heads * keys


def topk_bytes(lengths, num_kv_heads, topk, recent):
    """Selection: every candidate score read once, indices and counts written."""
    cand = sum(max(0, int(n) - recent) for n in lengths)
    return 4 * num_kv_heads * cand + len(lengths) * num_kv_heads * (topk + 1) * 4


def _randn_device(shape, gen, device, dtype, chunk_rows=1 << 18):
    """N(0, 1) rounded to `dtype`, drawn on `device` a slab of rows at a time (so
    that no fp32 copy of a multi-GB tensor is ever held)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device).to(dtype)
    return out


def make_prefill_device(seq_lens, num_q_heads, num_kv_heads, head_dim, seed, device):
    """make_prefill for streams too large to draw on the host: bf16 q/k/v drawn on
    `device` by a seeded device generator (different values from make_prefill for
    the same seed), fp32 sinks and int32 cu_seqlens on the host."""
    lens = [int(x) for x in seq_lens]
    n = sum(lens)
    gen = torch.Generator(device=device).manual_seed(int(seed))
    q = _randn_device((n, num_q_heads, head_dim), gen, device, torch.bfloat16)
    k = _randn_device((n, num_kv_heads, head_dim), gen, device, torch.bfloat16)
    v = _randn_device((n, num_kv_heads, head_dim), gen, device, torch.bfloat16)
    sinks = torch.randn(num_q_heads, generator=torch.Generator().manual_seed(int(seed)))
    return {"q": q, "k": k, "v": v, "sinks": sinks, "cu_seqlens": cu_from_lengths(lens),
            "max_seqlen": max(lens), "lengths": lens}


def make_decode_device(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, seed, device):
    """make_decode with bf16 tensors drawn on `device` (for batches whose caches
    are too large to draw on the host); ring heads and sinks on the host."""
    gen = torch.Generator(device=device).manual_seed(int(seed))
    hgen = torch.Generator().manual_seed(int(seed))
    bf = torch.bfloat16
    return {"q": _randn_device((batch, t_new, num_q_heads, head_dim), gen, device, bf),
            "k_new": _randn_device((batch, t_new, num_kv_heads, head_dim), gen, device, bf),
            "v_new": _randn_device((batch, t_new, num_kv_heads, head_dim), gen, device, bf),
            "k_cache": _randn_device((batch, num_kv_heads, window, head_dim), gen, device, bf, 4096),
            "v_cache": _randn_device((batch, num_kv_heads, window, head_dim), gen, device, bf, 4096),
            "ring_head": torch.randint(0, window, (batch,), generator=hgen, dtype=torch.int64).to(torch.int32),
            "sinks": torch.randn(num_q_heads, generator=hgen)}


def e4m3_codes(shape, gen, exp_center=10.0, exp_spread=2.0):
    """One-byte E4M3 codes shaped like a quantised N(0, s) tensor: random sign,
    exponent field ~ round(N(exp_center, exp_spread)) clipped to 1..14 (normal
    numbers, never the NaN pattern), uniform mantissa.  uint8, on the generator's
    device."""
    dev = gen.device
    e = torch.clamp(torch.round(exp_center + exp_spread * torch.randn(shape, generator=gen, device=dev)), 1, 14)
    m = torch.randint(0, 8, shape, generator=gen, device=dev)
    sgn = torch.randint(0, 2, shape, generator=gen, device=dev)
    return ((sgn << 7) | (e.to(torch.int64) << 3) | m).to(torch.uint8)


def make_prefill_fp8(seq_lens, num_q_heads, num_kv_heads, head_dim, dtype, seed, with_sinks=True):
    """make_prefill with K and V as E4M3 codes [N, Hkv, D] uint8 and per-tensor scales
    k_scale = 1/32, v_scale = 1/64 (values of about N(0, 1))."""
    x = make_prefill(seq_lens, num_q_heads, num_kv_heads, head_dim, dtype, seed, with_sinks)
    gen = torch.Generator().manual_seed(int(seed) + 17)
    shape = tuple(x["k"].shape)
    x["k"] = e4m3_codes(shape, gen)
    x["v"] = e4m3_codes(shape, gen)
    x["k_scale"], x["v_scale"] = 1.0 / 32, 1.0 / 64
    return x


def make_decode_fp8(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed):
    """make_decode with the caches as E4M3 codes [B, Hkv, W, D] uint8 and per-tensor
    scales: k_scale = 1/32 and v_scale = 1/64 bring the values to about N(0, 1)."""
    x = make_decode(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed)
    gen = torch.Generator().manual_seed(int(seed) + 17)
    shape = (batch, num_kv_heads, window, head_dim)
    x["k_cache"] = e4m3_codes(shape, gen)
    x["v_cache"] = e4m3_codes(shape, gen)
    x["k_scale"], x["v_scale"] = 1.0 / 32, 1.0 / 64
    return x


def make_decode_rope_fp8(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed):
    """make_decode_rope with the caches as E4M3 codes (make_decode_fp8's codes and
    scales, drawn from the same seeds)."""
    x = make_decode_rope(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed)
    y = make_decode_fp8(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, dtype, seed)
    for k in ("k_cache", "v_cache", "k_scale", "v_scale"):
        x[k] = y[k]
    return x


def make_workload(name: str, layer: int = 0):
    """Inputs of a named workload (for 'hybrid_5to1_32k', layer 0..4 are SWA, 5 is GA)."""
    w = WORKLOADS[name]
    if w.kind == "prefill":
        return make_prefill([w.seq_len], w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.seed)
    if w.kind == "prefill_fp8":
        return make_prefill_fp8([w.seq_len], w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.seed)
    if w.kind == "hybrid":
        return make_prefill([w.seq_len], w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype,
                            w.seed + layer, with_sinks=layer < 5)
    if w.kind == "varlen":
        lens = lognormal_lengths(w.seq_len, w.num_seqs, w.seed)
        return make_prefill(lens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.seed)
    if w.kind == "decode":
        return make_decode(w.batch, w.t_new, w.num_q_heads, w.num_kv_heads, w.head_dim, w.window,
                           w.dtype, w.seed)
    if w.kind == "decode_fp8":
        return make_decode_fp8(w.batch, w.t_new, w.num_q_heads, w.num_kv_heads, w.head_dim,
                               w.window, w.dtype, w.seed)
    if w.kind == "decode_rope":
        return make_decode_rope(w.batch, w.t_new, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                w.window, w.dtype, w.seed)
    if w.kind == "decode_rope_fp8":
        return make_decode_rope_fp8(w.batch, w.t_new, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    w.window, w.dtype, w.seed)
    raise KeyError(name)


# ---------------------------------------------------------------------------
# Closed-form work counters (algorithmic work only: masked tile work never counts)
# ---------------------------------------------------------------------------

def pairs(length: int, window) -> int:
    """Unmasked (query, key) pairs of one causal sequence of `length` tokens with
    a window of `window` keys (None = unbounded)."""
    n = int(length)
    if window is None or n <= window:
        return n * (n + 1) // 2
    w = int(window)
    return w * (w + 1) // 2 + w * (n - w)


def prefill_flops(lengths, num_q_heads, head_dim, window) -> int:
    """QK^T plus PV: 4 * D FLOPs per unmasked (query, key) pair per query head."""
    return 4 * head_dim * num_q_heads * sum(pairs(n, window) for n in lengths)


def prefill_bytes(total_tokens, num_q_heads, num_kv_heads, head_dim, elem_bytes, with_lse=True,
                  kv_elem_bytes=None):
    """Q, K, V read once, O written once, LSE (fp32) written once.  kv_elem_bytes: K/V
    element size when it differs from the rest (1 for E4M3 codes)."""
    kb = elem_bytes if kv_elem_bytes is None else kv_elem_bytes
    per_tok = 2 * num_q_heads * head_dim * elem_bytes + 2 * num_kv_heads * head_dim * kb
    if with_lse:
        per_tok += 4 * num_q_heads
    return total_tokens * per_tok


def backward_flops(lengths, num_q_heads, head_dim, window) -> int:
    """Gradients of O: per visible (query, key) pair and head, the recomputed logits,
    dO . v, and the dv, dk and dq products: 5 contractions of 2 * head_dim."""
    return 10 * head_dim * num_q_heads * sum(pairs(l, window) for l in lengths)


def backward_bytes(total_tokens, num_q_heads, num_kv_heads, head_dim, elem_bytes, with_out=False):
    """q, dout, dq ([N, Hq, D]); k, v, dk, dv ([N, Hkv, D]); the fp32 LSE: each read or
    written once.  The forward output `out` is counted only with with_out: the matrix-core
    backward forms delta_i = dout_i . O_i as sum_j p_ij (dout_i . v_j) from the weights it
    recomputes and does not read it."""
    nq = (4 if with_out else 3) * total_tokens * num_q_heads * head_dim * elem_bytes
    return nq + 4 * total_tokens * num_kv_heads * head_dim * elem_bytes + 4 * total_tokens * num_q_heads


def decode_flops(batch, t_new, num_q_heads, head_dim, window) -> int:
    """Every query row sees exactly `window` keys (W-1-t ring slots + t+1 new)."""
    return 4 * head_dim * num_q_heads * batch * t_new * window


def decode_bytes(batch, t_new, num_q_heads, num_kv_heads, head_dim, window, elem_bytes,
                 with_lse=True, cache_elem_bytes=None):
    """Live ring slots (W-1: the oldest slot is outside every query's window),
    the T new K/V rows, Q and O; LSE fp32.  cache_elem_bytes: ring element size
    when it differs from the rest (1 for an FP8 ring)."""
    cb = elem_bytes if cache_elem_bytes is None else cache_elem_bytes
    kv = 2 * batch * num_kv_heads * head_dim * (cb * (window - 1) + elem_bytes * t_new)
    qo = 2 * batch * t_new * num_q_heads * head_dim * elem_bytes
    lse = 4 * batch * t_new * num_q_heads if with_lse else 0
    return kv + qo + lse


def append_bytes(batch, n_accepted_total, num_kv_heads, head_dim, elem_bytes, cache_elem_bytes=None):
    """Ring append: the accepted tokens' K and V read once and written once (in the
    ring's element size: 1 for an FP8 ring), plus the accept counts, positions and heads
    (read, heads written)."""
    cb = elem_bytes if cache_elem_bytes is None else cache_elem_bytes
    return 2 * n_accepted_total * num_kv_heads * head_dim * (elem_bytes + cb) + 4 * 4 * batch


def mtp_commit_bytes(batch, n_accepted_total, num_kv_heads, head_dim, elem_bytes):
    """What the one-launch MTP step adds to the verify's bytes: the committed tokens' K and
    V written to the ring in its element size (elem_bytes: 2 for bf16, 1 for E4M3), the
    previous step's rows they come from standing in for the ring slots they fill (so the
    reads are the verify's), plus the accept counts, previous positions and heads (two
    heads: read and written)."""
    return 2 * n_accepted_total * num_kv_heads * head_dim * elem_bytes + 4 * 4 * batch


def rope_bytes(rows, heads, head_dim, elem_bytes):
    """In-place rotation: every element read and written once, plus one int32 position per row."""
    return 2 * rows * heads * head_dim * elem_bytes + 4 * rows


def workload_work(name: str):
    """(flops, bytes) of one pass of a named workload as its kind defines it."""
    w = WORKLOADS[name]
    eb = 4 if w.dtype == "f32" else 2
    if w.kind in ("decode", "decode_fp8", "decode_rope", "decode_rope_fp8"):
        return (decode_flops(w.batch, w.t_new, w.num_q_heads, w.head_dim, w.window),
                decode_bytes(w.batch, w.t_new, w.num_q_heads, w.num_kv_heads, w.head_dim,
                             w.window, eb, cache_elem_bytes=1 if "fp8" in w.kind else None))
    if w.kind == "varlen":
        lens = lognormal_lengths(w.seq_len, w.num_seqs, w.seed)
    else:
        lens = [w.seq_len]
    fl = prefill_flops(lens, w.num_q_heads, w.head_dim, w.window)
    by = prefill_bytes(sum(lens), w.num_q_heads, w.num_kv_heads, w.head_dim, eb,
                       kv_elem_bytes=1 if w.kind == "prefill_fp8" else None)
    if w.kind == "hybrid":
        ga = prefill_flops(lens, w.num_q_heads, w.head_dim, None)
        return 5 * fl + ga, 6 * by
    return fl, by
