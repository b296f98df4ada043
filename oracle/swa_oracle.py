"""fp64 numpy oracle for SWA-with-sink, global causal attention and ring-buffer decode.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  Every public function is pinned
by tests/test_oracle.py or tests/test_golden.py against something other than itself
(closed forms, library routines, brute force, hand-worked fixtures, invariants),
including the row-sampled evaluation (prefill_sample_rows: against the full oracle on
every row of multi-sequence streams with empty sequences, and brute force) and the
FP8 decode with RoPE (brute-force ring enumeration over hand-decoded codes with
distinct K and V scales, and exponent-shift identities of the two scales).

The operator (MiMo-V2-Flash Technical Report digest, section 2.2.2; the formula
block there lost its symbols in extraction, so the reading below is rebuilt from
the prose of that section and of the MiMo-V2 blog, section 2.2):

  for query row i of head h, with key set J(i) = the last W keys of the same
  sequence up to and including i (section 2.2.1: window of 128 tokens),
      a_j  = scale * <q_i, k_j>                        (scaled logits)
      m    = max(max_j a_j, sink_h)                    (stabilising max)
      Z    = exp(sink_h - m) + sum_j exp(a_j - m)      (sink in the denominator)
      o_i  = sum_j exp(a_j - m) v_j / Z                (the sink has no value)
      lse  = m + ln Z
  The sink is one learnable scalar per query head, compared with the scaled
  logits (it is not multiplied by the scale).  Global-attention layers use the
  same operator with an unbounded window and no sink (sink = -inf).
  GQA: query head h reads KV head h // (Hq // Hkv).

Decode against an FP8 ring (swa_sink_decode_fp8kv) is the same decode on caches
dequantised exactly (E4M3 code value times a per-tensor scale); the prefill with FP8
K/V (swa_sink_prefill_fp8kv) is likewise the prefill on dequantised K and V, and
the decode with RoPE against an FP8 ring (swa_sink_decode_rope_fp8kv) the decode with
RoPE on dequantised caches.  The append into an FP8 ring (swa_ring_append_fp8kv) stores E4M3 codes of element / scale,
rounded once to the nearest E4M3 value with ties to the even mantissa, saturating at
448 (e4m3_encode: the pages name the format, not the rounding, so this is the
plainest reading of a rounding conversion).

RoPE around decode (swa_rope, swa_sink_decode_rope, swa_ring_append_rope, and the MTP
step swa_sink_decode_rope_commit, which is the append followed by the decode, with
swa_sink_decode_rope_commit_fp8kv its FP8-ring form): the
rotary position embedding with a per-layer base (10,000 in SWA layers, 640,000 in
GA layers, raised to 5,000,000 for the 256K stage: MiMo-V2-Flash Technical Report
digest, section 3.1; the positions keep increasing as the window slides, ICML 2026
keynote write-up, section 06).  The pages give neither the pairing nor the
frequencies; the reading here is the common rotate-half form (element i pairs with
i + D/2, inverse frequency base^(-2i/D), angle = position times frequency), and
rotated vectors are rounded to the I/O type, as a separate rotation pass that
stores its result would.

Token-level sparse attention with a forced recent window (topk_select,
sparse_decode): the HySparse2 selection of the MiMo-V3 / HySparse2 report (page on
the MiMo-V3 news, HySparse2 sections): the full-attention layer's scores pick the top
k tokens (1024 there) and the most recent 128 tokens are always kept, the sparse
layers attending to that set over the shared KV cache (sparse_decode_mtp: the newest
T tokens as queries, each with its own recent window; sparse_decode_mtp_fp8kv: over a
cache of E4M3 codes).  Readings where the pages are
silent: the scores arrive per (sequence, KV head) over the cached positions; the top
k are taken among the tokens older than the recent window (larger score first, the
lower position on equal scores) and returned in increasing position; the query (the
newest token) attends to those plus the recent window, with the sink of the other
layers when one is given.

Arithmetic is fp64 on the exact input values (bf16, fp32 and E4M3 convert to fp64
exactly).  Rows are processed in blocks only to bound memory: every row is the
definition above, computed independently, with no online rescaling and no
reordering of its sums beyond numpy's own.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _as_f64(x) -> np.ndarray:
    """Exact fp64 copy of a numpy array or a CPU torch tensor (bf16/fp32/fp64)."""
    if hasattr(x, "detach"):  # torch tensor; imported lazily so numpy users need no torch
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _attend_rows(qr, keys, vals, q_pos, k_pos, seq_start, window, sink, scale):
    """The definition for a set of query rows of ONE head against candidate keys.

    qr [R, D] query vectors; keys/vals [J, D]; q_pos [R] and k_pos [J] are positions
    in one packed stream; seq_start [R] is the first position of each row's
    sequence; window is an int >= 1 or None (unbounded); sink is a float or -inf.
    Returns o [R, D], lse [R].
    """
    a = scale * (qr @ keys.T)  # [R, J] scaled logits
    valid = (k_pos[None, :] <= q_pos[:, None]) & (k_pos[None, :] >= seq_start[:, None])
    if window is not None:
        valid &= k_pos[None, :] >= q_pos[:, None] - window + 1
    a = np.where(valid, a, NEG_INF)
    m = np.maximum(a.max(axis=1), sink)
    e = np.exp(a - m[:, None])  # exp(-inf) == 0 for masked keys
    z = np.exp(sink - m) + e.sum(axis=1)
    o = (e @ vals) / z[:, None]
    lse = m + np.log(z)
    return o, lse


def _check_common(q, k, v, cu_seqlens):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [tokens, heads, head_dim]")
    n, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != n or k.shape[2] != d:
        raise ValueError("k and v must be [tokens, kv_heads, head_dim] matching q")
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != n or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to total_tokens")
    return n, hq, hkv, d, cu


def _prefill(q, k, v, sinks, cu_seqlens, window, scale, block):
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    n, hq, hkv, d, cu = _check_common(q, k, v, cu_seqlens)
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sink = np.full(hq, NEG_INF) if sinks is None else _as_f64(sinks).reshape(hq)
    o = np.zeros((n, hq, d))
    lse = np.zeros((n, hq))
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        for i0 in range(c0, c1, block):
            i1 = min(i0 + block, c1)
            k0 = c0 if window is None else max(c0, i0 - window + 1)
            q_pos = np.arange(i0, i1)
            k_pos = np.arange(k0, i1)
            start = np.full(i1 - i0, c0)
            for h in range(hq):
                kvh = h // g
                oo, ll = _attend_rows(q[i0:i1, h], k[k0:i1, kvh], v[k0:i1, kvh],
                                      q_pos, k_pos, start, window, sink[h], scale)
                o[i0:i1, h] = oo
                lse[i0:i1, h] = ll
    return o, lse


def _grad_rows(qr, keys, vals, q_pos, k_pos, seq_start, window, sink, scale, do_r):
    """Gradients of the definition for query rows of ONE head (see swa_sink_prefill_backward).

    Returns (dq [R, D], dk [J, D], dv [J, D], dsink scalar) for these rows; dk and dv
    are this head's contributions to the candidate keys.
    """
    a = scale * (qr @ keys.T)
    valid = (k_pos[None, :] <= q_pos[:, None]) & (k_pos[None, :] >= seq_start[:, None])
    if window is not None:
        valid &= k_pos[None, :] > q_pos[:, None] - window
    a = np.where(valid, a, NEG_INF)
    m = np.maximum(a.max(axis=1), sink)
    z = np.exp(sink - m) + np.exp(a - m[:, None]).sum(axis=1)
    lse = m + np.log(z)
    p = np.exp(a - lse[:, None])            # softmax weights of the keys (sink excluded)
    p_sink = np.exp(sink - lse)             # the sink's weight
    o = p @ vals
    delta = (do_r * o).sum(axis=1)          # dO . O
    dp = do_r @ vals.T                      # dO . v_j
    da = p * (dp - delta[:, None])          # gradient of the scaled logits
    dq = scale * (da @ keys)
    dk = scale * (da.T @ qr)
    dv = p.T @ do_r
    dsink = -(p_sink * delta).sum()
    return dq, dk, dv, dsink


def swa_sink_prefill_backward(q, k, v, sinks, cu_seqlens, dout, window=128, scale=None,
                              block=128):
    """Gradients of swa_sink_prefill's output O with respect to q, k, v and the sinks.

    For row i of head h with weights p_ij = exp(a_ij - lse_i) and sink weight
    p_s = exp(sink_h - lse_i) (p_s + sum_j p_ij = 1), O_i = sum_j p_ij v_j, so
        dv_j += p_ij dO_i,   delta_i = dO_i . O_i,   da_ij = p_ij (dO_i . v_j - delta_i),
        dq_i = scale sum_j da_ij k_j,   dk_j += scale da_ij q_i,
        dsink_h = -sum_i p_s(i) delta_i     (the sink carries no value: dO_i . (0 - O_i) p_s),
    sums over every row and, for dk and dv, over the query heads sharing a KV head.
    The sink is the learnable scalar of the technical report digest, section 2.2.2,
    whose training stability the ICML keynote's Q&A (section 06) singles out; window=None
    gives the GA layers (no sink).  Returns (dq [N, Hq, D], dk, dv [N, Hkv, D],
    dsinks [Hq]) in fp64; LSE is not an input of the loss here.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    n, hq, hkv, d, cu = _check_common(q, k, v, cu_seqlens)
    if do.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sink = np.full(hq, NEG_INF) if sinks is None else _as_f64(sinks).reshape(hq)
    w = None if window is None else int(window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = np.zeros(hq)
    for s in range(len(cu) - 1):
        c0, c1 = int(cu[s]), int(cu[s + 1])
        for i0 in range(c0, c1, block):
            i1 = min(i0 + block, c1)
            k0 = c0 if w is None else max(c0, i0 - w + 1)
            q_pos = np.arange(i0, i1)
            k_pos = np.arange(k0, i1)
            start = np.full(i1 - i0, c0)
            for h in range(hq):
                kvh = h // g
                dqr, dkr, dvr, dsr = _grad_rows(q[i0:i1, h], k[k0:i1, kvh], v[k0:i1, kvh], q_pos,
                                                k_pos, start, w, sink[h], scale, do[i0:i1, h])
                dq[i0:i1, h] = dqr
                dk[k0:i1, kvh] += dkr
                dv[k0:i1, kvh] += dvr
                dsink[h] += dsr
    return dq, dk, dv, dsink


def swa_sink_prefill(q, k, v, sinks, cu_seqlens, window=128, scale=None, block=128):
    """Causal GQA sliding-window attention with a per-head sink over packed sequences.

    q [N, Hq, D], k/v [N, Hkv, D], sinks [Hq], cu_seqlens [S+1] (0 .. N).  Keys of
    row i are the last `window` positions of its own sequence up to i.  Returns
    (o [N, Hq, D], lse [N, Hq]) in fp64.  Follows the operator of the technical
    report digest, section 2.2.2, with the window of section 2.2.1.
    """
    if window is None or int(window) < 1:
        raise ValueError("window must be an integer >= 1")
    return _prefill(q, k, v, sinks, cu_seqlens, int(window), scale, block)


def ga_causal_prefill(q, k, v, cu_seqlens, scale=None, block=128):
    """Global-attention layer: the same operator with no window and no sink
    (technical report digest, section 2.2: GA layers interleaved 1 per 5 SWA)."""
    return _prefill(q, k, v, None, cu_seqlens, None, scale, block)


def prefill_sample_rows(q, k, v, sinks, cu_seqlens, rows, window=128, scale=None):
    """The definition evaluated only at the (token, head) pairs in `rows`.

    For checks at sizes where the full fp64 output is too large.  window=None
    means unbounded (GA); sinks=None means no sink.  Returns (o [R, D], lse [R]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    n, hq, hkv, d, cu = _check_common(q, k, v, cu_seqlens)
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sink = np.full(hq, NEG_INF) if sinks is None else _as_f64(sinks).reshape(hq)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, (t, h) in enumerate(rows):
        s = int(np.searchsorted(cu, t, side="right")) - 1
        c0 = int(cu[s])
        k0 = c0 if window is None else max(c0, int(t) - int(window) + 1)
        kvh = int(h) // g
        oo, ll = _attend_rows(q[t:t + 1, h], k[k0:t + 1, kvh], v[k0:t + 1, kvh],
                              np.array([t]), np.arange(k0, t + 1), np.array([c0]),
                              window, sink[h], scale)
        o[r], lse[r] = oo[0], ll[0]
    return o, lse


def ring_logical_order(cache_b, head, window):
    """Cache of one sequence [Hkv, W, D] reordered so logical slot l is first-to-last.

    Logical slot l (0 = oldest cached token) lives at physical slot (head + l) mod W.
    """
    idx = (int(head) + np.arange(window)) % window
    return cache_b[:, idx, :]


def swa_sink_decode(q, k_new, v_new, k_cache, v_cache, ring_head, sinks, window=128,
                    scale=None):
    """Decode / MTP verify against a W-slot ring buffer per (sequence, KV head).

    q [B, T, Hq, D]; k_new/v_new [B, T, Hkv, D] are the T new tokens (the current
    one and T-1 drafts), not yet in the ring; k_cache/v_cache [B, Hkv, W, D];
    ring_head [B] is the physical slot of the oldest cached token.  Each sequence
    is the prefill definition applied to [ring in logical order] ++ [new tokens]
    with the same window and sinks; the T new rows are returned.  Query t thus
    sees cache slots t+1..W-1 and new tokens 0..t (drafts causal among
    themselves).  The MTP drafts verified in one pass follow the technical report
    digest, section 2.3.  Returns (o [B, T, Hq, D], lse [B, T, Hq]).
    """
    q, k_new, v_new = _as_f64(q), _as_f64(k_new), _as_f64(v_new)
    k_cache, v_cache = _as_f64(k_cache), _as_f64(v_cache)
    bsz, t_new, hq, d = q.shape
    hkv = k_new.shape[2]
    w = int(window)
    if k_cache.shape[2] != w:
        raise ValueError("cache slot count must equal the window")
    heads = np.asarray(_as_f64(ring_head), dtype=np.int64).reshape(bsz)
    o = np.zeros((bsz, t_new, hq, d))
    lse = np.zeros((bsz, t_new, hq))
    for b in range(bsz):
        ks = np.concatenate([ring_logical_order(k_cache[b], heads[b], w).transpose(1, 0, 2),
                             k_new[b]], axis=0)  # [W+T, Hkv, D]
        vs = np.concatenate([ring_logical_order(v_cache[b], heads[b], w).transpose(1, 0, 2),
                             v_new[b]], axis=0)
        qs = np.zeros((w + t_new, hq, d))
        qs[w:] = q[b]
        ob, lb = _prefill(qs, ks, vs, sinks, [0, w + t_new], w, scale, block=w + t_new)
        o[b] = ob[w:]
        lse[b] = lb[w:]
    return o, lse


def e4m3_to_float(codes) -> np.ndarray:
    """Exact fp64 value of one-byte E4M3 codes (the FP8 (E4M3) format the MiMo-V2
    blog, section 6, names for MiMo-V2.5-Pro; the bit layout is the OCP 8-bit
    floating-point one): sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
    2..0.  Exponent field 0 holds the subnormals m/8 * 2^-6; otherwise the value is
    (1 + m/8) * 2^(e - 7).  There are no infinities: S.1111.111 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def e4m3_encode(x, scale=1.0) -> np.ndarray:
    """E4M3 codes (uint8) of x / scale, with scale an fp32 value.

    Rounding follows the usual reading of a rounding conversion: the exact quotient
    goes to the nearest E4M3 value; on a tie, to the neighbour whose code has mantissa
    LSB 0 (round half to even).  Finite magnitudes beyond the largest finite value 448
    saturate to it, the sign of zero is kept, and an x that is not finite becomes the
    NaN code S.1111.111 with x's sign.  The quotient is formed in fp64: x here has at
    most 24 significant bits and so has the scale, so a quotient that is not exactly
    halfway between two E4M3 values differs from every such point by far more than
    fp64's rounding, and the nearest value found from the fp64 quotient is the one of
    the exact quotient.  The nearest value is looked up in the table of all E4M3
    values (e4m3_to_float of codes 0..126).
    """
    x = np.asarray(x, dtype=np.float64)
    s = float(np.float32(scale))
    if not (np.isfinite(s) and s > 0):
        raise ValueError("scale must be finite and > 0")
    table = e4m3_to_float(np.arange(127))           # 0, 2^-9, ..., 448, increasing
    sign = np.signbit(x)
    with np.errstate(invalid="ignore", over="ignore"):
        a = np.abs(x) / s
    finite = np.isfinite(a)
    a = np.where(finite, np.minimum(a, table[-1]), 0.0)
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, 126)    # table[hi-1] < a <= table[hi]
    lo = hi - 1
    d_lo, d_hi = a - table[lo], table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    code = np.where(finite, code, 0x7F)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def swa_sink_decode_fp8kv(q, k_new, v_new, k_codes, v_codes, k_scale, v_scale, ring_head, sinks,
                          window=128, scale=None):
    """Decode / MTP verify against a ring whose K and V are stored as E4M3 codes.

    The FP8 KV cache of the MiMo-V3 / HySparse2 report (cache sizes quoted "with an
    FP8 cache") with one fp32 scale per tensor: cache element value = the code's
    E4M3 value times k_scale (K) or v_scale (V).  The T new tokens keep their own
    precision.  Everything else is swa_sink_decode on the dequantised caches.
    """
    kc = e4m3_to_float(k_codes) * float(k_scale)
    vc = e4m3_to_float(v_codes) * float(v_scale)
    return swa_sink_decode(q, k_new, v_new, kc, vc, ring_head, sinks, window=window, scale=scale)


def swa_sink_prefill_fp8kv(q, k_codes, v_codes, k_scale, v_scale, sinks, cu_seqlens, window=128,
                           scale=None, block=128):
    """Prefill whose K and V are stored as E4M3 codes (the same FP8 KV format and
    per-tensor scales as swa_sink_decode_fp8kv): key / value element = the code's E4M3
    value times k_scale / v_scale.  sinks=None means no sink and window=None an
    unbounded window (the GA layer).  Everything else is the prefill operator on the
    dequantised K and V.
    """
    k = e4m3_to_float(k_codes) * float(k_scale)
    v = e4m3_to_float(v_codes) * float(v_scale)
    if window is None and sinks is None:
        return ga_causal_prefill(q, k, v, cu_seqlens, scale, block)
    return _prefill(q, k, v, sinks, cu_seqlens, None if window is None else int(window), scale, block)


def rope(x, positions, base):
    """Rotary position embedding of x [R, H, D] (or [R, D]) with row r at integer
    position positions[r], in fp64: for i < D/2, angle = positions[r] * base^(-2i/D),
        y[i]       = x[i] cos(angle) - x[i + D/2] sin(angle)
        y[i + D/2] = x[i + D/2] cos(angle) + x[i] sin(angle).
    """
    x = _as_f64(x)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("head_dim must be even")
    half = d // 2
    inv_freq = float(base) ** (-2.0 * np.arange(half) / d)                 # [D/2]
    ang = np.asarray(positions, dtype=np.float64).reshape(-1)[:, None] * inv_freq[None, :]  # [R, D/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, s_ = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s_, x2 * c + x1 * s_], axis=-1)


def round_to(x, io_dtype):
    """Round fp64 values to the I/O type ("bf16": round to nearest even through
    torch's conversion; "f32": numpy's float32 cast; None: no rounding)."""
    x = np.asarray(x, dtype=np.float64)
    if io_dtype is None:
        return x
    if io_dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    import torch

    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


def swa_sink_decode_rope(q, k_new, v_new, k_cache, v_cache, ring_head, positions, sinks, rope_base,
                         window=128, scale=None, io_dtype="bf16"):
    """Decode / MTP verify with the rotary embedding applied to the query tokens and
    the new keys first.  q [B, T, Hq, D] and k_new [B, T, Hkv, D] arrive unrotated;
    new token t of sequence b sits at position positions[b] + t.  The ring holds
    keys already rotated at their own positions.  Rotated q and k_new are rounded to
    io_dtype, then this is swa_sink_decode."""
    q, k_new = _as_f64(q), _as_f64(k_new)
    bsz, t_new = q.shape[:2]
    pos = np.asarray(positions, dtype=np.int64).reshape(bsz)[:, None] + np.arange(t_new)[None, :]
    qr = round_to(rope(q.reshape((bsz * t_new,) + q.shape[2:]), pos.reshape(-1), rope_base), io_dtype)
    kr = round_to(rope(k_new.reshape((bsz * t_new,) + k_new.shape[2:]), pos.reshape(-1), rope_base),
                  io_dtype)
    return swa_sink_decode(qr.reshape(q.shape), kr.reshape(k_new.shape), v_new, k_cache, v_cache,
                           ring_head, sinks, window=window, scale=scale)


def swa_sink_decode_rope_fp8kv(q, k_new, v_new, k_codes, v_codes, k_scale, v_scale, ring_head, positions,
                               sinks, rope_base, window=128, scale=None, io_dtype="bf16"):
    """swa_sink_decode_rope against an FP8 ring: the caches dequantised exactly (E4M3
    code value times the per-tensor scale), then the decode with q and the new keys
    rotated at their positions and rounded to io_dtype."""
    kc = e4m3_to_float(k_codes) * float(k_scale)
    vc = e4m3_to_float(v_codes) * float(v_scale)
    return swa_sink_decode_rope(q, k_new, v_new, kc, vc, ring_head, positions, sinks, rope_base,
                                window=window, scale=scale, io_dtype=io_dtype)


def swa_ring_append_rope(k_new, v_new, n_accept, positions, k_cache, v_cache, ring_head, rope_base,
                         io_dtype="bf16"):
    """Commit the first n_accept[b] of the T new tokens of each sequence to its ring
    (the accepted MTP tokens; rejected drafts never enter the cache).  Appending n
    tokens evicts the n oldest: accepted token t goes to physical slot
    (ring_head[b] + t) mod W, its key rotated at position positions[b] + t and
    rounded to io_dtype, its value copied; the head then advances by n.  With
    rope_base None the keys are copied unrotated.  Returns (k_cache, v_cache,
    ring_head) as new arrays."""
    k_new, v_new = _as_f64(k_new), _as_f64(v_new)
    kc, vc = _as_f64(k_cache).copy(), _as_f64(v_cache).copy()
    bsz, t_new = k_new.shape[:2]
    w = kc.shape[2]
    heads = np.asarray(_as_f64(ring_head), dtype=np.int64).reshape(bsz) % w
    n_acc = np.asarray(n_accept, dtype=np.int64).reshape(bsz)
    pos = np.asarray(positions, dtype=np.int64).reshape(bsz)
    new_heads = heads.copy()
    for b in range(bsz):
        n = int(n_acc[b])
        if n < 0 or n > t_new:
            raise ValueError("n_accept out of range")
        if n == 0:
            continue
        if rope_base is None:
            kr = k_new[b, :n]
        else:
            kr = round_to(rope(k_new[b, :n], pos[b] + np.arange(n), rope_base), io_dtype)  # [n, Hkv, D]
        for t in range(n):
            slot = (heads[b] + t) % w
            kc[b, :, slot, :] = kr[t]
            vc[b, :, slot, :] = v_new[b, t]
        new_heads[b] = (heads[b] + n) % w
    return kc, vc, new_heads


def swa_sink_decode_rope_commit(q, k_new, v_new, positions, prev_k, prev_v, prev_accept, prev_positions,
                                k_cache, v_cache, ring_head, sinks, rope_base, window=128, scale=None,
                                io_dtype="bf16"):
    """One MTP step (technical report digest, section 2.3): the previous step's accepted
    tokens enter the ring, then the step's T tokens are verified against the ring so
    updated.  The commit is swa_ring_append_rope of the first prev_accept[b] (clamped to
    [0, prev_T]) of prev_k / prev_v at prev_positions[b] + t; the verify is
    swa_sink_decode_rope of q / k_new / v_new at positions[b] + t.  Returns (out, lse,
    k_cache, v_cache, ring_head) with the caches and head after the commit."""
    prev_k = _as_f64(prev_k)
    n = np.clip(np.asarray(prev_accept, dtype=np.int64).reshape(-1), 0, prev_k.shape[1])
    kc, vc, heads = swa_ring_append_rope(prev_k, prev_v, n, prev_positions, k_cache, v_cache, ring_head,
                                         rope_base, io_dtype=io_dtype)
    out, lse = swa_sink_decode_rope(q, k_new, v_new, kc, vc, heads, positions, sinks, rope_base,
                                    window=window, scale=scale, io_dtype=io_dtype)
    return out, lse, kc, vc, heads


def swa_ring_append_fp8kv(k_new, v_new, n_accept, positions, k_codes, v_codes, ring_head, rope_base,
                          k_scale, v_scale, io_dtype="bf16"):
    """swa_ring_append_rope into an FP8 ring: each committed element -- the key rotated
    at its position and rounded to io_dtype, or the value as given -- enters the ring as
    its E4M3 code of element / k_scale (keys) or element / v_scale (values)
    (e4m3_encode).  k_codes / v_codes [B, Hkv, W, D] uint8; returns (k_codes, v_codes,
    ring_head) as new arrays."""
    k_new, v_new = _as_f64(k_new), _as_f64(v_new)
    kc = np.asarray(k_codes, dtype=np.uint8).copy()
    vc = np.asarray(v_codes, dtype=np.uint8).copy()
    bsz, t_new = k_new.shape[:2]
    w = kc.shape[2]
    heads = np.asarray(ring_head, dtype=np.int64).reshape(bsz) % w
    n_acc = np.asarray(n_accept, dtype=np.int64).reshape(bsz)
    pos = None if rope_base is None else np.asarray(positions, dtype=np.int64).reshape(bsz)
    new_heads = heads.copy()
    for b in range(bsz):
        n = int(n_acc[b])
        if n < 0 or n > t_new:
            raise ValueError("n_accept out of range")
        if n == 0:
            continue
        if rope_base is None:
            kr = k_new[b, :n]
        else:
            kr = round_to(rope(k_new[b, :n], pos[b] + np.arange(n), rope_base), io_dtype)
        kq = e4m3_encode(kr, k_scale)
        vq = e4m3_encode(v_new[b, :n], v_scale)
        for t in range(n):
            slot = (heads[b] + t) % w
            kc[b, :, slot, :] = kq[t]
            vc[b, :, slot, :] = vq[t]
        new_heads[b] = (heads[b] + n) % w
    return kc, vc, new_heads


def swa_sink_decode_rope_commit_fp8kv(q, k_new, v_new, positions, prev_k, prev_v, prev_accept, prev_positions,
                                      k_codes, v_codes, k_scale, v_scale, ring_head, sinks, rope_base, window=128,
                                      scale=None, io_dtype="bf16"):
    """swa_sink_decode_rope_commit against an FP8 ring: swa_ring_append_fp8kv of the first
    prev_accept[b] (clamped to [0, prev_T]) previous tokens, then swa_sink_decode_rope_fp8kv
    of the new ones on the ring so updated.  Returns (out, lse, k_codes, v_codes, ring_head)."""
    prev_k = _as_f64(prev_k)
    n = np.clip(np.asarray(prev_accept, dtype=np.int64).reshape(-1), 0, prev_k.shape[1])
    kc, vc, heads = swa_ring_append_fp8kv(prev_k, prev_v, n, prev_positions, k_codes, v_codes, ring_head,
                                          rope_base, k_scale, v_scale, io_dtype=io_dtype)
    out, lse = swa_sink_decode_rope_fp8kv(q, k_new, v_new, kc, vc, k_scale, v_scale, heads, positions, sinks,
                                          rope_base, window=window, scale=scale, io_dtype=io_dtype)
    return out, lse, kc, vc, heads


def sparse_decode_mtp(q, k_cache, v_cache, lengths, indices, counts, sinks, recent=128, scale=None):
    """MTP verify in a sparse layer: the newest T tokens of each sequence (positions
    p_t = L-T+t, t < T, all in the cache) are queries.  Query t attends the selected
    positions older than its own recent window, indices[b, g, :counts[b, g]] below
    p_t-recent+1, plus that window max(0, p_t-recent+1) .. p_t -- with T = 1 this is
    sparse_decode.  q [B, T, Hq, D]; caches [B, Hkv, Lmax, D]; sinks [Hq] or None.
    Returns (o [B, T, Hq, D], lse [B, T, Hq])."""
    q, kc, vc = _as_f64(q), _as_f64(k_cache), _as_f64(v_cache)
    bsz, t_new, hq, d = q.shape
    hkv = kc.shape[1]
    grp = hq // hkv
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lens = np.asarray(lengths, dtype=np.int64).reshape(bsz)
    idx = np.asarray(indices, dtype=np.int64)
    cnt = np.asarray(counts, dtype=np.int64)
    o = np.zeros((bsz, t_new, hq, d))
    lse = np.zeros((bsz, t_new, hq))
    for b in range(bsz):
        L = int(lens[b])
        for t in range(t_new):
            p = L - t_new + t
            lo = max(0, p - recent + 1)
            for h in range(hq):
                g = h // grp
                sel = idx[b, g, :cnt[b, g]]
                keys = np.concatenate([sel[sel < lo], np.arange(lo, p + 1)])
                a = sc * (kc[b, g, keys] @ q[b, t, h])
                sink = NEG_INF if sinks is None else float(_as_f64(sinks)[h])
                m = max(a.max(), sink)
                e = np.exp(a - m)
                z = e.sum() + (np.exp(sink - m) if sink != NEG_INF else 0.0)
                o[b, t, h] = (e @ vc[b, g, keys]) / z
                lse[b, t, h] = m + np.log(z)
    return o, lse


def sparse_decode_mtp_fp8kv(q, k_codes, v_codes, k_scale, v_scale, lengths, indices, counts, sinks, recent=128,
                            scale=None):
    """sparse_decode_mtp over a cache of E4M3 codes with per-tensor scales: the caches
    dequantised exactly (code value times k_scale / v_scale).  k_codes / v_codes
    [B, Hkv, Lmax, D] uint8; T = 1 is the single-token sparse decode."""
    kc = e4m3_to_float(k_codes) * float(k_scale)
    vc = e4m3_to_float(v_codes) * float(v_scale)
    return sparse_decode_mtp(q, kc, vc, lengths, indices, counts, sinks, recent=recent, scale=scale)


def topk_select(scores, lengths, k=1024, recent=128):
    """Token selection for the sparse layers.  scores [B, Hkv, Lmax] (finite floats);
    lengths [B]: sequence b holds positions 0 .. lengths[b]-1 (the newest, the query's,
    last).  Candidates are the positions older than the recent window, j < lengths[b] -
    recent; the min(k, #candidates) with the largest scores are chosen, equal scores
    broken towards the lower position.  Returns (indices [B, Hkv, k] int64 in increasing
    position, padded with -1; counts [B, Hkv] int64)."""
    sc = _as_f64(scores)
    bsz, hkv, _ = sc.shape
    lens = np.asarray(lengths, dtype=np.int64).reshape(bsz)
    idx = np.full((bsz, hkv, k), -1, dtype=np.int64)
    cnt = np.zeros((bsz, hkv), dtype=np.int64)
    for b in range(bsz):
        ncand = max(0, int(lens[b]) - recent)
        for h in range(hkv):
            cand = np.arange(ncand)
            order = np.lexsort((cand, -sc[b, h, :ncand]))  # score descending, then position
            chosen = np.sort(cand[order[:k]])
            idx[b, h, :len(chosen)] = chosen
            cnt[b, h] = len(chosen)
    return idx, cnt


def sparse_decode(q, k_cache, v_cache, lengths, indices, counts, sinks, recent=128, scale=None):
    """One query token per sequence (the newest, at position lengths[b]-1) over the
    selected older positions indices[b, g, :counts[b, g]] of its KV head g plus the
    recent window max(0, L-recent) .. L-1.  q [B, Hq, D]; caches [B, Hkv, Lmax, D]
    (token t of sequence b at [b, :, t]); sinks [Hq] or None.  Every query head reads its
    group's selection.  Returns (o [B, Hq, D], lse [B, Hq])."""
    q, kc, vc = _as_f64(q), _as_f64(k_cache), _as_f64(v_cache)
    bsz, hq, d = q.shape
    hkv = kc.shape[1]
    grp = hq // hkv
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lens = np.asarray(lengths, dtype=np.int64).reshape(bsz)
    idx = np.asarray(indices, dtype=np.int64)
    cnt = np.asarray(counts, dtype=np.int64)
    o = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for b in range(bsz):
        L = int(lens[b])
        rec = np.arange(max(0, L - recent), L)
        for h in range(hq):
            g = h // grp
            keys = np.concatenate([idx[b, g, :cnt[b, g]], rec])
            a = sc * (kc[b, g, keys] @ q[b, h])
            sink = NEG_INF if sinks is None else float(_as_f64(sinks)[h])
            m = max(a.max(), sink)
            e = np.exp(a - m)
            z = e.sum() + (np.exp(sink - m) if sink != NEG_INF else 0.0)
            o[b, h] = (e @ vc[b, g, keys]) / z
            lse[b, h] = m + np.log(z)
    return o, lse
