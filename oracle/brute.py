"""Brute-force enumeration of the SWA-with-sink operator (TEST INFRASTRUCTURE ONLY).

Pure-Python loops over (sequence, query, head, key) with math.fsum, for tiny inputs.
It states the operator of the MiMo-V2-Flash Technical Report digest, section 2.2.2
(sink term in the softmax denominator, no value attached to it) one query at a
time, with the 128-token causal window of section 2.2.1 generalised to `window`
(None = unbounded, as in the global-attention layers).  It exists only to pin
oracle.swa_oracle; it shares no code with it.
"""
from __future__ import annotations

import math


def _dot(x, y):
    return math.fsum(a * b for a, b in zip(x, y))


def attention(q, k, v, sinks, cu_seqlens, window, scale=None, return_weights=False):
    """q: nested lists [N][Hq][D]; k, v: [N][Hkv][D]; sinks: [Hq] or None.

    Returns o [N][Hq][D], lse [N][Hq] and, if asked, the per-row weights
    {(n, h): ([(j, p_j) ...], p_sink)} so that mass conservation can be checked.
    """
    n = len(q)
    hq = len(q[0])
    hkv = len(k[0])
    d = len(q[0][0])
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = [[[0.0] * d for _ in range(hq)] for _ in range(n)]
    lse = [[0.0] * hq for _ in range(n)]
    weights = {}
    for s in range(len(cu_seqlens) - 1):
        start, end = cu_seqlens[s], cu_seqlens[s + 1]
        for i in range(start, end):
            lo = start if window is None else max(start, i - window + 1)
            for h in range(hq):
                kvh = h // g
                logits = [(j, scale * _dot(q[i][h], k[j][kvh])) for j in range(lo, i + 1)]
                sink = -math.inf if sinks is None else float(sinks[h])
                m = max(max(a for _, a in logits), sink)
                ex = [(j, math.exp(a - m)) for j, a in logits]
                ex_sink = math.exp(sink - m) if sink != -math.inf else 0.0
                z = math.fsum([e for _, e in ex] + [ex_sink])
                for dd in range(d):
                    o[i][h][dd] = math.fsum(e * v[j][kvh][dd] for j, e in ex) / z
                lse[i][h] = m + math.log(z)
                if return_weights:
                    weights[(i, h)] = ([(j, e / z) for j, e in ex], ex_sink / z)
    if return_weights:
        return o, lse, weights
    return o, lse


def decode(q, k_new, v_new, k_cache, v_cache, ring_head, sinks, window, scale=None):
    """One query at a time against the ring: query t of sequence b sees logical
    cache slots t+1..W-1 (physical (head + l) mod W) and new tokens 0..t.

    q [B][T][Hq][D]; k_new/v_new [B][T][Hkv][D]; k_cache/v_cache [B][Hkv][W][D].
    """
    bsz = len(q)
    t_new = len(q[0])
    hq = len(q[0][0])
    d = len(q[0][0][0])
    hkv = len(k_new[0][0])
    g = hq // hkv
    w = window
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = [[[[0.0] * d for _ in range(hq)] for _ in range(t_new)] for _ in range(bsz)]
    lse = [[[0.0] * hq for _ in range(t_new)] for _ in range(bsz)]
    for b in range(bsz):
        for t in range(t_new):
            for h in range(hq):
                kvh = h // g
                keys = []  # (key vector, value vector)
                for slot in range(t + 1, w):
                    phys = (ring_head[b] + slot) % w
                    keys.append((k_cache[b][kvh][phys], v_cache[b][kvh][phys]))
                for u in range(t + 1):
                    keys.append((k_new[b][u][kvh], v_new[b][u][kvh]))
                logits = [scale * _dot(q[b][t][h], kk) for kk, _ in keys]
                sink = float(sinks[h])
                m = max(max(logits), sink)
                ex = [math.exp(a - m) for a in logits]
                z = math.fsum(ex + [math.exp(sink - m)])
                for dd in range(d):
                    o[b][t][h][dd] = math.fsum(e * vv[dd] for e, (_, vv) in zip(ex, keys)) / z
                lse[b][t][h] = m + math.log(z)
    return o, lse
