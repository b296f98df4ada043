"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties oracle.swa_oracle to something other than itself: a library routine
(torch's scaled_dot_product_attention / logsumexp in fp64 on the CPU), a closed
form, an invariant, or brute-force enumeration (oracle.brute).  The operator is
the one of the MiMo-V2-Flash Technical Report digest, section 2.2.2 (learnable
sink term in the softmax denominator), with the causal 128-token window of
section 2.2.1 and GQA (ICML 2026 keynote write-up, section 02).
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import brute
from oracle import swa_oracle as orc
from sliding_window_attention_amd import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _inputs(lens, hq, hkv, d, seed, sink_scale=1.0):
    rng = np.random.default_rng(seed)
    n = sum(lens)
    q = _rand((n, hq, d), rng)
    k = _rand((n, hkv, d), rng)
    v = _rand((n, hkv, d), rng)
    sinks = sink_scale * _rand((hq,), rng)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, sinks, cu


def _sdpa_reference(q, k, v, lens, window, scale):
    """torch SDPA (fp64, CPU) with an explicit boolean band mask per sequence; no sink."""
    hq, hkv = q.shape[1], k.shape[1]
    outs, lses = [], []
    c0 = 0
    for n in lens:
        qs = torch.from_numpy(q[c0:c0 + n]).permute(1, 0, 2)  # [Hq, n, D]
        ks = torch.from_numpy(k[c0:c0 + n]).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
        vs = torch.from_numpy(v[c0:c0 + n]).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
        i = torch.arange(n)[:, None]
        j = torch.arange(n)[None, :]
        mask = j <= i
        if window is not None:
            mask &= j >= i - window + 1
        o = torch.nn.functional.scaled_dot_product_attention(
            qs.unsqueeze(0), ks.unsqueeze(0), vs.unsqueeze(0), attn_mask=mask, scale=scale)[0]
        logits = scale * (qs @ ks.transpose(1, 2))
        logits = logits.masked_fill(~mask, float("-inf"))
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(torch.logsumexp(logits, dim=-1).permute(1, 0).numpy())
        c0 += n
    return np.concatenate(outs), np.concatenate(lses)


# ---- pin 1: sink -> -inf is ordinary causal-window softmax attention -------------

@pytest.mark.parametrize("lens,window", [([37], 5), ([64, 3, 30], 16), ([50], 1), ([20, 20], 128)])
def test_pin1_no_sink_equals_library_sdpa(lens, window):
    q, k, v, _, cu = _inputs(lens, 4, 2, 8, seed=1)
    sinks = np.full(4, -np.inf)
    o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, window, block=7)
    o_ref, lse_ref = _sdpa_reference(q, k, v, lens, window, 1 / math.sqrt(8))
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


# ---- pin 2: W >= L is full causal attention; GA equals library causal SDPA --------

def test_pin2_large_window_is_global_and_ga_is_causal_sdpa():
    lens = [33, 17]
    q, k, v, _, cu = _inputs(lens, 4, 4, 16, seed=2)
    ga_o, ga_l = orc.ga_causal_prefill(q, k, v, cu)
    sw_o, sw_l = orc.swa_sink_prefill(q, k, v, np.full(4, -np.inf), cu, window=max(lens))
    np.testing.assert_allclose(sw_o, ga_o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(sw_l, ga_l, atol=1e-12, rtol=0)
    o_ref, l_ref = _sdpa_reference(q, k, v, lens, None, 0.25)
    np.testing.assert_allclose(ga_o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(ga_l, l_ref, atol=1e-12, rtol=0)


# ---- pin 3: a large sink drives outputs to 0 and lse to the sink -----------------

def test_pin3_large_sink_drives_output_to_zero():
    lens = [40]
    q, k, v, _, cu = _inputs(lens, 2, 1, 8, seed=3)
    sinks = np.array([50.0, 60.0])
    o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, 16)
    a_max = np.abs(q).sum(-1).max() * np.abs(k).max() / math.sqrt(8)  # crude logit bound
    bound = math.exp(a_max - 50.0) * 16 * np.abs(v).max()
    assert np.abs(o).max() < max(bound, 1e-15)
    assert np.abs(o).max() < 1e-12
    np.testing.assert_allclose(lse[:, 0], 50.0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 1], 60.0, atol=1e-12)


# ---- pin 4: brute-force enumeration equals the vectorised oracle ------------------

@settings(max_examples=40, deadline=None)
@given(
    lens=st.lists(st.integers(1, 9), min_size=1, max_size=3),
    d=st.integers(1, 6),
    g=st.sampled_from([1, 2, 4]),
    hkv=st.integers(1, 2),
    window=st.sampled_from([1, 2, 3, 5, None]),
    sink_mode=st.sampled_from(["normal", "none", "big"]),
    seed=st.integers(0, 10_000),
)
def test_pin4_brute_force_matches_oracle(lens, d, g, hkv, window, sink_mode, seed):
    hq = g * hkv
    q, k, v, sinks, cu = _inputs(lens, hq, hkv, d, seed, sink_scale=3.0)
    if sink_mode == "none":
        sinks = None
    elif sink_mode == "big":
        sinks = sinks + 20.0
    if window is None and sinks is None:
        o, lse = orc.ga_causal_prefill(q, k, v, cu, block=4)
    else:
        o, lse = orc.swa_sink_prefill(q, k, v, np.full(hq, -np.inf) if sinks is None else sinks,
                                      cu, 10_000 if window is None else window, block=4)
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                             None if sinks is None else sinks.tolist(), cu.tolist(), window)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-13, rtol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-13, rtol=1e-13)


# ---- pin 5: closed form at W = 1 (and for the first row at any W) ----------------

def test_pin5_window_one_closed_form():
    lens = [12, 5]
    q, k, v, sinks, cu = _inputs(lens, 4, 2, 8, seed=5)
    o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, 1)
    g = 2
    for n in range(sum(lens)):
        for h in range(4):
            a = float(q[n, h] @ k[n, h // g]) / math.sqrt(8)
            sig = 1.0 / (1.0 + math.exp(-(a - sinks[h])))
            np.testing.assert_allclose(o[n, h], sig * v[n, h // g], atol=1e-14, rtol=1e-13)
            np.testing.assert_allclose(lse[n, h], np.logaddexp(a, sinks[h]), atol=1e-13)
    o128, l128 = orc.swa_sink_prefill(q, k, v, sinks, cu, 128)
    for c0 in cu[:-1]:  # row 0 of every sequence sees only itself at any window
        np.testing.assert_allclose(o128[c0], o[c0], atol=1e-14)
        np.testing.assert_allclose(l128[c0], lse[c0], atol=1e-14)


# ---- pin 6: exact sink identity against plain (sink-free) attention -------------

@pytest.mark.parametrize("window", [1, 4, 128])
def test_pin6_sink_identity(window):
    lens = [30, 9]
    q, k, v, sinks, cu = _inputs(lens, 4, 1, 8, seed=6, sink_scale=2.0)
    o_s, l_s = orc.swa_sink_prefill(q, k, v, sinks, cu, window)
    o_0, l_0 = orc.swa_sink_prefill(q, k, v, np.full(4, -np.inf), cu, window)
    factor = 1.0 / (1.0 + np.exp(sinks[None, :] - l_0))  # sigmoid(lse0 - sink)
    np.testing.assert_allclose(o_s, o_0 * factor[..., None], atol=1e-13, rtol=1e-12)
    np.testing.assert_allclose(l_s, np.logaddexp(l_0, sinks[None, :]), atol=1e-13)


# ---- pin 7: mass conservation -----------------------------------------------------

def test_pin7_mass_conservation():
    lens = [11, 6]
    q, k, v, sinks, cu = _inputs(lens, 2, 1, 4, seed=7)
    window = 4
    _, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, window)
    _, _, weights = brute.attention(q.tolist(), k.tolist(), v.tolist(), sinks.tolist(),
                                    cu.tolist(), window, return_weights=True)
    for (n, h), (pk, ps) in weights.items():
        assert math.isclose(math.fsum([p for _, p in pk] + [ps]), 1.0, abs_tol=1e-14)
        # the oracle's lse normalises the same weights
        s = next(i for i in range(len(cu) - 1) if cu[i] <= n < cu[i + 1])
        lo = max(cu[s], n - window + 1)
        a = [float(q[n, h] @ k[j, 0]) / 2.0 for j in range(lo, n + 1)]
        tot = math.fsum([math.exp(x - lse[n, h]) for x in a] + [math.exp(sinks[h] - lse[n, h])])
        assert math.isclose(tot, 1.0, abs_tol=1e-13)


# ---- pin 8: constant V gives o = c * (1 - p_sink) --------------------------------

def test_pin8_constant_values():
    lens = [25]
    q, k, v, sinks, cu = _inputs(lens, 4, 2, 8, seed=8)
    c = np.linspace(-2, 3, 8)
    v[:] = c
    o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, 6)
    expect = c[None, None, :] * (1.0 - np.exp(sinks[None, :] - lse))[..., None]
    np.testing.assert_allclose(o, expect, atol=1e-14, rtol=1e-13)


# ---- pin 9: decode == prefill on [ring in logical order ++ new]; brute; rotation ---

def _decode_inputs(b, t, hq, hkv, w, d, seed):
    rng = np.random.default_rng(seed)
    return dict(q=_rand((b, t, hq, d), rng), k_new=_rand((b, t, hkv, d), rng),
                v_new=_rand((b, t, hkv, d), rng), k_cache=_rand((b, hkv, w, d), rng),
                v_cache=_rand((b, hkv, w, d), rng), ring_head=rng.integers(0, w, b),
                sinks=_rand((hq,), rng))


@pytest.mark.parametrize("t", [1, 2, 4])
def test_pin9_decode_brute_and_prefill_equivalence(t):
    w, d = 6, 4
    x = _decode_inputs(3, t, 4, 2, w, d, seed=9 + t)
    o, lse = orc.swa_sink_decode(**x, window=w)
    ob, lb = brute.decode(x["q"].tolist(), x["k_new"].tolist(), x["v_new"].tolist(),
                          x["k_cache"].tolist(), x["v_cache"].tolist(), x["ring_head"].tolist(),
                          x["sinks"].tolist(), w)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-13, rtol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-13)
    # prefill of the concatenated stream, built here by explicit slot arithmetic
    for b in range(3):
        order = [(x["ring_head"][b] + l) % w for l in range(w)]
        ks = np.concatenate([x["k_cache"][b][:, order].transpose(1, 0, 2), x["k_new"][b]])
        vs = np.concatenate([x["v_cache"][b][:, order].transpose(1, 0, 2), x["v_new"][b]])
        qs = np.concatenate([np.zeros((w, 4, d)), x["q"][b]])
        op, lp = orc.swa_sink_prefill(qs, ks, vs, x["sinks"], [0, w + t], w)
        np.testing.assert_allclose(o[b], op[w:], atol=1e-13)
        np.testing.assert_allclose(lse[b], lp[w:], atol=1e-13)


def test_pin9_ring_rotation_invariance():
    w = 8
    x = _decode_inputs(4, 3, 2, 1, w, 4, seed=90)
    o, lse = orc.swa_sink_decode(**x, window=w)
    for s in (1, 3, 7):
        y = dict(x)
        y["k_cache"] = np.roll(x["k_cache"], s, axis=2)
        y["v_cache"] = np.roll(x["v_cache"], s, axis=2)
        y["ring_head"] = (x["ring_head"] + s) % w
        o2, l2 = orc.swa_sink_decode(**y, window=w)
        np.testing.assert_allclose(o2, o, atol=1e-14)
        np.testing.assert_allclose(l2, lse, atol=1e-14)


def test_pin9_oldest_slot_is_never_read():
    w = 5
    x = _decode_inputs(2, 2, 2, 1, w, 4, seed=91)
    o, _ = orc.swa_sink_decode(**x, window=w)
    y = {kk: np.array(vv, copy=True) for kk, vv in x.items()}
    for b in range(2):
        y["k_cache"][b, :, y["ring_head"][b]] = 1e6
        y["v_cache"][b, :, y["ring_head"][b]] = -1e6
    o2, _ = orc.swa_sink_decode(**y, window=w)
    np.testing.assert_allclose(o2, o, atol=1e-14)


# ---- pin 10: GQA equals MHA with K, V repeated along heads -----------------------

def test_pin10_gqa_equals_repeated_mha():
    lens = [21, 8]
    q, k, v, sinks, cu = _inputs(lens, 8, 2, 8, seed=10)
    o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, 5)
    o2, l2 = orc.swa_sink_prefill(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), sinks, cu, 5)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, l2, atol=1e-14)
    # a head reads KV head h // G: changing KV head 1 must leave heads 0..3 untouched
    k3 = k.copy()
    k3[:, 1] += 1.0
    o3, _ = orc.swa_sink_prefill(q, k3, v, sinks, cu, 5)
    np.testing.assert_allclose(o3[:, :4], o[:, :4], atol=0)
    assert np.abs(o3[:, 4:] - o[:, 4:]).max() > 1e-6


# ---- pin 11: varlen == independent sequences; packing order does not matter --------

def test_pin11_varlen_independence_and_order():
    lens = [13, 1, 40, 7]
    q, k, v, sinks, cu = _inputs(lens, 4, 2, 8, seed=11)
    o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, 16)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        os_, ls_ = orc.swa_sink_prefill(q[a:b], k[a:b], v[a:b], sinks, [0, b - a], 16)
        np.testing.assert_allclose(o[a:b], os_, atol=1e-14)
        np.testing.assert_allclose(lse[a:b], ls_, atol=1e-14)
    perm = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in perm])
    cu_p = np.concatenate([[0], np.cumsum([lens[s] for s in perm])])
    o_p, l_p = orc.swa_sink_prefill(q[idx], k[idx], v[idx], sinks, cu_p, 16)
    np.testing.assert_allclose(o_p, o[idx], atol=1e-14)
    np.testing.assert_allclose(l_p, lse[idx], atol=1e-14)


# ---- pin 12: the unmasked-pair counter equals the mask it counts -----------------

@pytest.mark.parametrize("n,w", [(1, 128), (5, 128), (128, 128), (129, 128), (1000, 128),
                                 (37, 1), (37, 5), (64, None)])
def test_pin12_pair_count(n, w):
    count = 0
    for i in range(n):
        lo = 0 if w is None else max(0, i - w + 1)
        count += i - lo + 1
    assert wl.pairs(n, w) == count


# ---- pin 13: hybrid vs full attention FLOPs against the pages' "7x" claim ---------

def test_pin13_hybrid_flop_ratio_consistent_with_pages():
    # Keynote write-up, section 02: a 7:1 hybrid at 1M context cuts attention
    # FLOPs and KV cache about 7x.  8 full layers vs 1 full + 7 SWA(128) layers:
    n = 1 << 20
    full = 8 * wl.pairs(n, None)
    hyb = 1 * wl.pairs(n, None) + 7 * wl.pairs(n, 128)
    ratio = full / hyb
    assert 7.0 <= ratio < 8.0
    assert abs(ratio - 7.99) < 0.01
    kv_ratio = (8 * n) / (1 * n + 7 * 128)
    assert 7.0 <= kv_ratio < 8.0


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache
# ---------------------------------------------------------------------------

def test_e4m3_decoder_matches_library_routine():
    """All 256 codes against torch's float8_e4m3fn (the same format: finite, NaN at S.1111.111)."""
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_to_float(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    assert np.array_equal(np.signbit(ours[~np.isnan(ours)]), np.signbit(ref[~np.isnan(ref)]))


def test_e4m3_hand_values():
    from tests.golden.load import load, value

    fx = load("e4m3_hand.json")
    for code, val in fx["values"].items():
        assert orc.e4m3_to_float(np.array([int(code, 16)]))[0] == value(val), code
    for code in fx["nan_codes"]:
        assert np.isnan(orc.e4m3_to_float(np.array([int(code, 16)]))[0])
    finite = orc.e4m3_to_float(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(finite) > 0)  # codes 0x00..0x7E increase strictly
    assert np.isnan(orc.e4m3_to_float(np.arange(256, dtype=np.uint8))).sum() == 2


def test_fp8kv_decode_never_reads_oldest_slot():
    """The largest codes (+-448) planted in the oldest ring slot of every (sequence, KV head) leave
    the result bit-identical (the definition multiplies masked keys' zero weights by their values,
    so NaN itself would propagate through the oracle's matrix product)."""
    rng = np.random.default_rng(8)
    b, t, hq, hkv, d, w = 3, 2, 4, 2, 16, 8
    q = rng.standard_normal((b, t, hq, d))
    kn = rng.standard_normal((b, t, hkv, d))
    vn = rng.standard_normal((b, t, hkv, d))
    kc = rng.integers(0, 0x70, (b, hkv, w, d)).astype(np.uint8) | (rng.integers(0, 2, (b, hkv, w, d)) << 7).astype(np.uint8)
    vc = rng.integers(0, 0x70, (b, hkv, w, d)).astype(np.uint8)
    heads = np.array([0, 5, 7])
    sinks = rng.standard_normal(hq)
    o1, l1 = orc.swa_sink_decode_fp8kv(q, kn, vn, kc, vc, 0.25, 0.5, heads, sinks, window=w)
    kc2, vc2 = kc.copy(), vc.copy()
    for bi in range(b):
        kc2[bi, :, heads[bi]] = 0x7E
        vc2[bi, :, heads[bi]] = 0xFE
    o2, l2 = orc.swa_sink_decode_fp8kv(q, kn, vn, kc2, vc2, 0.25, 0.5, heads, sinks, window=w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fp8kv_scales_act_on_the_ring_only():
    """Doubling v_scale equals raising every V code's exponent by one (ring values doubled exactly),
    and k_scale multiplies ring logits: with k_scale = 2 and codes whose exponent is lowered by
    one the result is unchanged."""
    rng = np.random.default_rng(9)
    b, t, hq, hkv, d, w = 2, 3, 4, 1, 8, 6
    q = rng.standard_normal((b, t, hq, d))
    kn = rng.standard_normal((b, t, hkv, d))
    vn = rng.standard_normal((b, t, hkv, d))
    exp_field = rng.integers(2, 12, (b, hkv, w, d))
    mant = rng.integers(0, 8, (b, hkv, w, d))
    sign = rng.integers(0, 2, (b, hkv, w, d))
    codes = ((sign << 7) | (exp_field << 3) | mant).astype(np.uint8)
    lower = ((sign << 7) | ((exp_field - 1) << 3) | mant).astype(np.uint8)
    higher = ((sign << 7) | ((exp_field + 1) << 3) | mant).astype(np.uint8)
    heads = np.array([1, 4])
    sinks = rng.standard_normal(hq)
    base = orc.swa_sink_decode_fp8kv(q, kn, vn, codes, codes, 1.0, 1.0, heads, sinks, window=w)
    v2 = orc.swa_sink_decode_fp8kv(q, kn, vn, codes, codes, 1.0, 2.0, heads, sinks, window=w)
    vh = orc.swa_sink_decode_fp8kv(q, kn, vn, codes, higher, 1.0, 1.0, heads, sinks, window=w)
    k2 = orc.swa_sink_decode_fp8kv(q, kn, vn, lower, codes, 2.0, 1.0, heads, sinks, window=w)
    np.testing.assert_allclose(v2[0], vh[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2[0], base[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2[1], base[1], rtol=0, atol=1e-12)


def _codes(rng, shape, lo=1, hi=13):
    """Random finite E4M3 codes with exponent fields in [lo, hi] (hand-built, not from the oracle)."""
    e = rng.integers(lo, hi + 1, shape)
    m = rng.integers(0, 8, shape)
    sgn = rng.integers(0, 2, shape)
    return ((sgn << 7) | (e << 3) | m).astype(np.uint8), sgn, e, m


@pytest.mark.parametrize("window,with_sinks", [(3, True), (5, False), (None, True), (None, False)])
def test_fp8kv_prefill_brute_force(window, with_sinks):
    """The FP8 prefill on codes equals brute-force enumeration over values decoded by hand
    from the bit fields ((-1)^s (1 + m/8) 2^(e-7), the E4M3 normal numbers) times the scales."""
    rng = np.random.default_rng(11)
    lens, hq, hkv, d = [5, 7], 4, 2, 6
    n = sum(lens)
    cu = np.array([0, 5, 12])
    q = rng.standard_normal((n, hq, d))
    kc, ks_, ke, km = _codes(rng, (n, hkv, d))
    vc, vs_, ve, vm = _codes(rng, (n, hkv, d))
    k_scale, v_scale = 0.375, 1.5
    kv = np.where(ks_ == 1, -1.0, 1.0) * (1 + km / 8.0) * 2.0 ** (ke - 7) * k_scale
    vv = np.where(vs_ == 1, -1.0, 1.0) * (1 + vm / 8.0) * 2.0 ** (ve - 7) * v_scale
    sinks = rng.standard_normal(hq) if with_sinks else None
    o, lse = orc.swa_sink_prefill_fp8kv(q, kc, vc, k_scale, v_scale, sinks, cu, window=window, block=4)
    ob, lb = brute.attention(q.tolist(), kv.tolist(), vv.tolist(),
                             None if sinks is None else sinks.tolist(), cu.tolist(), window)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12, rtol=1e-12)


def test_fp8kv_prefill_scales_are_exponent_shifts():
    """Doubling v_scale equals raising every V code's exponent by one; k_scale = 2 with every K
    exponent lowered by one leaves the result unchanged (K and V scales are not swapped)."""
    rng = np.random.default_rng(12)
    n, hq, hkv, d = 9, 4, 1, 8
    cu = np.array([0, 9])
    q = rng.standard_normal((n, hq, d))
    codes, sgn, e, m = _codes(rng, (n, hkv, d), 2, 12)
    lower = ((sgn << 7) | ((e - 1) << 3) | m).astype(np.uint8)
    higher = ((sgn << 7) | ((e + 1) << 3) | m).astype(np.uint8)
    sinks = rng.standard_normal(hq)
    base = orc.swa_sink_prefill_fp8kv(q, codes, codes, 1.0, 1.0, sinks, cu, window=4)
    v2 = orc.swa_sink_prefill_fp8kv(q, codes, codes, 1.0, 2.0, sinks, cu, window=4)
    vh = orc.swa_sink_prefill_fp8kv(q, codes, higher, 1.0, 1.0, sinks, cu, window=4)
    k2 = orc.swa_sink_prefill_fp8kv(q, lower, codes, 2.0, 1.0, sinks, cu, window=4)
    np.testing.assert_allclose(v2[0], vh[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2[0], base[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2[1], base[1], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# E4M3 encoding (the append into an FP8 ring)
# ---------------------------------------------------------------------------

def test_e4m3_encode_round_trips_every_finite_code():
    """Every finite code's value (the pinned decoder) encodes back to that code, -0 included."""
    codes = np.arange(256, dtype=np.uint8)
    fin = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_to_float(fin)), fin)


def test_e4m3_encode_matches_library_cast():
    """fp32 values spread over the E4M3 range and beyond its subnormals, against torch's
    float8_e4m3fn cast (round to nearest even).  That cast turns magnitudes from 464 on into
    NaN rather than saturating, so the comparison stays below 464; power-of-two scales keep the
    quotient exact in fp32, which is what the cast receives."""
    g = torch.Generator().manual_seed(31)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-16, 9, (200000,), generator=g).float())
    for s in (1.0, 1.0 / 32, 4.0):
        q = x / s
        keep = q.abs() < 464
        ref = q[keep].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = orc.e4m3_encode(x[keep].double().numpy(), s)
        assert np.array_equal(got, ref), s


def test_e4m3_encode_is_the_nearest_value_in_exact_arithmetic():
    """With a scale that is no power of two, each code is the nearest E4M3 value to x / scale
    found by exact rational search over the hand-decoded value set (ties to the even code),
    saturating at 448; quotients sitting exactly on ties are included."""
    from fractions import Fraction

    s32 = float(np.float32(0.0173))
    vals = [Fraction(m, 8) * Fraction(2) ** -6 for m in range(8)]          # codes 0..7
    vals += [(1 + Fraction(m, 8)) * Fraction(2) ** (e - 7) for e in range(1, 16) for m in range(8)
             if not (e == 15 and m == 7)]                                  # codes 8..126
    rng = np.random.default_rng(32)
    xs = list((rng.standard_normal(1500) * np.exp2(rng.integers(-14, 4, 1500))).astype(np.float32))
    # exact ties: halfway points times the scale, where that product is an fp32 value
    for c in rng.integers(0, 126, 400):
        t = (vals[c] + vals[c + 1]) / 2 * Fraction(s32)
        if float(np.float32(float(t))) == t:
            xs.append(np.float32(float(t)))
    xs += [np.float32(449 * s32), np.float32(-1e3)]
    got = orc.e4m3_encode(np.array(xs, dtype=np.float64), s32)
    for x, c in zip(xs, got):
        q = abs(Fraction(float(x))) / Fraction(s32)
        q = min(q, vals[-1])
        best = min(range(127), key=lambda k: (abs(q - vals[k]), k % 2))
        want = best | (0x80 if x < 0 else 0)
        assert int(c) == want, (float(x), hex(int(c)), hex(want))


def test_e4m3_encode_hand_values():
    from tests.golden.load import load, value

    for case in load("e4m3_encode_hand.json")["cases"]:
        x = float(case["x"]) if case["x"] in ("inf", "-inf", "nan", "-0") else value(case["x"])
        code = orc.e4m3_encode(np.array([x]), value(case["scale"]))[0]
        assert int(code) == int(case["code"], 16), case


def test_fp8_ring_append_matches_a_list_model():
    """The FP8 append places the same slots as the list model of the ring (last W of ring ++
    accepted tokens); keys and values that are E4M3 values times the scales come back as their
    codes unchanged, and rotated keys decode to within half an E4M3 step of the rotation."""
    rng = np.random.default_rng(33)
    bsz, t_new, hkv, d, w = 4, 4, 2, 8, 6
    k_scale, v_scale = 1.0 / 32, 0.25
    kc0 = _codes(rng, (bsz, hkv, w, d))[0]
    vc0 = _codes(rng, (bsz, hkv, w, d))[0]
    kcodes, ks_, ke, km = _codes(rng, (bsz, t_new, hkv, d))
    vcodes, vs_, ve, vm = _codes(rng, (bsz, t_new, hkv, d))
    kn = np.where(ks_ == 1, -1.0, 1.0) * (1 + km / 8.0) * 2.0 ** (ke - 7) * k_scale
    vn = np.where(vs_ == 1, -1.0, 1.0) * (1 + vm / 8.0) * 2.0 ** (ve - 7) * v_scale
    heads = np.array([0, 5, 3, 2])
    n_acc = np.array([0, 1, 4, 3])
    pos = np.array([10, 0, 77, 123456])
    k2, v2, h2 = orc.swa_ring_append_fp8kv(kn, vn, n_acc, pos, kc0, vc0, heads, None, k_scale, v_scale)
    k3, v3, h3 = orc.swa_ring_append_fp8kv(kn, vn, n_acc, pos, kc0, vc0, heads, 10000.0, k_scale, v_scale,
                                           io_dtype=None)
    assert np.array_equal(h2, h3) and np.array_equal(v2, v3)
    for b in range(bsz):
        klist = [kc0[b, :, (heads[b] + l) % w, :] for l in range(w)]
        vlist = [vc0[b, :, (heads[b] + l) % w, :] for l in range(w)]
        rlist = [None] * w
        for t in range(n_acc[b]):
            klist.append(kcodes[b, t])
            vlist.append(vcodes[b, t])
            rlist.append(orc.rope(kn[b, t][None], [pos[b] + t], 10000.0)[0])
        klist, vlist, rlist = klist[-w:], vlist[-w:], rlist[-w:]
        assert h2[b] == (heads[b] + n_acc[b]) % w
        for l in range(w):
            slot = (h2[b] + l) % w
            np.testing.assert_array_equal(k2[b, :, slot, :], klist[l])
            np.testing.assert_array_equal(v2[b, :, slot, :], vlist[l])
            if rlist[l] is None:
                np.testing.assert_array_equal(k3[b, :, slot, :], klist[l])
            else:
                dec = orc.e4m3_to_float(k3[b, :, slot, :]) * k_scale
                ref = rlist[l]
                assert np.all(np.abs(dec - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * k_scale)
    assert not np.shares_memory(k2, kc0)


# ---------------------------------------------------------------------------
# backward (gradients of O)
# ---------------------------------------------------------------------------

def _fd_grads(q, k, v, sinks, cu, do, window, eps=1e-6):
    """Central finite differences of sum(O * dO) through the forward oracle."""
    def loss(q_, k_, v_, s_):
        return float((orc.swa_sink_prefill(q_, k_, v_, s_, cu, window)[0] * do).sum()) if window \
            else float((orc.ga_causal_prefill(q_, k_, v_, cu)[0] * do).sum())
    out = []
    for which, x in enumerate((q, k, v, sinks)):
        if x is None:
            out.append(None)
            continue
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v, sinks]
            args_m = [q, k, v, sinks]
            args_p[which], args_m[which] = xp, xm
            g[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        out.append(g)
    return out


@pytest.mark.parametrize("window,hq,hkv,sink", [(1, 2, 1, True), (3, 4, 2, True), (5, 2, 2, True),
                                                (None, 4, 2, False), (4, 2, 1, False)])
def test_backward_matches_finite_differences(window, hq, hkv, sink):
    rng = np.random.default_rng(window or 99)
    n, d = 9, 4
    cu = np.array([0, 4, 9])
    q, k, v = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    sinks = rng.standard_normal(hq) if sink else None
    do = rng.standard_normal((n, hq, d))
    if window is None:
        dq, dk, dv, ds = orc.swa_sink_prefill_backward(q, k, v, None, cu, do, window=None)
    else:
        dq, dk, dv, ds = orc.swa_sink_prefill_backward(q, k, v, sinks, cu, do, window=window)
    fq, fk, fv, fs = _fd_grads(q, k, v, sinks, cu, do, window)
    np.testing.assert_allclose(dq, fq, atol=1e-7, rtol=0)
    np.testing.assert_allclose(dk, fk, atol=1e-7, rtol=0)
    np.testing.assert_allclose(dv, fv, atol=1e-7, rtol=0)
    if sink:
        np.testing.assert_allclose(ds, fs, atol=1e-7, rtol=0)
    else:
        assert np.all(ds == 0)


def test_backward_matches_torch_autograd():
    """Autograd through a plain fp64 torch forward (band mask, sink as an extra logit with zero value)."""
    rng = np.random.default_rng(3)
    n, hq, hkv, d, w = 20, 4, 2, 8, 6
    cu = [0, 7, 20]
    q0, k0, v0 = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    s0 = rng.standard_normal(hq)
    do = rng.standard_normal((n, hq, d))
    q, k, v, s = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q0, k0, v0, s0))
    g = hq // hkv
    outs = []
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        pos = torch.arange(L)
        band = (pos[None, :] <= pos[:, None]) & (pos[None, :] > pos[:, None] - w)
        kk = k[a:b].repeat_interleave(g, dim=1).transpose(0, 1)  # [Hq, L, D]
        vv = v[a:b].repeat_interleave(g, dim=1).transpose(0, 1)
        qq = q[a:b].transpose(0, 1)
        logits = (qq @ kk.transpose(1, 2)) / math.sqrt(d)
        logits = logits.masked_fill(~band, float("-inf"))
        sink_col = s[:, None, None].expand(hq, L, 1)
        pr = torch.softmax(torch.cat([logits, sink_col], dim=2), dim=2)[:, :, :L]
        outs.append((pr @ vv).transpose(0, 1))
    o = torch.cat(outs, dim=0)
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv, ds = orc.swa_sink_prefill_backward(q0, k0, v0, s0, np.array(cu), do, window=w)
    for ours, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad), (ds, s.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), atol=1e-12, rtol=0)


def test_backward_constant_keys_closed_form():
    """All keys equal to k: the logits of a row are equal, raising them moves weight from the sink
    (which carries no value) onto the keys, so dO_i . dO_i/dlogit = p_sink(i) delta_i and
    dq_i = scale * p_sink(i) * delta_i * k (with delta_i = dO_i . O_i)."""
    rng = np.random.default_rng(4)
    n, d, w = 11, 6, 4
    kbar = rng.standard_normal(d)
    q = rng.standard_normal((n, 1, d))
    k = np.tile(kbar, (n, 1, 1))
    v = rng.standard_normal((n, 1, d))
    s = np.array([0.3])
    do = rng.standard_normal((n, 1, d))
    cu = np.array([0, n])
    o, lse = orc.swa_sink_prefill(q, k, v, s, cu, w)
    dq, _, _, _ = orc.swa_sink_prefill_backward(q, k, v, s, cu, do, window=w)
    scale = 1 / math.sqrt(d)
    delta = (do[:, 0] * o[:, 0]).sum(axis=1)
    p_sink = np.exp(s[0] - lse[:, 0])
    np.testing.assert_allclose(dq[:, 0], scale * (p_sink * delta)[:, None] * kbar[None, :], atol=1e-13)


def test_backward_shift_invariance_and_gqa():
    """Adding one constant to every logit of a row and to the sink changes nothing, so per head
    the logit gradients (row sums p_sink(i) delta_i) cancel the sink gradient; and GQA gradients
    equal those of MHA with repeated K/V, summed over each group."""
    rng = np.random.default_rng(5)
    n, hq, hkv, d, w = 12, 4, 2, 8, 5
    cu = np.array([0, 5, 12])
    q, k, v = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(hq)
    do = rng.standard_normal((n, hq, d))
    dq, dk, dv, ds = orc.swa_sink_prefill_backward(q, k, v, s, cu, do, window=w)
    g = hq // hkv
    dq2, dk2, dv2, ds2 = orc.swa_sink_prefill_backward(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1),
                                                       s, cu, do, window=w)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(n, hkv, g, d).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(n, hkv, g, d).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(ds, ds2, atol=1e-13)
    o, lse = orc.swa_sink_prefill(q, k, v, s, cu, w)
    for h in range(hq):
        delta = (do[:, h] * o[:, h]).sum(axis=1)
        logit_grad_sum = (np.exp(s[h] - lse[:, h]) * delta).sum()
        assert abs(logit_grad_sum + ds[h]) < 1e-12


def test_backward_delta_equals_weighted_value_products():
    """delta_i = dO_i . O_i equals sum_j p_ij (dO_i . v_j) with p_ij = exp(a_ij - lse_i) the key
    weights and lse the forward's (sink included): O_i = sum_j p_ij v_j because the sink carries
    no value.  The matrix-core backward forms delta this way; checked on the forward oracle's O
    and LSE, with key positions and masks brute-forced from the definition."""
    rng = np.random.default_rng(11)
    n, hq, hkv, d, w = 23, 4, 2, 8, 6
    cu = np.array([0, 9, 9, 23])
    q, k, v = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    s = rng.standard_normal(hq) * 3
    do = rng.standard_normal((n, hq, d))
    o, lse = orc.swa_sink_prefill(q, k, v, s, cu, w)
    scale = 1.0 / math.sqrt(d)
    g = hq // hkv
    for i in range(n):
        seq = int(np.searchsorted(cu, i, side="right")) - 1
        keys = range(max(int(cu[seq]), i - w + 1), i + 1)
        for h in range(hq):
            p = np.array([math.exp(scale * float(q[i, h] @ k[j, h // g]) - lse[i, h]) for j in keys])
            dp = np.array([float(do[i, h] @ v[j, h // g]) for j in keys])
            assert abs(float(p @ dp) - float(do[i, h] @ o[i, h])) < 1e-12
            assert abs(p.sum() + math.exp(s[h] - lse[i, h]) - 1.0) < 1e-12


# ---------------------------------------------------------------------------
# RoPE around decode: rotation, decode with rotated inputs, ring append
# (bases: Technical Report digest, section 3.1; rotate-half reading)
# ---------------------------------------------------------------------------

def test_rope_hand_values():
    from tests.golden.load import load

    fx = load("rope_hand.json")
    for c in fx["cases"]:
        y = orc.rope(np.array([c["x"]], dtype=np.float64), [c["pos"]], fx["base"])[0]
        np.testing.assert_allclose(y, c["y"], rtol=0, atol=1e-15, err_msg=c["why"])


def test_rope_equals_complex_rotation():
    """Pairs (i, i + D/2) as complex numbers x_i + j x_{i+D/2}, multiplied by
    exp(j * pos * base^(-2i/D)) with numpy's complex arithmetic."""
    rng = np.random.default_rng(7)
    for base in (10000.0, 640000.0, 5e6):
        x = rng.standard_normal((6, 3, 16))
        pos = np.array([0, 1, 7, 128, 4095, 262143])
        z = x[..., :8] + 1j * x[..., 8:]
        freq = base ** (-2.0 * np.arange(8) / 16)
        z = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
        np.testing.assert_allclose(orc.rope(x, pos, base), np.concatenate([z.real, z.imag], axis=-1),
                                   rtol=0, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 2, 32))
    pos = np.array([0, 3, 99, 1000, 70000])
    y = orc.rope(x, pos, 10000.0)
    # position 0 is the identity; each pair keeps its length
    np.testing.assert_array_equal(y[0], x[0])
    np.testing.assert_allclose(y[..., :16] ** 2 + y[..., 16:] ** 2, x[..., :16] ** 2 + x[..., 16:] ** 2,
                               rtol=1e-12)
    # composition: rotating by a then by b is rotating by a + b
    np.testing.assert_allclose(orc.rope(orc.rope(x, pos, 10000.0), pos + 5, 10000.0),
                               orc.rope(x, 2 * pos + 5, 10000.0), atol=1e-9)
    # relative positions: <rope(q, m), rope(k, n)> = <rope(q, m - n), k>
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    for m, n in ((5, 2), (300, 299), (1000, 17)):
        lhs = orc.rope(q[None], [m], 640000.0)[0] @ orc.rope(k[None], [n], 640000.0)[0]
        rhs = orc.rope(q[None], [m - n], 640000.0)[0] @ k
        assert abs(lhs - rhs) < 1e-10, (m, n, lhs, rhs)


def _rope_decode_case(bsz, t_new, hq, hkv, d, w, seed, start):
    """Raw (unrotated) keys of a sequence's last w tokens plus T new tokens, the ring
    built by rotating each cached key at its own position."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((bsz, t_new, hq, d))
    kn = rng.standard_normal((bsz, t_new, hkv, d))
    vn = rng.standard_normal((bsz, t_new, hkv, d))
    k_raw = rng.standard_normal((bsz, w, hkv, d))  # logical order, oldest first
    v_ring = rng.standard_normal((bsz, hkv, w, d))
    heads = rng.integers(0, w, size=bsz)
    sinks = rng.standard_normal(hq)
    return q, kn, vn, k_raw, v_ring, heads, sinks


def _ring_from_raw(k_raw, heads, pos0, base, io_dtype):
    bsz, w, hkv, d = k_raw.shape
    kc = np.zeros((bsz, hkv, w, d))
    for b in range(bsz):
        rot = orc.round_to(orc.rope(k_raw[b], pos0[b] - w + np.arange(w), base), io_dtype)  # [w, hkv, d]
        for l in range(w):
            kc[b, :, (heads[b] + l) % w, :] = rot[l]
    return kc


def test_decode_rope_depends_on_relative_positions_only():
    """Shifting every position (cached and new) leaves the decode unchanged: the
    rotation of q and of the new keys agrees with the ring's."""
    q, kn, vn, k_raw, v_ring, heads, sinks = _rope_decode_case(2, 3, 4, 2, 16, 8, 11, 0)
    outs = []
    for shift in (8, 1000, 123457):
        pos0 = np.array([shift, shift + 40])
        kc = _ring_from_raw(k_raw, heads, pos0, 10000.0, None)
        o, lse = orc.swa_sink_decode_rope(q, kn, vn, kc, v_ring, heads, pos0, sinks, 10000.0, window=8,
                                          io_dtype=None)
        outs.append((o, lse))
    for o, lse in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], atol=1e-9)
        np.testing.assert_allclose(lse, outs[0][1], atol=1e-9)


def test_decode_rope_equals_prefill_on_rotated_stream():
    """A ring whose keys were rotated at positions p-W..p-1, plus new tokens at p..p+T-1,
    decodes like the windowed prefill of the whole rotated stream (sink included)."""
    q, kn, vn, k_raw, v_ring, heads, sinks = _rope_decode_case(1, 2, 2, 1, 8, 6, 12, 0)
    p = 50
    kc = _ring_from_raw(k_raw, heads, np.array([p]), 10000.0, None)
    o, lse = orc.swa_sink_decode_rope(q, kn, vn, kc, v_ring, heads, [p], sinks, 10000.0, window=6,
                                      io_dtype=None)
    w, t = 6, 2
    pos = np.arange(p - w, p + t)
    kstream = np.concatenate([k_raw[0], kn[0]], axis=0)                     # [w + t, hkv, d] raw
    vlog = orc.ring_logical_order(v_ring[0], heads[0], w).transpose(1, 0, 2)
    vstream = np.concatenate([vlog, vn[0]], axis=0)
    qstream = np.zeros((w + t,) + q.shape[2:])
    qstream[w:] = q[0]
    qr, kr = orc.rope(qstream, pos, 10000.0), orc.rope(kstream, pos, 10000.0)
    o2, l2 = brute.attention(qr.tolist(), kr.tolist(), vstream.tolist(), sinks.tolist(), [0, w + t], w)
    np.testing.assert_allclose(o[0], np.asarray(o2)[w:], atol=1e-12)
    np.testing.assert_allclose(lse[0], np.asarray(l2)[w:], atol=1e-12)


def test_ring_append_matches_a_list_model():
    """The ring after appending equals the last W tokens of (logical ring ++ accepted
    tokens), tracked with a Python list: eviction order, slots, head and rejected drafts."""
    rng = np.random.default_rng(13)
    bsz, t_new, hkv, d, w = 4, 4, 2, 8, 6
    kc = rng.standard_normal((bsz, hkv, w, d))
    vc = rng.standard_normal((bsz, hkv, w, d))
    heads = np.array([0, 5, 3, 2])
    kn = rng.standard_normal((bsz, t_new, hkv, d))
    vn = rng.standard_normal((bsz, t_new, hkv, d))
    n_acc = np.array([0, 1, 4, 3])
    pos = np.array([10, 0, 77, 123456])
    k2, v2, h2 = orc.swa_ring_append_rope(kn, vn, n_acc, pos, kc, vc, heads, 10000.0, io_dtype=None)
    for b in range(bsz):
        klist = [kc[b, :, (heads[b] + l) % w, :] for l in range(w)]
        vlist = [vc[b, :, (heads[b] + l) % w, :] for l in range(w)]
        for t in range(n_acc[b]):
            klist.append(orc.rope(kn[b, t][None], [pos[b] + t], 10000.0)[0])
            vlist.append(vn[b, t])
        klist, vlist = klist[-w:], vlist[-w:]
        assert h2[b] == (heads[b] + n_acc[b]) % w
        for l in range(w):
            np.testing.assert_array_equal(k2[b, :, (h2[b] + l) % w, :], klist[l])
            np.testing.assert_array_equal(v2[b, :, (h2[b] + l) % w, :], vlist[l])
    # inputs are untouched (new arrays returned)
    assert not np.shares_memory(k2, kc)
    # without a base the keys are copied as given
    k3, _, _ = orc.swa_ring_append_rope(kn, vn, n_acc, pos, kc, vc, heads, None)
    b, t = 2, 3
    np.testing.assert_array_equal(k3[b, :, (heads[b] + t) % w, :], kn[b, t])


def test_mtp_steps_equal_attention_over_the_accepted_stream():
    """A run of MTP steps (commit the previous step's accepted tokens, verify the new
    ones) sees exactly the stream of accepted tokens: each step's outputs equal brute
    force windowed attention with sink over (history ++ every accepted token ++ the
    step's T tokens), all rotated at their positions.  Covers accept counts 0, partial
    and all (and a count above prev_T, clamped), and the head carried between steps."""
    rng = np.random.default_rng(21)
    w, d, hq, hkv, t_new, base = 6, 8, 4, 2, 3, 10000.0
    q0, kn0, vn0, k_raw, v_ring, heads, sinks = _rope_decode_case(1, t_new, hq, hkv, d, w, 22, 0)
    p = 40  # history at positions p-w .. p-1
    kc = _ring_from_raw(k_raw, heads, np.array([p]), base, None)
    vc = v_ring.copy()
    hist_k = [k_raw[0, l] for l in range(w)]
    hist_v = [v_ring[0, :, (heads[0] + l) % w, :] for l in range(w)]
    prev_k, prev_v = kn0, vn0
    # the first step commits nothing (its "previous" tokens are arbitrary)
    accepts = [0, 2, 3, 1, 7, 0, 3]
    head = heads.copy()
    pos, prev_pos = p, p
    for step, acc in enumerate(accepts):
        n = min(acc, t_new)
        if step > 0:
            hist_k += [prev_k[0, t] for t in range(n)]
            hist_v += [prev_v[0, t] for t in range(n)]
            pos = prev_pos + n
        q = rng.standard_normal((1, t_new, hq, d))
        kn = rng.standard_normal((1, t_new, hkv, d))
        vn = rng.standard_normal((1, t_new, hkv, d))
        o, lse, kc, vc, head = orc.swa_sink_decode_rope_commit(
            q, kn, vn, [pos], prev_k, prev_v, [acc if step > 0 else 0], [prev_pos], kc, vc, head, sinks,
            base, window=w, io_dtype=None)
        ks = np.stack(hist_k + [kn[0, t] for t in range(t_new)])            # [L, hkv, d] raw
        vs = np.stack(hist_v + [vn[0, t] for t in range(t_new)])
        L = ks.shape[0]
        spos = pos - (L - t_new) + np.arange(L)
        assert spos[0] == p - w  # the stream is contiguous from the history's first position
        qs = np.zeros((L, hq, d))
        qs[L - t_new:] = q[0]
        qr, kr = orc.rope(qs, spos, base), orc.rope(ks, spos, base)
        o2, l2 = brute.attention(qr.tolist(), kr.tolist(), vs.tolist(), sinks.tolist(), [0, L], w)
        np.testing.assert_allclose(o[0], np.asarray(o2)[L - t_new:], atol=1e-12)
        np.testing.assert_allclose(lse[0], np.asarray(l2)[L - t_new:], atol=1e-12)
        assert head[0] == (heads[0] + len(hist_k) - w) % w
        prev_k, prev_v, prev_pos = kn, vn, pos


def test_fp8_mtp_steps_equal_attention_over_the_accepted_stream():
    """FP8 ring: each MTP step's outputs equal brute-force windowed attention with sink over
    the accepted stream, where the ring's keys and values are their E4M3 code values times
    the scales (distinct K and V scales), a committed key is rotated at its position before
    it is encoded, and the step's drafts enter unquantised."""
    rng = np.random.default_rng(31)
    w, d, hq, hkv, t_new, base, ks, vs = 6, 8, 4, 2, 3, 10000.0, 0.1875, 0.3
    kcode = rng.integers(1, 0x70, size=(1, hkv, w, d)).astype(np.uint8) | (rng.integers(0, 2, (1, hkv, w, d)) << 7).astype(np.uint8)
    vcode = rng.integers(1, 0x70, size=(1, hkv, w, d)).astype(np.uint8) | (rng.integers(0, 2, (1, hkv, w, d)) << 7).astype(np.uint8)
    heads = np.array([4])
    sinks = rng.standard_normal(hq)
    # the stream as the reference sees it: keys already rotated (ring) or raw (to rotate)
    hist_k = [orc.e4m3_to_float(kcode[0, :, (heads[0] + l) % w, :]) * ks for l in range(w)]
    hist_v = [orc.e4m3_to_float(vcode[0, :, (heads[0] + l) % w, :]) * vs for l in range(w)]
    p = 90
    prev_k = rng.standard_normal((1, t_new, hkv, d))
    prev_v = rng.standard_normal((1, t_new, hkv, d))
    kc, vc, head = kcode, vcode, heads
    pos, prev_pos = p, p
    for step, acc in enumerate([0, 3, 1, 2, 0, 3]):
        n = min(acc, t_new)
        if step > 0:
            for t in range(n):
                kr = orc.rope(prev_k[0, t][None], [prev_pos + t], base)[0]
                hist_k.append(orc.e4m3_to_float(orc.e4m3_encode(kr, ks)) * ks)
                hist_v.append(orc.e4m3_to_float(orc.e4m3_encode(prev_v[0, t], vs)) * vs)
            pos = prev_pos + n
        q = rng.standard_normal((1, t_new, hq, d))
        kn = rng.standard_normal((1, t_new, hkv, d))
        vn = rng.standard_normal((1, t_new, hkv, d))
        o, lse, kc, vc, head = orc.swa_sink_decode_rope_commit_fp8kv(
            q, kn, vn, [pos], prev_k, prev_v, [acc if step > 0 else 0], [prev_pos], kc, vc, ks, vs, head, sinks,
            base, window=w, io_dtype=None)
        newk = orc.rope(kn[0], pos + np.arange(t_new), base)
        ks_ = np.concatenate([np.stack(hist_k), newk])
        vs_ = np.concatenate([np.stack(hist_v), vn[0]])
        L = ks_.shape[0]
        qs = np.zeros((L, hq, d))
        qs[L - t_new:] = orc.rope(q[0], pos + np.arange(t_new), base)
        o2, l2 = brute.attention(qs.tolist(), ks_.tolist(), vs_.tolist(), sinks.tolist(), [0, L], w)
        np.testing.assert_allclose(o[0], np.asarray(o2)[L - t_new:], atol=1e-12)
        np.testing.assert_allclose(lse[0], np.asarray(l2)[L - t_new:], atol=1e-12)
        prev_k, prev_v, prev_pos = kn, vn, pos


# ---------------------------------------------------------------------------
# Token-level sparse attention with a forced recent window (MiMo-V3 / HySparse2 page)
# ---------------------------------------------------------------------------

def _brute_topk(scores_row, n_cand, k):
    """Python's sorted() on (score descending, position ascending), then increasing position."""
    pairs = sorted(((-float(scores_row[j]), j) for j in range(n_cand)))
    return sorted(j for _, j in pairs[:k])


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 40), st.integers(0, 12), st.integers(1, 6), st.integers(0, 3))
def test_topk_select_matches_brute_force(length, k, recent, levels):
    rng = np.random.default_rng(length * 1000 + k * 10 + recent)
    lmax = 48
    # levels > 0: scores drawn from a few values, so equal scores are common
    sc = rng.standard_normal((2, 3, lmax)) if levels == 0 else rng.integers(0, levels + 1, (2, 3, lmax)) * 0.5
    lens = np.array([length, max(0, length - 7)])
    idx, cnt = orc.topk_select(sc, lens, k=k, recent=recent)
    for b in range(2):
        for h in range(3):
            want = _brute_topk(sc[b, h], max(0, int(lens[b]) - recent), k)
            assert cnt[b, h] == len(want)
            assert list(idx[b, h, :cnt[b, h]]) == want
            assert np.all(idx[b, h, cnt[b, h]:] == -1)


def _sparse_case(bsz, hq, hkv, d, lmax, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((bsz, hq, d))
    kc = rng.standard_normal((bsz, hkv, lmax, d))
    vc = rng.standard_normal((bsz, hkv, lmax, d))
    sinks = rng.standard_normal(hq)
    scores = rng.standard_normal((bsz, hkv, lmax))
    return q, kc, vc, sinks, scores


def _prefill_last_row(q, kc, vc, sinks, b, L, window):
    """The oracle's windowed prefill of sequence b's first L tokens, newest row only
    (q placed on the newest token, zeros elsewhere)."""
    hq, d = q.shape[1], q.shape[2]
    qs = np.zeros((L, hq, d))
    qs[L - 1] = q[b]
    ks = kc[b, :, :L].transpose(1, 0, 2)
    vs = vc[b, :, :L].transpose(1, 0, 2)
    o, lse = orc.swa_sink_prefill(qs, ks, vs, sinks, [0, L], window)
    return o[L - 1], lse[L - 1]


def test_sparse_decode_special_cases_reduce_to_dense_attention():
    """k covering every older token: full causal attention (window = L); k = 0: the
    128-window SWA of the same layer -- both through the pinned prefill oracle."""
    q, kc, vc, sinks, scores = _sparse_case(3, 4, 2, 16, 60, 21)
    lens = np.array([60, 9, 33])
    recent = 8
    idx, cnt = orc.topk_select(scores, lens, k=64, recent=recent)  # k >= every candidate count
    o, lse = orc.sparse_decode(q, kc, vc, lens, idx, cnt, sinks, recent=recent)
    idx0, cnt0 = orc.topk_select(scores, lens, k=0, recent=recent)
    o0, lse0 = orc.sparse_decode(q, kc, vc, lens, idx0, cnt0, sinks, recent=recent)
    for b in range(3):
        L = int(lens[b])
        of, lf = _prefill_last_row(q, kc, vc, sinks, b, L, L)
        np.testing.assert_allclose(o[b], of, atol=1e-12)
        np.testing.assert_allclose(lse[b], lf, atol=1e-12)
        ow, lw = _prefill_last_row(q, kc, vc, sinks, b, L, recent)
        np.testing.assert_allclose(o0[b], ow, atol=1e-12)
        np.testing.assert_allclose(lse0[b], lw, atol=1e-12)


def test_sparse_decode_matches_brute_force_and_ignores_index_order():
    q, kc, vc, sinks, scores = _sparse_case(2, 4, 2, 8, 40, 22)
    lens = np.array([40, 25])
    recent, k = 5, 6
    idx, cnt = orc.topk_select(scores, lens, k=k, recent=recent)
    o, lse = orc.sparse_decode(q, kc, vc, lens, idx, cnt, sinks, recent=recent)
    for b in range(2):
        L = int(lens[b])
        for g in range(2):
            keys = list(idx[b, g, :cnt[b, g]]) + list(range(L - recent, L))
            m = len(keys)
            # the key list as a causal sequence whose last row is the query: brute force
            qs = [[[0.0] * 8 for _ in range(4)] for _ in range(m)]
            for h in range(2 * g, 2 * g + 2):
                qs[m - 1][h] = list(q[b, h])
            ks = [[list(kc[b, gg, j]) for gg in range(2)] for j in keys]
            vs = [[list(vc[b, gg, j]) for gg in range(2)] for j in keys]
            ob, lb = brute.attention(qs, ks, vs, list(sinks), [0, m], None)
            for h in range(2 * g, 2 * g + 2):
                np.testing.assert_allclose(o[b, h], ob[m - 1][h], atol=1e-12)
                assert abs(lse[b, h] - lb[m - 1][h]) < 1e-12
    # reversing each selection list changes nothing
    rev = idx.copy()
    for b in range(2):
        for g in range(2):
            rev[b, g, :cnt[b, g]] = idx[b, g, :cnt[b, g]][::-1]
    o2, l2 = orc.sparse_decode(q, kc, vc, lens, rev, cnt, sinks, recent=recent)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(l2, lse, atol=1e-12)


def _prefill_rows(q_t, kc, vc, sinks, b, L, window):
    """The oracle's windowed prefill of sequence b's first L tokens, rows L-T .. L-1
    (q_t [T, Hq, D] placed on the newest T tokens, zeros elsewhere)."""
    t_new, hq, d = q_t.shape
    qs = np.zeros((L, hq, d))
    qs[L - t_new:] = q_t
    ks = kc[b, :, :L].transpose(1, 0, 2)
    vs = vc[b, :, :L].transpose(1, 0, 2)
    o, lse = orc.swa_sink_prefill(qs, ks, vs, sinks, [0, L], window)
    return o[L - t_new:], lse[L - t_new:]


def test_sparse_mtp_special_cases_reduce_to_dense_attention():
    """T verified tokens in a sparse layer: T = 1 is sparse_decode; every older token
    selected gives full causal attention for each of the T rows, none selected the
    recent-window SWA (each row with its own window) -- through the pinned prefill oracle."""
    rng = np.random.default_rng(23)
    _, kc, vc, sinks, scores = _sparse_case(3, 4, 2, 16, 60, 24)
    lens = np.array([60, 10, 33])
    recent = 8
    for t_new in (1, 2, 3):
        q = rng.standard_normal((3, t_new, 4, 16))
        idx, cnt = orc.topk_select(scores, lens, k=64, recent=recent)
        o, lse = orc.sparse_decode_mtp(q, kc, vc, lens, idx, cnt, sinks, recent=recent)
        idx0, cnt0 = orc.topk_select(scores, lens, k=0, recent=recent)
        o0, lse0 = orc.sparse_decode_mtp(q, kc, vc, lens, idx0, cnt0, sinks, recent=recent)
        if t_new == 1:
            o1, l1 = orc.sparse_decode(q[:, 0], kc, vc, lens, idx, cnt, sinks, recent=recent)
            np.testing.assert_allclose(o[:, 0], o1, atol=1e-12)
            np.testing.assert_allclose(lse[:, 0], l1, atol=1e-12)
        for b in range(3):
            L = int(lens[b])
            of, lf = _prefill_rows(q[b], kc, vc, sinks, b, L, L)
            np.testing.assert_allclose(o[b], of, atol=1e-12)
            np.testing.assert_allclose(lse[b], lf, atol=1e-12)
            ow, lw = _prefill_rows(q[b], kc, vc, sinks, b, L, recent)
            np.testing.assert_allclose(o0[b], ow, atol=1e-12)
            np.testing.assert_allclose(lse0[b], lw, atol=1e-12)


def test_sparse_mtp_matches_brute_force_with_the_windows_overlapping_the_selection():
    """Brute force over explicit key lists: query t sees the selected positions below its
    own window and the window itself, each once, including a selection that reaches into
    the older drafts' windows (positions just below the newest token's window)."""
    rng = np.random.default_rng(25)
    hq, hkv, d, lmax, recent, t_new = 4, 2, 8, 40, 5, 3
    _, kc, vc, sinks, _ = _sparse_case(2, hq, hkv, d, lmax, 26)
    q = rng.standard_normal((2, t_new, hq, d))
    lens = np.array([40, 9])
    idx = np.full((2, hkv, 6), -1, dtype=np.int64)
    cnt = np.zeros((2, hkv), dtype=np.int64)
    for b in range(2):
        L = int(lens[b])
        for g in range(hkv):  # the newest candidates (just below the newest window) always chosen
            cand = np.arange(L - recent)
            pick = np.sort(np.concatenate([cand[-2:], rng.choice(cand[:-2], size=min(4, len(cand) - 2), replace=False)]))
            idx[b, g, :len(pick)] = pick
            cnt[b, g] = len(pick)
    o, lse = orc.sparse_decode_mtp(q, kc, vc, lens, idx, cnt, sinks, recent=recent)
    for b in range(2):
        L = int(lens[b])
        for t in range(t_new):
            p = L - t_new + t
            for g in range(hkv):
                win = list(range(max(0, p - recent + 1), p + 1))
                keys = [j for j in idx[b, g, :cnt[b, g]] if j not in win] + win
                assert len(set(keys)) == len(keys)
                m = len(keys)
                qs = [[[0.0] * d for _ in range(hq)] for _ in range(m)]
                for h in range(2 * g, 2 * g + 2):
                    qs[m - 1][h] = list(q[b, t, h])
                ks = [[list(kc[b, gg, j]) for gg in range(hkv)] for j in keys]
                vs = [[list(vc[b, gg, j]) for gg in range(hkv)] for j in keys]
                ob, lb = brute.attention(qs, ks, vs, list(sinks), [0, m], None)
                for h in range(2 * g, 2 * g + 2):
                    np.testing.assert_allclose(o[b, t, h], ob[m - 1][h], atol=1e-12)
                    assert abs(lse[b, t, h] - lb[m - 1][h]) < 1e-12


def test_sparse_mtp_fp8kv_brute_force_with_distinct_scales():
    """FP8 cache: brute force over explicit key lists whose K and V values are decoded by
    hand from the E4M3 bit fields (sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals) times distinct scales, T = 2, the selection reaching into the older
    draft's window."""
    rng = np.random.default_rng(27)
    hq, hkv, d, lmax, recent, t_new, ks, vs = 4, 2, 8, 30, 5, 2, 0.1875, 0.3
    kcode = _codes(rng, (2, hkv, lmax, d), lo=0)[0]
    vcode = _codes(rng, (2, hkv, lmax, d), lo=0)[0]
    sinks = rng.standard_normal(hq)
    q = rng.standard_normal((2, t_new, hq, d))
    lens = np.array([30, 12])
    idx = np.full((2, hkv, 4), -1, dtype=np.int64)
    cnt = np.zeros((2, hkv), dtype=np.int64)
    for b in range(2):
        L = int(lens[b])
        for g in range(hkv):
            pick = np.sort(np.concatenate([[L - recent - 1], rng.choice(L - recent - 1, size=3, replace=False)]))
            idx[b, g, :4] = pick
            cnt[b, g] = 4

    def hand(c):
        s_, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        return -v if s_ else v

    o, lse = orc.sparse_decode_mtp_fp8kv(q, kcode, vcode, ks, vs, lens, idx, cnt, sinks, recent=recent)
    for b in range(2):
        L = int(lens[b])
        for t in range(t_new):
            p = L - t_new + t
            for g in range(hkv):
                win = list(range(max(0, p - recent + 1), p + 1))
                keys = [int(j) for j in idx[b, g, :cnt[b, g]] if j not in win] + win
                m = len(keys)
                qs = [[[0.0] * d for _ in range(hq)] for _ in range(m)]
                for h in range(2 * g, 2 * g + 2):
                    qs[m - 1][h] = list(q[b, t, h])
                kk = [[[hand(int(c)) * ks for c in kcode[b, gg, j]] for gg in range(hkv)] for j in keys]
                vv = [[[hand(int(c)) * vs for c in vcode[b, gg, j]] for gg in range(hkv)] for j in keys]
                ob, lb = brute.attention(qs, kk, vv, list(sinks), [0, m], None)
                for h in range(2 * g, 2 * g + 2):
                    np.testing.assert_allclose(o[b, t, h], ob[m - 1][h], atol=1e-12)
                    assert abs(lse[b, t, h] - lb[m - 1][h]) < 1e-12


# ---------------------------------------------------------------------------
# the row-sampled evaluation used at sizes where the full fp64 output is too large
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window,with_sinks", [(3, True), (16, True), (None, False), (None, True)])
def test_prefill_sample_rows_equals_full_oracle_on_every_row(window, with_sinks):
    """prefill_sample_rows at every (token, head) pair of a multi-sequence stream with
    zero-length sequences (before the first, between and after the others) equals the full
    swa_sink_prefill / ga_causal_prefill: each sequence's first and last token, the rows
    inside its first window and the rows past it all take their own sequence's keys."""
    lens = [0, 5, 0, 0, 23, 1, 0, 40, 2, 0]
    q, k, v, sinks, cu = _inputs(lens, 4, 2, 8, seed=31)
    sinks = sinks if with_sinks else None
    if window is None and sinks is None:
        o, lse = orc.ga_causal_prefill(q, k, v, cu)
    elif window is None:
        o, lse = orc._prefill(q, k, v, sinks, cu, None, None, 128)
    else:
        o, lse = orc.swa_sink_prefill(q, k, v, sinks, cu, window)
    n, hq = q.shape[:2]
    rows = np.array([(t, h) for t in range(n) for h in range(hq)])
    os_, ls_ = orc.prefill_sample_rows(q, k, v, sinks, cu, rows, window=window)
    np.testing.assert_allclose(os_, o[rows[:, 0], rows[:, 1]], atol=1e-13, rtol=0)
    np.testing.assert_allclose(ls_, lse[rows[:, 0], rows[:, 1]], atol=1e-13, rtol=0)
    # and against brute-force enumeration for the first tokens of each non-empty sequence
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), None if sinks is None else sinks.tolist(),
                             cu.tolist(), window)
    firsts = [(int(cu[s]), h) for s in range(len(lens)) if lens[s] for h in range(hq)]
    fo, fl = orc.prefill_sample_rows(q, k, v, sinks, cu, np.array(firsts), window=window)
    for r, (t, h) in enumerate(firsts):
        np.testing.assert_allclose(fo[r], ob[t][h], atol=1e-13)
        assert abs(fl[r] - lb[t][h]) < 1e-13


def test_prefill_sample_rows_first_token_sees_only_itself():
    """Row 0 of every sequence attends to its own key alone: o = sigmoid(a - sink) v, the
    closed form of the first row, whatever the previous sequence holds."""
    lens = [7, 0, 9, 4]
    q, k, v, sinks, cu = _inputs(lens, 2, 1, 6, seed=32)
    d = q.shape[2]
    for s in (0, 2, 3):
        t = int(cu[s])
        for h in range(2):
            o, lse = orc.prefill_sample_rows(q, k, v, sinks, cu, np.array([[t, h]]), window=128)
            a = (q[t, h] @ k[t, 0]) / math.sqrt(d)
            w_ = 1.0 / (1.0 + math.exp(sinks[h] - a))
            np.testing.assert_allclose(o[0], w_ * v[t, 0], atol=1e-14)
            assert abs(lse[0] - np.logaddexp(a, sinks[h])) < 1e-14


# ---------------------------------------------------------------------------
# decode with RoPE against an FP8 ring
# ---------------------------------------------------------------------------

def test_decode_rope_fp8kv_brute_force_with_distinct_scales():
    """swa_sink_decode_rope_fp8kv equals brute-force ring enumeration (oracle.brute.decode) over
    cache values decoded by hand from the E4M3 bit fields times k_scale (keys) and v_scale
    (values), with q and the new keys rotated at positions p .. p+T-1 (the pinned rope)."""
    rng = np.random.default_rng(33)
    b, t, hq, hkv, d, w = 2, 3, 4, 2, 8, 7
    q = rng.standard_normal((b, t, hq, d))
    kn = rng.standard_normal((b, t, hkv, d))
    vn = rng.standard_normal((b, t, hkv, d))
    kc, ks_, ke, km = _codes(rng, (b, hkv, w, d), 3, 10)
    vc, vs_, ve, vm = _codes(rng, (b, hkv, w, d), 3, 10)
    k_scale, v_scale = 0.0625 * 3, 0.3
    kval = np.where(ks_ == 1, -1.0, 1.0) * (1 + km / 8.0) * 2.0 ** (ke - 7) * k_scale
    vval = np.where(vs_ == 1, -1.0, 1.0) * (1 + vm / 8.0) * 2.0 ** (ve - 7) * v_scale
    heads = np.array([2, 6])
    pos = np.array([40, 1234])
    sinks = rng.standard_normal(hq)
    base = 10000.0
    o, lse = orc.swa_sink_decode_rope_fp8kv(q, kn, vn, kc, vc, k_scale, v_scale, heads, pos, sinks, base,
                                            window=w, io_dtype=None)
    qr = np.stack([orc.rope(q[bi], pos[bi] + np.arange(t), base) for bi in range(b)])
    kr = np.stack([orc.rope(kn[bi], pos[bi] + np.arange(t), base) for bi in range(b)])
    ob, lb = brute.decode(qr.tolist(), kr.tolist(), vn.tolist(), kval.tolist(), vval.tolist(),
                          heads.tolist(), sinks.tolist(), w)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12, rtol=0)


def test_decode_rope_fp8kv_scales_are_exponent_shifts():
    """Doubling v_scale equals raising every V code's exponent by one; k_scale = 2 with every K
    exponent lowered by one leaves the result unchanged; so the two scales are neither swapped
    nor applied to the new tokens (which keep their own values)."""
    rng = np.random.default_rng(34)
    b, t, hq, hkv, d, w = 2, 2, 4, 1, 8, 6
    q = rng.standard_normal((b, t, hq, d))
    kn = rng.standard_normal((b, t, hkv, d))
    vn = rng.standard_normal((b, t, hkv, d))
    codes, sgn, e, m = _codes(rng, (b, hkv, w, d), 2, 12)
    lower = ((sgn << 7) | ((e - 1) << 3) | m).astype(np.uint8)
    higher = ((sgn << 7) | ((e + 1) << 3) | m).astype(np.uint8)
    heads, pos, sinks = np.array([0, 3]), np.array([7, 99]), rng.standard_normal(hq)

    def run(kc, vc, ksc, vsc):
        return orc.swa_sink_decode_rope_fp8kv(q, kn, vn, kc, vc, ksc, vsc, heads, pos, sinks, 640000.0,
                                              window=w, io_dtype=None)
    base = run(codes, codes, 1.0, 1.0)
    v2, vh = run(codes, codes, 1.0, 2.0), run(codes, higher, 1.0, 1.0)
    k2 = run(lower, codes, 2.0, 1.0)
    np.testing.assert_allclose(v2[0], vh[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(v2[1], vh[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2[0], base[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(k2[1], base[1], rtol=0, atol=1e-12)
    assert np.abs(v2[0] - base[0]).max() > 1e-3  # the V scale does act on the ring values
