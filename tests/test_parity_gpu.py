"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Inputs are seeded synthetic tensors (sliding_window_attention_amd.workloads);
the oracle runs on exactly the values the GPU saw.  Small cases compare every
output element and span several 16-query tiles, ragged tails, short and length-1
sequences, sequence boundaries inside tiles, windows below, at and above 128,
and ring heads at both ends.  The full-size workloads compare every output where
the oracle finishes in seconds and sampled rows otherwise.
"""
import numpy as np
import pytest
import torch

import sliding_window_attention_amd as swa
from oracle import swa_oracle as orc
from sliding_window_attention_amd import workloads as wl
from tests.golden.load import array, load
from tests.parity import TOL, assert_close, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _gpu(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _run_prefill(x, window, ga=False):
    g = _gpu(x)
    if ga:
        o, lse = swa.ga_causal_prefill(g["q"], g["k"], g["v"], g["cu_seqlens"], x["max_seqlen"])
    else:
        o, lse = swa.swa_sink_prefill(g["q"], g["k"], g["v"], g["sinks"], g["cu_seqlens"],
                                      x["max_seqlen"], window=window)
    torch.cuda.synchronize()
    return o, lse


def _oracle_prefill(x, window, ga=False):
    cu = x["cu_seqlens"].numpy()
    if ga:
        return orc.ga_causal_prefill(x["q"], x["k"], x["v"], cu)
    return orc.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], cu, window)


# ---------------------------------------------------------------------------
# hand-worked fixtures (exact rationals), fp32, through the library
# ---------------------------------------------------------------------------

def _pad_d(a, d=64):
    out = np.zeros(a.shape[:-1] + (d,))
    out[..., : a.shape[-1]] = a
    return torch.tensor(out, dtype=torch.float32, device=DEV).contiguous()


def test_golden_prefill_and_ga_through_library():
    fx = load()["prefill"]
    _say("golden prefill fp32 (head_dim 4 padded to 64, scale 1/2)")
    q, k, v = _pad_d(array(fx["q"])), _pad_d(array(fx["k"])), _pad_d(array(fx["v"]))
    sinks = torch.tensor(array(fx["sinks"]), dtype=torch.float32, device=DEV)
    cu = torch.tensor(fx["cu_seqlens"], dtype=torch.int32, device=DEV)
    o, lse = swa.swa_sink_prefill(q, k, v, sinks, cu, window=fx["window"], scale=0.5)
    np.testing.assert_allclose(to_np(o)[..., :4], array(fx["swa_o"]), atol=2e-6)
    np.testing.assert_allclose(to_np(lse), array(fx["swa_lse"]), atol=2e-6)
    o, lse = swa.ga_causal_prefill(q, k, v, cu, scale=0.5)
    np.testing.assert_allclose(to_np(o)[..., :4], array(fx["ga_o"]), atol=2e-6)
    np.testing.assert_allclose(to_np(lse), array(fx["ga_lse"]), atol=2e-6)


def test_golden_decode_through_library():
    for n, fx in enumerate(load()["decode"]):
        _say(f"golden decode {n} fp32 window {fx['window']}")
        t = {k: _pad_d(array(fx[k])) for k in ("q", "k_new", "v_new", "k_cache", "v_cache")}
        head = torch.tensor(fx["ring_head"], dtype=torch.int32, device=DEV)
        sinks = torch.tensor(array(fx["sinks"]), dtype=torch.float32, device=DEV)
        o, lse = swa.swa_sink_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     head, sinks, scale=0.5)
        np.testing.assert_allclose(to_np(o)[..., :4], array(fx["o"]), atol=2e-6)
        np.testing.assert_allclose(to_np(lse), array(fx["lse"]), atol=2e-6)


# ---------------------------------------------------------------------------
# prefill, small sizes, every element
# ---------------------------------------------------------------------------

def test_tiny_fp32_workload_full():
    _say("tiny_fp32: 512 tokens, 4/1 heads, D 64, W 128, fp32")
    x = wl.make_workload("tiny_fp32")
    o, lse = _run_prefill(x, 128)
    o_ref, l_ref = _oracle_prefill(x, 128)
    assert_close(torch.float32, o, o_ref, lse, l_ref, "tiny_fp32")


PREFILL_CASES = [
    # (lengths, Hq, Hkv, D, dtype, window)
    ([700], 32, 4, 128, "bf16", 128),           # window kernel, ragged tail (700 = 43*16 + 12)
    ([130, 1, 17, 300, 5, 64], 32, 4, 128, "bf16", 128),  # boundaries inside tiles, L=1, L<W
    ([400], 16, 2, 128, "bf16", 1),             # window 1: only the diagonal
    ([333, 90], 8, 1, 128, "bf16", 37),         # odd window, G = 8
    ([260], 16, 1, 128, "bf16", 100),           # G = 16 (two head octets per KV head)
    ([520, 45], 32, 4, 128, "bf16", 129),       # online kernel with window + sink
    ([1000], 8, 1, 128, "bf16", 300),           # online kernel, long window
    ([300, 77], 8, 2, 128, "bf16", 128),        # generic kernel (G = 4)
    ([250], 8, 1, 64, "bf16", 128),             # generic kernel (D = 64)
    ([200, 3], 4, 2, 128, "f32", 50),           # generic fp32
    ([7], 32, 4, 128, "bf16", 128),             # fewer tokens than one tile
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"{c[0]}-{c[1]}/{c[2]}-D{c[3]}-{c[4]}-W{c[5]}")
def test_swa_prefill_small(case):
    lens, hq, hkv, d, dt, window = case
    _say(f"swa prefill lens={lens} heads={hq}/{hkv} D={d} {dt} W={window}")
    x = wl.make_prefill(lens, hq, hkv, d, dt, seed=sum(lens) + hq + window)
    o, lse = _run_prefill(x, window)
    o_ref, l_ref = _oracle_prefill(x, window)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"swa {case}")


GA_CASES = [
    ([600], 32, 4, 128, "bf16"),
    ([129, 1, 400, 33], 16, 2, 128, "bf16"),
    ([300], 8, 1, 64, "bf16"),   # generic
    ([90, 40], 4, 4, 128, "f32"),  # generic fp32
]


@pytest.mark.parametrize("case", GA_CASES, ids=lambda c: f"{c[0]}-{c[1]}/{c[2]}-D{c[3]}-{c[4]}")
def test_ga_prefill_small(case):
    lens, hq, hkv, d, dt = case
    _say(f"ga prefill lens={lens} heads={hq}/{hkv} D={d} {dt}")
    x = wl.make_prefill(lens, hq, hkv, d, dt, seed=7 + sum(lens), with_sinks=False)
    o, lse = _run_prefill(x, None, ga=True)
    o_ref, l_ref = _oracle_prefill(x, None, ga=True)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"ga {case}")


def _growing_keys(x, factor):
    """Scale each key by 1 + factor * (position in its sequence) / length, so that
    row maxima keep rising along the sequence (forces repeated online rescales)."""
    cu = x["cu_seqlens"].tolist()
    k = x["k"].float()
    for s in range(len(cu) - 1):
        n = cu[s + 1] - cu[s]
        ramp = 1.0 + factor * torch.arange(n, dtype=torch.float32) / max(n, 1)
        k[cu[s]:cu[s + 1]] *= ramp[:, None, None]
    x["k"] = k.to(x["k"].dtype)
    return x


def test_ga_prefill_rising_maxima():
    _say("ga prefill with key norms rising 6x along each sequence (lazy rescale path)")
    x = _growing_keys(wl.make_prefill([900, 260], 16, 2, 128, "bf16", seed=31, with_sinks=False), 5.0)
    o, lse = _run_prefill(x, None, ga=True)
    o_ref, l_ref = _oracle_prefill(x, None, ga=True)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "ga rising maxima")


def test_long_window_sink_rising_maxima():
    _say("swa prefill W=200 (online kernel) with sinks in [-3, 12] and rising key norms")
    x = _growing_keys(wl.make_prefill([700, 90], 8, 1, 128, "bf16", seed=32), 4.0)
    x["sinks"] = torch.linspace(-3.0, 12.0, 8)
    o, lse = _run_prefill(x, 200)
    o_ref, l_ref = _oracle_prefill(x, 200)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "W=200 rising maxima")


def test_prefill_large_sink_and_no_lse():
    _say("swa prefill with sinks +40 (outputs ~0) and lse=None")
    x = wl.make_prefill([300], 32, 4, 128, "bf16", seed=99)
    x["sinks"] = x["sinks"] + 40.0
    g = _gpu(x)
    o, lse = swa.swa_sink_prefill(g["q"], g["k"], g["v"], g["sinks"], g["cu_seqlens"], return_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    assert float(o.float().abs().max()) < 1e-6
    o_ref, _ = _oracle_prefill(x, 128)
    assert_close(torch.bfloat16, o, o_ref, what="large sink")


def test_prefill_deterministic():
    _say("swa prefill run twice: bitwise identical (LDS race detector)")
    x = wl.make_prefill([2000, 48], 32, 4, 128, "bf16", seed=5)
    o1, l1 = _run_prefill(x, 128)
    o2, l2 = _run_prefill(x, 128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o1, l1 = _run_prefill(x, None, ga=True)
    o2, l2 = _run_prefill(x, None, ga=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# decode / MTP verify
# ---------------------------------------------------------------------------

def _run_decode(x, window):
    g = _gpu(x)
    o, lse = swa.swa_sink_decode(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"],
                                 g["ring_head"], g["sinks"])
    torch.cuda.synchronize()
    return o, lse


def _oracle_decode(x, window):
    return orc.swa_sink_decode(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                               x["ring_head"].numpy(), x["sinks"], window)


@pytest.mark.parametrize("t_new", [1, 2, 3, 4])
def test_decode_small_all_ring_heads(t_new):
    _say(f"decode B=16 T={t_new} 32/4 D128 bf16, ring heads incl. 0 and 127")
    x = wl.make_decode(16, t_new, 32, 4, 128, 128, "bf16", seed=300 + t_new)
    x["ring_head"][0] = 0
    x["ring_head"][1] = 127
    x["ring_head"][2] = 1
    o, lse = _run_decode(x, 128)
    o_ref, l_ref = _oracle_decode(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"decode T={t_new}")


@pytest.mark.parametrize("case", [(6, 16, 2, 128, 128, "bf16"), (3, 8, 1, 64, 128, "bf16"),
                                  (4, 8, 8, 128, 64, "bf16"), (5, 4, 1, 64, 128, "f32"),
                                  (2, 8, 1, 128, 128, "bf16", 8)])
def test_decode_generic_shapes(case):
    b, hq, hkv, d, w, dt = case[:6]
    t_new = case[6] if len(case) > 6 else 3
    _say(f"decode generic B={b} T={t_new} {hq}/{hkv} D{d} W{w} {dt}")
    x = wl.make_decode(b, t_new, hq, hkv, d, w, dt, seed=b * 7 + w)
    o, lse = _run_decode(x, w)
    o_ref, l_ref = _oracle_decode(x, w)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"decode generic {case}")


def test_decode_never_reads_oldest_slot():
    _say("decode: the oldest ring slot holds NaN and must not matter")
    x = wl.make_decode(8, 4, 32, 4, 128, 128, "bf16", seed=77)
    o_ref, l_ref = _oracle_decode(x, 128)
    for b in range(8):
        h = int(x["ring_head"][b])
        x["k_cache"][b, :, h] = float("nan")
        x["v_cache"][b, :, h] = float("nan")
    o, lse = _run_decode(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "decode NaN oldest slot")


# ---------------------------------------------------------------------------
# degenerate inputs
# ---------------------------------------------------------------------------

ZERO_LEN_CASES = [
    (32, 4, 128, "bf16", 128),  # window kernel
    (32, 4, 128, "bf16", 200),  # online kernel with window and sink
    (8, 2, 128, "bf16", 128),   # generic kernel
]


@pytest.mark.parametrize("case", ZERO_LEN_CASES, ids=lambda c: f"{c[0]}/{c[1]}-D{c[2]}-{c[3]}-W{c[4]}")
def test_prefill_zero_length_sequences(case):
    hq, hkv, d, dt, w = case
    lens = [0, 37, 0, 0, 150, 1, 0, 16, 0]
    _say(f"prefill with empty sequences {lens} {hq}/{hkv} W{w}")
    x = wl.make_prefill(lens, hq, hkv, d, dt, seed=900 + w + hq)
    o, lse = _run_prefill(x, w)
    o_ref, l_ref = _oracle_prefill(x, w)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"zero-length sequences W{w}")
    o, lse = _run_prefill(x, None, ga=True)
    o_ref, l_ref = _oracle_prefill(x, None, ga=True)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, "zero-length sequences GA")


@pytest.mark.parametrize("lens", [[0, 0, 1], [0, 0, 0, 2, 0, 0, 3, 0, 0, 0]], ids=["0-0-1", "trailing-empty"])
def test_more_sequences_than_tokens(lens):
    """Packed batches with more (mostly empty) sequences than tokens, e.g. cu_seqlens =
    [0, 0, 0, 1]: every prefill path, the FP8-K/V prefill and the backward."""
    _say(f"prefill with more sequences than tokens: {lens}")
    for hq, hkv, w in ((32, 4, 128), (32, 4, 200), (8, 2, 128)):
        x = wl.make_prefill(lens, hq, hkv, 128, "bf16", seed=950 + w + hq + len(lens))
        assert x["cu_seqlens"].numel() - 1 > x["q"].shape[0]
        o, lse = _run_prefill(x, w)
        o_ref, l_ref = _oracle_prefill(x, w)
        assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"{lens} {hq}/{hkv} W{w}")
        o, lse = _run_prefill(x, None, ga=True)
        o_ref, l_ref = _oracle_prefill(x, None, ga=True)
        assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"{lens} {hq}/{hkv} GA")
    f = wl.make_prefill_fp8(lens, 32, 4, 128, "bf16", seed=960 + len(lens))
    o, lse = _run_prefill_fp8(f, 128)
    o_ref, l_ref = _oracle_prefill_fp8(f, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"{lens} FP8 K/V")
    for hq, hkv in ((32, 4), (8, 2)):  # matrix-core and vector backward paths
        _backward_case(lens, hq, hkv, 128, "bf16", 128, True, seed=970 + hq + len(lens))


def test_empty_stream_and_batch():
    _say("empty prefill stream and empty decode batch")
    x = wl.make_prefill([0, 0], 32, 4, 128, "bf16", seed=1)
    for ga in (False, True):
        o, lse = _run_prefill(x, None if ga else 128, ga=ga)
        assert tuple(o.shape) == (0, 32, 128) and tuple(lse.shape) == (0, 32)
    xd = wl.make_decode(0, 2, 32, 4, 128, 128, "bf16", seed=1)
    o, lse = _run_decode(xd, 128)
    assert tuple(o.shape) == (0, 2, 32, 128) and tuple(lse.shape) == (0, 2, 32)


@pytest.mark.parametrize("case", [(32, 4, 128), (32, 4, 300), (8, 2, 128)],
                         ids=["window", "online", "generic"])
def test_prefill_minus_inf_sinks(case):
    hq, hkv, w = case
    _say(f"prefill with sinks = -inf on a third of the heads ({hq}/{hkv}, W{w})")
    x = wl.make_prefill([333, 64], hq, hkv, 128, "bf16", seed=70 + w)
    x["sinks"][::3] = float("-inf")  # a sink of -inf contributes exp(-inf) = 0: plain SWA
    o, lse = _run_prefill(x, w)
    o_ref, l_ref = _oracle_prefill(x, w)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"-inf sinks W{w}")


def test_decode_longest_draft_run():
    _say("decode T = W - 1 = 127 (generic path)")
    x = wl.make_decode(2, 127, 8, 1, 128, 128, "bf16", seed=127)
    o, lse = _run_decode(x, 128)
    o_ref, l_ref = _oracle_decode(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "decode T=127")


# ---------------------------------------------------------------------------
# full-size workloads (launch configuration of the benchmark)
# ---------------------------------------------------------------------------

def test_swa_prefill_32k_full():
    _say("swa_prefill_32k: 32768 tokens, 32/4, D128, W128, every element")
    x = wl.make_workload("swa_prefill_32k")
    o, lse = _run_prefill(x, 128)
    o_ref, l_ref = _oracle_prefill(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "swa_prefill_32k")


@pytest.mark.parametrize("name", ["decode_t1", "decode_t4"])
def test_decode_full(name):
    _say(f"{name}: 256 sequences, every element")
    x = wl.make_workload(name)
    o, lse = _run_decode(x, 128)
    o_ref, l_ref = _oracle_decode(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, name)


def _sample_rows(x, n_random, seed):
    cu = x["cu_seqlens"].tolist()
    n, hq = x["q"].shape[0], x["q"].shape[1]
    rng = np.random.default_rng(seed)
    toks = set(int(t) for t in rng.integers(0, n, n_random))
    for s in range(len(cu) - 1):  # sequence starts, the first window, ends
        for off in (0, 1, 15, 16, 127, 128, 129):
            if cu[s] + off < cu[s + 1]:
                toks.add(cu[s] + off)
        toks.add(cu[s + 1] - 1)
    rows = [(t, int(h)) for t in sorted(toks) for h in rng.choice(hq, 2, replace=False)]
    return np.array(rows)


def _check_rows(x, o, lse, rows, window, what):
    sinks = None if window is None else x["sinks"]
    o_ref, l_ref = orc.prefill_sample_rows(x["q"], x["k"], x["v"], sinks, x["cu_seqlens"].numpy(),
                                           rows, window=window)
    og = to_np(o)[rows[:, 0], rows[:, 1]]
    lg = to_np(lse)[rows[:, 0], rows[:, 1]]
    assert_close(torch.bfloat16, og, o_ref, lg, l_ref, what)


def test_hybrid_block_full_size():
    _say("hybrid_5to1_32k: 5 SWA layers (every element of layer 0, sampled rows of 1-4) + GA sampled")
    for layer in range(6):
        x = wl.make_workload("hybrid_5to1_32k", layer)
        ga = layer == 5
        o, lse = _run_prefill(x, None if ga else 128, ga=ga)
        if layer == 0:
            o_ref, l_ref = _oracle_prefill(x, 128)
            assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "hybrid layer 0")
        else:
            rows = _sample_rows(x, 96 if ga else 256, seed=layer)
            _check_rows(x, o, lse, rows, None if ga else 128, f"hybrid layer {layer}")


class _Err:
    """Errors of one operator call accumulated over pieces of its output: max-abs of O and
    LSE over all pieces, rel-L2 of O over the whole output."""

    def __init__(self):
        self.max_abs, self.num, self.den, self.lse, self.finite = 0.0, 0.0, 0.0, 0.0, True

    def add(self, o_gpu, o_ref, l_gpu, l_ref):
        og, lg = to_np(o_gpu), to_np(l_gpu)
        diff = og - o_ref
        self.max_abs = max(self.max_abs, float(np.abs(diff).max(initial=0.0)))
        self.num += float((diff * diff).sum())
        self.den += float((o_ref * o_ref).sum())
        self.lse = max(self.lse, float(np.abs(lg - l_ref).max(initial=0.0)))
        self.finite &= bool(np.isfinite(og).all() and np.isfinite(lg).all())

    def check(self, what):
        tol = TOL[torch.bfloat16]
        e = {"max_abs": self.max_abs, "rel_l2": (self.num / max(self.den, 1e-300)) ** 0.5, "finite": self.finite,
             "lse_max_abs": self.lse}
        msg = f"{what}: {e} vs {tol}"
        print(msg, flush=True)
        assert self.finite and e["max_abs"] <= tol["max_abs"] and e["rel_l2"] <= tol["rel_l2"], msg
        assert e["lse_max_abs"] <= tol["lse"], msg


def test_ga_layer_32k_every_row_of_one_head_per_kv_head():
    """The 32K GA layer of the 5:1 block: every query row of four query heads, one per KV head
    (heads 3, 14, 17 and 28), so every tile and workgroup of the launch is compared; the four
    single-head oracle runs go to threads (numpy releases the GIL in its kernels)."""
    from concurrent.futures import ThreadPoolExecutor

    _say("hybrid_5to1_32k GA layer: every row of heads 3, 14, 17, 28 against the oracle")
    x = wl.make_workload("hybrid_5to1_32k", 5)
    o, lse = _run_prefill(x, None, ga=True)
    heads = [3, 14, 17, 28]
    g = x["q"].shape[1] // x["k"].shape[1]
    cu = x["cu_seqlens"].numpy()

    def one(h):
        kvh = h // g
        return orc.ga_causal_prefill(x["q"][:, h:h + 1].contiguous(), x["k"][:, kvh:kvh + 1].contiguous(),
                                     x["v"][:, kvh:kvh + 1].contiguous(), cu)

    with ThreadPoolExecutor(len(heads)) as ex:
        refs = list(ex.map(one, heads))
    err = _Err()
    for h, (o_ref, l_ref) in zip(heads, refs):
        err.add(o[:, h], o_ref[:, 0], lse[:, h], l_ref[:, 0])
    err.check("GA 32K, 4 heads every row")


def test_varlen_262k_full():
    """The 262,144-token varlen workload: every element against the oracle, one sequence at a
    time (sequences are independent: no attention crosses a boundary), so the fp64 copies
    stay bounded by the longest sequence."""
    from concurrent.futures import ThreadPoolExecutor

    _say("varlen_262k: 8 log-normal sequences, 262144 tokens, every element")
    x = wl.make_workload("varlen_262k")
    o, lse = _run_prefill(x, 128)
    cu = x["cu_seqlens"].tolist()

    def one(s):
        c0, c1 = cu[s], cu[s + 1]
        return orc.swa_sink_prefill(x["q"][c0:c1], x["k"][c0:c1], x["v"][c0:c1], x["sinks"],
                                    np.array([0, c1 - c0]), 128)

    err = _Err()
    order = sorted(range(len(cu) - 1), key=lambda s: cu[s] - cu[s + 1])  # longest first
    with ThreadPoolExecutor(2) as ex:
        for s, (o_ref, l_ref) in zip(order, ex.map(one, order)):
            err.add(o[cu[s]:cu[s + 1]], o_ref, lse[cu[s]:cu[s + 1]], l_ref)
            del o_ref, l_ref
    err.check("varlen_262k every element")


# ---------------------------------------------------------------------------
# maximum sizes: byte offsets of q / out beyond 2^32, caches beyond 2^31 elements
# ---------------------------------------------------------------------------

def _oracle_rows_from_device(x, rows, window):
    """Oracle values at (token, head) pairs of a device-resident stream too large
    for the host.  Each pair becomes the one-sequence problem made of its visible
    keys (its window inside its own sequence, or the whole prefix for window=None),
    to which the definition gives the same value."""
    import bisect

    cu = x["cu_seqlens"].tolist()
    hq, d = x["q"].shape[1], x["q"].shape[2]
    sinks = None if window is None else x["sinks"]
    o_ref, l_ref = [], []
    for t, h in rows:
        t, h = int(t), int(h)
        s = bisect.bisect_right(cu, t) - 1
        k0 = cu[s] if window is None else max(cu[s], t - window + 1)
        qs = torch.zeros((t - k0 + 1, hq, d), dtype=torch.bfloat16)
        qs[-1] = x["q"][t].cpu()
        ks, vs = x["k"][k0:t + 1].cpu(), x["v"][k0:t + 1].cpu()
        oo, ll = orc.prefill_sample_rows(qs, ks, vs, sinks, np.array([0, t - k0 + 1]),
                                         np.array([[t - k0, h]]), window=window)
        o_ref.append(oo[0])
        l_ref.append(ll[0])
    return np.array(o_ref), np.array(l_ref)


def _device_rows(o, lse, rows):
    idx_t = torch.tensor(rows[:, 0], device=o.device)
    idx_h = torch.tensor(rows[:, 1], device=o.device)
    return to_np(o[idx_t, idx_h]), to_np(lse[idx_t, idx_h])


def test_swa_prefill_max_size_sampled():
    n1, n = 1_300_001, (1 << 21) + 37
    _say(f"SWA prefill {n} tokens in 2 sequences, 32/4 D128 W128: q/out byte offsets past 2^33")
    x = wl.make_prefill_device([n1, n - n1], 32, 4, 128, seed=6000, device=DEV)
    o, lse = swa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"].to(DEV), x["cu_seqlens"].to(DEV),
                                  x["max_seqlen"], window=128)
    torch.cuda.synchronize()
    per_tok = 32 * 128  # q elements per token: token 2^19 starts past 2^31 elements (2^32 bytes)
    special = [0, 1, 15, 16, 127, 128, (1 << 31) // per_tok - 1, (1 << 31) // per_tok,
               (1 << 32) // per_tok - 1, (1 << 32) // per_tok, n1 - 1, n1, n1 + 1, n1 + 127, n1 + 128,
               n - 17, n - 1]
    rng = np.random.default_rng(6000)
    toks = special + [int(t) for t in rng.integers(0, n, 40)]
    rows = np.array([(t, int(h)) for t in toks for h in rng.choice(32, 2, replace=False)])
    og, lg = _device_rows(o, lse, rows)
    o_ref, l_ref = _oracle_rows_from_device(x, rows, 128)
    assert_close(torch.bfloat16, og, o_ref, lg, l_ref, "SWA max size")
    del x, o, lse
    torch.cuda.empty_cache()


def test_ga_prefill_many_sequences_sampled():
    lens = [4096] * 512
    _say("GA prefill 512 x 4096 tokens, 32/4 D128: q/out byte offsets past 2^33")
    x = wl.make_prefill_device(lens, 32, 4, 128, seed=6100, device=DEV)
    o, lse = swa.ga_causal_prefill(x["q"], x["k"], x["v"], x["cu_seqlens"].to(DEV), x["max_seqlen"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(6100)
    toks = [0, 4095, 4096, 4097, (1 << 19) - 1, 1 << 19, (1 << 20) + 4095, (1 << 21) - 1]
    toks += [int(t) for t in rng.integers(0, 1 << 21, 24)]
    rows = np.array([(t, int(h)) for t in toks for h in rng.choice(32, 2, replace=False)])
    og, lg = _device_rows(o, lse, rows)
    o_ref, l_ref = _oracle_rows_from_device(x, rows, None)
    assert_close(torch.bfloat16, og, o_ref, lg, l_ref, "GA many sequences")
    del x, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("t_new", [1, 3])
def test_decode_max_batch_sampled(t_new):
    b = 32771  # caches hold 4 x 128 x 128 elements per sequence: past 2^31 at sequence 32768
    _say(f"decode B={b} T={t_new} 32/4 D128 W128: caches past 2^31 elements")
    x = wl.make_decode_device(b, t_new, 32, 4, 128, 128, seed=6200 + t_new, device=DEV)
    o, lse = swa.swa_sink_decode(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                 x["ring_head"].to(DEV), x["sinks"].to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(6200)
    picks = sorted(set([0, 1, 16383, 32766, 32767, 32768, 32769, b - 1] + [int(v) for v in rng.integers(0, b, 8)]))
    for bi in picks:
        sl = {k: (v[bi:bi + 1].cpu() if k not in ("sinks",) else v) for k, v in x.items()}
        o_ref, l_ref = _oracle_decode(sl, 128)
        assert_close(torch.bfloat16, o[bi:bi + 1], o_ref, lse[bi:bi + 1], l_ref, f"decode max batch b={bi}")
    del x, o, lse
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# decode against an FP8 (E4M3) ring
# ---------------------------------------------------------------------------

def _run_decode_fp8(x):
    g = _gpu(x)
    o, lse = swa.swa_sink_decode_fp8kv(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"],
                                       x["k_scale"], x["v_scale"], g["ring_head"], g["sinks"])
    torch.cuda.synchronize()
    return o, lse


def _oracle_decode_fp8(x, window):
    return orc.swa_sink_decode_fp8kv(x["q"], x["k_new"], x["v_new"], x["k_cache"].numpy(),
                                     x["v_cache"].numpy(), x["k_scale"], x["v_scale"],
                                     x["ring_head"].numpy(), x["sinks"], window)


@pytest.mark.parametrize("t_new", [1, 2, 3, 4])
def test_decode_fp8_small_all_ring_heads(t_new):
    _say(f"FP8 ring decode B=16 T={t_new} 32/4 D128 bf16, ring heads incl. 0 and 127")
    x = wl.make_decode_fp8(16, t_new, 32, 4, 128, 128, "bf16", seed=700 + t_new)
    x["ring_head"][0], x["ring_head"][1], x["ring_head"][2] = 0, 127, 1
    o, lse = _run_decode_fp8(x)
    o_ref, l_ref = _oracle_decode_fp8(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"FP8 decode T={t_new}")


def test_decode_fp8_every_finite_code():
    _say("FP8 ring decode: every finite E4M3 code (subnormals, +-448) in K and V")
    x = wl.make_decode_fp8(8, 3, 32, 4, 128, 128, "bf16", seed=777)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    n = x["k_cache"].numel()
    idx = torch.arange(n)
    x["k_cache"] = finite[idx % len(finite)].reshape(x["k_cache"].shape)
    x["v_cache"] = finite[(idx * 7 + 3) % len(finite)].reshape(x["v_cache"].shape)
    x["k_scale"], x["v_scale"] = 1.0 / 448, 1.0 / 448
    o, lse = _run_decode_fp8(x)
    o_ref, l_ref = _oracle_decode_fp8(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "FP8 every code")


@pytest.mark.parametrize("case", [(6, 16, 2, 128, 128, "bf16", 3), (3, 8, 1, 64, 128, "bf16", 2),
                                  (4, 8, 8, 128, 64, "bf16", 5), (5, 4, 1, 64, 128, "f32", 3),
                                  (2, 8, 1, 128, 128, "bf16", 8)])
def test_decode_fp8_generic_shapes(case):
    b, hq, hkv, d, w, dt, t_new = case
    _say(f"FP8 ring decode generic B={b} T={t_new} {hq}/{hkv} D{d} W{w} {dt}")
    x = wl.make_decode_fp8(b, t_new, hq, hkv, d, w, dt, seed=b * 11 + w)
    o, lse = _run_decode_fp8(x)
    o_ref, l_ref = _oracle_decode_fp8(x, w)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"FP8 decode generic {case}")


def test_decode_fp8_never_reads_oldest_slot():
    _say("FP8 ring decode: the oldest ring slot holds the NaN code and must not matter")
    x = wl.make_decode_fp8(8, 4, 32, 4, 128, 128, "bf16", seed=78)
    o_ref, l_ref = _oracle_decode_fp8(x, 128)
    for bi in range(8):
        h = int(x["ring_head"][bi])
        x["k_cache"][bi, :, h] = 0x7F
        x["v_cache"][bi, :, h] = 0xFF
    o, lse = _run_decode_fp8(x)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "FP8 decode NaN oldest slot")


@pytest.mark.parametrize("name", ["decode_fp8_t1", "decode_fp8_t4"])
def test_decode_fp8_full(name):
    _say(f"{name}: 256 sequences, FP8 ring, every element")
    x = wl.make_workload(name)
    o, lse = _run_decode_fp8(x)
    o_ref, l_ref = _oracle_decode_fp8(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, name)


def test_decode_fp8_max_batch_sampled():
    b = 32771  # FP8 caches of 4 x 128 x 128 bytes per sequence: past 2^31 bytes at sequence 32768
    _say(f"FP8 ring decode B={b} T=2 32/4 D128: caches past 2^31 bytes")
    x = wl.make_decode_device(b, 2, 32, 4, 128, 128, seed=6300, device=DEV)
    gen = torch.Generator().manual_seed(6301)
    shape = (b, 4, 128, 128)
    x["k_cache"] = wl.e4m3_codes(shape, gen).to(DEV)
    x["v_cache"] = wl.e4m3_codes(shape, gen).to(DEV)
    x["k_scale"], x["v_scale"] = 1.0 / 32, 1.0 / 64
    o, lse = swa.swa_sink_decode_fp8kv(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                       x["k_scale"], x["v_scale"], x["ring_head"].to(DEV),
                                       x["sinks"].to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(6300)
    picks = sorted(set([0, 1, 32767, 32768, 32769, b - 1] + [int(v) for v in rng.integers(0, b, 8)]))
    for bi in picks:
        sl = {k: (v[bi:bi + 1].cpu() if isinstance(v, torch.Tensor) and k != "sinks" else v)
              for k, v in x.items()}
        o_ref, l_ref = _oracle_decode_fp8(sl, 128)
        assert_close(torch.bfloat16, o[bi:bi + 1], o_ref, lse[bi:bi + 1], l_ref, f"FP8 max batch b={bi}")
    del x, o, lse
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# prefill with FP8 (E4M3) K and V
# ---------------------------------------------------------------------------

def _run_prefill_fp8(x, window, k_scale=None, v_scale=None):
    g = _gpu(x)
    o, lse = swa.swa_sink_prefill_fp8kv(
        g["q"], g["k"], g["v"], x["k_scale"] if k_scale is None else k_scale,
        x["v_scale"] if v_scale is None else v_scale, g["sinks"], g["cu_seqlens"], x["max_seqlen"],
        window=window)
    torch.cuda.synchronize()
    return o, lse


def _oracle_prefill_fp8(x, window):
    return orc.swa_sink_prefill_fp8kv(x["q"], x["k"].numpy(), x["v"].numpy(), x["k_scale"], x["v_scale"],
                                      x["sinks"], x["cu_seqlens"].numpy(), window=window)


PREFILL_FP8_CASES = [
    # (lengths, Hq, Hkv, D, dtype, window (None: unbounded), sinks)
    ([700], 32, 4, 128, "bf16", 128, True),                 # window kernel, ragged tail
    ([130, 1, 17, 300, 5], 16, 2, 128, "bf16", 100, True),  # boundaries inside tiles, G = 8
    ([7], 32, 4, 128, "bf16", 128, True),                   # fewer tokens than one tile
    ([520, 45], 32, 4, 128, "bf16", 200, True),             # online kernel, window + sink
    ([600, 33], 16, 2, 128, "bf16", None, False),           # GA kernel
    ([300, 77], 8, 2, 128, "bf16", 128, True),              # generic kernel (G = 4)
    ([250], 8, 1, 64, "bf16", None, False),                 # generic kernel, D = 64, GA
    ([200, 3], 4, 2, 128, "f32", 50, True),                 # generic fp32
]


@pytest.mark.parametrize("case", PREFILL_FP8_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}/{c[2]}-D{c[3]}-{c[4]}-W{c[5]}-{'sink' if c[6] else 'nosink'}")
def test_prefill_fp8kv_small(case):
    lens, hq, hkv, d, dt, window, with_sinks = case
    _say(f"FP8 K/V prefill lens={lens} heads={hq}/{hkv} D={d} {dt} W={window} sinks={with_sinks}")
    x = wl.make_prefill_fp8(lens, hq, hkv, d, dt, seed=2300 + sum(lens) + hq, with_sinks=with_sinks)
    o, lse = _run_prefill_fp8(x, window)
    o_ref, l_ref = _oracle_prefill_fp8(x, window)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"fp8 prefill {case}")


@pytest.mark.parametrize("window", [128, 100, None])
def test_prefill_fp8kv_unit_scales_equal_bf16_prefill(window):
    """Every E4M3 value is a bf16 value and the kernels widen codes exactly, so with unit scales
    the FP8 prefill is bitwise the bf16 prefill on the decoded K/V (decoded by torch's
    float8_e4m3fn): window kernel, and with no window and no sink the GA kernel."""
    _say(f"FP8 K/V prefill, unit scales, against the bf16 prefill (W={window})")
    lens = [900, 140, 3]
    x = wl.make_prefill_fp8(lens, 32, 4, 128, "bf16", seed=2400, with_sinks=window is not None)
    o8, l8 = _run_prefill_fp8(x, window, 1.0, 1.0)
    g = _gpu(x)
    kd = g["k"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    vd = g["v"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    if window is None:
        ob, lb = swa.ga_causal_prefill(g["q"], kd, vd, g["cu_seqlens"], x["max_seqlen"])
    else:
        ob, lb = swa.swa_sink_prefill(g["q"], kd, vd, g["sinks"], g["cu_seqlens"], x["max_seqlen"],
                                      window=window)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob) and torch.equal(l8, lb)


def test_prefill_fp8kv_32k_full():
    _say("swa_prefill_fp8kv_32k: 32768 tokens, 32/4, D128, W128, E4M3 K/V, every element")
    x = wl.make_workload("swa_prefill_fp8kv_32k")
    o, lse = _run_prefill_fp8(x, 128)
    o_ref, l_ref = _oracle_prefill_fp8(x, 128)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "swa_prefill_fp8kv_32k")


# ---------------------------------------------------------------------------
# backward (gradients of O)
# ---------------------------------------------------------------------------

INT_MAX = 2 ** 31 - 1


def assert_grads_close(dtype, got, ref, what):
    """Gradient bar derived from the arithmetic: fp32 accumulation on exact inputs, outputs
    rounded to the I/O type (bf16: 2^-9 relative), and delta = dO . O taken on the forward output
    as stored (bf16-rounded; the matrix-core path forms delta from its recomputed weights
    instead, which only brings it closer to the oracle's), so bf16 errors are a few 2^-9 of the
    largest gradient: max-abs <= 1e-2 * max(1, max |ref|) and rel-L2 <= 1e-2; fp32: 1e-4 and 1e-5."""
    g = to_np(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), what
    err = np.abs(g - r)
    scale = max(1.0, float(np.abs(r).max(initial=0.0)))
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    tol_abs, tol_rel = (1e-2, 1e-2) if dtype == torch.bfloat16 else (1e-4, 1e-5)
    msg = f"{what}: max_abs {err.max(initial=0.0):.3e} (scale {scale:.3e}), rel_l2 {rel:.3e}"
    print(msg, flush=True)
    assert err.max(initial=0.0) <= tol_abs * scale, msg
    assert rel <= tol_rel or np.linalg.norm(r) < 1e-6, msg


def _backward_case(lens, hq, hkv, d, dt, window, sink=True, seed=0):
    """GPU backward against the oracle.  The forward output (rounded to the I/O type) and its
    LSE come from the oracle, so no GPU value feeds the comparison."""
    x = wl.make_prefill(lens, hq, hkv, d, dt, seed, with_sinks=sink)
    gen = torch.Generator().manual_seed(seed + 1)
    td = x["q"].dtype
    dout = torch.randn(x["q"].shape, generator=gen).to(td)
    cu = x["cu_seqlens"].numpy()
    w = None if window is None else window
    if w is None:
        o_ref, l_ref = orc.ga_causal_prefill(x["q"], x["k"], x["v"], cu)
    else:
        o_ref, l_ref = orc.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], cu, w)
    g = _gpu(x)
    out = torch.tensor(o_ref).to(td).to(DEV)
    lse = torch.tensor(l_ref, dtype=torch.float32, device=DEV)
    dq, dk, dv, ds = swa.swa_sink_prefill_backward(
        g["q"], g["k"], g["v"], g["sinks"] if sink else None, g["cu_seqlens"], out, lse, dout.to(DEV),
        x["max_seqlen"], window=INT_MAX if w is None else w)
    torch.cuda.synchronize()
    rq, rk, rv, rs = orc.swa_sink_prefill_backward(x["q"], x["k"], x["v"], x["sinks"] if sink else None,
                                                   cu, dout, window=w)
    tag = f"{lens} {hq}/{hkv} D{d} {dt} W{window}"
    assert_grads_close(td, dq, rq, f"dq {tag}")
    assert_grads_close(td, dk, rk, f"dk {tag}")
    assert_grads_close(td, dv, rv, f"dv {tag}")
    if sink:
        # dsink_h = -sum_i p_s(i) delta_i with delta_i = dO_i . O_i taken on O as stored (the
        # vector path; the matrix-core path forms delta from its recomputed weights, nearer the
        # oracle's): rounding each O element (2^-9 relative in bf16, 2^-24 in fp32) moves dsink_h
        # by at most u * sum_i p_s(i) sum_d |dO_id O_id|; the bar is twice that plus fp32
        # accumulation slack
        u = 2.0 ** -9 if td == torch.bfloat16 else 2.0 ** -24
        p_s = np.exp(x["sinks"].double().numpy()[None, :] - l_ref)          # [N, Hq]
        mag = (np.abs(dout.double().numpy()) * np.abs(o_ref)).sum(axis=2)   # [N, Hq]
        bound = 2 * u * (p_s * mag).sum(axis=0) + 1e-5 * (p_s * mag).sum(axis=0) + 1e-6
        err = np.abs(to_np(ds) - rs)
        msg = f"dsinks {tag}: max err {err.max():.3e}, max err / bound {(err / bound).max():.3f}"
        print(msg, flush=True)
        assert np.all(err <= bound), msg
    else:
        assert ds is None
    return dq, dk, dv, ds


BACKWARD_CASES = [
    ([300, 45], 32, 4, 128, "bf16", 128, True),
    ([130, 1, 17], 8, 1, 128, "bf16", 37, True),
    ([200], 8, 2, 64, "bf16", 128, True),        # group size 4, head_dim 64
    ([150, 3], 4, 2, 128, "f32", 50, True),
    ([200, 31], 16, 2, 128, "bf16", None, False),  # GA: no window, no sink
    ([0, 37, 0, 60, 0], 8, 1, 128, "bf16", 128, True),  # zero-length sequences
    # matrix-core path (bf16, D128, groups of 8k heads, window <= 128)
    ([7], 8, 1, 128, "bf16", 128, True),                 # one partial tile
    ([5, 0, 33, 17, 1, 200, 64], 32, 2, 128, "bf16", 128, True),  # group 16, boundaries inside tiles
    ([333], 8, 1, 128, "bf16", 1, True),                 # window 1: the diagonal only
    ([260, 19], 16, 2, 128, "bf16", 100, False),         # no sink, window 100
    ([129, 127, 16], 8, 1, 128, "bf16", 16, True),       # window of one key block
]


@pytest.mark.parametrize("case", BACKWARD_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}/{c[2]}-D{c[3]}-{c[4]}-W{c[5]}-{'sink' if c[6] else 'nosink'}")
def test_backward_small(case):
    lens, hq, hkv, d, dt, w, sink = case
    _say(f"backward {lens} {hq}/{hkv} D{d} {dt} W{w} sink={sink}")
    _backward_case(lens, hq, hkv, d, dt, w, sink, seed=8000 + sum(lens) + (w or 0))


def test_backward_empty_stream_and_determinism():
    _say("backward: empty stream writes zero sink gradients; two calls are bitwise identical")
    x = wl.make_prefill([0, 0], 8, 1, 128, "bf16", seed=1)
    z = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    dq, dk, dv, ds = swa.swa_sink_prefill_backward(
        z, torch.zeros((0, 1, 128), dtype=torch.bfloat16, device=DEV),
        torch.zeros((0, 1, 128), dtype=torch.bfloat16, device=DEV), x["sinks"].to(DEV),
        x["cu_seqlens"].to(DEV), z, torch.zeros((0, 8), device=DEV), z, 0)
    torch.cuda.synchronize()
    assert tuple(dq.shape) == (0, 8, 128) and bool((ds == 0).all())
    a = _backward_case([257, 100], 32, 4, 128, "bf16", 128, True, seed=8100)
    b = _backward_case([257, 100], 32, 4, 128, "bf16", 128, True, seed=8100)
    for u, w_ in zip(a, b):
        assert torch.equal(u, w_)


def test_backward_32k_layer():
    _say("backward of the 32K SWA-sink layer (32/4, D128, W128): every gradient element")
    _backward_case([32768], 32, 4, 128, "bf16", 128, True, seed=wl.WORKLOADS["swa_prefill_32k"].seed)


def test_backward_max_size_sampled():
    """Backward of a 2^21 + 37-token stream in 2 sequences (q, dout, dq byte offsets past
    2^33), on sampled outputs: dq of (token, head) rows and dk, dv of (key, KV head) rows,
    each from the oracle's backward of the tokens around it -- dq_t depends only on row t's
    window, dk_j and dv_j only on queries j .. j + 127 of j's sequence, whose windows lie in
    the window before j -- so each small problem gives exactly the values of the full one.
    The GPU backward takes its out and lse from the library's forward (its inputs, as in the
    bench); every expected value comes from the oracle on the seeded q, k, v and dout.  The
    sink gradient sums over every token and is checked at full size by the 32K test."""
    import bisect

    n1, n = 1_300_001, (1 << 21) + 37
    _say(f"backward {n} tokens in 2 sequences, 32/4 D128 W128: byte offsets past 2^33")
    x = wl.make_prefill_device([n1, n - n1], 32, 4, 128, seed=6400, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(6401)
    dout = wl._randn_device(x["q"].shape, gen, DEV, torch.bfloat16)
    sinks, cu_d = x["sinks"].to(DEV), x["cu_seqlens"].to(DEV)
    out, lse = swa.swa_sink_prefill(x["q"], x["k"], x["v"], sinks, cu_d, x["max_seqlen"], window=128)
    dq, dk, dv, _ = swa.swa_sink_prefill_backward(x["q"], x["k"], x["v"], sinks, cu_d, out, lse, dout,
                                                  x["max_seqlen"], window=128)
    torch.cuda.synchronize()
    del out, lse
    cu = x["cu_seqlens"].tolist()
    per_tok = 32 * 128
    special = [0, 1, 127, 128, (1 << 31) // per_tok, (1 << 32) // per_tok - 1, (1 << 32) // per_tok,
               n1 - 1, n1, n1 + 1, n1 + 128, n - 1]
    rng = np.random.default_rng(6400)
    toks = special + [int(t) for t in rng.integers(0, n, 12)]

    def local(a, b):  # oracle backward of tokens a .. b (one sequence)
        sl = slice(a, b + 1)
        return orc.swa_sink_prefill_backward(x["q"][sl].cpu(), x["k"][sl].cpu(), x["v"][sl].cpu(),
                                             x["sinks"], np.array([0, b - a + 1]), dout[sl].cpu(), window=128)

    got_q, ref_q, got_kv, ref_k, ref_v = [], [], [], [], []
    for t in toks:
        s0 = cu[bisect.bisect_right(cu, t) - 1]
        s1 = cu[bisect.bisect_right(cu, t)]
        a = max(s0, t - 127)
        rq, _, _, _ = local(a, t)                      # row t's window is whole
        got_q.append(to_np(dq[t]))
        ref_q.append(rq[t - a])
        b = min(s1 - 1, t + 127)
        _, rk, rv, _ = local(a, b)                     # every query that sees key t
        got_kv.append((to_np(dk[t]), to_np(dv[t])))
        ref_k.append(rk[t - a])
        ref_v.append(rv[t - a])
    tag = f"{n} tokens, {len(toks)} sampled tokens"
    assert_grads_close(torch.bfloat16, torch.tensor(np.array(got_q)), np.array(ref_q), f"dq {tag}")
    assert_grads_close(torch.bfloat16, torch.tensor(np.array([g[0] for g in got_kv])), np.array(ref_k), f"dk {tag}")
    assert_grads_close(torch.bfloat16, torch.tensor(np.array([g[1] for g in got_kv])), np.array(ref_v), f"dv {tag}")
    del x, dout, dq, dk, dv
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# rotary embedding around decode: in place, inside the decode, ring append
# ---------------------------------------------------------------------------

def _ulp(y, dtype):
    """Spacing of the I/O type at |y| (bf16: 8 significant bits; fp32: 24)."""
    bits = 8 if dtype == torch.bfloat16 else 24
    a = np.maximum(np.abs(y), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - (bits - 1))


def assert_rotated_close(got, x, ref, dtype, what):
    """Rotated values against the fp64 oracle: within half a unit in the last place of
    the I/O type (the oracle's rounding) plus the fp32 rotation error, bounded by
    1e-5 (|x_i| + |x_pair|) for angles reduced in fp64.  For bf16 output, where the
    fp32 rotation is far finer than the output spacing, at least 99.9% must also be
    bit-identical to the oracle rounded to bf16 (fp32 output differs from a rounded
    fp64 result in the last bit about half the time, so no such check there)."""
    g = to_np(got).astype(np.float64)
    xs = np.abs(np.asarray(x, dtype=np.float64))
    half = xs.shape[-1] // 2
    pair = np.concatenate([xs[..., half:], xs[..., :half]], axis=-1)
    bound = 0.5 * _ulp(ref, dtype) + 1e-5 * (xs + pair)
    err = np.abs(g - ref)
    same = float(np.mean(g == orc.round_to(ref, "bf16" if dtype == torch.bfloat16 else "f32")))
    msg = f"{what}: max err/bound {float((err / bound).max()):.3f}, identical {same:.5f}"
    print(msg, flush=True)
    assert np.isfinite(g).all() and np.all(err <= bound), msg
    if dtype == torch.bfloat16:
        assert same >= 0.999, msg


@pytest.mark.parametrize("case", [(1000, 8, 128, "bf16", 10000.0), (513, 4, 64, "bf16", 640000.0),
                                  (300, 2, 128, "f32", 5e6), (77, 32, 128, "bf16", 5e6)],
                         ids=lambda c: f"{c[0]}x{c[1]}-D{c[2]}-{c[3]}-base{c[4]:g}")
def test_rope_in_place(case):
    rows, heads, d, dt, base = case
    _say(f"rope in place {rows}x{heads} D{d} {dt} base {base:g}")
    gen = torch.Generator().manual_seed(rows + heads)
    x = torch.randn(rows, heads, d, generator=gen).to(wl._torch_dtype(dt))
    pos = torch.randint(0, 1 << 20, (rows,), generator=gen, dtype=torch.int64)
    pos[:4] = torch.tensor([0, 1, 2 ** 31 - 1, -12345])  # identity, first step, extremes
    pos = pos.to(torch.int32)
    xd = x.to(DEV)
    swa.swa_rope(xd, pos.to(DEV), base)
    torch.cuda.synchronize()
    ref = orc.rope(x, pos.numpy(), base)
    assert_rotated_close(xd, x.double().numpy(), ref, x.dtype, f"rope {case}")
    assert torch.equal(xd[0].cpu(), x[0])  # position 0 is the identity, bit for bit


def _run_decode_rope(x, base):
    g = _gpu(x)
    o, lse = swa.swa_sink_decode_rope(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"],
                                      g["ring_head"], g["positions"], g["sinks"], base)
    torch.cuda.synchronize()
    return o, lse


def _oracle_decode_rope(x, window, base):
    io = "bf16" if x["q"].dtype == torch.bfloat16 else "f32"
    return orc.swa_sink_decode_rope(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                    x["ring_head"].numpy(), x["positions"].numpy(), x["sinks"], base,
                                    window, io_dtype=io)


@pytest.mark.parametrize("t_new", [1, 4])
def test_decode_without_lse(t_new):
    """return_lse=False takes the decode kernels' branch that writes no LSE: the outputs are
    bitwise those of the same call with the LSE written (bf16 ring, FP8 ring, RoPE in the
    kernel), and the bf16 ring's match the oracle."""
    _say(f"decode T={t_new} without LSE (bf16 ring, FP8 ring, RoPE): bitwise vs with LSE, and vs the oracle")
    x = wl.make_decode(16, t_new, 32, 4, 128, 128, "bf16", seed=4400 + t_new)
    g = _gpu(x)
    args = (g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"], g["ring_head"], g["sinks"])
    o1, lse1 = swa.swa_sink_decode(*args)
    o0, lse0 = swa.swa_sink_decode(*args, return_lse=False)
    torch.cuda.synchronize()
    assert lse0 is None
    assert torch.equal(o0, o1)
    o_ref, l_ref = _oracle_decode(x, 128)
    assert_close(torch.bfloat16, o0, o_ref, lse1, l_ref, f"decode T={t_new} without LSE")

    xf = wl.make_decode_fp8(16, t_new, 32, 4, 128, 128, "bf16", seed=4500 + t_new)
    gf = _gpu(xf)
    fargs = (gf["q"], gf["k_new"], gf["v_new"], gf["k_cache"], gf["v_cache"], xf["k_scale"], xf["v_scale"],
             gf["ring_head"], gf["sinks"])
    o1, _ = swa.swa_sink_decode_fp8kv(*fargs)
    o0, lse0 = swa.swa_sink_decode_fp8kv(*fargs, return_lse=False)
    torch.cuda.synchronize()
    assert lse0 is None
    assert torch.equal(o0, o1)

    xr = wl.make_decode_rope(16, t_new, 32, 4, 128, 128, "bf16", seed=4600 + t_new)
    gr = _gpu(xr)
    rargs = (gr["q"], gr["k_new"], gr["v_new"], gr["k_cache"], gr["v_cache"], gr["ring_head"], gr["positions"],
             gr["sinks"], 10000.0)
    o1, _ = swa.swa_sink_decode_rope(*rargs)
    o0, lse0 = swa.swa_sink_decode_rope(*rargs, return_lse=False)
    torch.cuda.synchronize()
    assert lse0 is None
    assert torch.equal(o0, o1)


@pytest.mark.parametrize("t_new", [1, 2, 3, 4])
def test_decode_rope_small(t_new):
    _say(f"decode with RoPE B=16 T={t_new} 32/4 D128 bf16 (matrix cores), positions up to 2^31")
    x = wl.make_decode_rope(16, t_new, 32, 4, 128, 128, "bf16", seed=3600 + t_new)
    x["positions"][0] = 128
    x["positions"][1] = 2 ** 31 - 8  # new tokens up to 2^31 - 5
    x["ring_head"][2] = 127
    for base in (10000.0, 5e6):
        o, lse = _run_decode_rope(x, base)
        o_ref, l_ref = _oracle_decode_rope(x, 128, base)
        assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"decode rope T={t_new} base {base:g}")


@pytest.mark.parametrize("case", [(6, 16, 2, 128, 128, "bf16", 3), (3, 8, 1, 64, 128, "bf16", 2),
                                  (4, 8, 8, 128, 64, "bf16", 4), (5, 4, 1, 64, 128, "f32", 3),
                                  (2, 8, 1, 128, 128, "bf16", 8)])
def test_decode_rope_generic_shapes(case):
    b, hq, hkv, d, w, dt, t_new = case
    _say(f"decode with RoPE generic B={b} T={t_new} {hq}/{hkv} D{d} W{w} {dt}")
    x = wl.make_decode_rope(b, t_new, hq, hkv, d, w, dt, seed=3700 + b * 7 + w)
    o, lse = _run_decode_rope(x, 640000.0)
    o_ref, l_ref = _oracle_decode_rope(x, w, 640000.0)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"decode rope generic {case}")


def test_decode_rope_base_zero_is_plain_decode():
    _say("decode with rope_base 0 equals swa_sink_decode bit for bit")
    x = wl.make_decode_rope(8, 4, 32, 4, 128, 128, "bf16", seed=3800)
    o, lse = _run_decode_rope(x, 0.0)
    o2, l2 = _run_decode(x, 128)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("case", [(16, 4, 4, 128, 128, "bf16", 10000.0), (9, 3, 2, 64, 32, "f32", 640000.0),
                                  (5, 2, 1, 128, 128, "bf16", 0.0),
                                  (6, 12, 2, 128, 128, "bf16", 10000.0)],  # T > 8: angles per element
                         ids=lambda c: f"B{c[0]}-T{c[1]}-kv{c[2]}-D{c[3]}-W{c[4]}-{c[5]}-base{c[6]:g}")
def test_ring_append(case):
    b, t_new, hkv, d, w, dt, base = case
    _say(f"ring append B={b} T={t_new} kv {hkv} D{d} W{w} {dt} base {base:g}")
    x = wl.make_decode_rope(b, t_new, hkv, hkv, d, w, dt, seed=3900 + b)
    gen = torch.Generator().manual_seed(3901 + b)
    n_acc = torch.randint(0, t_new + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32)
    n_acc[0], n_acc[1] = t_new + 3, -2  # clamped to T and to 0
    x["ring_head"][2] = w - 1           # writes wrap around the ring
    x["ring_head"][3] = 3 * w + 1       # reduced modulo W
    g = _gpu(x)
    heads = g["ring_head"].clone()
    swa.swa_ring_append_rope(g["k_new"], g["v_new"], n_acc.to(DEV), g["positions"], g["k_cache"],
                             g["v_cache"], heads, base)
    torch.cuda.synchronize()
    io = "bf16" if dt == "bf16" else "f32"
    kc, vc, h2 = orc.swa_ring_append_rope(x["k_new"], x["v_new"], np.clip(n_acc.numpy(), 0, t_new),
                                          x["positions"].numpy(), x["k_cache"], x["v_cache"],
                                          x["ring_head"].numpy(), base or None, io_dtype=io)
    assert np.array_equal(heads.cpu().numpy(), h2)
    assert np.array_equal(to_np(g["v_cache"]), vc)  # values copied bit for bit
    got_k = to_np(g["k_cache"])
    written = np.zeros(got_k.shape[:3], dtype=bool)  # [B, Hkv, W]
    for bb in range(b):
        n = int(np.clip(n_acc[bb], 0, t_new))
        for t in range(n):
            written[bb, :, (int(x["ring_head"][bb]) % w + t) % w] = True
    assert np.array_equal(got_k[~written], to_np(x["k_cache"])[~written])  # untouched slots
    if base == 0.0:
        assert np.array_equal(got_k, kc)
    else:
        kraw = np.zeros_like(kc)
        for bb in range(b):
            n = int(np.clip(n_acc[bb], 0, t_new))
            for t in range(n):
                kraw[bb, :, (int(x["ring_head"][bb]) % w + t) % w] = x["k_new"][bb, t].double().numpy()
        kref = orc.swa_ring_append_rope(x["k_new"], x["v_new"], np.clip(n_acc.numpy(), 0, t_new),
                                        x["positions"].numpy(), x["k_cache"], x["v_cache"],
                                        x["ring_head"].numpy(), base, io_dtype=None)[0]
        assert_rotated_close(torch.from_numpy(got_k[written]), kraw[written], kref[written],
                             x["k_new"].dtype, f"append keys {case}")


def test_decode_and_append_steps_follow_the_oracle():
    """Five MTP steps: verify T = 4 tokens against the ring (RoPE in the kernel), accept a
    seeded 0..4 of them, commit those to the ring (keys rotated), advance the positions;
    the GPU state and every step's outputs follow the oracle run on the same inputs."""
    _say("decode + append: 5 MTP steps, B=8, 32/4 D128 bf16")
    b, t_new, hq, hkv, d, w, base = 8, 4, 32, 4, 128, 128, 10000.0
    x = wl.make_decode_rope(b, t_new, hq, hkv, d, w, "bf16", seed=4100)
    gen = torch.Generator().manual_seed(4101)
    g = _gpu(x)
    kc, vc, heads = x["k_cache"].double().numpy(), x["v_cache"].double().numpy(), x["ring_head"].numpy()
    pos = x["positions"].numpy().astype(np.int64)
    for step in range(5):
        q = torch.randn(b, t_new, hq, d, generator=gen).to(torch.bfloat16)
        kn = torch.randn(b, t_new, hkv, d, generator=gen).to(torch.bfloat16)
        vn = torch.randn(b, t_new, hkv, d, generator=gen).to(torch.bfloat16)
        n_acc = torch.randint(0, t_new + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32)
        pos_t = torch.from_numpy(pos.astype(np.int32))
        o, lse = swa.swa_sink_decode_rope(q.to(DEV), kn.to(DEV), vn.to(DEV), g["k_cache"], g["v_cache"],
                                          g["ring_head"], pos_t.to(DEV), g["sinks"], base)
        swa.swa_ring_append_rope(kn.to(DEV), vn.to(DEV), n_acc.to(DEV), pos_t.to(DEV), g["k_cache"],
                                 g["v_cache"], g["ring_head"], base)
        torch.cuda.synchronize()
        o_ref, l_ref = orc.swa_sink_decode_rope(q, kn, vn, kc, vc, heads, pos, x["sinks"], base, w)
        assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"step {step}")
        kc, vc, heads = orc.swa_ring_append_rope(kn, vn, n_acc.numpy(), pos, kc, vc, heads, base)
        assert np.array_equal(g["ring_head"].cpu().numpy(), heads)
        pos = pos + n_acc.numpy()
        # the GPU ring carries its own rotated keys forward: compare them to the oracle's
        diff = np.abs(to_np(g["k_cache"]) - kc)
        assert diff.max() <= 2.0 ** -6 * max(1.0, float(np.abs(kc).max())), f"step {step} ring keys"
        assert np.array_equal(to_np(g["v_cache"]), vc)


@pytest.mark.parametrize("name", ["decode_rope_t1", "decode_rope_t4"])
def test_decode_rope_full(name):
    _say(f"{name}: every element of the benchmarked decode with RoPE (B=256)")
    x = wl.make_workload(name)
    o, lse = _run_decode_rope(x, 10000.0)
    o_ref, l_ref = _oracle_decode_rope(x, 128, 10000.0)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, name)


def test_ring_append_full_batch():
    _say("ring append after the T = 4 verify of the benchmarked workload (B=256), every slot")
    x = wl.make_workload("decode_rope_t4")
    gen = torch.Generator().manual_seed(3501)
    n_acc = torch.randint(0, 5, (256,), generator=gen, dtype=torch.int64).to(torch.int32)
    g = _gpu(x)
    swa.swa_ring_append_rope(g["k_new"], g["v_new"], n_acc.to(DEV), g["positions"], g["k_cache"],
                             g["v_cache"], g["ring_head"], 10000.0)
    torch.cuda.synchronize()
    kc, vc, h2 = orc.swa_ring_append_rope(x["k_new"], x["v_new"], n_acc.numpy(), x["positions"].numpy(),
                                          x["k_cache"], x["v_cache"], x["ring_head"].numpy(), 10000.0)
    assert np.array_equal(g["ring_head"].cpu().numpy(), h2)
    assert np.array_equal(to_np(g["v_cache"]), vc)
    got = to_np(g["k_cache"])
    # rotated keys: the fp32 rotation may round to the neighbouring bf16 value of the
    # oracle's in rare near-ties; everything else is bit-identical
    diff = got != kc
    assert float(diff.mean()) < 1e-4
    assert np.all(np.abs(got - kc)[diff] <= 2.0 ** -7 * np.abs(kc)[diff] + 1e-30)


# ---------------------------------------------------------------------------
# one-launch MTP step: commit the previous step's accepted tokens, then verify
# ---------------------------------------------------------------------------

def _commit_case(b, t_new, prev_t, hq, hkv, d, w, dt, seed):
    """Decode-with-RoPE inputs plus a previous step: prev_k / prev_v [B, prev_T, Hkv, D]
    (keys unrotated), accept counts ~ U{0..prev_T} and the previous step's positions
    (new token 0 of this step minus the accepted count)."""
    x = wl.make_decode_rope(b, t_new, hq, hkv, d, w, dt, seed=seed)
    gen = torch.Generator().manual_seed(seed + 7)
    td = x["q"].dtype
    x["prev_k"] = torch.randn(b, prev_t, hkv, d, generator=gen).to(td)
    x["prev_v"] = torch.randn(b, prev_t, hkv, d, generator=gen).to(td)
    x["prev_accept"] = torch.randint(0, prev_t + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32)
    x["prev_positions"] = x["positions"] - x["prev_accept"]
    return x


def _run_commit(g, base, ring_head_out=None):
    head_out = torch.empty_like(g["ring_head"]) if ring_head_out is None else ring_head_out
    o, lse = swa.swa_sink_decode_rope_commit(g["q"], g["k_new"], g["v_new"], g["positions"], g["prev_k"],
                                             g["prev_v"], g["prev_accept"], g["prev_positions"], g["k_cache"],
                                             g["v_cache"], g["ring_head"], head_out, g["sinks"], base)
    torch.cuda.synchronize()
    return o, lse, head_out


def _run_append_then_decode(g, base):
    """The same step as two calls: swa_ring_append_rope on a copy of the head, then
    swa_sink_decode_rope against the updated ring."""
    head = g["ring_head"].clone()
    swa.swa_ring_append_rope(g["prev_k"], g["prev_v"], g["prev_accept"], g["prev_positions"], g["k_cache"],
                             g["v_cache"], head, base)
    o, lse = swa.swa_sink_decode_rope(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"], head,
                                      g["positions"], g["sinks"], base)
    torch.cuda.synchronize()
    return o, lse, head


def _oracle_commit(x, base, io):
    t = x["prev_k"].shape[1]
    return orc.swa_sink_decode_rope_commit(x["q"], x["k_new"], x["v_new"], x["positions"].numpy(), x["prev_k"],
                                           x["prev_v"], np.clip(x["prev_accept"].numpy(), 0, t),
                                           x["prev_positions"].numpy(), x["k_cache"], x["v_cache"],
                                           x["ring_head"].numpy(), x["sinks"], base,
                                           window=x["k_cache"].shape[2], io_dtype=io)


COMMIT_FUSED_CASES = [(16, 4, 4), (16, 1, 1), (16, 3, 2), (16, 2, 3), (16, 1, 4), (16, 4, 1)]


@pytest.mark.parametrize("case", COMMIT_FUSED_CASES, ids=lambda c: f"B{c[0]}-T{c[1]}-prevT{c[2]}")
def test_mtp_commit_equals_append_then_decode(case):
    """The one-launch step gives the bits of swa_ring_append_rope + swa_sink_decode_rope:
    outputs, lse, every ring slot and the new head (accept counts 0, prev_T, and out of
    range on both sides; heads 127, negative and beyond the window)."""
    b, t_new, prev_t = case
    _say(f"MTP step in one launch vs append + decode: B={b} T={t_new} prev_T={prev_t} 32/4 D128 bf16")
    x = _commit_case(b, t_new, prev_t, 32, 4, 128, 128, "bf16", seed=4300 + 10 * t_new + prev_t)
    x["prev_accept"][0], x["prev_accept"][1] = 0, prev_t
    x["prev_accept"][2], x["prev_accept"][3] = prev_t + 3, -2   # clamped to prev_T and to 0
    x["ring_head"][4], x["ring_head"][5], x["ring_head"][6] = 127, -5, 3 * 128 + 1
    x["positions"][7], x["prev_positions"][7] = 2 ** 31 - 8, 2 ** 31 - 8 - prev_t
    g1, g2 = _gpu(x), _gpu(x)
    head0 = g1["ring_head"].clone()
    o1, l1, h1 = _run_commit(g1, 10000.0)
    o2, l2, h2 = _run_append_then_decode(g2, 10000.0)
    assert torch.equal(g1["ring_head"], head0)  # read only
    assert torch.equal(h1, h2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1["k_cache"], g2["k_cache"]) and torch.equal(g1["v_cache"], g2["v_cache"])


def test_mtp_commit_follows_the_oracle():
    _say("MTP step in one launch vs the oracle: B=16 T=4 prev_T=4 32/4 D128 bf16")
    x = _commit_case(16, 4, 4, 32, 4, 128, 128, "bf16", seed=4400)
    g = _gpu(x)
    o, lse, h = _run_commit(g, 10000.0)
    o_ref, l_ref, kc, vc, h_ref = _oracle_commit(x, 10000.0, "bf16")
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "mtp commit")
    assert np.array_equal(h.cpu().numpy(), h_ref)
    assert np.array_equal(to_np(g["v_cache"]), vc)
    got = to_np(g["k_cache"])
    diff = got != kc  # rotated keys: rare neighbouring-bf16 near-ties, as the append's
    assert float(diff.mean()) < 1e-3
    assert np.all(np.abs(got - kc)[diff] <= 2.0 ** -7 * np.abs(kc)[diff] + 1e-30)


def test_mtp_commit_steps_ping_pong_heads():
    """Six steps, each passing the last one's new tokens as prev and its head_out as the
    head (two head buffers in turn); every step matches the two-call sequence bit for
    bit and the ring state follows it."""
    _say("MTP steps in one launch, heads ping-ponged: B=8 T=4 32/4 D128 bf16")
    b, t_new, hq, hkv, d, w, base = 8, 4, 32, 4, 128, 128, 10000.0
    x = _commit_case(b, t_new, t_new, hq, hkv, d, w, "bf16", seed=4500)
    x["prev_accept"].zero_()  # the first step commits nothing
    gen = torch.Generator().manual_seed(4501)
    g1, g2 = _gpu(x), _gpu(x)
    heads = [g1["ring_head"], torch.empty_like(g1["ring_head"])]
    head2 = g2["ring_head"].clone()
    for step in range(6):
        q = torch.randn(b, t_new, hq, d, generator=gen).to(torch.bfloat16).to(DEV)
        kn = torch.randn(b, t_new, hkv, d, generator=gen).to(torch.bfloat16).to(DEV)
        vn = torch.randn(b, t_new, hkv, d, generator=gen).to(torch.bfloat16).to(DEV)
        pos = (g1["prev_positions"] + g1["prev_accept"].clamp(0, t_new)).to(torch.int32)
        for g in (g1, g2):
            g["q"], g["k_new"], g["v_new"], g["positions"] = q, kn, vn, pos
        g1["ring_head"] = heads[step % 2]
        o1, l1, _ = _run_commit(g1, base, ring_head_out=heads[(step + 1) % 2])
        g2["ring_head"] = head2
        o2, l2, head2 = _run_append_then_decode(g2, base)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {step}"
        assert torch.equal(heads[(step + 1) % 2], head2), f"step {step}"
        assert torch.equal(g1["k_cache"], g2["k_cache"]) and torch.equal(g1["v_cache"], g2["v_cache"])
        n_acc = torch.randint(0, t_new + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32).to(DEV)
        for g in (g1, g2):
            g["prev_k"], g["prev_v"], g["prev_accept"], g["prev_positions"] = kn, vn, n_acc, pos


@pytest.mark.parametrize("case", [(6, 3, 8, 16, 2, 128, 128, "bf16"), (5, 2, 3, 4, 1, 64, 128, "f32"),
                                  (4, 4, 4, 8, 8, 128, 64, "bf16"), (3, 1, 2, 8, 1, 64, 128, "bf16")],
                         ids=lambda c: f"B{c[0]}-T{c[1]}-prevT{c[2]}-{c[3]}/{c[4]}-D{c[5]}-W{c[6]}-{c[7]}")
def test_mtp_commit_other_shapes(case):
    """Shapes outside the one-launch kernel (prev_T > 4, fp32, D 64, other windows) run
    as the head copy and the two calls: the same bits as those calls, and the oracle."""
    b, t_new, prev_t, hq, hkv, d, w, dt = case
    _say(f"MTP step, other shapes: {case}")
    x = _commit_case(b, t_new, prev_t, hq, hkv, d, w, dt, seed=4600 + b)
    x["prev_accept"][0] = prev_t
    g1, g2 = _gpu(x), _gpu(x)
    o1, l1, h1 = _run_commit(g1, 640000.0)
    o2, l2, h2 = _run_append_then_decode(g2, 640000.0)
    assert torch.equal(h1, h2) and torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1["k_cache"], g2["k_cache"]) and torch.equal(g1["v_cache"], g2["v_cache"])
    io = "bf16" if dt == "bf16" else "f32"
    o_ref, l_ref, _, vc, h_ref = _oracle_commit(x, 640000.0, io)
    assert_close(x["q"].dtype, o1, o_ref, l1, l_ref, f"mtp commit {case}")
    assert np.array_equal(h1.cpu().numpy(), h_ref)
    assert np.array_equal(to_np(g1["v_cache"]), vc)
    # without rotation: the step is the plain append (keys copied) and the plain decode
    g3, g4 = _gpu(x), _gpu(x)
    o3, l3, h3 = _run_commit(g3, 0.0)
    o4, l4, h4 = _run_append_then_decode(g4, 0.0)
    assert torch.equal(h3, h4) and torch.equal(o3, o4) and torch.equal(l3, l4)
    assert torch.equal(g3["k_cache"], g4["k_cache"])


def test_mtp_commit_full():
    """The benchmarked step (B = 256, T = 4, prev_T = 4, accept counts ~ U{0..4}): every
    output element against the oracle, the head and every ring slot."""
    _say("MTP step in one launch, full: B=256 T=4 prev_T=4 32/4 D128 bf16")
    x = wl.make_workload("decode_rope_t4")
    gen = torch.Generator().manual_seed(4701)
    x["prev_k"] = torch.randn(256, 4, 4, 128, generator=gen).to(torch.bfloat16)
    x["prev_v"] = torch.randn(256, 4, 4, 128, generator=gen).to(torch.bfloat16)
    x["prev_accept"] = torch.randint(0, 5, (256,), generator=gen, dtype=torch.int64).to(torch.int32)
    x["prev_positions"] = x["positions"] - x["prev_accept"]
    g = _gpu(x)
    o, lse, h = _run_commit(g, 10000.0)
    o_ref, l_ref, kc, vc, h_ref = _oracle_commit(x, 10000.0, "bf16")
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "mtp commit full")
    assert np.array_equal(h.cpu().numpy(), h_ref)
    assert np.array_equal(to_np(g["v_cache"]), vc)
    got = to_np(g["k_cache"])
    diff = got != kc
    assert float(diff.mean()) < 1e-4
    assert np.all(np.abs(got - kc)[diff] <= 2.0 ** -7 * np.abs(kc)[diff] + 1e-30)


def _commit_case_fp8(b, t_new, prev_t, hq, hkv, d, w, dt, seed, scales=None):
    x = _commit_case(b, t_new, prev_t, hq, hkv, d, w, dt, seed)
    y = wl.make_decode_rope_fp8(b, t_new, hq, hkv, d, w, dt, seed=seed)
    for k in ("k_cache", "v_cache", "k_scale", "v_scale"):
        x[k] = y[k]
    if scales is not None:
        x["k_scale"], x["v_scale"] = scales
    return x


def _run_commit_fp8(g, x, base, ring_head_out=None):
    head_out = torch.empty_like(g["ring_head"]) if ring_head_out is None else ring_head_out
    o, lse = swa.swa_sink_decode_rope_commit_fp8kv(g["q"], g["k_new"], g["v_new"], g["positions"], g["prev_k"],
                                                   g["prev_v"], g["prev_accept"], g["prev_positions"],
                                                   g["k_cache"], g["v_cache"], x["k_scale"], x["v_scale"],
                                                   g["ring_head"], head_out, g["sinks"], base)
    torch.cuda.synchronize()
    return o, lse, head_out


def _run_append_then_decode_fp8(g, x, base):
    head = g["ring_head"].clone()
    swa.swa_ring_append_fp8kv(g["prev_k"], g["prev_v"], g["prev_accept"], g["prev_positions"], g["k_cache"],
                              g["v_cache"], x["k_scale"], x["v_scale"], head, base)
    o, lse = swa.swa_sink_decode_rope_fp8kv(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"],
                                            x["k_scale"], x["v_scale"], head, g["positions"], g["sinks"], base)
    torch.cuda.synchronize()
    return o, lse, head


@pytest.mark.parametrize("case", [(16, 4, 4, None), (16, 1, 1, None), (16, 3, 2, (0.0173, 0.0311)),
                                  (16, 2, 3, None), (16, 1, 4, (0.0173, 0.0311)), (16, 4, 1, None)],
                         ids=lambda c: f"B{c[0]}-T{c[1]}-prevT{c[2]}-{'s' if c[3] else 'p2'}")
def test_mtp_commit_fp8_equals_append_then_decode(case):
    """FP8 ring: the one-launch step gives the bits of swa_ring_append_fp8kv +
    swa_sink_decode_rope_fp8kv (outputs, lse, every code of both rings, the head), with
    power-of-two scales (exact E4M3 ties) and others."""
    b, t_new, prev_t, scales = case
    _say(f"FP8 MTP step in one launch vs append + decode: B={b} T={t_new} prev_T={prev_t} scales {scales}")
    x = _commit_case_fp8(b, t_new, prev_t, 32, 4, 128, 128, "bf16", seed=4800 + 10 * t_new + prev_t,
                         scales=scales)
    x["prev_accept"][0], x["prev_accept"][1] = 0, prev_t
    x["prev_accept"][2], x["prev_accept"][3] = prev_t + 3, -2
    x["ring_head"][4], x["ring_head"][5], x["ring_head"][6] = 127, -5, 3 * 128 + 1
    g1, g2 = _gpu(x), _gpu(x)
    head0 = g1["ring_head"].clone()
    o1, l1, h1 = _run_commit_fp8(g1, x, 10000.0)
    o2, l2, h2 = _run_append_then_decode_fp8(g2, x, 10000.0)
    assert torch.equal(g1["ring_head"], head0)
    assert torch.equal(h1, h2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1["k_cache"], g2["k_cache"]) and torch.equal(g1["v_cache"], g2["v_cache"])


@pytest.mark.parametrize("case", [(6, 3, 8, 16, 2, 128, 128, "bf16"), (5, 2, 3, 4, 1, 64, 128, "f32"),
                                  (4, 4, 4, 8, 8, 128, 64, "bf16")],
                         ids=lambda c: f"B{c[0]}-T{c[1]}-prevT{c[2]}-{c[3]}/{c[4]}-D{c[5]}-W{c[6]}-{c[7]}")
def test_mtp_commit_fp8_other_shapes(case):
    """FP8 ring, shapes outside the one-launch kernel: the same bits as the two calls, and
    the oracle (rotated keys' codes up to one-step neighbours)."""
    b, t_new, prev_t, hq, hkv, d, w, dt = case
    _say(f"FP8 MTP step, other shapes: {case}")
    x = _commit_case_fp8(b, t_new, prev_t, hq, hkv, d, w, dt, seed=4900 + b)
    x["prev_accept"][0] = prev_t
    g1, g2 = _gpu(x), _gpu(x)
    o1, l1, h1 = _run_commit_fp8(g1, x, 640000.0)
    o2, l2, h2 = _run_append_then_decode_fp8(g2, x, 640000.0)
    assert torch.equal(h1, h2) and torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(g1["k_cache"], g2["k_cache"]) and torch.equal(g1["v_cache"], g2["v_cache"])
    io = "bf16" if dt == "bf16" else "f32"
    o_ref, l_ref, kc, vc, h_ref = orc.swa_sink_decode_rope_commit_fp8kv(
        x["q"], x["k_new"], x["v_new"], x["positions"].numpy(), x["prev_k"], x["prev_v"],
        np.clip(x["prev_accept"].numpy(), 0, prev_t), x["prev_positions"].numpy(), x["k_cache"].numpy(),
        x["v_cache"].numpy(), x["k_scale"], x["v_scale"], x["ring_head"].numpy(), x["sinks"], 640000.0,
        window=w, io_dtype=io)
    assert_close(x["q"].dtype, o1, o_ref, l1, l_ref, f"FP8 mtp commit {case}")
    assert np.array_equal(h1.cpu().numpy(), h_ref)
    assert np.array_equal(g1["v_cache"].cpu().numpy(), vc)
    _codes_close(g1["k_cache"].cpu().numpy(), kc, f"FP8 mtp commit keys {case}")


def test_mtp_commit_fp8_full():
    """The FP8-ring step at the benchmarked size (B = 256, T = 4, prev_T = 4, accept counts
    ~ U{0..4}): every output element against the oracle, the head, every code."""
    _say("FP8 MTP step in one launch, full: B=256 T=4 prev_T=4 32/4 D128 bf16")
    x = wl.make_workload("decode_rope_fp8_t4")
    gen = torch.Generator().manual_seed(4951)
    x["prev_k"] = torch.randn(256, 4, 4, 128, generator=gen).to(torch.bfloat16)
    x["prev_v"] = torch.randn(256, 4, 4, 128, generator=gen).to(torch.bfloat16)
    x["prev_accept"] = torch.randint(0, 5, (256,), generator=gen, dtype=torch.int64).to(torch.int32)
    x["prev_positions"] = x["positions"] - x["prev_accept"]
    g = _gpu(x)
    o, lse, h = _run_commit_fp8(g, x, 10000.0)
    o_ref, l_ref, kc, vc, h_ref = orc.swa_sink_decode_rope_commit_fp8kv(
        x["q"], x["k_new"], x["v_new"], x["positions"].numpy(), x["prev_k"], x["prev_v"],
        x["prev_accept"].numpy(), x["prev_positions"].numpy(), x["k_cache"].numpy(), x["v_cache"].numpy(),
        x["k_scale"], x["v_scale"], x["ring_head"].numpy(), x["sinks"], 10000.0)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "FP8 mtp commit full")
    assert np.array_equal(h.cpu().numpy(), h_ref)
    assert np.array_equal(g["v_cache"].cpu().numpy(), vc)
    _codes_close(g["k_cache"].cpu().numpy(), kc, "FP8 mtp commit full keys", min_same=0.9999)


# ---------------------------------------------------------------------------
# FP8 ring with RoPE: decode (rotation in the kernel) and the append that encodes
# ---------------------------------------------------------------------------

def _run_decode_rope_fp8(x, base):
    g = _gpu(x)
    o, lse = swa.swa_sink_decode_rope_fp8kv(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"],
                                            x["k_scale"], x["v_scale"], g["ring_head"], g["positions"],
                                            g["sinks"], base)
    torch.cuda.synchronize()
    return o, lse


def _oracle_decode_rope_fp8(x, window, base):
    io = "bf16" if x["q"].dtype == torch.bfloat16 else "f32"
    return orc.swa_sink_decode_rope_fp8kv(x["q"], x["k_new"], x["v_new"], x["k_cache"].numpy(),
                                          x["v_cache"].numpy(), x["k_scale"], x["v_scale"],
                                          x["ring_head"].numpy(), x["positions"].numpy(), x["sinks"], base,
                                          window, io_dtype=io)


@pytest.mark.parametrize("t_new", [1, 2, 3, 4])
def test_decode_rope_fp8(t_new):
    _say(f"FP8 ring decode with RoPE B=16 T={t_new} 32/4 D128 bf16 (matrix cores)")
    x = wl.make_decode_rope_fp8(16, t_new, 32, 4, 128, 128, "bf16", seed=3620 + t_new)
    x["positions"][0] = 128
    x["positions"][1] = 2 ** 31 - 8
    x["ring_head"][2] = 127
    for base in (10000.0, 5e6):
        o, lse = _run_decode_rope_fp8(x, base)
        o_ref, l_ref = _oracle_decode_rope_fp8(x, 128, base)
        assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"FP8 decode rope T={t_new} base {base:g}")


@pytest.mark.parametrize("case", [(3, 8, 1, 64, 128, "bf16", 2), (5, 4, 1, 64, 128, "f32", 3),
                                  (4, 8, 8, 128, 64, "bf16", 4)])
def test_decode_rope_fp8_generic_shapes(case):
    b, hq, hkv, d, w, dt, t_new = case
    _say(f"FP8 ring decode with RoPE generic B={b} T={t_new} {hq}/{hkv} D{d} W{w} {dt}")
    x = wl.make_decode_rope_fp8(b, t_new, hq, hkv, d, w, dt, seed=3640 + b * 7 + w)
    o, lse = _run_decode_rope_fp8(x, 640000.0)
    o_ref, l_ref = _oracle_decode_rope_fp8(x, w, 640000.0)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"FP8 decode rope generic {case}")


def test_decode_rope_fp8_base_zero_is_fp8_decode():
    _say("FP8 ring decode with rope_base 0 equals swa_sink_decode_fp8kv bit for bit")
    x = wl.make_decode_rope_fp8(8, 4, 32, 4, 128, 128, "bf16", seed=3660)
    o, lse = _run_decode_rope_fp8(x, 0.0)
    o2, l2 = _run_decode_fp8(x)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def _codes_close(got, ref, what, min_same=0.999):
    """E4M3 codes that come from rotated keys: the fp32 rotation may round to the
    neighbouring I/O value of the oracle's, which moves a code by at most one step when the
    quotient sits near a rounding point.  At least min_same must be identical; every other
    code must decode to a neighbour (same sign, magnitudes one step apart)."""
    got = np.asarray(got, dtype=np.int64)
    ref = np.asarray(ref, dtype=np.int64)
    same = got == ref
    frac = float(same.mean()) if same.size else 1.0
    diff = ~same
    adjacent = ((got & 0x80) == (ref & 0x80)) & (np.abs((got & 0x7F) - (ref & 0x7F)) == 1)
    msg = f"{what}: identical {frac:.6f}, non-adjacent {int((diff & ~adjacent).sum())}"
    print(msg, flush=True)
    assert frac >= min_same and not np.any(diff & ~adjacent), msg


def _written(ring_head, n_acc, b, t_new, w, shape):
    m = np.zeros(shape[:3], dtype=bool)  # [B, Hkv, W]
    for bb in range(b):
        n = int(np.clip(n_acc[bb], 0, t_new))
        for t in range(n):
            m[bb, :, (int(ring_head[bb]) % w + t) % w] = True
    return m


@pytest.mark.parametrize("case", [(16, 4, 4, 128, 128, "bf16", 0.0, 1 / 32, 1 / 64),
                                  (16, 4, 4, 128, 128, "bf16", 10000.0, 0.0173, 0.0311),
                                  (9, 3, 2, 64, 32, "f32", 640000.0, 0.0173, 0.0311),
                                  (7, 2, 1, 128, 128, "f32", 0.0, 0.0173, 0.0311),
                                  (6, 12, 2, 128, 128, "bf16", 10000.0, 0.0173, 0.0311)],
                         ids=lambda c: f"B{c[0]}-T{c[1]}-kv{c[2]}-D{c[3]}-W{c[4]}-{c[5]}-base{c[6]:g}-s{c[7]:g}")
def test_ring_append_fp8kv(case):
    """Codes written to an FP8 ring: bit-exact against the oracle's encoding where the keys
    are copied (base 0; specials, saturation and subnormals planted; with power-of-two scales
    bf16 quotients sit exactly halfway between E4M3 values about once in sixteen, with other
    scales they round), values always bit-exact, rotated keys identical up to one-step
    neighbours; untouched slots and the heads exact."""
    b, t_new, hkv, d, w, dt, base, ks, vs = case
    _say(f"FP8 ring append B={b} T={t_new} kv {hkv} D{d} W{w} {dt} base {base:g} scales {ks:g}/{vs:g}")
    x = wl.make_decode_rope_fp8(b, t_new, hkv, hkv, d, w, dt, seed=3680 + b)
    gen = torch.Generator().manual_seed(3681 + b)
    n_acc = torch.randint(0, t_new + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32)
    n_acc[0], n_acc[1], n_acc[4] = t_new + 3, -2, t_new  # clamped to T and to 0
    x["ring_head"][2] = w - 1
    x["ring_head"][3] = 3 * w + 1
    if base == 0.0:
        s32 = float(np.float32(ks))
        specials = [float("nan"), float("inf"), -float("inf"), -0.0, 1e30, -1e30, 449 * s32, 1e-30,
                    2.0 ** -10 * s32, 3 * 2.0 ** -10 * s32, 17 / 16 * s32, 19 / 16 * s32]
        sp = torch.tensor(specials, dtype=torch.float64).to(x["k_new"].dtype)
        x["k_new"][4, 0, 0, :len(specials)] = sp
        x["v_new"][4, 0, 0, :len(specials)] = torch.tensor(specials, dtype=torch.float64).to(x["k_new"].dtype)
        x["v_new"][4, 0, 0, :len(specials)] *= float(np.float32(vs)) / s32
    g = _gpu(x)
    heads = g["ring_head"].clone()
    swa.swa_ring_append_fp8kv(g["k_new"], g["v_new"], n_acc.to(DEV), g["positions"], g["k_cache"],
                              g["v_cache"], ks, vs, heads, base)
    torch.cuda.synchronize()
    io = "bf16" if dt == "bf16" else "f32"
    kc, vc, h2 = orc.swa_ring_append_fp8kv(x["k_new"], x["v_new"], np.clip(n_acc.numpy(), 0, t_new),
                                           x["positions"].numpy(), x["k_cache"].numpy(), x["v_cache"].numpy(),
                                           x["ring_head"].numpy(), base or None, ks, vs, io_dtype=io)
    assert np.array_equal(heads.cpu().numpy(), h2)
    got_k, got_v = g["k_cache"].cpu().numpy(), g["v_cache"].cpu().numpy()
    assert np.array_equal(got_v, vc)
    written = _written(x["ring_head"].numpy(), n_acc.numpy(), b, t_new, w, got_k.shape)
    assert np.array_equal(got_k[~written], x["k_cache"].numpy()[~written])
    if base == 0.0:
        assert np.array_equal(got_k, kc)
    else:
        _codes_close(got_k[written], kc[written], f"FP8 append keys {case}")


def test_fp8_mtp_steps_follow_the_oracle():
    """Five MTP steps against an FP8 ring: verify T = 4 tokens (RoPE in the kernel), commit a
    seeded 0..4 of them (keys rotated, both encoded), advance the positions; each step's
    outputs and the ring follow the oracle run on the same inputs."""
    _say("FP8 decode + append: 5 MTP steps, B=8, 32/4 D128 bf16")
    b, t_new, hq, hkv, d, w, base = 8, 4, 32, 4, 128, 128, 10000.0
    x = wl.make_decode_rope_fp8(b, t_new, hq, hkv, d, w, "bf16", seed=4150)
    ks, vs = x["k_scale"], x["v_scale"]
    gen = torch.Generator().manual_seed(4151)
    g = _gpu(x)
    kc, vc, heads = x["k_cache"].numpy(), x["v_cache"].numpy(), x["ring_head"].numpy()
    pos = x["positions"].numpy().astype(np.int64)
    for step in range(5):
        q = torch.randn(b, t_new, hq, d, generator=gen).to(torch.bfloat16)
        kn = torch.randn(b, t_new, hkv, d, generator=gen).to(torch.bfloat16)
        vn = torch.randn(b, t_new, hkv, d, generator=gen).to(torch.bfloat16)
        n_acc = torch.randint(0, t_new + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32)
        pos_t = torch.from_numpy(pos.astype(np.int32))
        o, lse = swa.swa_sink_decode_rope_fp8kv(q.to(DEV), kn.to(DEV), vn.to(DEV), g["k_cache"], g["v_cache"],
                                                ks, vs, g["ring_head"], pos_t.to(DEV), g["sinks"], base)
        swa.swa_ring_append_fp8kv(kn.to(DEV), vn.to(DEV), n_acc.to(DEV), pos_t.to(DEV), g["k_cache"],
                                  g["v_cache"], ks, vs, g["ring_head"], base)
        torch.cuda.synchronize()
        o_ref, l_ref = orc.swa_sink_decode_rope_fp8kv(q, kn, vn, kc, vc, ks, vs, heads, pos, x["sinks"], base, w)
        assert_close(torch.bfloat16, o, o_ref, lse, l_ref, f"FP8 step {step}")
        kc, vc, heads = orc.swa_ring_append_fp8kv(kn, vn, n_acc.numpy(), pos, kc, vc, heads, base, ks, vs)
        assert np.array_equal(g["ring_head"].cpu().numpy(), heads)
        assert np.array_equal(g["v_cache"].cpu().numpy(), vc)
        _codes_close(g["k_cache"].cpu().numpy(), kc, f"FP8 step {step} ring keys", min_same=0.9999)
        pos = pos + n_acc.numpy()


def test_ring_append_fp8kv_full_batch():
    _say("FP8 ring append after the T = 4 verify (B=256), every slot")
    x = wl.make_workload("decode_rope_fp8_t4")
    gen = torch.Generator().manual_seed(3501)
    n_acc = torch.randint(0, 5, (256,), generator=gen, dtype=torch.int64).to(torch.int32)
    g = _gpu(x)
    swa.swa_ring_append_fp8kv(g["k_new"], g["v_new"], n_acc.to(DEV), g["positions"], g["k_cache"],
                              g["v_cache"], x["k_scale"], x["v_scale"], g["ring_head"], 10000.0)
    torch.cuda.synchronize()
    kc, vc, h2 = orc.swa_ring_append_fp8kv(x["k_new"], x["v_new"], n_acc.numpy(), x["positions"].numpy(),
                                           x["k_cache"].numpy(), x["v_cache"].numpy(), x["ring_head"].numpy(),
                                           10000.0, x["k_scale"], x["v_scale"])
    assert np.array_equal(g["ring_head"].cpu().numpy(), h2)
    assert np.array_equal(g["v_cache"].cpu().numpy(), vc)
    _codes_close(g["k_cache"].cpu().numpy(), kc, "FP8 append B=256 keys", min_same=0.9999)


# ---------------------------------------------------------------------------
# token-level sparse attention: selection (exact) and sparse decode
# ---------------------------------------------------------------------------

def _topk_gpu(scores, lengths, k, recent):
    idx, cnt = swa.swa_topk_select(scores.to(DEV), lengths.to(DEV), k=k, recent=recent)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("case", [(6, 3, 5000, 1024, 128, "normal"), (5, 2, 3000, 300, 7, "ties"),
                                  (4, 4, 9000, 64, 128, "few"), (3, 2, 700, 1024, 128, "short"),
                                  (4, 2, 2000, 0, 128, "k0"), (3, 2, 4100, 500, 16, "special"),
                                  (3, 2, 9000, 1024, 128, "two"), (2, 2, 40000, 1024, 128, "normal"),
                                  (4, 3, 3001, 256, 64, "normal"),  # rows at every 4-byte alignment
                                  (4, 2, 3000, 1024, 128, "zeros"), (3, 2, 2500, 700, 33, "zeros")],
                         ids=lambda c: f"B{c[0]}-kv{c[1]}-L{c[2]}-k{c[3]}-r{c[4]}-{c[5]}")
def test_topk_select_exact(case):
    b, hkv, lmax, k, recent, kind = case
    _say(f"top-k selection {case}")
    gen = torch.Generator().manual_seed(lmax + k)
    scores = torch.randn(b, hkv, lmax, generator=gen)
    if kind == "ties":  # a handful of distinct values: most ranks are decided by position
        scores = torch.randint(0, 4, (b, hkv, lmax), generator=gen).float() * 0.25
    if kind == "two":  # two values: the threshold's first-digit bin holds thousands of keys
        scores = torch.randint(0, 2, (b, hkv, lmax), generator=gen).float() * 0.5
    if kind == "few":  # values equal to the threshold straddle chunk boundaries
        scores = torch.randint(0, 40, (b, hkv, lmax), generator=gen).float()
    if kind == "special":  # NaN ranks below every number (numpy's sort puts it last too); +-inf; +-0.0
        scores[:, :, ::7] = float("nan")
        scores[:, :, 3::11] = float("inf")
        scores[:, :, 5::13] = float("-inf")
        scores[:, :, 1::17] = -0.0
        scores[:, :, 2::19] = 0.0   # the two zeros are equal scores: the lower position wins
    if kind == "zeros":  # mostly signed zeros: the threshold lands on zero, ties across both signs
        scores = torch.randn(b, hkv, lmax, generator=gen).clamp(min=0.0)
        scores = torch.where(torch.rand(b, hkv, lmax, generator=gen) < 0.5, scores, -scores)
    lengths = torch.randint(1, lmax + 1, (b,), generator=gen, dtype=torch.int64).to(torch.int32)
    lengths[0] = lmax
    if kind == "short":
        lengths[1] = recent      # no candidate
        lengths[2] = recent + 5  # fewer candidates than k
    idx, cnt = _topk_gpu(scores, lengths, k, recent)
    ridx, rcnt = orc.topk_select(scores, lengths.numpy(), k=k, recent=recent)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(idx, ridx)


def _sparse_gpu(x, idx, cnt, recent):
    g = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in x.items()}
    o, lse = swa.swa_sparse_decode(g["q"], g["k_cache"], g["v_cache"], g["lengths"],
                                   torch.as_tensor(idx, dtype=torch.int32).to(DEV),
                                   torch.as_tensor(cnt, dtype=torch.int32).to(DEV), g["sinks"], recent=recent)
    torch.cuda.synchronize()
    return o, lse


def test_prefill_and_sparse_without_lse():
    """return_lse=False on the GA prefill, the prefill over E4M3 K/V and the sparse decode:
    outputs bitwise those of the same call with the LSE written."""
    _say("GA prefill, FP8-K/V prefill and sparse decode without LSE: bitwise vs with LSE")
    x = wl.make_prefill([300, 77, 140], 32, 4, 128, "bf16", seed=4700)
    g = _gpu(x)
    o1, _ = swa.ga_causal_prefill(g["q"], g["k"], g["v"], g["cu_seqlens"])
    o0, lse0 = swa.ga_causal_prefill(g["q"], g["k"], g["v"], g["cu_seqlens"], return_lse=False)
    torch.cuda.synchronize()
    assert lse0 is None
    assert torch.equal(o0, o1)

    f = wl.make_prefill_fp8([200, 45, 300], 32, 4, 128, "bf16", seed=4701)
    gf = _gpu(f)
    fargs = (gf["q"], gf["k"], gf["v"], f["k_scale"], f["v_scale"], gf["sinks"], gf["cu_seqlens"])
    o1, _ = swa.swa_sink_prefill_fp8kv(*fargs, window=128)
    o0, lse0 = swa.swa_sink_prefill_fp8kv(*fargs, window=128, return_lse=False)
    torch.cuda.synchronize()
    assert lse0 is None
    assert torch.equal(o0, o1)

    xs = wl.make_sparse(4, 32, 4, 128, 3000, "bf16", seed=4702, min_len=300)
    idx, cnt = _topk_gpu(xs["scores"], xs["lengths"], 1024, 128)
    gs = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in xs.items()}
    sargs = (gs["q"], gs["k_cache"], gs["v_cache"], gs["lengths"], torch.as_tensor(idx, dtype=torch.int32).to(DEV),
             torch.as_tensor(cnt, dtype=torch.int32).to(DEV), gs["sinks"])
    o1, _ = swa.swa_sparse_decode(*sargs)
    o0, lse0 = swa.swa_sparse_decode(*sargs, return_lse=False)
    torch.cuda.synchronize()
    assert lse0 is None
    assert torch.equal(o0, o1)


def test_every_output_element_written():
    """Outputs and LSE handed in filled with NaN come back equal, bit for bit, to freshly
    allocated ones: every kernel writes every element of its outputs (ragged tails, an empty
    sequence, sequence ends, the duplicate query columns of a decode with T < 4)."""
    _say("every output element written: prefill (SWA, GA, FP8 K/V), decode T=1..4 (bf16, FP8, RoPE), sparse")

    def check(fn, what):
        o1, l1 = fn()
        o2 = torch.full_like(o1, float("nan"))
        l2 = torch.full_like(l1, float("nan"))
        fn(out=o2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o2, o1), what
        assert torch.equal(l2, l1), what

    x = wl.make_prefill([300, 0, 77, 141], 32, 4, 128, "bf16", seed=4800)
    g = _gpu(x)
    check(lambda **kw: swa.swa_sink_prefill(g["q"], g["k"], g["v"], g["sinks"], g["cu_seqlens"], **kw), "swa prefill")
    check(lambda **kw: swa.ga_causal_prefill(g["q"], g["k"], g["v"], g["cu_seqlens"], **kw), "ga prefill")
    f = wl.make_prefill_fp8([200, 0, 45, 133], 32, 4, 128, "bf16", seed=4801)
    gf = _gpu(f)
    check(lambda **kw: swa.swa_sink_prefill_fp8kv(gf["q"], gf["k"], gf["v"], f["k_scale"], f["v_scale"], gf["sinks"],
                                                  gf["cu_seqlens"], **kw), "fp8 prefill")
    for t_new in (1, 2, 3, 4):
        d = _gpu(wl.make_decode(8, t_new, 32, 4, 128, 128, "bf16", seed=4810 + t_new))
        check(lambda **kw: swa.swa_sink_decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                               d["ring_head"], d["sinks"], **kw), f"decode T={t_new}")
        df = wl.make_decode_fp8(8, t_new, 32, 4, 128, 128, "bf16", seed=4820 + t_new)
        gd = _gpu(df)
        check(lambda **kw: swa.swa_sink_decode_fp8kv(gd["q"], gd["k_new"], gd["v_new"], gd["k_cache"], gd["v_cache"],
                                                     df["k_scale"], df["v_scale"], gd["ring_head"], gd["sinks"], **kw),
              f"fp8 decode T={t_new}")
        r = _gpu(wl.make_decode_rope(8, t_new, 32, 4, 128, 128, "bf16", seed=4830 + t_new))
        check(lambda **kw: swa.swa_sink_decode_rope(r["q"], r["k_new"], r["v_new"], r["k_cache"], r["v_cache"],
                                                    r["ring_head"], r["positions"], r["sinks"], 10000.0, **kw),
              f"rope decode T={t_new}")
    xs = wl.make_sparse(4, 32, 4, 128, 3000, "bf16", seed=4840, min_len=300)
    idx, cnt = _topk_gpu(xs["scores"], xs["lengths"], 1024, 128)
    gs = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in xs.items()}
    ti, tc = torch.as_tensor(idx, dtype=torch.int32).to(DEV), torch.as_tensor(cnt, dtype=torch.int32).to(DEV)
    check(lambda **kw: swa.swa_sparse_decode(gs["q"], gs["k_cache"], gs["v_cache"], gs["lengths"], ti, tc,
                                             gs["sinks"], **kw), "sparse decode")


def test_side_stream_and_repeat_are_bitwise_equal():
    """Each entry point, called on torch's current stream, again on the same stream, and on a
    second (default-priority) stream made current, gives the same bits: the kernels are
    deterministic (no atomics, fixed reduction orders) and run on the stream they are given."""
    _say("side stream and repeated calls: bitwise equal (SWA/GA prefill, decode T=4, FP8 decode, sparse)")
    x = _gpu(wl.make_prefill([700, 33, 250], 32, 4, 128, "bf16", seed=4900))
    d = _gpu(wl.make_decode(16, 4, 32, 4, 128, 128, "bf16", seed=4901))
    df = wl.make_decode_fp8(16, 2, 32, 4, 128, 128, "bf16", seed=4902)
    gd = _gpu(df)
    xs = wl.make_sparse(4, 32, 4, 128, 3000, "bf16", seed=4903, min_len=300)
    gs = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in xs.items()}

    def run_all():
        outs = list(swa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], x["cu_seqlens"]))
        outs += swa.ga_causal_prefill(x["q"], x["k"], x["v"], x["cu_seqlens"])
        outs += swa.swa_sink_decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ring_head"],
                                    d["sinks"])
        outs += swa.swa_sink_decode_fp8kv(gd["q"], gd["k_new"], gd["v_new"], gd["k_cache"], gd["v_cache"],
                                          df["k_scale"], df["v_scale"], gd["ring_head"], gd["sinks"])
        idx, cnt = swa.swa_topk_select(gs["scores"], gs["lengths"], k=1024, recent=128)
        outs += [idx, cnt]
        outs += swa.swa_sparse_decode(gs["q"], gs["k_cache"], gs["v_cache"], gs["lengths"], idx, cnt, gs["sinks"])
        return outs

    first = run_all()
    again = run_all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        on_side = run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a_, b_, c_ in zip(first, again, on_side):
        assert torch.equal(a_, b_)
        assert torch.equal(a_, c_)


def test_hip_graph_replays_match_eager():
    """The library allocates nothing and issues no memset or synchronisation, so its calls can
    be captured in a HIP graph: a graph holding a prefill, a decode (T = 4), a token selection
    with its sparse decode and the backward on the library's own scratch array is replayed
    three times, with new inputs copied in and eager work and synchronisations between the
    replays, and every replay equals the eager calls on the same inputs bit for bit."""
    _say("HIP graph: prefill + decode + selection/sparse decode + no-alloc backward, 3 replays vs eager")
    x = _gpu(wl.make_prefill([500, 77], 32, 4, 128, "bf16", seed=5000))
    d = _gpu(wl.make_decode(16, 4, 32, 4, 128, 128, "bf16", seed=5001))
    xs = wl.make_sparse(4, 32, 4, 128, 3000, "bf16", seed=5002, min_len=300)
    gs = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in xs.items()}
    n, hq = x["q"].shape[0], x["q"].shape[1]
    po, pl = torch.empty_like(x["q"]), torch.empty(n, hq, dtype=torch.float32, device=DEV)
    do_, dl = torch.empty_like(d["q"]), torch.empty(d["q"].shape[:3], dtype=torch.float32, device=DEV)
    ti = torch.empty(gs["scores"].shape[0], gs["scores"].shape[1], 1024, dtype=torch.int32, device=DEV)
    tc = torch.empty(gs["scores"].shape[:2], dtype=torch.int32, device=DEV)
    so, sl = torch.empty_like(gs["q"]), torch.empty(gs["q"].shape[:2], dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5003)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]),
             torch.empty(hq, dtype=torch.float32, device=DEV))

    def body():
        swa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], x["cu_seqlens"], out=po, lse=pl)
        swa.swa_sink_decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["ring_head"], d["sinks"],
                            out=do_, lse=dl)
        swa.swa_topk_select(gs["scores"], gs["lengths"], k=1024, recent=128, indices=ti, counts=tc)
        swa.swa_sparse_decode(gs["q"], gs["k_cache"], gs["v_cache"], gs["lengths"], ti, tc, gs["sinks"], out=so, lse=sl)
        swa.swa_sink_prefill_backward(x["q"], x["k"], x["v"], x["sinks"], x["cu_seqlens"], po, pl, dout,
                                      library_scratch=True, grads=grads)

    side = torch.cuda.Stream()  # torch's capture recipe: warm up eagerly on a side stream
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    outs = (po, pl, do_, dl, ti, tc, so, sl) + grads
    for rep in range(3):
        x["q"].copy_(torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16))
        d["q"].copy_(torch.randn(d["q"].shape, generator=gen, device=DEV).to(torch.bfloat16))
        gs["scores"].copy_(torch.randn(gs["scores"].shape, generator=gen, device=DEV))
        dout.copy_(torch.randn(dout.shape, generator=gen, device=DEV).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        body()  # eager, same inputs, same buffers
        torch.cuda.synchronize()
        for i_, (a_, b_) in enumerate(zip(got, outs)):
            assert torch.equal(a_, b_), f"replay {rep}: output {i_} differs from the eager call"


@pytest.mark.parametrize("case", [(8, 32, 4, 128, 6000, "bf16", 1024, 128, True),
                                  (6, 16, 2, 128, 3000, "bf16", 300, 37, False),
                                  (5, 8, 1, 128, 900, "bf16", 1024, 128, True),
                                  (4, 8, 2, 64, 2000, "bf16", 200, 64, True),
                                  (3, 4, 1, 128, 1500, "f32", 256, 128, True),
                                  (4, 32, 4, 128, 2500, "bf16", 2000, 128, False),
                                  (70, 32, 4, 128, 800, "bf16", 300, 128, True)],  # > 256 workgroups
                         ids=lambda c: f"B{c[0]}-{c[1]}/{c[2]}-D{c[3]}-L{c[4]}-{c[5]}-k{c[6]}-r{c[7]}-{'sink' if c[8] else 'nosink'}")
def test_sparse_decode_against_oracle(case):
    b, hq, hkv, d, lmax, dt, k, recent, sink = case
    _say(f"sparse decode {case}")
    x = wl.make_sparse(b, hq, hkv, d, lmax, dt, seed=6100 + lmax + k, with_sinks=sink)
    x["lengths"][0] = lmax
    x["lengths"][1] = min(lmax, recent // 2 + 1)  # shorter than the recent window
    idx, cnt = _topk_gpu(x["scores"], x["lengths"], k, recent)
    ridx, rcnt = orc.topk_select(x["scores"], x["lengths"].numpy(), k=k, recent=recent)
    assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)
    o, lse = _sparse_gpu(x, idx, cnt, recent)
    o_ref, l_ref = orc.sparse_decode(x["q"], x["k_cache"], x["v_cache"], x["lengths"].numpy(), ridx, rcnt,
                                     x["sinks"], recent=recent)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"sparse {case}")


def test_sparse_decode_limits_match_dense_kernels():
    """k = 0 with the 128-token recent window is the newest row of swa_sink_prefill with
    window 128; a selection of every older token is the newest row of full causal
    attention (swa_sink_prefill with the window at the sequence length)."""
    _say("sparse decode limits vs the library's own dense prefill")
    b, hq, hkv, d, lmax = 4, 32, 4, 128, 1000
    x = wl.make_sparse(b, hq, hkv, d, lmax, "bf16", seed=6200, min_len=300)
    for k, window_of in ((0, lambda n: 128), (1024, lambda n: n)):
        idx, cnt = _topk_gpu(x["scores"], x["lengths"], k, 128)
        o, lse = _sparse_gpu(x, idx, cnt, 128)
        for bb in range(b):
            n = int(x["lengths"][bb])
            qs = torch.zeros(n, hq, d, dtype=torch.bfloat16)
            qs[n - 1] = x["q"][bb]
            ks = x["k_cache"][bb, :, :n].transpose(0, 1).contiguous()
            vs = x["v_cache"][bb, :, :n].transpose(0, 1).contiguous()
            od, ld = swa.swa_sink_prefill(qs.to(DEV), ks.to(DEV), vs.to(DEV), x["sinks"].to(DEV),
                                          torch.tensor([0, n], dtype=torch.int32, device=DEV), n,
                                          window=window_of(n))
            torch.cuda.synchronize()
            err = (o[bb].float() - od[n - 1].float()).abs().max().item()
            lerr = (lse[bb] - ld[n - 1]).abs().max().item()
            assert err <= 2e-2 and lerr <= 1e-3, (k, bb, err, lerr)


@pytest.mark.parametrize("case", [(8, 32, 4, 128, 6000, "bf16", 1024, 128, True, 2),
                                  (6, 16, 2, 128, 3000, "bf16", 300, 37, False, 2),
                                  (5, 8, 1, 128, 900, "bf16", 1024, 128, True, 1),
                                  (4, 32, 4, 128, 2500, "bf16", 2000, 128, True, 3),
                                  (4, 8, 2, 64, 2000, "bf16", 200, 64, True, 2),
                                  (3, 4, 1, 128, 1500, "f32", 256, 128, True, 2),
                                  (72, 32, 4, 128, 700, "bf16", 256, 64, True, 2)],  # > 256 workgroups
                         ids=lambda c: f"B{c[0]}-{c[1]}/{c[2]}-D{c[3]}-L{c[4]}-{c[5]}-k{c[6]}-r{c[7]}-"
                                       f"{'sink' if c[8] else 'nosink'}-T{c[9]}")
def test_sparse_mtp_against_oracle(case):
    """MTP verify in the sparse layer: the newest T tokens, each with its own recent window
    and the selection below it; the newest candidate (just below the newest token's window)
    forced into the selection, so it falls inside the older drafts' windows; a sequence
    shorter than the window and one of exactly T tokens."""
    b, hq, hkv, d, lmax, dt, k, recent, sink, t_new = case
    _say(f"sparse MTP verify {case}")
    x = wl.make_sparse(b, hq, hkv, d, lmax, dt, seed=6300 + lmax + k, with_sinks=sink)
    gen = torch.Generator().manual_seed(6301 + lmax)
    x["q"] = torch.randn(b, t_new, hq, d, generator=gen).to(x["q"].dtype)
    x["lengths"][0] = lmax
    x["lengths"][1] = min(lmax, recent // 2 + 1)
    x["lengths"][2] = t_new
    x["scores"][0, :, lmax - recent - 1] = 1e4  # selected, and inside the older drafts' windows
    if b > 3 and int(x["lengths"][3]) > recent + 1:
        x["scores"][3, :, int(x["lengths"][3]) - recent - 1] = 1e4
    idx, cnt = _topk_gpu(x["scores"], x["lengths"], k, recent)
    ridx, rcnt = orc.topk_select(x["scores"], x["lengths"].numpy(), k=k, recent=recent)
    assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)
    g = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in x.items()}
    o, lse = swa.swa_sparse_decode_mtp(g["q"], g["k_cache"], g["v_cache"], g["lengths"],
                                       torch.as_tensor(idx, dtype=torch.int32).to(DEV),
                                       torch.as_tensor(cnt, dtype=torch.int32).to(DEV), g["sinks"], recent=recent)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.sparse_decode_mtp(x["q"], x["k_cache"], x["v_cache"], x["lengths"].numpy(), ridx, rcnt,
                                         x["sinks"], recent=recent)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"sparse MTP {case}")
    if t_new == 1:  # the same kernel as the single-token entry point
        o1, l1 = _sparse_gpu({**x, "q": x["q"][:, 0].contiguous()}, idx, cnt, recent)
        assert torch.equal(o1, o[:, 0]) and torch.equal(l1, lse[:, 0])


def test_sparse_mtp_limits_match_dense_kernels():
    """k = 0 gives each of the T rows the windowed prefill's row (window 128); every older
    token selected gives full causal attention -- against the library's own dense prefill."""
    _say("sparse MTP verify limits vs the library's dense prefill, T = 2")
    b, hq, hkv, d, lmax, t_new = 4, 32, 4, 128, 1000, 2
    x = wl.make_sparse(b, hq, hkv, d, lmax, "bf16", seed=6400, min_len=300)
    x["q"] = torch.randn(b, t_new, hq, d, generator=torch.Generator().manual_seed(6401)).to(torch.bfloat16)
    for k, window_of in ((0, lambda n: 128), (1024, lambda n: n)):
        idx, cnt = _topk_gpu(x["scores"], x["lengths"], k, 128)
        o, lse = swa.swa_sparse_decode_mtp(x["q"].to(DEV), x["k_cache"].to(DEV), x["v_cache"].to(DEV),
                                           x["lengths"].to(DEV), torch.as_tensor(idx, dtype=torch.int32).to(DEV),
                                           torch.as_tensor(cnt, dtype=torch.int32).to(DEV), x["sinks"].to(DEV))
        torch.cuda.synchronize()
        for bb in range(b):
            n = int(x["lengths"][bb])
            qs = torch.zeros(n, hq, d, dtype=torch.bfloat16)
            qs[n - t_new:] = x["q"][bb]
            ks = x["k_cache"][bb, :, :n].transpose(0, 1).contiguous()
            vs = x["v_cache"][bb, :, :n].transpose(0, 1).contiguous()
            od, ld = swa.swa_sink_prefill(qs.to(DEV), ks.to(DEV), vs.to(DEV), x["sinks"].to(DEV),
                                          torch.tensor([0, n], dtype=torch.int32, device=DEV), n,
                                          window=window_of(n))
            torch.cuda.synchronize()
            err = (o[bb].float() - od[n - t_new:].float()).abs().max().item()
            lerr = (lse[bb] - ld[n - t_new:]).abs().max().item()
            assert err <= 2e-2 and lerr <= 1e-3, (k, bb, err, lerr)


@pytest.mark.parametrize("case", [(8, 32, 4, 128, 6000, "bf16", 1024, 128, True, 1),
                                  (6, 16, 2, 128, 3000, "bf16", 300, 37, False, 2),
                                  (5, 8, 1, 128, 900, "bf16", 1024, 128, True, 2),
                                  (4, 32, 4, 128, 2500, "bf16", 2000, 128, True, 3),
                                  (4, 8, 2, 64, 2000, "bf16", 200, 64, True, 1),
                                  (3, 4, 1, 128, 1500, "f32", 256, 128, True, 2),
                                  (72, 32, 4, 128, 700, "bf16", 256, 64, True, 1),  # > 256 workgroups
                                  (66, 32, 4, 128, 900, "bf16", 512, 128, False, 2)],
                         ids=lambda c: f"B{c[0]}-{c[1]}/{c[2]}-D{c[3]}-L{c[4]}-{c[5]}-k{c[6]}-r{c[7]}-"
                                       f"{'sink' if c[8] else 'nosink'}-T{c[9]}")
def test_sparse_fp8_against_oracle(case):
    """The sparse decode and MTP verify over an FP8 cache (E4M3 codes, per-tensor scales):
    the matrix-core kernel (bf16, head_dim 128, T <= 2) and the vector kernel, the selection
    reaching into the older drafts' windows, a sequence shorter than the window and one of
    exactly T tokens."""
    b, hq, hkv, d, lmax, dt, k, recent, sink, t_new = case
    _say(f"sparse FP8 {case}")
    x = wl.make_sparse_fp8(b, hq, hkv, d, lmax, dt, seed=6500 + lmax + k, with_sinks=sink)
    gen = torch.Generator().manual_seed(6501 + lmax)
    x["q"] = torch.randn(b, t_new, hq, d, generator=gen).to(x["q"].dtype)
    x["lengths"][0] = lmax
    x["lengths"][1] = min(lmax, recent // 2 + 1)
    x["lengths"][2] = t_new
    x["scores"][0, :, lmax - recent - 1] = 1e4
    idx, cnt = _topk_gpu(x["scores"], x["lengths"], k, recent)
    ridx, rcnt = orc.topk_select(x["scores"], x["lengths"].numpy(), k=k, recent=recent)
    assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)
    g = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in x.items()}
    o, lse = swa.swa_sparse_decode_fp8kv(g["q"], g["k_cache"], g["v_cache"], x["k_scale"], x["v_scale"],
                                         g["lengths"], torch.as_tensor(idx, dtype=torch.int32).to(DEV),
                                         torch.as_tensor(cnt, dtype=torch.int32).to(DEV), g["sinks"],
                                         recent=recent)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.sparse_decode_mtp_fp8kv(x["q"], x["k_cache"].numpy(), x["v_cache"].numpy(), x["k_scale"],
                                               x["v_scale"], x["lengths"].numpy(), ridx, rcnt, x["sinks"],
                                               recent=recent)
    assert_close(x["q"].dtype, o, o_ref, lse, l_ref, f"sparse FP8 {case}")


def test_sparse_fp8_every_finite_code():
    """Every finite E4M3 code (both signs, zeros and subnormals included) appears in each
    (sequence, kv head)'s recent window, which every query row reads, in the matrix-core
    kernel, T = 2."""
    _say("sparse FP8 every finite code")
    b, hq, hkv, d, lmax, k, recent = 4, 32, 4, 128, 2000, 512, 128
    x = wl.make_sparse_fp8(b, hq, hkv, d, lmax, "bf16", seed=6600, min_len=lmax)
    finite = torch.tensor([c for c in range(256) if c & 0x7F != 0x7F], dtype=torch.uint8).repeat(64)
    gen = torch.Generator().manual_seed(6601)
    for key in ("k_cache", "v_cache"):
        for bb in range(b):
            for gg in range(hkv):
                win = x[key][bb, gg, lmax - recent:].reshape(-1)
                win[:finite.numel()] = finite[torch.randperm(finite.numel(), generator=gen)]
                x[key][bb, gg, lmax - recent:] = win.view(recent, d)
    x["q"] = torch.randn(b, 2, hq, d, generator=gen).to(torch.bfloat16)
    idx, cnt = _topk_gpu(x["scores"], x["lengths"], k, recent)
    ridx, rcnt = orc.topk_select(x["scores"], x["lengths"].numpy(), k=k, recent=recent)
    assert np.array_equal(idx, ridx) and np.array_equal(cnt, rcnt)
    g = {k_: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k_, v in x.items()}
    o, lse = swa.swa_sparse_decode_fp8kv(g["q"], g["k_cache"], g["v_cache"], x["k_scale"], x["v_scale"],
                                         g["lengths"], torch.as_tensor(idx, dtype=torch.int32).to(DEV),
                                         torch.as_tensor(cnt, dtype=torch.int32).to(DEV), g["sinks"],
                                         recent=recent)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.sparse_decode_mtp_fp8kv(x["q"], x["k_cache"].numpy(), x["v_cache"].numpy(), x["k_scale"],
                                               x["v_scale"], x["lengths"].numpy(), ridx, rcnt, x["sinks"],
                                               recent=recent)
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "sparse FP8 every code")


def test_sparse_full_size_workload():
    """The benchmarked workload (64 sequences of 16K-32K tokens, [64, 4, 32768, 128]
    caches drawn on the GPU): every selection index exactly, every output row against the
    oracle on the rows it gathers."""
    w = wl.WORKLOADS["sparse_b64"]
    k, recent = w.extra["topk"], w.extra["recent"]
    _say("sparse_b64 full size: top-k exact, all 64 x 32 output rows")
    x = wl.make_sparse_device(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seq_len, w.seed, DEV,
                              min_len=w.extra["min_len"])
    idx, cnt = swa.swa_topk_select(x["scores"], x["lengths"].to(DEV), k=k, recent=recent)
    o, lse = swa.swa_sparse_decode(x["q"], x["k_cache"], x["v_cache"], x["lengths"].to(DEV), idx, cnt, None,
                                   recent=recent)
    torch.cuda.synchronize()
    ridx, rcnt = orc.topk_select(x["scores"].cpu(), x["lengths"].numpy(), k=k, recent=recent)
    assert np.array_equal(idx.cpu().numpy(), ridx) and np.array_equal(cnt.cpu().numpy(), rcnt)
    # the oracle on each sequence's gathered rows (selected + recent), read back from the GPU
    hkv, d = w.num_kv_heads, w.head_dim
    o_ref = np.zeros((w.batch, w.num_q_heads, d))
    l_ref = np.zeros((w.batch, w.num_q_heads))
    for bb in range(w.batch):
        n = int(x["lengths"][bb])
        keys = [np.concatenate([ridx[bb, g, :rcnt[bb, g]], np.arange(n - recent, n)]) for g in range(hkv)]
        m = len(keys[0])
        kg = torch.stack([x["k_cache"][bb, g, torch.as_tensor(keys[g], device=DEV)] for g in range(hkv)])
        vg = torch.stack([x["v_cache"][bb, g, torch.as_tensor(keys[g], device=DEV)] for g in range(hkv)])
        ob, lb = orc.sparse_decode(x["q"][bb:bb + 1].cpu(), kg[None].cpu(), vg[None].cpu(), [m],
                                   np.full((1, hkv, 1), -1), np.zeros((1, hkv)), None, recent=m)
        o_ref[bb], l_ref[bb] = ob[0], lb[0]
    assert_close(torch.bfloat16, o, o_ref, lse, l_ref, "sparse_b64")
