"""Seeded generators and the closed-form FLOP/byte counters used for roofline figures."""
import torch

from sliding_window_attention_amd import workloads as wl


def test_counters_match_hand_closed_forms():
    # SWA prefill, 32768 tokens, 32 q / 4 kv heads, D 128, W 128, bf16:
    # pairs = 128*129/2 + 128*(32768-128); per token Q 8192 + O 8192 + K 1024 + V 1024 + LSE 128 B
    p = 128 * 129 // 2 + 128 * (32768 - 128)
    assert p == 4_186_176
    fl, by = wl.workload_work("swa_prefill_32k")
    assert fl == 4 * 128 * 32 * p == 68_586_307_584
    assert by == 32768 * 18_560 == 608_174_080
    # decode: 127 live ring slots + T new K/V rows, Q and O bf16, LSE fp32
    fl, by = wl.workload_work("decode_t1")
    assert by == 2 * 256 * 4 * 128 * 2 * 128 + 2 * 256 * 32 * 128 * 2 + 4 * 256 * 32 == 71_335_936
    assert fl == 4 * 128 * 32 * 256 * 128
    _, by = wl.workload_work("decode_t4")
    assert by == 85_590_016
    fl, by = wl.workload_work("hybrid_5to1_32k")
    assert by == 6 * 608_174_080
    assert fl == 5 * 68_586_307_584 + 4 * 128 * 32 * (32768 * 32769 // 2)
    fl, _ = wl.workload_work("tiny_fp32")
    assert fl == 4 * 64 * 4 * (128 * 129 // 2 + 128 * (512 - 128))


def test_lognormal_lengths_sum_and_positive():
    for seed in (0, 5000, 123):
        lens = wl.lognormal_lengths(262144, 8, seed)
        assert sum(lens) == 262144 and min(lens) >= 1 and len(lens) == 8
    assert wl.lognormal_lengths(262144, 8, 5000) == wl.lognormal_lengths(262144, 8, 5000)
    lens = wl.lognormal_lengths(20, 16, 1)
    assert sum(lens) == 20 and min(lens) >= 1


def test_generators_are_seeded_and_shaped():
    a = wl.make_prefill([7, 9], 8, 1, 128, "bf16", 42)
    b = wl.make_prefill([7, 9], 8, 1, 128, "bf16", 42)
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["sinks"], b["sinks"])
    assert a["q"].dtype == torch.bfloat16 and a["sinks"].dtype == torch.float32
    assert a["cu_seqlens"].tolist() == [0, 7, 16] and a["max_seqlen"] == 9
    d = wl.make_decode(3, 4, 32, 4, 128, 128, "bf16", 7)
    assert d["k_cache"].shape == (3, 4, 128, 128) and d["q"].shape == (3, 4, 32, 128)
    assert d["ring_head"].dtype == torch.int32
    assert 0 <= int(d["ring_head"].min()) and int(d["ring_head"].max()) < 128
