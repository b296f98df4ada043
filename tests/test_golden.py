"""The oracle against hand-worked fixtures (tests/golden/hand_worked.json) and the
pages' stated hyper-parameters (tests/golden/pages_constants.json)."""
import numpy as np

from oracle import swa_oracle as orc
from sliding_window_attention_amd import workloads as wl
from tests.golden.load import array, load


def test_hand_worked_prefill_swa_and_ga():
    fx = load()["prefill"]
    q, k, v = array(fx["q"]), array(fx["k"]), array(fx["v"])
    o, lse = orc.swa_sink_prefill(q, k, v, array(fx["sinks"]), fx["cu_seqlens"], fx["window"])
    np.testing.assert_allclose(o, array(fx["swa_o"]), atol=1e-15, rtol=1e-15)
    np.testing.assert_allclose(lse, array(fx["swa_lse"]), atol=1e-15, rtol=1e-15)
    o, lse = orc.ga_causal_prefill(q, k, v, fx["cu_seqlens"])
    np.testing.assert_allclose(o, array(fx["ga_o"]), atol=1e-15, rtol=1e-15)
    np.testing.assert_allclose(lse, array(fx["ga_lse"]), atol=1e-15, rtol=1e-15)


def test_hand_worked_decode():
    for fx in load()["decode"]:
        o, lse = orc.swa_sink_decode(array(fx["q"]), array(fx["k_new"]), array(fx["v_new"]),
                                     array(fx["k_cache"]), array(fx["v_cache"]),
                                     np.array(fx["ring_head"]), array(fx["sinks"]),
                                     window=fx["window"])
        np.testing.assert_allclose(o, array(fx["o"]), atol=1e-15, rtol=1e-15)
        np.testing.assert_allclose(lse, array(fx["lse"]), atol=1e-15, rtol=1e-15)


def test_workloads_follow_pages_constants():
    pc = load("pages_constants.json")
    w = pc["window"]["value"]
    for name, cfg in wl.WORKLOADS.items():
        assert cfg.window == w, name
    assert wl.WORKLOADS["swa_prefill_32k"].num_kv_heads == pc["swa_kv_heads_v25"]["value"]
    # 1 + (mtp layers) tokens verified per sequence in the MTP-verify workload
    assert wl.WORKLOADS["decode_t4"].t_new == 1 + pc["mtp_layers"]["value"]
    ratio = pc["swa_to_ga_ratio_flash"]["value"]
    assert ratio == [5, 1]
