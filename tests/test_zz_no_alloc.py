"""swa_sink_prefill_backward_noalloc (the library-owned scratch array) against
swa_sink_prefill_backward (a caller-provided workspace), through the C ABI."""
import ctypes

import pytest
import torch

import sliding_window_attention_amd as swa
from oracle import swa_oracle as orc
from sliding_window_attention_amd import workloads as wl

DEV = "cuda:0"


def _case(lens, hq, hkv, seed):
    x = wl.make_prefill(lens, hq, hkv, 128, "bf16", seed)
    o_ref, l_ref = orc.swa_sink_prefill(x["q"], x["k"], x["v"], x["sinks"], x["cu_seqlens"].numpy(), 128)
    g = {k: v.to(DEV) for k, v in x.items() if isinstance(v, torch.Tensor)}
    g["out"] = torch.tensor(o_ref).to(torch.bfloat16).to(DEV)
    g["lse"] = torch.tensor(l_ref, dtype=torch.float32, device=DEV)
    g["dout"] = torch.randn(x["q"].shape, generator=torch.Generator().manual_seed(seed + 1)).to(
        torch.bfloat16).to(DEV)
    g["max_seqlen"] = x["max_seqlen"]
    return g


def _grads(g):
    return (torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"]),
            torch.empty(g["q"].shape[1], dtype=torch.float32, device=DEV))


def _call(g, grads, ws=None):
    """One raw C call: the existing entry point with a workspace, or the scratch variant."""
    lib = swa.library()
    n, hq, d = g["q"].shape
    common = (g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(), g["sinks"].data_ptr(),
              g["cu_seqlens"].data_ptr(), g["cu_seqlens"].numel() - 1, n, g["max_seqlen"], hq, g["k"].shape[1],
              d, 128, 0.0, 1, g["out"].data_ptr(), g["lse"].data_ptr(), g["dout"].data_ptr(),
              *(t.data_ptr() for t in grads))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if ws is None:
        rc = lib.swa_sink_prefill_backward_noalloc(*common, stream)
    else:
        rc = lib.swa_sink_prefill_backward(*common, ws.data_ptr(), ws.numel(), stream)
    assert rc == 0, lib.swa_last_error().decode()


@pytest.mark.gpu
def test_noalloc_backward_equals_workspace_backward_on_calls_in_a_row():
    lib = swa.library()
    # two calls in a row on one GPU, the second smaller (the array keeps the first call's
    # contents), then a call on the vector-ALU kernels (group size 4)
    cases = [([4096, 1000, 3], 32, 4, 21), ([300, 45], 32, 4, 22), ([200, 31], 8, 2, 23)]
    for lens, hq, hkv, seed in cases:
        print(f"no-alloc backward {lens} {hq}/{hkv}", flush=True)
        g = _case(lens, hq, hkv, seed)
        n = g["q"].shape[0]
        ref = _grads(g)
        ws = torch.empty(int(lib.swa_sink_prefill_backward_workspace(n, hq)), dtype=torch.uint8, device=DEV)
        _call(g, ref, ws)
        got = _grads(g)
        for t in got:
            t.fill_(float("nan"))
        _call(g, got)
        torch.cuda.synchronize()
        for a, b, nm in zip(got, ref, ("dq", "dk", "dv", "dsinks")):
            assert torch.equal(a, b), f"{lens}: {nm} differs from the workspace entry point"
