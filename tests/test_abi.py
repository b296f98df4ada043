"""C-ABI contract checks that need no GPU: the library loads, exports every symbol
include/swasink.h declares, and rejects bad arguments on the host (before any HIP
call) with the documented status codes and a message."""
import ctypes
import os
import re

import pytest

import sliding_window_attention_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swasink.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP = 0, -1, -2, -3, -4
NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"SWASINK_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == {"swa_sink_prefill", "ga_causal_prefill", "swa_sink_prefill_fp8kv", "swa_sink_decode",
                          "swa_sink_decode_fp8kv", "swa_sink_prefill_backward",
                          "swa_sink_prefill_backward_workspace", "swa_sink_prefill_backward_noalloc",
                          "swa_rope", "swa_sink_decode_rope",
                          "swa_ring_append_rope", "swa_topk_select", "swa_sparse_decode", "swa_sparse_decode_mtp",
                          "swa_sparse_decode_fp8kv",
                          "swa_sink_decode_rope_fp8kv", "swa_ring_append_fp8kv", "swa_sink_decode_rope_commit", "swa_sink_decode_rope_commit_fp8kv",
                          "swa_last_error", "swa_abi_version"}


def test_library_exports_every_declared_symbol():
    lib = swa.library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define SWASINK_ABI_VERSION (\d+)", open(HEADER).read())
    assert swa.abi_version() == int(m.group(1))


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, cu=FAKE, num_seqs=1, n=16, max_seqlen=16, hq=8,
             hkv=1, d=128, window=128, scale=0.0, dtype=1, out=FAKE, lse=NULL, stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_prefill(a["q"], a["k"], a["v"], a["sinks"], a["cu"], a["num_seqs"],
                                          a["n"], a["max_seqlen"], a["hq"], a["hkv"], a["d"],
                                          a["window"], a["scale"], a["dtype"], a["out"], a["lse"],
                                          a["stream"])


def _decode(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, head=FAKE, sinks=FAKE, b=4, t=1, hq=8,
             hkv=1, d=128, window=128, scale=0.0, dtype=1, out=FAKE, lse=NULL, stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_decode(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["head"],
                                         a["sinks"], a["b"], a["t"], a["hq"], a["hkv"], a["d"],
                                         a["window"], a["scale"], a["dtype"], a["out"], a["lse"],
                                         a["stream"])


def _last():
    return swa.library().swa_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=NULL), E_NULL, "non-NULL"),
    (dict(sinks=NULL), E_NULL, "sinks"),
    (dict(cu=NULL), E_NULL, "cu_seqlens"),
    (dict(out=NULL), E_NULL, "out"),
    (dict(hq=6, hkv=4), E_SHAPE, "multiple"),
    (dict(hq=0), E_SHAPE, ">= 1"),
    (dict(d=96), E_UNSUP, "head_dim"),
    (dict(window=0), E_SHAPE, "window"),
    (dict(dtype=7), E_DTYPE, "dtype"),
    (dict(n=-1), E_SHAPE, "total_tokens"),
    (dict(num_seqs=0), E_SHAPE, "num_seqs"),
    (dict(max_seqlen=0), E_SHAPE, "max_seqlen"),
    (dict(max_seqlen=17), E_SHAPE, "max_seqlen"),
])
def test_prefill_rejects_bad_arguments(kw, code, needle):
    assert _prefill(**kw) == code
    assert needle in _last()


def test_prefill_accepts_more_sequences_than_tokens():
    # zero-length sequences are valid, so a packed batch may hold more sequences than
    # tokens (cu_seqlens = [0, 0, 0, 1]); with no tokens nothing is launched, and with
    # tokens the size checks must not reject it (that case runs in the GPU parity tests)
    assert _prefill(n=0, max_seqlen=0, num_seqs=3) == OK
    assert _backward(n=0, max_seqlen=0, num_seqs=5, sinks=NULL, dsinks=NULL) == OK
    src = open(os.path.join(ROOT, "sliding_window_attention_amd", "csrc", "abi.hip")).read()
    assert "exceeds total_tokens" not in src


def test_prefill_empty_is_ok_and_launches_nothing():
    assert _prefill(n=0, max_seqlen=0) == OK
    assert _last() == ""


def test_ga_rejects_bad_arguments():
    lib = swa.library()
    rc = lib.ga_causal_prefill(FAKE, FAKE, FAKE, NULL, 1, 16, 16, 8, 1, 128, 0.0, 1, FAKE, NULL, NULL)
    assert rc == E_NULL and "cu_seqlens" in _last()
    rc = lib.ga_causal_prefill(FAKE, FAKE, FAKE, FAKE, 1, 16, 16, 8, 3, 128, 0.0, 1, FAKE, NULL, NULL)
    assert rc == E_SHAPE
    # no sinks argument exists for GA; a NULL lse is fine but NULL out is not
    rc = lib.ga_causal_prefill(FAKE, FAKE, FAKE, FAKE, 1, 16, 16, 8, 1, 128, 0.0, 1, NULL, NULL, NULL)
    assert rc == E_NULL


@pytest.mark.parametrize("kw,code,needle", [
    (dict(t=0), E_SHAPE, "T must"),
    (dict(t=128), E_SHAPE, "T must"),
    (dict(window=1, t=1), E_SHAPE, "window"),
    (dict(head=NULL), E_NULL, "ring_head"),
    (dict(sinks=NULL), E_NULL, "sinks"),
    (dict(kc=NULL), E_NULL, "k_cache"),
    (dict(b=-2), E_SHAPE, "batch"),
    (dict(hq=12, hkv=8), E_SHAPE, "multiple"),
    (dict(d=32), E_UNSUP, "head_dim"),
    (dict(dtype=-1), E_DTYPE, "dtype"),
])
def test_decode_rejects_bad_arguments(kw, code, needle):
    assert _decode(**kw) == code
    assert needle in _last()


FAKE2 = ctypes.c_void_p(0x2000)


def _commit(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, pos=FAKE, pk=FAKE, pv=FAKE, acc=FAKE, ppos=FAKE, pt=4, kc=FAKE,
             vc=FAKE, head=FAKE, head_out=FAKE2, sinks=FAKE, b=4, t=4, hq=8, hkv=1, d=128, window=128,
             scale=0.0, base=10000.0, dtype=1, out=FAKE, lse=NULL, stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_decode_rope_commit(
        a["q"], a["kn"], a["vn"], a["pos"], a["pk"], a["pv"], a["acc"], a["ppos"], a["pt"], a["kc"], a["vc"],
        a["head"], a["head_out"], a["sinks"], a["b"], a["t"], a["hq"], a["hkv"], a["d"], a["window"],
        a["scale"], a["base"], a["dtype"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(pt=0), E_SHAPE, "prev_T"),
    (dict(pt=128), E_SHAPE, "prev_T"),
    (dict(pt=0, b=0), E_SHAPE, "prev_T"),  # sizes validate before the empty batch returns
    (dict(t=0), E_SHAPE, "T must"),
    (dict(head_out=FAKE), E_SHAPE, "must not be ring_head"),
    (dict(head_out=NULL), E_NULL, "ring_head_out"),
    (dict(pk=NULL), E_NULL, "prev_k"),
    (dict(acc=NULL), E_NULL, "prev_accept"),
    (dict(ppos=NULL), E_NULL, "prev_positions"),
    (dict(pos=NULL), E_NULL, "positions"),
    (dict(base=-1.0), E_SHAPE, "rope_base"),
    (dict(dtype=3), E_DTYPE, "dtype"),
])
def test_decode_rope_commit_rejects_bad_arguments(kw, code, needle):
    assert _commit(**kw) == code
    assert needle in _last()


def test_decode_rope_commit_fp8kv_rejects_bad_scales():
    lib = swa.library()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 0.0, 0.5, FAKE, FAKE2, FAKE, 4, 4, 8, 1,
            128, 128, 0.0, 10000.0, 1, FAKE, NULL, NULL]
    assert lib.swa_sink_decode_rope_commit_fp8kv(*args) == E_SHAPE and "k_scale" in _last()
    args[11], args[12] = 0.5, float("nan")
    assert lib.swa_sink_decode_rope_commit_fp8kv(*args) == E_SHAPE and "finite" in _last()
    args[12], args[8] = 0.5, 0
    assert lib.swa_sink_decode_rope_commit_fp8kv(*args) == E_SHAPE and "prev_T" in _last()


def test_decode_rope_commit_empty_batch_and_no_rotation():
    assert _commit(b=0, q=NULL, kn=NULL, vn=NULL, pos=NULL, pk=NULL, pv=NULL, acc=NULL, ppos=NULL, kc=NULL,
                   vc=NULL, head=NULL, head_out=NULL, sinks=NULL, out=NULL) == OK
    # without rotation the positions are not needed, but prev_accept still is
    assert _commit(base=0.0, ppos=NULL, acc=NULL) == E_NULL and "prev_accept" in _last()


def test_decode_empty_batch_is_ok():
    assert _decode(b=0) == OK


def test_empty_inputs_accept_null_pointers_but_still_validate_sizes():
    lib = swa.library()
    assert _prefill(n=0, max_seqlen=0, q=NULL, k=NULL, v=NULL, sinks=NULL, cu=NULL, out=NULL) == OK
    assert lib.ga_causal_prefill(NULL, NULL, NULL, NULL, 1, 0, 0, 8, 1, 128, 0.0, 1, NULL, NULL,
                                 NULL) == OK
    assert _decode(b=0, q=NULL, kn=NULL, vn=NULL, kc=NULL, vc=NULL, head=NULL, sinks=NULL,
                   out=NULL) == OK
    assert _prefill(n=0, max_seqlen=0, hq=12, hkv=8) == E_SHAPE
    assert _prefill(n=0, max_seqlen=0, window=0) == E_SHAPE
    assert _decode(b=0, t=0) == E_SHAPE
    assert _decode(b=0, d=32) == E_UNSUP


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(4, 8, 128)
    with pytest.raises(ValueError, match="GPU tensor"):
        swa.swa_sink_prefill(q, q[:, :1].contiguous(), q[:, :1].contiguous(), torch.zeros(8),
                             torch.tensor([0, 4], dtype=torch.int32))


def _prefill_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.5, vs=0.25, sinks=FAKE, cu=FAKE, num_seqs=1, n=16,
             max_seqlen=16, hq=8, hkv=1, d=128, window=128, scale=0.0, dtype=1, out=FAKE, lse=NULL,
             stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_prefill_fp8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["sinks"],
                                                a["cu"], a["num_seqs"], a["n"], a["max_seqlen"], a["hq"],
                                                a["hkv"], a["d"], a["window"], a["scale"], a["dtype"],
                                                a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=0.0), E_SHAPE, "k_scale"),
    (dict(vs=-2.0), E_SHAPE, "v_scale"),
    (dict(ks=float("nan")), E_SHAPE, "finite"),
    (dict(vs=float("inf")), E_SHAPE, "finite"),
    (dict(window=0), E_SHAPE, "window"),
    (dict(k=NULL), E_NULL, "non-NULL"),
    (dict(cu=NULL), E_NULL, "non-NULL"),
    (dict(hq=6, hkv=4), E_SHAPE, "multiple"),
    (dict(d=96), E_UNSUP, "head_dim"),
    (dict(dtype=5), E_DTYPE, "dtype"),
])
def test_prefill_fp8kv_rejects_bad_arguments(kw, code, needle):
    assert _prefill_fp8(**kw) == code
    assert needle in _last()


def test_prefill_fp8kv_empty_stream_accepts_null_pointers():
    assert _prefill_fp8(n=0, q=NULL, k=NULL, v=NULL, sinks=NULL, cu=NULL, out=NULL) == OK
    assert _prefill_fp8(n=0, vs=0.0) == E_SHAPE  # the scales are still checked


def test_binding_prefill_fp8_refuses_non_byte_kv():
    import torch

    q = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        swa.swa_sink_prefill_fp8kv(q, torch.zeros(4, 1, 128), torch.zeros(4, 1, 128), 1.0, 1.0,
                                   torch.zeros(8), torch.tensor([0, 4], dtype=torch.int32))


def _decode_fp8(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, ks=0.5, vs=0.25, head=FAKE, sinks=FAKE, b=4,
             t=1, hq=8, hkv=1, d=128, window=128, scale=0.0, dtype=1, out=FAKE, lse=NULL, stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_decode_fp8kv(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["ks"],
                                               a["vs"], a["head"], a["sinks"], a["b"], a["t"], a["hq"],
                                               a["hkv"], a["d"], a["window"], a["scale"], a["dtype"],
                                               a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=0.0), E_SHAPE, "k_scale"),
    (dict(vs=-1.0), E_SHAPE, "v_scale"),
    (dict(ks=float("inf")), E_SHAPE, "finite"),
    (dict(vs=float("nan")), E_SHAPE, "finite"),
    (dict(t=0), E_SHAPE, "T must"),
    (dict(kc=NULL), E_NULL, "k_cache"),
    (dict(vc=NULL), E_NULL, "v_cache"),
    (dict(d=32), E_UNSUP, "head_dim"),
    (dict(dtype=7), E_DTYPE, "dtype"),
])
def test_decode_fp8kv_rejects_bad_arguments(kw, code, needle):
    assert _decode_fp8(**kw) == code
    assert needle in _last()
    if code in (E_SHAPE, E_NULL):  # messages written by the decode checks name the entry point
        assert "swa_sink_decode_fp8kv" in _last()


def test_decode_fp8kv_empty_batch_accepts_null_pointers():
    assert _decode_fp8(b=0, q=NULL, kn=NULL, vn=NULL, kc=NULL, vc=NULL, head=NULL, sinks=NULL,
                       out=NULL) == OK
    assert _decode_fp8(b=0, ks=0.0) == E_SHAPE  # the scales are still checked


def test_binding_fp8_refuses_non_byte_caches():
    import torch

    q = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        swa.swa_sink_decode_fp8kv(q, q[:, :, :1], q[:, :, :1], torch.zeros(1, 1, 128, 128),
                                  torch.zeros(1, 1, 128, 128), 1.0, 1.0,
                                  torch.zeros(1, dtype=torch.int32), torch.zeros(8), scale=None)


def _backward(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, cu=FAKE, num_seqs=1, n=16, max_seqlen=16, hq=8,
             hkv=1, d=128, window=128, scale=0.0, dtype=1, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE,
             dk=FAKE, dv=FAKE, dsinks=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_prefill_backward(
        a["q"], a["k"], a["v"], a["sinks"], a["cu"], a["num_seqs"], a["n"], a["max_seqlen"], a["hq"],
        a["hkv"], a["d"], a["window"], a["scale"], a["dtype"], a["out"], a["lse"], a["dout"], a["dq"],
        a["dk"], a["dv"], a["dsinks"], a["ws"], a["ws_bytes"], a["stream"])


def test_backward_workspace_size():
    lib = swa.library()
    assert lib.swa_sink_prefill_backward_workspace(16, 8) == 1024  # 2 x 128 floats, 256-aligned
    assert lib.swa_sink_prefill_backward_workspace(1000, 32) == 256000
    assert lib.swa_sink_prefill_backward_workspace(0, 8) == 0
    assert lib.swa_sink_prefill_backward_workspace(-1, 8) == -1


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ws_bytes=1000), E_SHAPE, "workspace of 1024"),
    (dict(ws=NULL), E_SHAPE, "workspace"),
    (dict(lse=NULL), E_NULL, "lse"),
    (dict(dout=NULL), E_NULL, "dout"),
    (dict(dk=NULL), E_NULL, "dk"),
    (dict(dsinks=NULL), E_NULL, "both"),
    (dict(sinks=NULL), E_NULL, "both"),
    (dict(window=0), E_SHAPE, "window"),
    (dict(hq=12, hkv=8), E_SHAPE, "multiple"),
    (dict(d=96), E_UNSUP, "head_dim"),
    (dict(num_seqs=0), E_SHAPE, "num_seqs"),
])
def test_backward_rejects_bad_arguments(kw, code, needle):
    assert _backward(**kw) == code
    assert needle in _last()


def _backward_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=FAKE, cu=FAKE, num_seqs=1, n=16, max_seqlen=16, hq=8,
             hkv=1, d=128, window=128, scale=0.0, dtype=1, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE,
             dk=FAKE, dv=FAKE, dsinks=FAKE, stream=NULL)
    a.update(kw)
    return swa.library().swa_sink_prefill_backward_noalloc(
        a["q"], a["k"], a["v"], a["sinks"], a["cu"], a["num_seqs"], a["n"], a["max_seqlen"], a["hq"],
        a["hkv"], a["d"], a["window"], a["scale"], a["dtype"], a["out"], a["lse"], a["dout"], a["dq"],
        a["dk"], a["dv"], a["dsinks"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(n=65537, max_seqlen=65537, hq=32, hkv=4), E_UNSUP, "16777216"),  # 2 x 65537 x 32 fp32 > 16 MiB
    (dict(n=1 << 20, max_seqlen=1 << 20, hq=8, hkv=1), E_UNSUP, "2097152"),
    (dict(lse=NULL), E_NULL, "lse"),
    (dict(dsinks=NULL), E_NULL, "both"),
    (dict(window=0), E_SHAPE, "window"),
    (dict(num_seqs=0), E_SHAPE, "num_seqs"),
])
def test_backward_noalloc_rejects_bad_arguments_and_sizes_beyond_its_scratch(kw, code, needle):
    assert _backward_noalloc(**kw) == code
    assert needle in _last()


def test_backward_empty_stream_without_sinks_reads_nothing():
    assert _backward(n=0, max_seqlen=0, q=NULL, k=NULL, v=NULL, cu=NULL, out=NULL, lse=NULL, dout=NULL,
                     dq=NULL, dk=NULL, dv=NULL, sinks=NULL, dsinks=NULL, ws=NULL, ws_bytes=0) == OK


# ---------------------------------------------------------------------------
# rotary embedding around decode
# ---------------------------------------------------------------------------

def _rope(**kw):
    a = dict(x=FAKE, pos=FAKE, rows=4, heads=2, d=128, base=10000.0, dtype=1)
    a.update(kw)
    return swa.library().swa_rope(a["x"], a["pos"], a["rows"], a["heads"], a["d"], a["base"], a["dtype"], NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(base=-1.0), E_SHAPE, "rope_base"),
    (dict(base=float("nan")), E_SHAPE, "rope_base"),
    (dict(base=float("inf")), E_SHAPE, "rope_base"),
    (dict(d=96), E_SHAPE, "head_dim"),
    (dict(rows=-1), E_SHAPE, "rows"),
    (dict(heads=0), E_SHAPE, "heads"),
    (dict(x=NULL), E_NULL, "positions"),
    (dict(pos=NULL), E_NULL, "positions"),
    (dict(dtype=5), E_DTYPE, "dtype"),
])
def test_rope_rejects_bad_arguments(kw, code, needle):
    assert _rope(**kw) == code
    assert needle in _last()


def test_rope_nothing_to_do_is_ok():
    assert _rope(rows=0, x=NULL, pos=NULL) == OK
    assert _rope(base=0.0, x=NULL, pos=NULL) == OK  # base 0: no rotation, nothing launched


def _decode_rope(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, head=FAKE, pos=FAKE, sinks=FAKE, b=2, t=1, hq=8,
             hkv=1, d=128, window=128, scale=0.0, base=10000.0, dtype=1, out=FAKE, lse=NULL)
    a.update(kw)
    return swa.library().swa_sink_decode_rope(
        a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["head"], a["pos"], a["sinks"], a["b"], a["t"], a["hq"],
        a["hkv"], a["d"], a["window"], a["scale"], a["base"], a["dtype"], a["out"], a["lse"], NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(pos=NULL), E_NULL, "positions"),
    (dict(base=-2.0), E_SHAPE, "rope_base"),
    (dict(t=0), E_SHAPE, "T must"),
    (dict(head=NULL), E_NULL, "ring_head"),
    (dict(d=32), E_UNSUP, "head_dim"),
])
def test_decode_rope_rejects_bad_arguments(kw, code, needle):
    assert _decode_rope(**kw) == code
    assert needle in _last()


def test_decode_rope_empty_batch_accepts_null_pointers():
    assert _decode_rope(b=0, q=NULL, kn=NULL, vn=NULL, kc=NULL, vc=NULL, head=NULL, pos=NULL, sinks=NULL,
                        out=NULL) == OK


def _append(**kw):
    a = dict(kn=FAKE, vn=FAKE, nacc=FAKE, pos=FAKE, kc=FAKE, vc=FAKE, head=FAKE, b=2, t=4, hkv=4, d=128,
             window=128, base=10000.0, dtype=1)
    a.update(kw)
    return swa.library().swa_ring_append_rope(
        a["kn"], a["vn"], a["nacc"], a["pos"], a["kc"], a["vc"], a["head"], a["b"], a["t"], a["hkv"], a["d"],
        a["window"], a["base"], a["dtype"], NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(t=0), E_SHAPE, "T must"),
    (dict(t=128), E_SHAPE, "T must"),
    (dict(window=1, t=1), E_SHAPE, "window"),
    (dict(hkv=0), E_SHAPE, "num_kv_heads"),
    (dict(d=80), E_SHAPE, "head_dim"),
    (dict(b=-1), E_SHAPE, "batch"),
    (dict(nacc=NULL), E_NULL, "n_accept"),
    (dict(head=NULL), E_NULL, "ring_head"),
    (dict(pos=NULL), E_NULL, "positions"),
    (dict(base=float("nan")), E_SHAPE, "rope_base"),
    (dict(dtype=9), E_DTYPE, "dtype"),
])
def test_ring_append_rejects_bad_arguments(kw, code, needle):
    assert _append(**kw) == code
    assert needle in _last()


def test_ring_append_edge_cases_validate_without_launching():
    assert _append(b=0, kn=NULL, vn=NULL, nacc=NULL, pos=NULL, kc=NULL, vc=NULL, head=NULL) == OK
    # base 0 copies the keys unrotated, so positions may be NULL; every other pointer is still
    # required (the call fails before any launch)
    assert _append(pos=NULL, base=0.0, kc=NULL) == E_NULL and "k_cache" in _last()


def _append_fp8(**kw):
    a = dict(kn=FAKE, vn=FAKE, nacc=FAKE, pos=FAKE, kc=FAKE, vc=FAKE, ks=0.5, vs=0.25, head=FAKE, b=2, t=4,
             hkv=4, d=128, window=128, base=10000.0, dtype=1)
    a.update(kw)
    return swa.library().swa_ring_append_fp8kv(
        a["kn"], a["vn"], a["nacc"], a["pos"], a["kc"], a["vc"], a["ks"], a["vs"], a["head"], a["b"], a["t"],
        a["hkv"], a["d"], a["window"], a["base"], a["dtype"], NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=0.0), E_SHAPE, "k_scale"),
    (dict(vs=-0.5), E_SHAPE, "v_scale"),
    (dict(ks=float("inf")), E_SHAPE, "finite"),
    (dict(vs=float("nan")), E_SHAPE, "finite"),
    (dict(t=0), E_SHAPE, "T must"),
    (dict(d=80), E_SHAPE, "head_dim"),
    (dict(kc=NULL), E_NULL, "k_cache"),
    (dict(pos=NULL), E_NULL, "positions"),
    (dict(dtype=9), E_DTYPE, "dtype"),
])
def test_ring_append_fp8kv_rejects_bad_arguments(kw, code, needle):
    assert _append_fp8(**kw) == code
    assert needle in _last()
    if code in (E_SHAPE, E_NULL):
        assert "swa_ring_append_fp8kv" in _last()


def test_ring_append_fp8kv_edge_cases_validate_without_launching():
    assert _append_fp8(b=0, kn=NULL, vn=NULL, nacc=NULL, pos=NULL, kc=NULL, vc=NULL, head=NULL) == OK
    assert _append_fp8(b=0, ks=-1.0) == E_SHAPE  # the scales are still checked
    assert _append_fp8(pos=NULL, base=0.0, vc=NULL) == E_NULL and "v_cache" in _last()


def _decode_rope_fp8(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, ks=0.5, vs=0.25, head=FAKE, pos=FAKE, sinks=FAKE,
             b=2, t=1, hq=8, hkv=1, d=128, window=128, scale=0.0, base=10000.0, dtype=1, out=FAKE, lse=NULL)
    a.update(kw)
    return swa.library().swa_sink_decode_rope_fp8kv(
        a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["ks"], a["vs"], a["head"], a["pos"], a["sinks"], a["b"],
        a["t"], a["hq"], a["hkv"], a["d"], a["window"], a["scale"], a["base"], a["dtype"], a["out"], a["lse"],
        NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(ks=0.0), E_SHAPE, "k_scale"),
    (dict(vs=float("inf")), E_SHAPE, "finite"),
    (dict(pos=NULL), E_NULL, "positions"),
    (dict(base=-2.0), E_SHAPE, "rope_base"),
    (dict(t=128), E_SHAPE, "T must"),
    (dict(sinks=NULL), E_NULL, "sinks"),
    (dict(d=32), E_UNSUP, "head_dim"),
])
def test_decode_rope_fp8kv_rejects_bad_arguments(kw, code, needle):
    assert _decode_rope_fp8(**kw) == code
    assert needle in _last()


def test_decode_rope_fp8kv_empty_batch_accepts_null_pointers():
    assert _decode_rope_fp8(b=0, q=NULL, kn=NULL, vn=NULL, kc=NULL, vc=NULL, head=NULL, pos=NULL, sinks=NULL,
                            out=NULL) == OK


def test_binding_fp8_append_refuses_non_byte_caches():
    import torch

    kn = torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16)
    ring = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        swa.swa_ring_append_fp8kv(kn, kn, torch.ones(1, dtype=torch.int32), None, ring, ring, 1.0, 1.0,
                                  torch.zeros(1, dtype=torch.int32), rope_base=0.0)
    with pytest.raises((ValueError, TypeError)):
        swa.swa_sink_decode_rope_fp8kv(kn, kn, kn, ring, ring, 1.0, 1.0, torch.zeros(1, dtype=torch.int32),
                                       torch.zeros(1, dtype=torch.int32), torch.zeros(1))


# ---------------------------------------------------------------------------
# token-level sparse attention
# ---------------------------------------------------------------------------

def _topk(**kw):
    a = dict(sc=FAKE, lens=FAKE, b=2, hkv=4, lmax=4096, k=1024, recent=128, idx=FAKE, cnt=FAKE)
    a.update(kw)
    return swa.library().swa_topk_select(a["sc"], a["lens"], a["b"], a["hkv"], a["lmax"], a["k"], a["recent"],
                                         a["idx"], a["cnt"], NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(k=-1), E_SHAPE, "k must"),
    (dict(recent=0), E_SHAPE, "recent"),
    (dict(lmax=0), E_SHAPE, "max_len"),
    (dict(hkv=0), E_SHAPE, "num_kv_heads"),
    (dict(b=-3), E_SHAPE, "batch"),
    (dict(sc=NULL), E_NULL, "scores"),
    (dict(idx=NULL), E_NULL, "indices"),
    (dict(cnt=NULL), E_NULL, "counts"),
])
def test_topk_rejects_bad_arguments(kw, code, needle):
    assert _topk(**kw) == code
    assert needle in _last()


def test_topk_empty_and_k_zero_need_no_index_array():
    assert _topk(b=0, sc=NULL, lens=NULL, idx=NULL, cnt=NULL) == OK
    assert _topk(k=0, idx=NULL, sc=NULL) == E_NULL  # scores are still required


def _sparse(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, idx=FAKE, cnt=FAKE, sinks=NULL, b=2, hq=32, hkv=4, d=128,
             lmax=4096, k=1024, recent=128, scale=0.0, dtype=1, out=FAKE, lse=NULL)
    a.update(kw)
    return swa.library().swa_sparse_decode(
        a["q"], a["kc"], a["vc"], a["lens"], a["idx"], a["cnt"], a["sinks"], a["b"], a["hq"], a["hkv"], a["d"],
        a["lmax"], a["k"], a["recent"], a["scale"], a["dtype"], a["out"], a["lse"], NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(recent=0), E_SHAPE, "recent"),
    (dict(k=8000, recent=200), E_SHAPE, "8192"),
    (dict(k=-5), E_SHAPE, "k >= 0"),
    (dict(lmax=0), E_SHAPE, "max_len"),
    (dict(hq=12, hkv=8), E_SHAPE, "multiple"),
    (dict(d=32), E_UNSUP, "head_dim"),
    (dict(q=NULL), E_NULL, "q, k_cache"),
    (dict(idx=NULL), E_NULL, "indices"),
    (dict(dtype=7), E_DTYPE, "dtype"),
])
def test_sparse_decode_rejects_bad_arguments(kw, code, needle):
    assert _sparse(**kw) == code
    assert needle in _last()


def test_sparse_decode_mtp_rejects_bad_arguments():
    lib = swa.library()
    # every call below fails validation (or has an empty batch): nothing is launched
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 2, 0, 8, 1, 128, 4096, 1024, 128, 0.0, 1, FAKE, NULL, NULL]
    assert lib.swa_sparse_decode_mtp(*args) == E_SHAPE and "T must" in _last()
    args[8] = 4097
    assert lib.swa_sparse_decode_mtp(*args) == E_SHAPE and "T must" in _last()
    args[8], args[13], args[14] = 2, 8000, 192  # 8000 + 192 + 1 > 8192
    assert lib.swa_sparse_decode_mtp(*args) == E_SHAPE and "k + recent + T - 1" in _last()
    args[14], args[7] = 128, 0  # empty batch: sizes still validated, nothing launched
    assert lib.swa_sparse_decode_mtp(*args) == OK


def test_sparse_decode_fp8kv_rejects_bad_arguments():
    lib = swa.library()
    # every call below fails validation (or has an empty batch): nothing is launched
    args = [FAKE, FAKE, FAKE, 0.0, 0.5, FAKE, FAKE, FAKE, NULL, 2, 1, 8, 1, 128, 4096, 1024, 128, 0.0, 1, FAKE,
            NULL, NULL]
    assert lib.swa_sparse_decode_fp8kv(*args) == E_SHAPE and "k_scale" in _last()
    args[3], args[4] = 0.5, float("inf")
    assert lib.swa_sparse_decode_fp8kv(*args) == E_SHAPE and "finite" in _last()
    args[4], args[10] = 0.5, 0
    assert lib.swa_sparse_decode_fp8kv(*args) == E_SHAPE and "T must" in _last()
    args[10], args[16] = 2, 0
    assert lib.swa_sparse_decode_fp8kv(*args) == E_SHAPE and "recent" in _last()
    args[16], args[9] = 128, 0
    assert lib.swa_sparse_decode_fp8kv(*args) == OK


def test_sparse_decode_empty_batch_and_optional_sinks():
    assert _sparse(b=0, q=NULL, kc=NULL, vc=NULL, lens=NULL, idx=NULL, cnt=NULL, out=NULL) == OK
    assert _sparse(sinks=NULL, out=NULL) == E_NULL and "out" in _last()


MIS = ctypes.c_void_p(0x1008)  # 8-byte aligned, not 16


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0


@pytest.mark.parametrize("call", [
    lambda: _prefill(k=MIS), lambda: _prefill(out=MIS), lambda: _decode(vc=MIS), lambda: _decode(kn=MIS),
    lambda: _commit(pk=MIS), lambda: _commit(q=MIS), lambda: _prefill_fp8(v=MIS), lambda: _decode_fp8(out=MIS),
    lambda: _backward(dq=MIS), lambda: _backward(ws=MIS), lambda: _rope(x=MIS), lambda: _append(kc=MIS),
    lambda: _append_fp8(vn=MIS), lambda: _decode_rope_fp8(kc=MIS), lambda: _decode_rope(q=MIS),
    lambda: _sparse(vc=MIS), lambda: _sparse(q=MIS),
], ids=lambda f: "")
def test_misaligned_tensor_pointers_are_refused(call):
    # every argument but one pointer is valid: the alignment check is the last before a
    # launch, so on a machine with a GPU a missing check would launch on fake pointers
    if _gpu_visible():
        pytest.skip("runs where no GPU is visible")
    assert call() == E_UNSUP and "16-byte aligned" in _last()
