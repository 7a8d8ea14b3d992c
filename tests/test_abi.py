"""The C ABI without a GPU: the library loads, exports every entry point the header
declares, and rejects invalid arguments on the host (before any HIP call) with the
documented status codes and messages."""
import ctypes
import os
import subprocess
import re

import pytest

import transformer_attention_03_amd as ta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

P = 0x10000          # a fake 16-byte-aligned device address; never dereferenced
MIS = 0x10004        # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("attn_prefill", "attn_prefill_device_kv_len", "attn_vision", "attn_decode",
              "attn_decode_ring", "attn_decode_paged_q8", "attn_decode_tiered_q8",
              "attn_decode_workspace_bytes",
              "attn_last_error", "attn_set_decode_split"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ta.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    # and the binding offers a function of the same name for each
    for n in declared_functions():
        assert callable(getattr(ta, n)), n


def test_library_links_no_torch():
    r = subprocess.run(["ldd", ta.LIB_PATH], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    # library names only: the hexadecimal load addresses can hold any digit string
    names = [ln.split()[0] for ln in r.stdout.splitlines() if ln.strip()]
    assert not any("torch" in n or "c10" in n for n in names), names
    assert any("amdhip64" in n for n in names), r.stdout + r.stderr


def prefill(**kw):
    a = dict(q=P, k=P, v=P, o=P, dtype=1, seq_len=16, kv_len=16, H=4, Hkv=2, D=128, causal=1,
             W=0, cap=0.0, scale=0.125)
    a.update(kw)
    return ta.lib().attn_prefill(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["seq_len"],
                                 a["kv_len"], a["H"], a["Hkv"], a["D"], a["causal"], a["W"],
                                 a["cap"], a["scale"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), ta.ATTN_ERR_INVALID_ARG, "q must not be null"),
    (dict(v=MIS), ta.ATTN_ERR_INVALID_ARG, "16-byte aligned"),
    (dict(dtype=7), ta.ATTN_ERR_INVALID_ARG, "dtype"),
    (dict(kv_len=0, seq_len=0), ta.ATTN_ERR_INVALID_ARG, "invalid kv_len 0"),
    (dict(seq_len=17), ta.ATTN_ERR_INVALID_ARG, "seq_len 17"),
    (dict(H=3), ta.ATTN_ERR_INVALID_ARG, "multiple of num_kv_heads"),
    (dict(Hkv=0), ta.ATTN_ERR_INVALID_ARG, ">= 1"),
    (dict(D=96), ta.ATTN_ERR_UNSUPPORTED, "requires head_dim in"),
    (dict(D=0), ta.ATTN_ERR_INVALID_ARG, "head_dim"),
    (dict(causal=2), ta.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(W=-1), ta.ATTN_ERR_INVALID_ARG, "sliding_window"),
    (dict(cap=-1.0), ta.ATTN_ERR_INVALID_ARG, "attn_softcap"),
    (dict(cap=float("inf")), ta.ATTN_ERR_INVALID_ARG, "attn_softcap"),
    (dict(scale=0.0), ta.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), ta.ATTN_ERR_INVALID_ARG, "scale"),
])
def test_prefill_validation(kw, code, msg):
    assert prefill(**kw) == code
    assert msg in ta.attn_last_error()


def test_vision_validation():
    L = ta.lib()
    assert L.attn_vision(P, P, P, P, 0, 16, 64, 0.125, None) == ta.ATTN_ERR_INVALID_ARG
    assert L.attn_vision(P, P, None, P, 8, 16, 64, 0.125, None) == ta.ATTN_ERR_INVALID_ARG
    assert L.attn_vision(P, P, P, P, 8, 16, 80, 0.125, None) == ta.ATTN_ERR_UNSUPPORTED
    assert L.attn_vision(P, P, P, P, 8, 16, 64, -1.0, None) == ta.ATTN_ERR_INVALID_ARG


def decode(**kw):
    a = dict(q=P, k=P, v=P, o=P, H=32, Hkv=8, D=128, L=4096, W=0, cap=0.0, scale=0.088, ws=P,
             wsb=1 << 30)
    a.update(kw)
    return ta.lib().attn_decode(a["q"], a["k"], a["v"], a["o"], a["H"], a["Hkv"], a["D"], a["L"],
                                a["W"], a["cap"], a["scale"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(k=None), ta.ATTN_ERR_INVALID_ARG, "k must not be null"),
    (dict(L=0), ta.ATTN_ERR_INVALID_ARG, "invalid kv_len 0"),
    (dict(H=30), ta.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(D=32), ta.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(ws=None), ta.ATTN_ERR_WORKSPACE, "workspace must not be null"),
    (dict(ws=P + 16), ta.ATTN_ERR_WORKSPACE, "256-byte aligned"),
    (dict(wsb=64), ta.ATTN_ERR_WORKSPACE, "smaller than"),
    (dict(W=-3), ta.ATTN_ERR_INVALID_ARG, "sliding_window"),
])
def test_decode_validation(kw, code, msg):
    assert decode(**kw) == code
    assert msg in ta.attn_last_error()


def prefill_dev(**kw):
    a = dict(q=P, k=P, v=P, o=P, dtype=1, seq_len=16, max_kv_len=64, kl=P, H=4, Hkv=2, D=128,
             causal=1, W=0, cap=0.0, scale=0.125)
    a.update(kw)
    return ta.lib().attn_prefill_device_kv_len(a["q"], a["k"], a["v"], a["o"], a["dtype"],
                                               a["seq_len"], a["max_kv_len"], a["kl"], a["H"],
                                               a["Hkv"], a["D"], a["causal"], a["W"], a["cap"],
                                               a["scale"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(kl=None), ta.ATTN_ERR_INVALID_ARG, "kv_len must not be null"),
    (dict(kl=P + 2), ta.ATTN_ERR_INVALID_ARG, "kv_len must be 4-byte aligned"),
    (dict(o=MIS), ta.ATTN_ERR_INVALID_ARG, "16-byte aligned"),
    (dict(max_kv_len=0), ta.ATTN_ERR_INVALID_ARG, "invalid max_kv_len 0"),
    (dict(seq_len=65), ta.ATTN_ERR_INVALID_ARG, "seq_len 65 must be in [1, max_kv_len = 64]"),
    (dict(dtype=3), ta.ATTN_ERR_INVALID_ARG, "dtype"),
    (dict(D=96), ta.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(scale=float("nan")), ta.ATTN_ERR_INVALID_ARG, "scale"),
])
def test_prefill_device_kv_len_validation(kw, code, msg):
    assert prefill_dev(**kw) == code
    assert msg in ta.attn_last_error()


def ring(**kw):
    a = dict(q=P, k=P, v=P, o=P, H=32, Hkv=8, D=128, R=4096, T=40000, W=0, cap=0.0, scale=0.088,
             ws=P, wsb=1 << 30)
    a.update(kw)
    return ta.lib().attn_decode_ring(a["q"], a["k"], a["v"], a["o"], a["H"], a["Hkv"], a["D"],
                                     a["R"], a["T"], a["W"], a["cap"], a["scale"], a["ws"],
                                     a["wsb"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(v=None), ta.ATTN_ERR_INVALID_ARG, "v must not be null"),
    (dict(R=0), ta.ATTN_ERR_INVALID_ARG, "invalid ring_len 0"),
    (dict(T=0), ta.ATTN_ERR_INVALID_ARG, "invalid total_len 0"),
    (dict(W=4097), ta.ATTN_ERR_INVALID_ARG, "sliding_window 4097 exceeds ring_len 4096"),
    (dict(W=-1), ta.ATTN_ERR_INVALID_ARG, "sliding_window"),
    (dict(D=48), ta.ATTN_ERR_UNSUPPORTED, "head_dim"),
    (dict(ws=None), ta.ATTN_ERR_WORKSPACE, "workspace must not be null"),
    (dict(wsb=64), ta.ATTN_ERR_WORKSPACE, "smaller than"),
])
def test_decode_ring_validation(kw, code, msg):
    assert ring(**kw) == code
    assert msg in ta.attn_last_error()


def paged(**kw):
    a = dict(q=P, kp=P, vp=P, ks=P, vs=P, pt=P, kl=P, o=P, B=8, H=32, Hkv=8, D=128, ps=16,
             npg=16000, mp=2048, W=0, cap=0.0, scale=0.088, ws=P, wsb=1 << 30)
    a.update(kw)
    return ta.lib().attn_decode_paged_q8(a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["pt"],
                                         a["kl"], a["o"], a["B"], a["H"], a["Hkv"], a["D"],
                                         a["ps"], a["npg"], a["mp"], a["W"], a["cap"],
                                         a["scale"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(pt=None), ta.ATTN_ERR_INVALID_ARG, "page_table must not be null"),
    (dict(kl=MIS), ta.ATTN_ERR_INVALID_ARG, "kv_lens must be 16-byte aligned"),
    (dict(B=0), ta.ATTN_ERR_INVALID_ARG, "batch"),
    (dict(ps=32), ta.ATTN_ERR_UNSUPPORTED, "page_size"),
    (dict(npg=0), ta.ATTN_ERR_INVALID_ARG, "num_pages"),
    (dict(ws=None), ta.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(wsb=1000), ta.ATTN_ERR_WORKSPACE, "smaller than"),
    (dict(cap=-2.0), ta.ATTN_ERR_INVALID_ARG, "attn_softcap"),
    (dict(B=1 << 20, H=1 << 20, Hkv=1), ta.ATTN_ERR_INVALID_ARG, "query rows"),   # q of 2^47 floats
])
def test_paged_validation(kw, code, msg):
    assert paged(**kw) == code
    assert msg in ta.attn_last_error()


def tiered(**kw):
    a = dict(q=P, hk=P, hv=P, kp=P, vp=P, ks=P, vs=P, pt=P, o=P, H=32, Hkv=8, D=128, cold=20000,
             hot=1000, R=1024, hs=0, ps=16, npg=2000, mp=1300, W=0, cap=0.0, scale=0.088, ws=P,
             wsb=1 << 30)
    a.update(kw)
    return ta.lib().attn_decode_tiered_q8(a["q"], a["hk"], a["hv"], a["kp"], a["vp"], a["ks"],
                                          a["vs"], a["pt"], a["o"], a["H"], a["Hkv"], a["D"],
                                          a["cold"], a["hot"], a["R"], a["hs"], a["ps"],
                                          a["npg"], a["mp"], a["W"], a["cap"], a["scale"],
                                          a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(hk=None), ta.ATTN_ERR_INVALID_ARG, "hot_k must not be null"),
    (dict(pt=MIS), ta.ATTN_ERR_INVALID_ARG, "cold_page_table must be 16-byte aligned"),
    (dict(D=96), ta.ATTN_ERR_UNSUPPORTED, "requires head_dim in"),
    (dict(cold=-1), ta.ATTN_ERR_INVALID_ARG, "must be >= 0"),
    (dict(cold=0, hot=0), ta.ATTN_ERR_INVALID_ARG, "cold_len + hot_len"),
    (dict(hot=1025), ta.ATTN_ERR_INVALID_ARG, "hot_len 1025 exceeds hot_window 1024"),
    (dict(hs=1024), ta.ATTN_ERR_INVALID_ARG, "hot_start 1024"),
    (dict(cold=20801), ta.ATTN_ERR_INVALID_ARG, "exceeds max_pages * page_size"),
    (dict(ps=8), ta.ATTN_ERR_UNSUPPORTED, "page_size"),
    (dict(W=-3), ta.ATTN_ERR_INVALID_ARG, "sliding_window"),
    (dict(ws=None), ta.ATTN_ERR_WORKSPACE, "workspace must not be null"),
    (dict(wsb=4096), ta.ATTN_ERR_WORKSPACE, "smaller than"),
])
def test_tiered_validation(kw, code, msg):
    assert tiered(**kw) == code
    assert msg in ta.attn_last_error()


def test_tiered_tiers_may_be_empty_and_null():
    """A tier with no positions needs no pointers: validation passes up to the workspace."""
    assert tiered(hot=0, hk=None, hv=None, ws=None) == ta.ATTN_ERR_WORKSPACE
    assert tiered(cold=0, kp=None, vp=None, ks=None, vs=None, pt=None, ws=None) == ta.ATTN_ERR_WORKSPACE


def test_workspace_bytes():
    n = ta.attn_decode_workspace_bytes(1, 32, 8, 128, 4096)
    assert n > 0 and n % 256 == 0
    assert ta.attn_decode_workspace_bytes(8, 32, 8, 128, 32768) > n
    assert ta.attn_decode_workspace_bytes(1, 30, 8, 128, 4096) == 0
    assert ta.attn_decode_workspace_bytes(1, 32, 8, 100, 4096) == 0


@pytest.mark.parametrize("args", [
    (2 ** 31 - 1, 2 ** 31 - 1, 1, 128, 2 ** 31 - 1),     # q of ~2^69 floats
    (1 << 20, 1 << 20, 1, 256, 1 << 20),
    (1, 8, 8, 128, 2 ** 31 - 1),                          # K of 2^41 elements
])
def test_workspace_bytes_refuses_shapes_no_buffer_can_hold(args):
    """Shapes whose q (batch x heads x head_dim) or K would exceed 2^40 elements are refused
    (0), so the size arithmetic never wraps to a small, allocatable number."""
    assert ta.attn_decode_workspace_bytes(*args) == 0


def test_workspace_bytes_grows_without_wrapping():
    """Large but representable shapes give sizes that grow with the shape."""
    sizes = [ta.attn_decode_workspace_bytes(b, 4096, 1, 128, 1 << 20) for b in (1, 64, 4096)]
    assert all(n > 0 for n in sizes) and sizes[0] < sizes[1] < sizes[2]


def test_split_override_sizes_workspace():
    base = ta.attn_decode_workspace_bytes(1, 32, 8, 128, 4096)
    try:
        ta.attn_set_decode_split(16)
        small = ta.attn_decode_workspace_bytes(1, 32, 8, 128, 4096)
        assert small > base
    finally:
        ta.attn_set_decode_split(0)
    assert ta.attn_decode_workspace_bytes(1, 32, 8, 128, 4096) == base
    with pytest.raises(ta.AttnError):
        ta.attn_set_decode_split(17)


def test_error_string_is_thread_local_and_cleared_on_success():
    import threading
    assert prefill(D=96) == ta.ATTN_ERR_UNSUPPORTED
    seen = {}

    def other():
        seen["msg"] = ta.attn_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "head_dim" in ta.attn_last_error()
    ta.attn_set_decode_split(0)   # a successful call clears it
    assert ta.attn_last_error() == ""


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """A decode whose split partials would not fit the library's scratch array is refused on
    the host, before any HIP call, with the limit in the message."""
    L = ta.lib()
    rc = L.attn_decode_noalloc(P, P, P, P, 64, 8, 256, 1000000, 0, 0.0, 0.0625, None)
    assert rc == ta.ATTN_ERR_UNSUPPORTED
    assert "scratch" in ta.attn_last_error() and "4194304" in ta.attn_last_error()
    rc = L.attn_decode_noalloc(None, P, P, P, 32, 8, 128, 4096, 0, 0.0, 0.088, None)
    assert rc == ta.ATTN_ERR_INVALID_ARG and "q must not be null" in ta.attn_last_error()


def block_local(**kw):
    a = dict(q=P, k=P, v=P, pos=P, o=P, seq=30, padded=36, rows=48, H=2, D=128, chunk=12,
             context=24, span=13, past=12, future=0, pad=12, cap=50.0)
    a.update(kw)
    return ta.lib().attn_block_local(a["q"], a["k"], a["v"], a["pos"], a["o"], a["seq"], a["padded"],
                                     a["rows"], a["H"], a["D"], a["chunk"], a["context"], a["span"],
                                     a["past"], a["future"], a["pad"], a["cap"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(pos=None), ta.ATTN_ERR_INVALID_ARG, "pos_proj must not be null"),
    (dict(D=64), ta.ATTN_ERR_UNSUPPORTED, "requires head_dim == 128"),
    (dict(seq=40), ta.ATTN_ERR_INVALID_ARG, "seq"),
    (dict(padded=30), ta.ATTN_ERR_INVALID_ARG, "multiple of chunk_size"),
    (dict(span=12), ta.ATTN_ERR_INVALID_ARG, "max_span"),
    (dict(context=25), ta.ATTN_ERR_INVALID_ARG, "context_size"),
    (dict(pad=0), ta.ATTN_ERR_INVALID_ARG, "pad_left"),
    (dict(rows=41), ta.ATTN_ERR_INVALID_ARG, "kv_rows"),
    (dict(past=20, future=9, span=30, context=41, pad=20, rows=56), ta.ATTN_ERR_UNSUPPORTED, "max_span <= 29"),
    (dict(cap=-1.0), ta.ATTN_ERR_INVALID_ARG, "logit_cap"),
    (dict(H=0), ta.ATTN_ERR_INVALID_ARG, "num_heads"),
])
def test_block_local_validation(kw, code, msg):
    assert block_local(**kw) == code
    assert msg in ta.attn_last_error()


def tiered_f16(**kw):
    a = dict(q=P, hk=P, hv=P, ck=P, cv=P, pt=P, o=P, H=8, Hkv=2, D=128, cold=100, hot=10, R=16, hs=0,
             layout=2, cap_rows=112, ps=16, npages=20, W=0, cap=0.0, scale=0.088, ws=P, wsb=1 << 30)
    a.update(kw)
    return ta.lib().attn_decode_tiered_f16(a["q"], a["hk"], a["hv"], a["ck"], a["cv"], a["pt"], a["o"], a["H"],
                                           a["Hkv"], a["D"], a["cold"], a["hot"], a["R"], a["hs"], a["layout"],
                                           a["cap_rows"], a["ps"], a["npages"], a["W"], a["cap"], a["scale"],
                                           a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(layout=1), ta.ATTN_ERR_INVALID_ARG, "cold_layout 1"),
    (dict(layout=0), ta.ATTN_ERR_INVALID_ARG, "takes no page table"),
    (dict(layout=0, pt=None, cap_rows=99), ta.ATTN_ERR_INVALID_ARG, "cold_capacity 99 is smaller"),
    (dict(cap_rows=100), ta.ATTN_ERR_INVALID_ARG, "multiple of 16"),
    (dict(cap_rows=96), ta.ATTN_ERR_INVALID_ARG, "exceeds max_pages * page_size"),
    (dict(pt=None), ta.ATTN_ERR_INVALID_ARG, "cold_page_table must not be null"),
    (dict(ps=32), ta.ATTN_ERR_UNSUPPORTED, "page_size 32"),
    (dict(ck=None), ta.ATTN_ERR_INVALID_ARG, "cold_k_pages must not be null"),
    (dict(hot=20), ta.ATTN_ERR_INVALID_ARG, "hot_len 20 exceeds hot_window 16"),
    (dict(ws=None), ta.ATTN_ERR_WORKSPACE, "workspace must not be null"),
])
def test_tiered_f16_validation(kw, code, msg):
    assert tiered_f16(**kw) == code
    assert msg in ta.attn_last_error()


def test_tiered_q8_packed_validation():
    L = ta.lib()
    rc = L.attn_decode_tiered_q8_packed(P, P, P, P, P, P, P, P, 8, 2, 128, 100, 10, 16, 0, 99, 0, 0.0, 0.088,
                                        P, 1 << 30, None)
    assert rc == ta.ATTN_ERR_INVALID_ARG and "cold_capacity 99 is smaller than cold_len 100" in ta.attn_last_error()
    rc = L.attn_decode_tiered_q8_packed(P, P, P, P, P, None, P, P, 8, 2, 128, 100, 10, 16, 0, 128, 0, 0.0, 0.088,
                                        P, 1 << 30, None)
    assert rc == ta.ATTN_ERR_INVALID_ARG and "cold_k_scales must not be null" in ta.attn_last_error()
