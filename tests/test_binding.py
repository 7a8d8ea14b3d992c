"""The Python binding refuses tensors of the wrong dtype or on the wrong device before
anything reaches the library (a wrong element size or a host pointer would make the
kernels read out of bounds).  CPU only: every case raises before the first HIP call."""
import pytest

torch = pytest.importorskip("torch")
import transformer_attention_03_amd as ta  # noqa: E402


def z(shape, dtype):
    return torch.zeros(shape, dtype=getattr(torch, dtype))


def ws():
    return z((4096,), "uint8")


def prefill_args(qd="float16", kd="float16", vd="float16", od="float16"):
    return (z((16, 4, 64), qd), z((16, 2, 64), kd), z((16, 2, 64), vd), z((16, 4, 64), od))


@pytest.mark.parametrize("kw,msg", [
    (dict(kd="float32"), "k must be float16"),
    (dict(vd="float32"), "v must be float16"),
    (dict(od="float32"), "o must be float16"),
    (dict(qd="float64", kd="float64", vd="float64", od="float64"), "q must be float32 or float16"),
    (dict(qd="float32", kd="float16", vd="float16", od="float32"), "k must be float32"),
])
def test_prefill_dtypes(kw, msg):
    with pytest.raises(ValueError, match=msg):
        ta.attn_prefill(*prefill_args(**kw), causal=True, scale=0.125)


def test_prefill_host_tensors_are_refused():
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_prefill(*prefill_args(), causal=True, scale=0.125)


def test_prefill_device_kv_len_needs_int32():
    q, k, v, o = prefill_args()
    with pytest.raises(ValueError, match="kv_len must be int32"):
        ta.attn_prefill_device_kv_len(q, k, v, o, z((1,), "int64"), causal=True, scale=0.125)


def test_vision_needs_f16():
    x = z((2, 16, 64), "float32")
    with pytest.raises(ValueError, match="q must be float16"):
        ta.attn_vision(x, x, x, x, scale=0.125)
    y = z((2, 16, 64), "float16")
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_vision(y, y, y, y, scale=0.125)


@pytest.mark.parametrize("fn", ["attn_decode", "attn_decode_ring"])
@pytest.mark.parametrize("bad,msg", [
    ("q", "q must be float32"), ("k", "k must be float16"), ("o", "o must be float32"),
    ("ws", "workspace must be uint8"),
])
def test_decode_dtypes(fn, bad, msg):
    a = dict(q=z((8, 64), "float32"), k=z((2, 32, 64), "float16"), v=z((2, 32, 64), "float16"),
             o=z((8, 64), "float32"), ws=ws())
    a[bad] = a[bad].to(torch.float16 if bad in ("q", "o") else torch.float32)
    kw = dict(scale=0.125)
    if fn == "attn_decode_ring":
        kw["total_len"] = 32
    with pytest.raises(ValueError, match=msg):
        getattr(ta, fn)(a["q"], a["k"], a["v"], a["o"], a["ws"], **kw)


def test_decode_host_tensors_are_refused():
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_decode(z((8, 64), "float32"), z((2, 32, 64), "float16"), z((2, 32, 64), "float16"),
                       z((8, 64), "float32"), ws(), scale=0.125)


def paged_args():
    return dict(q=z((2, 8, 64), "float32"), kp=z((10, 2, 16, 64), "int8"),
                vp=z((10, 2, 16, 64), "int8"), ks=z((10, 2, 16), "float32"),
                vs=z((10, 2, 16), "float32"), pt=z((2, 5), "int32"), kl=z((2,), "int32"),
                o=z((2, 8, 64), "float32"), ws=ws())


@pytest.mark.parametrize("bad,to,msg", [
    ("kp", "float16", "k_pages must be int8"),
    ("vs", "float16", "v_scales must be float32"),
    ("pt", "int64", "page_table must be int32"),
    ("kl", "int64", "kv_lens must be int32"),
    ("q", "float16", "q must be float32"),
])
def test_paged_dtypes(bad, to, msg):
    a = paged_args()
    a[bad] = a[bad].to(getattr(torch, to))
    with pytest.raises(ValueError, match=msg):
        ta.attn_decode_paged_q8(a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["pt"], a["kl"],
                                a["o"], a["ws"], scale=0.125)
    b = paged_args()
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_decode_paged_q8(b["q"], b["kp"], b["vp"], b["ks"], b["vs"], b["pt"], b["kl"],
                                b["o"], b["ws"], scale=0.125)


def test_tiered_dtypes():
    a = paged_args()
    hk = z((2, 32, 64), "float16")
    with pytest.raises(ValueError, match="hot_k must be float16"):
        ta.attn_decode_tiered_q8(a["q"][0], hk.float(), hk, a["kp"], a["vp"], a["ks"], a["vs"],
                                 a["pt"][0], a["o"][0], a["ws"], cold_len=16, hot_len=8,
                                 hot_start=0, scale=0.125)
    with pytest.raises(ValueError, match="cold_page_table must be int32"):
        ta.attn_decode_tiered_q8(a["q"][0], hk, hk, a["kp"], a["vp"], a["ks"], a["vs"],
                                 a["pt"][0].long(), a["o"][0], a["ws"], cold_len=16, hot_len=8,
                                 hot_start=0, scale=0.125)


def test_tiered_packed_and_f16_dtypes():
    hk = z((2, 32, 64), "float16")
    q, o = z((8, 64), "float32"), z((8, 64), "float32")
    ck8, cs = z((2, 40, 64), "int8"), z((2, 40), "float32")
    with pytest.raises(ValueError, match="cold_k must be int8"):
        ta.attn_decode_tiered_q8_packed(q, hk, hk, ck8.float(), ck8, cs, cs, o, ws(), cold_len=16, hot_len=8,
                                        hot_start=0, scale=0.125)
    with pytest.raises(ValueError, match="cold_v_scales must be float32"):
        ta.attn_decode_tiered_q8_packed(q, hk, hk, ck8, ck8, cs, cs.half(), o, ws(), cold_len=16, hot_len=8,
                                        hot_start=0, scale=0.125)
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_decode_tiered_q8_packed(q, hk, hk, ck8, ck8, cs, cs, o, ws(), cold_len=16, hot_len=8,
                                        hot_start=0, scale=0.125)
    ck16 = z((2, 40, 64), "float16")
    with pytest.raises(ValueError, match="cold_k must be float16"):
        ta.attn_decode_tiered_f16(q, hk, hk, ck16.float(), ck16, None, o, ws(), cold_len=16, hot_len=8,
                                  hot_start=0, scale=0.125)
    with pytest.raises(ValueError, match="cold_page_table must be int32"):
        ta.attn_decode_tiered_f16(q, hk, hk, z((3, 2, 16, 64), "float16"), z((3, 2, 16, 64), "float16"),
                                  z((3,), "int64"), o, ws(), cold_len=16, hot_len=8, hot_start=0, scale=0.125)
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_decode_tiered_f16(q, hk, hk, ck16, ck16, None, o, ws(), cold_len=16, hot_len=8,
                                  hot_start=0, scale=0.125)


def test_block_local_and_noalloc_dtypes():
    x = z((24, 2, 128), "float32")
    kv = z((36, 2, 128), "float32")
    pos = z((13, 2, 128), "float32")
    with pytest.raises(ValueError, match="q_pad must be float32"):
        ta.attn_block_local(x.half(), kv, kv, pos, x, seq=20, chunk_size=12, max_past=12, max_future=0)
    with pytest.raises(ValueError, match="pos_proj must be float32"):
        ta.attn_block_local(x, kv, kv, pos.half(), x, seq=20, chunk_size=12, max_past=12, max_future=0)
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_block_local(x, kv, kv, pos, x, seq=20, chunk_size=12, max_past=12, max_future=0)
    q, k = z((8, 64), "float32"), z((2, 32, 64), "float16")
    with pytest.raises(ValueError, match="k must be float16"):
        ta.attn_decode_noalloc(q, k.float(), k, q.clone(), scale=0.125)
    with pytest.raises(ValueError, match="must be on a GPU"):
        ta.attn_decode_noalloc(q, k, k, q.clone(), scale=0.125)
