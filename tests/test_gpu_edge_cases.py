"""GPU parity in the method's limiting regimes, against the float64 oracle at the usual
tolerances:

- near one-hot softmax: scores scaled 32x (a max-to-second gap of several units, the other
  weights below e^-10), which tests the running-max rescaling of the online softmax;
- a tiny logit cap (c = 1e-3: every capped score within 1e-3 of 0, near-uniform weights);
- a huge logit cap (c = 1e6: c tanh(s / c) = s to 1e-12, so the result must equal the
  uncapped one), which tests the cap's accuracy for small tanh arguments;
- identical keys (every score equal: exactly uniform weights);
- int8 rows with zero scales (zero K scales: equal scores; zero V scales: a zero output).
"""
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import transformer_attention_03_amd as ta  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_F16 = 3e-3
TOL_F32 = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def to_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def prefill(dev, q, k, v, causal, W, cap, scale):
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    od = torch.empty_like(qd)
    ta.attn_prefill(qd, kd, vd, od, causal=causal, scale=scale, sliding_window=W, attn_softcap=cap)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def decode(dev, q, k, v, W, cap, scale):
    H, D = q.shape
    Hkv, L, _ = k.shape
    od = torch.empty((H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, L, dev)
    ta.attn_decode(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), od, ws, scale=scale, sliding_window=W,
                   attn_softcap=cap)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def decode_oracle(q, k, v, W, cap, scale):
    kk = np.transpose(k, (1, 0, 2))[None]
    vv = np.transpose(v, (1, 0, 2))[None]
    return oracle.attention(q[None, None], kk, vv, causal=True, window=W, softcap=cap, scale=scale)[0, 0]


# (name, scale multiplier, cap): the regimes above; "equal keys" is a test of its own
REGIMES = [("one_hot", 32.0, 0.0), ("one_hot_capped", 32.0, 50.0), ("tiny_cap", 1.0, 1e-3),
           ("huge_cap", 1.0, 1e6)]


@pytest.mark.parametrize("name,mul,cap", REGIMES, ids=[r[0] for r in REGIMES])
@pytest.mark.parametrize("S,L,H,Hkv,D,W", [
    (300, 300, 4, 2, 64, 0),         # key-group configurations
    (300, 500, 4, 2, 128, 100),
    (200, 200, 4, 2, 256, 0),
    (1100, 1100, 16, 8, 64, 0),      # the standard configurations
    (1100, 1100, 16, 8, 128, 300),
])
def test_prefill_f16_regimes(dev, name, mul, cap, S, L, H, Hkv, D, W):
    say("edge prefill f16 %s S=%d L=%d H=%d D=%d W=%d" % (name, S, L, H, D, W))
    q, k, v = synth.prefill_inputs(synth.seed_of(11) + S + D, S, L, H, Hkv, D, "f16")
    scale = mul / math.sqrt(D)
    got = prefill(dev, q, k, v, True, W, cap, scale)
    assert np.all(np.isfinite(got))
    want = oracle.attention(q[None], k[None], v[None], causal=True, window=W, softcap=cap, scale=scale)[0]
    assert maxabs(got, want) < TOL_F16


@pytest.mark.parametrize("name,mul,cap", REGIMES, ids=[r[0] for r in REGIMES])
@pytest.mark.parametrize("S,L,H,Hkv,D", [(128, 128, 1, 1, 64), (520, 600, 8, 2, 128), (100, 100, 2, 2, 256)])
def test_prefill_f32_regimes(dev, name, mul, cap, S, L, H, Hkv, D):
    say("edge prefill f32 %s S=%d L=%d H=%d D=%d" % (name, S, L, H, D))
    q, k, v = synth.prefill_inputs(synth.seed_of(11) + 3 * S + D, S, L, H, Hkv, D, "f32")
    scale = mul / math.sqrt(D)
    got = prefill(dev, q, k, v, True, 0, cap, scale)
    want = oracle.attention(q[None], k[None], v[None], causal=True, softcap=cap, scale=scale)[0]
    assert maxabs(got, want) < TOL_F32


@pytest.mark.parametrize("H,P,D", [(16, 1000, 64), (2, 300, 128), (2, 200, 256)])
def test_vision_one_hot(dev, H, P, D):
    say("edge vision one-hot H=%d P=%d D=%d" % (H, P, D))
    q, k, v = synth.vision_inputs(synth.seed_of(11) + P + D, P, H, D)
    scale = 32.0 / math.sqrt(D)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    od = torch.empty_like(qd)
    ta.attn_vision(qd, kd, vd, od, scale=scale)
    torch.cuda.synchronize()
    got = od.cpu().numpy()
    want = oracle.attention(np.transpose(q, (1, 0, 2))[None], np.transpose(k, (1, 0, 2))[None],
                            np.transpose(v, (1, 0, 2))[None], causal=False, scale=scale)[0]
    assert maxabs(got, np.transpose(want, (1, 0, 2))) < TOL_F16


@pytest.mark.parametrize("name,mul,cap", REGIMES, ids=[r[0] for r in REGIMES])
@pytest.mark.parametrize("H,Hkv,D,L,W", [(32, 8, 128, 4096, 0), (8, 2, 64, 1000, 300), (16, 4, 256, 2000, 0)])
def test_decode_regimes(dev, name, mul, cap, H, Hkv, D, L, W):
    say("edge decode %s H=%d D=%d L=%d W=%d" % (name, H, D, L, W))
    q, k, v = synth.decode_inputs(synth.seed_of(11) + L + D, H, Hkv, D, L)
    scale = mul / math.sqrt(D)
    got = decode(dev, q, k, v, W, cap, scale)
    want = decode_oracle(q, k, v, W, cap, scale)
    # decode keeps f32 accuracy: the bound is relative to the largest output
    assert maxabs(got, want) < 2e-5 * max(1.0, float(np.abs(want).max()))


@pytest.mark.parametrize("name,mul,cap", REGIMES, ids=[r[0] for r in REGIMES])
def test_paged_regimes(dev, name, mul, cap):
    lens = [3000, 17, 5000, 1]
    say("edge paged %s lens=%s" % (name, lens))
    H, Hkv, D = 16, 4, 128
    d = synth.paged_inputs(synth.seed_of(11) + 7, len(lens), H, Hkv, D, lens)
    t = {k: to_dev(d[k], dev) for k in ("q", "k_pages", "v_pages", "k_scales", "v_scales", "page_table",
                                        "kv_lens")}
    o = torch.empty((len(lens), H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(len(lens), H, Hkv, D, d["page_table"].shape[1] * 16, dev)
    scale = mul / math.sqrt(D)
    ta.attn_decode_paged_q8(t["q"], t["k_pages"], t["v_pages"], t["k_scales"], t["v_scales"], t["page_table"],
                            t["kv_lens"], o, ws, scale=scale, attn_softcap=cap)
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    for b in range(len(lens)):
        k = oracle.dequant_i8(d["k_q"][b], d["k_s"][b])[None]
        v = oracle.dequant_i8(d["v_q"][b], d["v_s"][b])[None]
        want = oracle.attention(d["q"][b][None, None], k, v, causal=True, softcap=cap, scale=scale)[0, 0]
        assert maxabs(got[b], want) < 5e-5 * max(1.0, float(np.abs(want).max())), b


@pytest.mark.parametrize("name,mul,cap", REGIMES, ids=[r[0] for r in REGIMES])
def test_tiered_f16_regimes(dev, name, mul, cap):
    say("edge tiered f16 %s" % name)
    H, Hkv, D = 8, 2, 128
    t = synth.tiered_f16_inputs(synth.seed_of(11) + 9, H, Hkv, D, 3000, 400, 512, 100, True)
    o = torch.empty((H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, 3400, dev)
    scale = mul / math.sqrt(D)
    ta.attn_decode_tiered_f16(to_dev(t["q"], dev), to_dev(t["ring_k"], dev), to_dev(t["ring_v"], dev),
                              to_dev(t["cold_k_pages"], dev), to_dev(t["cold_v_pages"], dev),
                              to_dev(t["cold_page_table"], dev), o, ws, cold_len=3000, hot_len=400,
                              hot_start=100, scale=scale, attn_softcap=cap)
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    k = np.concatenate([t["cold_k"], t["hot_k"]]).astype(np.float64)
    v = np.concatenate([t["cold_v"], t["hot_v"]]).astype(np.float64)
    want = oracle.attention(t["q"][None, None], k[None], v[None], causal=True, softcap=cap, scale=scale)[0, 0]
    assert maxabs(got, want) < 5e-5 * max(1.0, float(np.abs(want).max()))


@pytest.mark.parametrize("qmul,cap", [(8.0, 0.0), (1.0, 1e-3), (1.0, 1e6)], ids=["one_hot", "tiny_cap", "huge_cap"])
def test_block_local_regimes(dev, qmul, cap):
    say("edge block-local q x %g cap %g" % (qmul, cap))
    seq, chunk, past, future, H = 600, 12, 12, 0, 4
    d = synth.block_local_inputs(synth.seed_of(11) + 13, seq, chunk, past, future, H,
                                 q_scale=qmul / math.sqrt(128))
    o = torch.empty(d["q"].shape, dtype=torch.float32, device=dev)
    ta.attn_block_local(to_dev(d["q"], dev), to_dev(d["k"], dev), to_dev(d["v"], dev), to_dev(d["pos"], dev), o,
                        seq=seq, chunk_size=chunk, max_past=past, max_future=future, logit_cap=cap)
    torch.cuda.synchronize()
    want = oracle.block_local(d["q"], d["k"], d["v"], d["pos"], seq=seq, chunk_size=chunk, max_past=past,
                              max_future=future, logit_cap=cap)
    assert maxabs(o.cpu().numpy(), want) < TOL_F32


def test_equal_keys_give_the_mean_of_the_visible_values(dev):
    """Every key row equal: all scores of a row are equal, the weights exactly uniform, and
    the output the mean of the visible V rows (the oracle's; here also checked directly)."""
    say("edge equal keys")
    S, L, H, Hkv, D = 200, 200, 4, 2, 128
    q, k, v = synth.prefill_inputs(synth.seed_of(11) + 21, S, L, H, Hkv, D, "f16")
    k[:] = k[0]
    got = prefill(dev, q, k, v, True, 0, 0.0, 1 / math.sqrt(D))
    mean = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, L + 1)[:, None, None]
    G = H // Hkv
    for h in range(H):
        assert maxabs(got[:, h], mean[:, h // G]) < TOL_F16, h
    qd = synth.decode_inputs(synth.seed_of(11) + 22, 8, 2, 128, 1000)
    q1, k1, v1 = qd
    k1[:] = k1[:, :1]
    got1 = decode(dev, q1, k1, v1, 0, 0.0, 1 / math.sqrt(128))
    mean1 = v1.astype(np.float64).mean(axis=1)
    for h in range(8):
        assert maxabs(got1[h], mean1[h // 4]) < 2e-5, h


def test_paged_zero_scales(dev):
    """int8 rows whose scales are zero: a sequence whose K scales are all zero has equal
    scores (uniform weights, the mean of its V rows); one whose V scales are all zero
    returns zeros; a third sequence is untouched."""
    lens = [700, 333, 1000]
    say("edge paged zero scales lens=%s" % lens)
    H, Hkv, D = 8, 2, 128
    d = synth.paged_inputs(synth.seed_of(11) + 31, len(lens), H, Hkv, D, lens)
    for b, key in ((0, "k"), (1, "v")):
        n_pages = (lens[b] + 15) // 16
        d[key + "_scales"][d["page_table"][b, :n_pages]] = 0.0
        d[key + "_s"][b][:] = 0.0
    t = {k: to_dev(d[k], dev) for k in ("q", "k_pages", "v_pages", "k_scales", "v_scales", "page_table",
                                        "kv_lens")}
    o = torch.empty((len(lens), H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(len(lens), H, Hkv, D, d["page_table"].shape[1] * 16, dev)
    ta.attn_decode_paged_q8(t["q"], t["k_pages"], t["v_pages"], t["k_scales"], t["v_scales"], t["page_table"],
                            t["kv_lens"], o, ws, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.all(got[1] == 0)
    mean0 = oracle.dequant_i8(d["v_q"][0], d["v_s"][0]).mean(axis=0)       # [Hkv, D]
    for h in range(H):
        assert maxabs(got[0, h], mean0[h // (H // Hkv)]) < 2e-5, h
    for b in range(len(lens)):
        k = oracle.dequant_i8(d["k_q"][b], d["k_s"][b])[None]
        v = oracle.dequant_i8(d["v_q"][b], d["v_s"][b])[None]
        want = oracle.attention(d["q"][b][None, None], k, v, causal=True, scale=1 / math.sqrt(D))[0, 0]
        assert maxabs(got[b], want) < 5e-5 * max(1.0, float(np.abs(want).max())), b
