"""GPU parity at the largest sizes: caches whose K or V tensors exceed 2^31 bytes, so that
every address the kernels form must be 64-bit.  The oracle runs on the heads it checks only
(each over the full key range), in float64, on the logical rows; the inputs are the seeded
synthetic generators' as everywhere else.

- contiguous f16 decode over 1,250,013 positions (K and V 2.56 GB each; the last KV head's
  rows all lie past 2^31 bytes);
- paged int8 decode whose page pool holds 140,000 pages (K and V pools 2.29 GB each), the
  live pages of two sequences scattered over it by the seeded permutation, the rest poison;
- a 64-token prefill chunk at the end of a 1,200,000-position f16 cache (K and V 2.46 GB;
  positions from 1,048,576 on lie past 2^31 bytes);
- Conformer block-local attention over 540,000 frames of 8 heads (q, K, V and the output
  2.21 GB each, f32; frames from 524,288 on lie past 2^31 bytes), checked on slices of 120
  frames that the oracle takes as sequences of their own.
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_beyond_2gib(dev):
    H, Hkv, D, L = 32, 8, 128, 1250013
    say("max size: decode H=%d Hkv=%d D=%d L=%d" % (H, Hkv, D, L))
    q, k, v = synth.decode_inputs(synth.seed_of(10), H, Hkv, D, L)
    assert k.nbytes > (1 << 31)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    qd = torch.from_numpy(q).to(dev)
    o = torch.empty((H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, L, dev)
    ta.attn_decode(qd, kd, vd, o, ws, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    assert int(ws[-256:].sum().item()) == 0
    del kd, vd, ws
    release()
    assert np.all(np.isfinite(got))
    G = H // Hkv
    for kvh in (0, 3, Hkv - 1):               # KV head 7's rows lie past 2^31 bytes
        assert kvh < Hkv - 1 or kvh * L * D * 2 > (1 << 31)
        heads = list(range(kvh * G, kvh * G + G))
        kk = k[kvh][None, :, None, :]           # [1, L, 1, D]
        vv = v[kvh][None, :, None, :]
        want = oracle.attention(q[heads][None, None], kk, vv, causal=True,
                                scale=1 / math.sqrt(D))[0, 0]
        assert maxabs(got[heads], want) < 2e-5, kvh


def test_paged_pool_beyond_2gib(dev):
    H, Hkv, D = 32, 8, 128
    lens = [70000, 33333]
    pool = 140000
    live = sum((n + 15) // 16 for n in lens)
    say("max size: paged lens=%s pool=%d pages" % (lens, pool))
    d = synth.paged_inputs(synth.seed_of(10) + 1, 2, H, Hkv, D, lens, n_poison=pool - live)
    assert d["k_pages"].nbytes > (1 << 31)
    assert int(d["page_table"].max()) * 16 * Hkv * D > (1 << 31)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
         for k in ("q", "k_pages", "v_pages", "k_scales", "v_scales", "page_table", "kv_lens")}
    o = torch.empty((2, H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(2, H, Hkv, D, d["page_table"].shape[1] * 16, dev)
    ta.attn_decode_paged_q8(t["q"], t["k_pages"], t["v_pages"], t["k_scales"], t["v_scales"],
                            t["page_table"], t["kv_lens"], o, ws, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    del t, ws
    release()
    assert np.all(np.isfinite(got))
    for b in range(2):
        k = oracle.dequant_i8(d["k_q"][b], d["k_s"][b])[None]
        v = oracle.dequant_i8(d["v_q"][b], d["v_s"][b])[None]
        want = oracle.attention(d["q"][b][None, None], k, v, causal=True,
                                scale=1 / math.sqrt(D))[0, 0]
        assert maxabs(got[b], want) < 5e-5 * max(1.0, float(np.abs(want).max())), b


def test_prefill_chunk_beyond_2gib(dev):
    S, L, H, Hkv, D = 64, 1200000, 16, 8, 128
    say("max size: prefill S=%d L=%d H=%d Hkv=%d D=%d" % (S, L, H, Hkv, D))
    q, k, v = synth.prefill_inputs(synth.seed_of(10) + 2, S, L, H, Hkv, D, "f16")
    assert k.nbytes > (1 << 31)
    qd = torch.from_numpy(q).to(dev)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    od = torch.empty_like(qd)
    ta.attn_prefill(qd, kd, vd, od, causal=True, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    got = od.cpu().numpy()
    del kd, vd
    release()
    assert np.all(np.isfinite(got))
    G = H // Hkv
    for kvh in (0, Hkv - 1):
        heads = [kvh * G, kvh * G + G - 1]
        kk = np.ascontiguousarray(k[:, kvh:kvh + 1])[None]     # [1, L, 1, D]
        vv = np.ascontiguousarray(v[:, kvh:kvh + 1])[None]
        for h in heads:
            want = oracle.attention(q[None, :, h:h + 1], kk, vv, causal=True,
                                    scale=1 / math.sqrt(D))[0, :, 0]
            assert maxabs(got[:, h], want) < TOL_F16, h


def test_block_local_beyond_2gib(dev):
    seq, chunk, past, future, H, cap = 540000, 12, 12, 0, 8, 50.0
    say("max size: block-local seq=%d chunk=%d past=%d future=%d H=%d" % (seq, chunk, past, future, H))
    d = synth.block_local_inputs(synth.seed_of(10) + 3, seq, chunk, past, future, H)
    q, k, v, pos = d["q"], d["k"], d["v"], d["pos"]
    assert q.nbytes > (1 << 31) and k.nbytes > (1 << 31)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    od = torch.empty_like(qd)
    ta.attn_block_local(qd, kd, vd, torch.from_numpy(pos).to(dev), od, seq=seq, chunk_size=chunk,
                        max_past=past, max_future=future, logit_cap=cap)
    torch.cuda.synchronize()
    got = od.cpu().numpy()
    del qd, kd, vd, od
    release()
    assert np.all(np.isfinite(got))
    # Frames [f0, f0 + n) as a sequence of their own (f0 and n multiples of the chunk): a row
    # whose key window lies inside the slice has the same output as in the full call.
    n = 120
    row_bytes = H * 128 * 4
    for f0 in (0, 264000, 524280, 529992, d["padded_len"] - n):
        assert f0 % chunk == 0
        want = oracle.block_local(q[f0:f0 + n], k[f0:f0 + n + past + future], v[f0:f0 + n + past + future],
                                  pos, seq=min(n, seq - f0), chunk_size=chunk, max_past=past,
                                  max_future=future, logit_cap=cap)
        lo = 0 if f0 == 0 else past + future
        assert maxabs(got[f0 + lo:f0 + n], want[lo:]) < 1e-4, f0
        if f0 >= 524280:
            assert (f0 + n) * row_bytes > (1 << 31)
