"""Every entry point captured once in a HIP graph and replayed several times, with eager
calls and synchronisations between the replays: each replay must equal the eager result
bit for bit (the benchmark times every workload as graph replays).  The decode, ring,
paged, tiered-int8 and device-kv-length graph tests sit beside their entry points' other
tests; these cover the rest."""
import math

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
import transformer_attention_03_amd as ta  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def replay_equals_eager(launch, out, reps=3):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        launch()
    torch.cuda.synchronize()
    for _ in range(reps):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        launch()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("dtype,S,L,H,Hkv,D,W,cap", [
    ("f16", 1100, 1100, 16, 8, 128, 300, 50.0),   # standard configuration, capped
    ("f16", 200, 700, 4, 2, 64, 0, 0.0),          # key groups
    ("f16", 300, 300, 8, 4, 256, 0, 0.0),
    ("f32", 128, 128, 1, 1, 64, 0, 0.0),          # the f32 workload's shape
])
def test_prefill_graph_replays(dev, dtype, S, L, H, Hkv, D, W, cap):
    print("graph prefill %s S=%d L=%d D=%d" % (dtype, S, L, D), flush=True)
    q, k, v = synth.prefill_inputs(synth.seed_of(12) + S + D, S, L, H, Hkv, D, dtype)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    o = torch.empty_like(qd)
    replay_equals_eager(lambda: ta.attn_prefill(qd, kd, vd, o, causal=True, scale=1 / math.sqrt(D),
                                                sliding_window=W, attn_softcap=cap), o)


def test_vision_graph_replays(dev):
    print("graph vision", flush=True)
    q, k, v = synth.vision_inputs(synth.seed_of(12) + 1, 1000, 16, 64)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    o = torch.empty_like(qd)
    replay_equals_eager(lambda: ta.attn_vision(qd, kd, vd, o, scale=0.125), o)


def test_block_local_graph_replays(dev):
    print("graph block-local", flush=True)
    d = synth.block_local_inputs(synth.seed_of(12) + 2, 700, 12, 12, 0, 8)
    q, k, v, pos = (to_dev(d[x], dev) for x in ("q", "k", "v", "pos"))
    o = torch.empty_like(q)
    replay_equals_eager(lambda: ta.attn_block_local(q, k, v, pos, o, seq=700, chunk_size=12, max_past=12,
                                                    max_future=0, logit_cap=50.0), o)


def test_tiered_packed_and_contiguous_f16_graph_replays(dev):
    print("graph tiered packed / contiguous f16", flush=True)
    t = synth.tiered_packed_inputs(synth.seed_of(12) + 3, 8, 2, 128, 2000, 300, 512, 50)
    d = {x: to_dev(t[x], dev) for x in ("q", "ring_k", "ring_v", "packed_k", "packed_v", "packed_k_scales",
                                        "packed_v_scales")}
    o = torch.empty((8, 128), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, 8, 2, 128, 2300, dev)
    replay_equals_eager(lambda: ta.attn_decode_tiered_q8_packed(
        d["q"], d["ring_k"], d["ring_v"], d["packed_k"], d["packed_v"], d["packed_k_scales"],
        d["packed_v_scales"], o, ws, cold_len=2000, hot_len=300, hot_start=50, scale=1 / math.sqrt(128)), o)
    f = synth.tiered_f16_inputs(synth.seed_of(12) + 4, 8, 2, 128, 2000, 300, 512, 50, False)
    e = {x: to_dev(f[x], dev) for x in ("q", "ring_k", "ring_v", "cold_k_contig", "cold_v_contig")}
    replay_equals_eager(lambda: ta.attn_decode_tiered_f16(
        e["q"], e["ring_k"], e["ring_v"], e["cold_k_contig"], e["cold_v_contig"], None, o, ws, cold_len=2000,
        hot_len=300, hot_start=50, scale=1 / math.sqrt(128)), o)


def test_noalloc_graph_replays(dev):
    """The allocation-free decode clears its counters with a kernel, not a memset node, so
    it can be captured too."""
    print("graph noalloc", flush=True)
    q, k, v = synth.decode_inputs(synth.seed_of(12) + 5, 32, 8, 128, 4096)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    o = torch.empty((32, 128), dtype=torch.float32, device=dev)
    replay_equals_eager(lambda: ta.attn_decode_noalloc(qd, kd, vd, o, scale=1 / math.sqrt(128)), o)
