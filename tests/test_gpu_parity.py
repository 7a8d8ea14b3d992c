"""GPU parity: every entry point of libattn.so against the float64 CPU oracle on the same
seeded inputs, element by element.

Tolerances (max-abs, on outputs of O(1)): 1e-4 for the float32 path, 3e-3 for the
float16 and int8 paths.  Every test compares every output element, full-size workloads
included.
Page-table indexing is checked bit-exactly: two placements of the same logical cache give
identical bits.
"""
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import transformer_attention_03_amd as ta  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_F16 = 3e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def say(msg):
    print(msg, flush=True)


# =============================================================================================
# contiguous f16 decode
# =============================================================================================

def run_decode(dev, q, k, v, W=0, cap=0.0, scale=None):
    H, D = q.shape
    Hkv, L, _ = k.shape
    scale = scale or 1.0 / math.sqrt(D)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    od = torch.empty((H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, L, dev)
    ta.attn_decode(qd, kd, vd, od, ws, scale=scale, sliding_window=W, attn_softcap=cap)
    torch.cuda.synchronize()
    # the arrival counters (at the end of the workspace) are left at zero
    assert int(ws[-256:].sum().item()) == 0
    return od.cpu().numpy(), ws


def decode_oracle(q, k, v, W=0, cap=0.0, scale=None):
    H, D = q.shape
    scale = scale or 1.0 / math.sqrt(D)
    kk = np.transpose(k, (1, 0, 2))[None]       # [1, L, Hkv, D]
    vv = np.transpose(v, (1, 0, 2))[None]
    return oracle.attention(q[None, None], kk, vv, causal=True, window=W, softcap=cap,
                            scale=scale)[0, 0]


@pytest.mark.parametrize("H,Hkv,D,L,W,cap", [
    (8, 2, 128, 300, 0, 0.0),
    (4, 4, 64, 1, 0, 0.0),
    (16, 2, 256, 777, 0, 0.0),
    (8, 8, 128, 129, 0, 0.0),
    (8, 2, 128, 1000, 100, 0.0),
    (8, 2, 128, 1000, 0, 50.0),
    (6, 3, 64, 500, 0, 0.0),
    (24, 4, 128, 333, 7, 0.0),
    (64, 8, 128, 2048, 0, 0.0),
    (32, 8, 128, 4096, 0, 0.0),          # the 32/8-head, 4096-token, head_dim 128 workload
])
def test_decode_f16(dev, H, Hkv, D, L, W, cap):
    say("decode H=%d Hkv=%d D=%d L=%d W=%d cap=%g" % (H, Hkv, D, L, W, cap))
    c = synth.seed_of(2) + 1000 * H + L
    q, k, v = synth.decode_inputs(c, H, Hkv, D, L)
    got, _ = run_decode(dev, q, k, v, W, cap)
    want = decode_oracle(q, k, v, W, cap)
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < TOL_F16


@pytest.mark.parametrize("H,Hkv,D,L,cap,tol", [
    (32, 8, 128, 4096, 0.0, 1e-5),
    (16, 2, 256, 777, 0.0, 1e-5),
    (8, 2, 128, 1000, 50.0, 2e-5),
])
def test_decode_keeps_f32_accuracy(dev, H, Hkv, D, L, cap, tol):
    """f16 K/V times the f32 query and softmax weights, each split into two f16 parts, are
    exact products: the result must sit at f32 rounding level, far inside the f16 bound."""
    say("decode f32-level accuracy H=%d Hkv=%d D=%d L=%d cap=%g" % (H, Hkv, D, L, cap))
    c = synth.seed_of(2) + 1000 * H + L
    q, k, v = synth.decode_inputs(c, H, Hkv, D, L)
    got, _ = run_decode(dev, q, k, v, 0, cap)
    assert maxabs(got, decode_oracle(q, k, v, 0, cap)) < tol


def test_decode_split_sizes_agree(dev):
    say("decode split sizes")
    q, k, v = synth.decode_inputs(synth.seed_of(2), 32, 8, 128, 4096)
    want = decode_oracle(q, k, v)
    outs = []
    try:
        for t in (16, 48, 128, 512, 4096):
            ta.attn_set_decode_split(t)
            got, ws = run_decode(dev, q, k, v)
            assert maxabs(got, want) < TOL_F16, t
            outs.append(got)
    finally:
        ta.attn_set_decode_split(0)
    for o in outs[1:]:
        assert maxabs(o, outs[0]) < 1e-5


def test_decode_repeat_is_deterministic_and_counters_reset(dev):
    say("decode repeat")
    q, k, v = synth.decode_inputs(synth.seed_of(2), 32, 8, 128, 4096)
    H, D = q.shape
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    ws = ta.decode_workspace(1, 32, 8, 128, 4096, dev)
    o1 = torch.empty((H, D), dtype=torch.float32, device=dev)
    o2 = torch.empty_like(o1)
    for _ in range(3):
        ta.attn_decode(qd, kd, vd, o1, ws, scale=1 / math.sqrt(128))
    ta.attn_decode(qd, kd, vd, o2, ws, scale=1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ---- ring-buffer cache of a sliding-window layer -----------------------------------------

def ring_cache(x, total, R, span):
    """The ring a cache of R rows holds after `total` tokens: position t at row t % R for the
    newest min(total, R) positions.  Rows of positions outside the newest `span` (and rows
    never written) hold NaN, so a stray read shows up in the output."""
    Hkv, _, D = x.shape
    ring = np.full((Hkv, R, D), np.nan, dtype=x.dtype)
    for t in range(max(0, total - span), total):
        ring[:, t % R] = x[:, t]
    return ring


def run_decode_ring(dev, q, kr, vr, total, W=0, cap=0.0):
    H, D = q.shape
    Hkv, R, _ = kr.shape
    qd, kd, vd = to_dev(q, dev), to_dev(kr, dev), to_dev(vr, dev)
    od = torch.empty((H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, R, dev)
    ta.attn_decode_ring(qd, kd, vd, od, ws, total_len=total, scale=1 / math.sqrt(D),
                        sliding_window=W, attn_softcap=cap)
    torch.cuda.synchronize()
    assert int(ws[-256:].sum().item()) == 0
    return od.cpu().numpy()


@pytest.mark.parametrize("H,Hkv,D,R,total,W,cap", [
    (8, 2, 128, 512, 512, 0, 0.0),         # full ring, no wrap
    (8, 2, 128, 512, 1300, 0, 0.0),        # wrapped
    (8, 2, 128, 512, 1300, 200, 0.0),      # window shorter than the ring
    (4, 4, 64, 100, 37, 0, 0.0),           # ring not yet full
    (16, 2, 256, 333, 5000, 333, 0.0),     # capacity not a multiple of 16
    (8, 8, 128, 1000, 7777, 0, 30.0),      # softcap
    (6, 3, 64, 48, 49, 17, 0.0),           # one step past a full ring, short window
    (32, 8, 128, 4096, 9000, 0, 0.0),      # 4096-token ring, 9000 tokens seen
])
def test_decode_ring(dev, H, Hkv, D, R, total, W, cap):
    """Oracle over the visible positions of the logical cache, and bit-identical to
    attn_decode over the same positions stored contiguously."""
    say("decode ring H=%d Hkv=%d D=%d R=%d total=%d W=%d cap=%g" % (H, Hkv, D, R, total, W, cap))
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 71 + R, H, Hkv, D, total)
    span = W if W > 0 else R
    lo = max(0, total - span)
    got = run_decode_ring(dev, q, ring_cache(k, total, R, span), ring_cache(v, total, R, span),
                          total, W, cap)
    assert np.all(np.isfinite(got))
    want = decode_oracle(q, k[:, lo:total], v[:, lo:total], cap=cap)
    assert maxabs(got, want) < TOL_F16
    ref, _ = run_decode(dev, q, np.ascontiguousarray(k[:, lo:total]),
                        np.ascontiguousarray(v[:, lo:total]), cap=cap)
    assert np.array_equal(got, ref)


def test_decode_ring_split_sizes_agree(dev):
    say("decode ring split sizes")
    H, Hkv, D, R, total = 8, 2, 128, 1000, 3333
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 81, H, Hkv, D, total)
    kr, vr = ring_cache(k, total, R, R), ring_cache(v, total, R, R)
    want = decode_oracle(q, k[:, total - R:], v[:, total - R:])
    try:
        for t in (16, 48, 256, 1024):
            ta.attn_set_decode_split(t)
            got = run_decode_ring(dev, q, kr, vr, total)
            assert maxabs(got, want) < TOL_F16, t
    finally:
        ta.attn_set_decode_split(0)


def test_decode_softcap_is_applied(dev):
    """With q scaled x8 and c = 5 the capped and uncapped results differ by >> tolerance."""
    say("decode softcap sensitivity")
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 7, 8, 2, 128, 512)
    q = (q * 8).astype(np.float32)
    got, _ = run_decode(dev, q, k, v, cap=5.0)
    capped = decode_oracle(q, k, v, cap=5.0)
    plain = decode_oracle(q, k, v)
    assert maxabs(capped, plain) > 30 * TOL_F16
    assert maxabs(got, capped) < TOL_F16


# =============================================================================================
# paged int8 decode
# =============================================================================================

def paged_to_dev(d, dev):
    return {k: to_dev(d[k], dev) for k in ("q", "k_pages", "v_pages", "k_scales", "v_scales",
                                           "page_table", "kv_lens")}


def run_paged(dev, d, W=0, cap=0.0, kv_lens=None, table=None):
    t = paged_to_dev(d, dev)
    if kv_lens is not None:
        t["kv_lens"] = to_dev(np.asarray(kv_lens, np.int32), dev)
    if table is not None:
        t["page_table"] = to_dev(table, dev)
    B, H, D = d["q"].shape
    Hkv = d["k_pages"].shape[1]
    mp = d["page_table"].shape[1]
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(B, H, Hkv, D, mp * 16, dev)
    ta.attn_decode_paged_q8(t["q"], t["k_pages"], t["v_pages"], t["k_scales"], t["v_scales"],
                            t["page_table"], t["kv_lens"], o, ws, scale=1 / math.sqrt(D),
                            sliding_window=W, attn_softcap=cap)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def paged_oracle(d, W=0, cap=0.0):
    """Oracle over the LOGICAL int8 rows (before paging): never reads the page table."""
    B, H, D = d["q"].shape
    Hkv = d["k_q"][0].shape[1]
    out = np.zeros((B, H, D))
    for b in range(B):
        k = oracle.dequant_i8(d["k_q"][b], d["k_s"][b])[None]
        v = oracle.dequant_i8(d["v_q"][b], d["v_s"][b])[None]
        out[b] = oracle.attention(d["q"][b][None, None], k, v, causal=True, window=W,
                                  softcap=cap, scale=1 / math.sqrt(D))[0, 0]
    return out


@pytest.mark.parametrize("lens,H,Hkv,D,W,cap", [
    ([37, 16, 1, 500], 8, 2, 128, 0, 0.0),
    ([1000, 2049, 333], 32, 8, 128, 0, 0.0),
    ([700, 129], 8, 2, 64, 0, 0.0),
    ([300, 1111], 8, 4, 256, 0, 0.0),
    ([1500, 900], 8, 2, 128, 256, 0.0),
    ([1500, 900], 8, 2, 128, 0, 30.0),
])
def test_paged_q8(dev, lens, H, Hkv, D, W, cap):
    say("paged lens=%s H=%d Hkv=%d D=%d W=%d cap=%g" % (lens, H, Hkv, D, W, cap))
    d = synth.paged_inputs(synth.seed_of(5) + sum(lens), len(lens), H, Hkv, D, lens, n_poison=9)
    got = run_paged(dev, d, W, cap)
    want = paged_oracle(d, W, cap)
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < TOL_F16


@pytest.mark.parametrize("lens,H,Hkv,D,vf", [
    ([1000, 2049, 333], 32, 8, 128, 1.0),
    ([700, 129], 16, 2, 128, 1.0),          # eight query heads per KV head
    ([1000, 517], 8, 2, 128, 1e4),          # large V scales
    ([1000, 517], 8, 2, 128, 1e-4),         # small V scales
])
def test_paged_q8_relative_accuracy(dev, lens, H, Hkv, D, vf):
    """int8 K/V enter the products exactly; the V scales are normalised by a power of two
    before the f16 split, so the relative error stays near f32 level for any scale range."""
    say("paged relative accuracy lens=%s H=%d Hkv=%d D=%d vf=%g" % (lens, H, Hkv, D, vf))
    d = synth.paged_inputs(synth.seed_of(5) + sum(lens), len(lens), H, Hkv, D, lens, n_poison=9)
    d["v_scales"] = (d["v_scales"] * np.float32(vf)).astype(np.float32)
    d["v_s"] = [(x * np.float32(vf)).astype(np.float32) for x in d["v_s"]]
    got = run_paged(dev, d)
    want = paged_oracle(d)
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < 5e-5 * np.abs(want).max()


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_merge_in_passes(dev, D, group):
    """16-token splits over 4096 tokens: 256 partials per (sequence, head chunk).  The last
    workgroup folds them through LDS a number of splits at a time that shrinks with the
    heads per workgroup and head_dim (down to 15 at 8 heads of 256), so most of these
    cases take several passes, each with its own maximum and rescale."""
    say("decode merge in passes D=%d group=%d" % (D, group))
    Hkv = 2
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 500 + D + group, Hkv * group, Hkv, D, 4096)
    try:
        ta.attn_set_decode_split(16)
        got, _ = run_decode(dev, q, k, v)
    finally:
        ta.attn_set_decode_split(0)
    assert maxabs(got, decode_oracle(q, k, v)) < TOL_F16


def test_paged_q8_error_does_not_grow_with_split_length(dev):
    """int8 V enters the products with a bias of 1.125 per weight, which leaves the
    accumulators block by block: a 4096-token split (32 blocks per wave) keeps the accuracy
    of a 256-token one."""
    say("paged error against split length")
    d = synth.paged_inputs(synth.seed_of(5) + 991, 1, 8, 2, 128, [32768], n_poison=3)
    want = paged_oracle(d)
    errs = []
    try:
        for ts in (256, 4096):
            ta.attn_set_decode_split(ts)
            got = run_paged(dev, d)
            errs.append(maxabs(got, want) / np.abs(want).max())
    finally:
        ta.attn_set_decode_split(0)
    say("relative errors %s" % errs)
    assert max(errs) < 1e-5


@pytest.mark.parametrize("lens,H,Hkv,D", [
    ([33, 4000, 1, 700, 16], 32, 2, 64),               # sixteen query heads per KV head
    ([1, 32768], 8, 2, 128),                            # one token next to a 32K sequence
    ([(7 * i) % 200 + 1 for i in range(40)], 8, 4, 128),  # forty short sequences
    # more than 64 sequences: the lengths are read 64 per load, so the owner of a workgroup
    # may sit in the second or third load
    ([(13 * i) % 300 + 1 for i in range(150)], 8, 4, 128),
    ([2000 if i % 9 == 0 else (5 * i) % 90 + 1 for i in range(70)], 8, 2, 64),
])
def test_paged_q8_batch_balance(dev, lens, H, Hkv, D):
    """The paged kernel shares its workgroups out over the batch by length: skewed and wide
    batches must still cover every token of every sequence exactly once."""
    say("paged balance lens=%s H=%d Hkv=%d D=%d" % (lens[:6], H, Hkv, D))
    mp = max((max(lens) + 15) // 16, 4)
    d = synth.paged_inputs(synth.seed_of(5) + 77 + len(lens), len(lens), H, Hkv, D, lens, n_poison=5,
                           max_pages=mp)
    got = run_paged(dev, d)
    want = paged_oracle(d)
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < 5e-5 * max(1.0, np.abs(want).max())


@pytest.fixture(scope="module")
def c5_inputs():
    """The batch-8, 32/8-head, head_dim 128 int8 paged workload with kv_len ~ U[16384, 32768]."""
    c = synth.seed_of(5)
    lens = synth.paged_kv_lens(c, 8, 16384, 32768)
    return synth.paged_inputs(c, 8, 32, 8, 128, lens, n_poison=64, max_pages=2048)


def test_paged_q8_full_workload(dev, c5_inputs):
    say("paged full workload")
    got = run_paged(dev, c5_inputs)
    want = paged_oracle(c5_inputs)
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < TOL_F16


def replay_matches_eager(launch, out, replays=3):
    """Capture `launch` once in a HIP graph and replay it several times, with eager work and
    synchronisations in between: every replay equals the eager result bitwise (the split
    merge's arrival counters reset themselves inside the kernel, with no memset node)."""
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
    for _ in range(replays):
        out.fill_(float("nan"))
        launch()                 # an eager call between replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    return eager.cpu().numpy()


def test_decode_graph_replays(dev):
    say("decode graph replays")
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 91, 32, 8, 128, 4096)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    o = torch.empty((32, 128), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, 32, 8, 128, 4096, dev)
    got = replay_matches_eager(lambda: ta.attn_decode(qd, kd, vd, o, ws, scale=1 / math.sqrt(128)), o)
    assert maxabs(got, decode_oracle(q, k, v)) < TOL_F16


def test_decode_ring_graph_replays(dev):
    say("decode ring graph replays")
    H, Hkv, D, R, total = 16, 4, 128, 1024, 2500
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 92, H, Hkv, D, total)
    qd = to_dev(q, dev)
    kd, vd = to_dev(ring_cache(k, total, R, R), dev), to_dev(ring_cache(v, total, R, R), dev)
    o = torch.empty((H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, R, dev)
    got = replay_matches_eager(lambda: ta.attn_decode_ring(qd, kd, vd, o, ws, total_len=total,
                                                           scale=1 / math.sqrt(D)), o)
    assert maxabs(got, decode_oracle(q, k[:, total - R:], v[:, total - R:])) < TOL_F16


def test_paged_graph_replays(dev):
    say("paged graph replays")
    lens = [3000, 77, 1500, 4096]
    d = synth.paged_inputs(synth.seed_of(5) + 93, 4, 16, 4, 128, lens, n_poison=8)
    t = paged_to_dev(d, dev)
    B, H, D = d["q"].shape
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(B, H, 4, D, d["page_table"].shape[1] * 16, dev)
    got = replay_matches_eager(lambda: ta.attn_decode_paged_q8(
        t["q"], t["k_pages"], t["v_pages"], t["k_scales"], t["v_scales"], t["page_table"],
        t["kv_lens"], o, ws, scale=1 / math.sqrt(D)), o)
    assert maxabs(got, paged_oracle(d)) < TOL_F16


# =============================================================================================
# tiered decode: int8 paged cold tier + f16 ring hot tier, one online softmax
# =============================================================================================

def run_tiered(dev, t, W=0, cap=0.0, ws=None):
    c = t["cold"]
    H, D = t["q"].shape
    Hkv = t["ring_k"].shape[0]
    d = {k: to_dev(v, dev) for k, v in (("q", t["q"]), ("hk", t["ring_k"]), ("hv", t["ring_v"]),
                                          ("kp", c["k_pages"]), ("vp", c["v_pages"]),
                                          ("ks", c["k_scales"]), ("vs", c["v_scales"]),
                                          ("pt", c["page_table"][0]))}
    o = torch.empty((H, D), dtype=torch.float32, device=dev)
    if ws is None:
        ws = ta.decode_workspace(1, H, Hkv, D, t["cold_len"] + t["hot_len"], dev)
    ta.attn_decode_tiered_q8(d["q"], d["hk"], d["hv"], d["kp"], d["vp"], d["ks"], d["vs"], d["pt"],
                             o, ws, cold_len=t["cold_len"], hot_len=t["hot_len"],
                             hot_start=t["hot_start"], scale=1 / math.sqrt(D), sliding_window=W,
                             attn_softcap=cap)
    torch.cuda.synchronize()
    assert int(ws[-256:].sum().item()) == 0
    return o.cpu().numpy()


def tiered_oracle(t, W=0, cap=0.0):
    """Oracle over the logical sequence: the dequantised cold rows followed by the hot f16
    rows (never reads the page table or the ring)."""
    c = t["cold"]
    H, D = t["q"].shape
    k = np.concatenate([oracle.dequant_i8(c["k_q"][0], c["k_s"][0]), t["hot_k"].astype(np.float64)])
    v = np.concatenate([oracle.dequant_i8(c["v_q"][0], c["v_s"][0]), t["hot_v"].astype(np.float64)])
    return oracle.attention(t["q"][None, None], k[None], v[None], causal=True, window=W, softcap=cap,
                            scale=1 / math.sqrt(D))[0, 0]


def poison_outside_window(t, W):
    """NaN in every stored row of a position the window hides (cold: its K and V scales; hot:
    its ring rows), so that a read of one shows up in the output."""
    total = t["cold_len"] + t["hot_len"]
    lo = max(0, total - W) if W > 0 else 0
    c = t["cold"]
    for p in range(min(lo, t["cold_len"])):
        pg = c["page_table"][0][p // 16]
        c["k_scales"][pg, :, p % 16] = np.nan
        c["v_scales"][pg, :, p % 16] = np.nan
    R = t["ring_k"].shape[1]
    for p in range(t["cold_len"], lo):
        r = (t["hot_start"] + p - t["cold_len"]) % R
        t["ring_k"][:, r] = np.nan
        t["ring_v"][:, r] = np.nan


@pytest.mark.parametrize("H,Hkv,D,cold,hot,R,hs,W,cap", [
    (8, 2, 128, 1000, 300, 512, 100, 0, 0.0),
    (32, 8, 128, 5000, 512, 512, 0, 0, 0.0),      # full hot ring
    (8, 2, 64, 37, 5, 64, 60, 0, 0.0),            # the hot tier wraps the ring end
    (4, 4, 64, 0, 50, 64, 20, 0, 0.0),            # empty cold tier
    (8, 2, 128, 777, 0, 16, 0, 0, 0.0),           # empty hot tier
    (8, 2, 128, 3000, 400, 500, 123, 1000, 0.0),  # window over both tiers
    (8, 2, 128, 3000, 400, 500, 123, 300, 0.0),   # window inside the hot tier
    (8, 8, 128, 2000, 256, 256, 7, 0, 30.0),      # softcap
    (16, 2, 128, 17, 1, 8, 3, 0, 0.0),            # a few tokens
    (24, 4, 64, 9000, 1000, 1024, 1000, 0, 0.0),  # six query heads per KV head
    (8, 2, 256, 2500, 300, 333, 200, 0, 0.0),     # head_dim 256
    (8, 4, 256, 1200, 100, 128, 127, 500, 20.0),  # head_dim 256, window over both tiers, softcap
])
def test_tiered_q8(dev, H, Hkv, D, cold, hot, R, hs, W, cap):
    say("tiered H=%d Hkv=%d D=%d cold=%d hot=%d R=%d hs=%d W=%d cap=%g" % (H, Hkv, D, cold, hot, R, hs, W, cap))
    t = synth.tiered_inputs(synth.seed_of(6) + cold + 7 * hot, H, Hkv, D, cold, hot, R, hs, n_poison=5)
    if W > 0:
        poison_outside_window(t, W)
    got = run_tiered(dev, t, W, cap)
    want = tiered_oracle(t, W, cap)
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < TOL_F16
    # int8 and f16 rows enter the products exactly: f32-level agreement
    assert maxabs(got, want) < 5e-5 * np.abs(want).max()


def test_tiered_split_sizes_agree(dev):
    say("tiered split sizes")
    t = synth.tiered_inputs(synth.seed_of(6) + 31, 8, 2, 128, 2500, 700, 1000, 900, n_poison=5)
    want = tiered_oracle(t)
    try:
        for ts in (16, 48, 256, 1024, 4096):
            ta.attn_set_decode_split(ts)
            got = run_tiered(dev, t)
            assert maxabs(got, want) < 5e-5 * np.abs(want).max(), ts
    finally:
        ta.attn_set_decode_split(0)


def test_tiered_graph_replays(dev):
    say("tiered graph replays")
    t = synth.tiered_inputs(synth.seed_of(6) + 33, 16, 4, 128, 3000, 600, 1024, 500, n_poison=5)
    c = t["cold"]
    d = {k: to_dev(v, dev) for k, v in (("q", t["q"]), ("hk", t["ring_k"]), ("hv", t["ring_v"]),
                                          ("kp", c["k_pages"]), ("vp", c["v_pages"]),
                                          ("ks", c["k_scales"]), ("vs", c["v_scales"]),
                                          ("pt", c["page_table"][0]))}
    o = torch.empty((16, 128), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, 16, 4, 128, 3600, dev)
    got = replay_matches_eager(lambda: ta.attn_decode_tiered_q8(
        d["q"], d["hk"], d["hv"], d["kp"], d["vp"], d["ks"], d["vs"], d["pt"], o, ws, cold_len=3000,
        hot_len=600, hot_start=500, scale=1 / math.sqrt(128)), o)
    assert maxabs(got, tiered_oracle(t)) < 5e-5 * np.abs(tiered_oracle(t)).max()


def test_paged_permutation_is_bit_identical(dev):
    say("paged permutation bit identity")
    lens = [2000, 1234, 17, 4096]
    c = synth.seed_of(5) + 99
    a = synth.paged_inputs(c, 4, 32, 8, 128, lens, n_poison=20)
    b = synth.paged_inputs(c, 4, 32, 8, 128, lens, n_poison=20, alt_perm=True)
    assert not np.array_equal(a["page_table"], b["page_table"])
    oa = run_paged(dev, a)
    ob = run_paged(dev, b)
    assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32))
    assert maxabs(oa, paged_oracle(a)) < TOL_F16


def test_paged_identity_table_equals_random_placement(dev):
    """The same logical pages stored in order (sequence b's page i at physical page
    start_b + i) and at seeded random places give bitwise identical outputs."""
    say("paged identity table")
    lens = [1500, 33, 4096]
    a = synth.paged_inputs(synth.seed_of(5) + 101, 3, 32, 8, 128, lens, n_poison=8)
    ident = dict(a)
    n_live = [(n + 15) // 16 for n in lens]
    P = sum(n_live)
    kp, vp = np.full_like(a["k_pages"][:P], -128), np.full_like(a["v_pages"][:P], -128)
    ks, vs = np.full_like(a["k_scales"][:P], np.nan), np.full_like(a["v_scales"][:P], np.nan)
    table = np.full_like(a["page_table"], -1)
    start = 0
    for b, n in enumerate(n_live):
        for i in range(n):
            src = a["page_table"][b, i]
            kp[start + i], vp[start + i] = a["k_pages"][src], a["v_pages"][src]
            ks[start + i], vs[start + i] = a["k_scales"][src], a["v_scales"][src]
            table[b, i] = start + i
        start += n
    ident.update(k_pages=kp, v_pages=vp, k_scales=ks, v_scales=vs, page_table=table)
    assert np.array_equal(run_paged(dev, a).view(np.uint32), run_paged(dev, ident).view(np.uint32))


def test_paged_int8_equals_f16_decode_on_dequantised_values(dev):
    """Cross-entry check: the int8 paged decode of a sequence and the contiguous f16 decode
    of the same rows dequantised (then rounded to f16) agree within the f16 tolerance."""
    say("paged int8 vs f16 decode")
    lens = [3000, 700]
    d = synth.paged_inputs(synth.seed_of(5) + 103, 2, 32, 8, 128, lens)
    got = run_paged(dev, d)
    for b in range(2):
        k16 = oracle.dequant_i8(d["k_q"][b], d["k_s"][b]).astype(np.float16)   # [L, Hkv, D]
        v16 = oracle.dequant_i8(d["v_q"][b], d["v_s"][b]).astype(np.float16)
        ref, _ = run_decode(dev, d["q"][b], np.ascontiguousarray(np.transpose(k16, (1, 0, 2))),
                            np.ascontiguousarray(np.transpose(v16, (1, 0, 2))))
        assert maxabs(got[b], ref) < TOL_F16, b


def test_paged_negative_control_detects_mis_indexing(dev):
    """A wrong page-table entry must show up.  One query sees every key, so the result is
    invariant to the ORDER of its pages; the controls therefore (a) point a logical page at
    a copy of another one and (b) swap a full page with the poisoned partial last page."""
    say("paged negative control")
    lens = [1000, 800]
    d = synth.paged_inputs(synth.seed_of(5) + 5, 2, 8, 2, 128, lens, n_poison=4)
    want = paged_oracle(d)
    assert maxabs(run_paged(dev, d), want) < TOL_F16
    dup = d["page_table"].copy()
    dup[0, 3] = dup[0, 40]
    got = run_paged(dev, d, table=dup)
    assert maxabs(got[0], want[0]) > 3 * TOL_F16
    assert maxabs(got[1], want[1]) < TOL_F16
    swp = d["page_table"].copy()
    last = (lens[0] + 15) // 16 - 1           # holds 8 live slots and 8 poisoned ones
    swp[0, 3], swp[0, last] = swp[0, last], swp[0, 3]
    got = run_paged(dev, d, table=swp)
    assert np.all(np.isnan(got[0]))
    assert maxabs(got[1], want[1]) < TOL_F16


def test_paged_out_of_contract_kv_len_gives_nan_row(dev):
    say("paged out-of-contract kv_len")
    lens = [300, 200, 100]
    d = synth.paged_inputs(synth.seed_of(5) + 6, 3, 8, 2, 128, lens, n_poison=2)
    mp = d["page_table"].shape[1]
    got = run_paged(dev, d, kv_lens=[300, 0, mp * 16 + 1])
    want = paged_oracle(d)
    assert maxabs(got[0], want[0]) < TOL_F16
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))


def test_paged_out_of_contract_kv_len_past_the_first_64_sequences(dev):
    """Seventy sequences, two of them (in the second load of 64 lengths) out of contract:
    their rows are NaN and every other row matches the oracle."""
    say("paged out-of-contract kv_len, 70 sequences")
    lens = [(11 * i) % 150 + 1 for i in range(70)]
    d = synth.paged_inputs(synth.seed_of(5) + 8, 70, 8, 2, 64, lens, n_poison=2)
    mp = d["page_table"].shape[1]
    bad = {66: 0, 69: mp * 16 + 1}
    got = run_paged(dev, d, kv_lens=[bad.get(b, L) for b, L in enumerate(lens)])
    want = paged_oracle(d)
    good = [b for b in range(70) if b not in bad]
    assert maxabs(got[good], want[good]) < TOL_F16
    assert all(np.all(np.isnan(got[b])) for b in bad)


# =============================================================================================
# prefill (token-major) and vision (head-major)
# =============================================================================================

def run_prefill(dev, q, k, v, causal, W=0, cap=0.0, scale=None):
    S, H, D = q.shape
    scale = scale or 1.0 / math.sqrt(D)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    od = torch.empty_like(qd)
    ta.attn_prefill(qd, kd, vd, od, causal=causal, scale=scale, sliding_window=W,
                    attn_softcap=cap)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def prefill_oracle_rows(q, k, v, rows, causal, W=0, cap=0.0, scale=None):
    """Oracle for selected query rows, one row at a time (keys up to its position)."""
    S, H, D = q.shape
    L = k.shape[0]
    scale = scale or 1.0 / math.sqrt(D)
    out = []
    for i in rows:
        p = L - S + i
        hi = p + 1 if causal else L
        o = oracle.attention(q[None, i:i + 1], k[None, :hi], v[None, :hi], causal=causal,
                             window=W, softcap=cap, scale=scale)[0, 0]
        out.append(o)
    return np.stack(out)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("S,L,causal,W,cap", [
    (200, 200, True, 0, 0.0),
    (200, 200, False, 0, 0.0),
    (77, 300, True, 0, 0.0),
    (300, 300, True, 37, 0.0),
    (300, 300, True, 0, 20.0),
    (130, 130, True, 64, 50.0),
])
def test_prefill_f16(dev, D, S, L, causal, W, cap):
    say("prefill f16 D=%d S=%d L=%d causal=%d W=%d cap=%g" % (D, S, L, causal, W, cap))
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + D + S, S, L, 4, 2, D, "f16")
    got = run_prefill(dev, q, k, v, causal, W, cap)
    want = oracle.attention(q[None], k[None], v[None], causal=causal, window=W, softcap=cap,
                            scale=1 / math.sqrt(D))[0]
    assert np.all(np.isfinite(got))
    assert maxabs(got, want) < TOL_F16


@pytest.mark.parametrize("D,S,L,H,Hkv,causal,W,cap", [
    (64, 128, 128, 1, 1, True, 0, 0.0),       # the causal 128-token, head_dim 64 f32 workload
    (64, 100, 250, 2, 1, True, 0, 0.0),
    (128, 70, 70, 4, 2, True, 16, 0.0),
    (256, 65, 65, 2, 2, False, 0, 10.0),
    (128, 40, 90, 3, 1, True, 0, 5.0),         # key groups with a cap and three heads per KV head
    (64, 520, 520, 8, 2, True, 0, 0.0),        # 72 workgroups of 64 rows: no key groups
])
def test_prefill_f32(dev, D, S, L, H, Hkv, causal, W, cap):
    say("prefill f32 D=%d S=%d L=%d" % (D, S, L))
    q, k, v = synth.prefill_inputs(synth.seed_of(1) + S + D, S, L, H, Hkv, D, "f32")
    got = run_prefill(dev, q, k, v, causal, W, cap)
    want = oracle.attention(q[None], k[None], v[None], causal=causal, window=W, softcap=cap,
                            scale=1 / math.sqrt(D))[0]
    assert maxabs(got, want) < TOL_F32


# f32 instantiations fwd_f32_kernel<D, CAP, KG> not reached above: key groups run below 64
# workgroups of 64 rows at head_dim 64 and 128, the 64-row blocks at and above it.
@pytest.mark.parametrize("D,S,L,H,Hkv,causal,W,cap", [
    (64, 100, 100, 2, 1, True, 0, 15.0),       # <64, true, true>
    (64, 520, 600, 8, 2, True, 200, 15.0),     # <64, true, false>: 72 workgroups
    (128, 520, 520, 8, 4, True, 0, 30.0),      # <128, true, false>
    (128, 520, 700, 8, 2, True, 100, 0.0),     # <128, false, false> with a window
    (256, 200, 200, 2, 1, True, 0, 0.0),       # <256, false, false>
    (256, 130, 300, 4, 2, False, 0, 0.0),
])
def test_prefill_f32_every_instantiation(dev, D, S, L, H, Hkv, causal, W, cap):
    say("prefill f32 instantiation D=%d S=%d L=%d H=%d cap=%g" % (D, S, L, H, cap))
    q, k, v = synth.prefill_inputs(synth.seed_of(1) + 7 * S + L + D, S, L, H, Hkv, D, "f32")
    got = run_prefill(dev, q, k, v, causal, W, cap)
    assert np.all(np.isfinite(got))
    want = oracle.attention(q[None], k[None], v[None], causal=causal, window=W, softcap=cap,
                            scale=1 / math.sqrt(D))[0]
    assert maxabs(got, want) < TOL_F32


@pytest.fixture(scope="module")
def c3_inputs():
    """Causal GQA prefill: 2048 tokens, 16/8 heads, head_dim 256, f16."""
    return synth.prefill_inputs(synth.seed_of(3), 2048, 2048, 16, 8, 256, "f16")


def test_prefill_full_workload_every_element(dev, c3_inputs):
    """The 2048-token windowed softcapped GQA prefill at head_dim 256, every output element
    against the oracle (the oracle runs all 32768 rows)."""
    say("prefill full workload, every element")
    q, k, v = c3_inputs
    got = run_prefill(dev, q, k, v, True, 512, 50.0)
    assert np.all(np.isfinite(got))
    want = oracle.attention(q[None], k[None], v[None], causal=True, window=512, softcap=50.0,
                            scale=1 / 16)[0]
    assert maxabs(got, want) < TOL_F16
    # row 0 sees only key 0: its output is v0 exactly, for every head
    G = 2
    for h in range(16):
        assert np.array_equal(got[0, h], v[0, h // G])


@pytest.mark.parametrize("S,L,H,Hkv,D,W", [
    (1024, 1024, 16, 8, 128, 0),     # 256 workgroups of 64 rows: the unsplit configuration
    (64, 4096, 4, 2, 128, 0),        # a short chunk after a long cache: four key groups
    (100, 3000, 2, 1, 64, 700),      # key groups with a window and a ragged chunk
    (1, 1, 4, 2, 128, 0),            # one query, one key: three of the four key groups idle
    (1, 5000, 8, 8, 64, 0),          # one query against a long cache
])
def test_prefill_both_configurations(dev, S, L, H, Hkv, D, W):
    """Grids that fill the device run 64-row workgroups; smaller ones run 32-row workgroups
    whose waves split the keys four ways and merge in LDS.  Both against the oracle, every
    element."""
    say("prefill configuration S=%d L=%d H=%d Hkv=%d D=%d W=%d" % (S, L, H, Hkv, D, W))
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + S + L, S, L, H, Hkv, D, "f16")
    got = run_prefill(dev, q, k, v, True, W, 0.0)
    assert np.all(np.isfinite(got))
    want = oracle.attention(q[None], k[None], v[None], causal=True, window=W,
                            scale=1 / math.sqrt(D))[0]
    assert maxabs(got, want) < TOL_F16


# Grids that fill the device (>= 256 workgroups of the standard block: 16 heads and >= 1100
# query rows, or head_dim 256), so that the configuration the full-size calls run is the one
# tested, with ragged last key tiles (1100 and 1700 keys are no multiple of 64 or 96), windows,
# softcaps (the capped instantiations) and chunks shorter than the cache.  Every element.
@pytest.mark.parametrize("S,L,H,Hkv,D,causal,W,cap", [
    (1100, 1100, 16, 8, 64, True, 0, 0.0),
    (1100, 1100, 16, 8, 64, True, 300, 50.0),
    (1100, 1700, 16, 8, 64, True, 0, 0.0),
    (1100, 1100, 16, 16, 64, False, 0, 20.0),
    (1100, 1100, 16, 8, 128, True, 0, 0.0),
    (1100, 1100, 16, 8, 128, True, 257, 50.0),
    (1100, 1700, 16, 4, 128, True, 0, 0.0),
    (1100, 1700, 16, 8, 128, True, 500, 30.0),
    (1100, 1100, 16, 16, 128, False, 0, 0.0),
    (700, 900, 24, 8, 256, True, 100, 30.0),
    (700, 700, 16, 16, 256, False, 0, 0.0),
])
def test_prefill_at_size_every_element(dev, S, L, H, Hkv, D, causal, W, cap):
    say("prefill at size S=%d L=%d H=%d Hkv=%d D=%d causal=%d W=%d cap=%g" % (S, L, H, Hkv, D, causal, W, cap))
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 3 * S + L + D + W, S, L, H, Hkv, D, "f16")
    got = run_prefill(dev, q, k, v, causal, W, cap)
    assert np.all(np.isfinite(got))
    want = oracle.attention(q[None], k[None], v[None], causal=causal, window=W, softcap=cap,
                            scale=1 / math.sqrt(D))[0]
    assert maxabs(got, want) < TOL_F16


@pytest.mark.parametrize("dtype,S,L,H,Hkv,D", [
    ("f16", 1100, 1100, 16, 8, 64),      # the standard configurations
    ("f16", 1100, 1300, 16, 8, 128),
    ("f16", 300, 300, 8, 4, 256),
    ("f16", 100, 400, 2, 1, 64),         # small grids (key groups)
    ("f16", 64, 64, 4, 2, 128),
    ("f32", 128, 128, 1, 1, 64),
    ("f32", 520, 600, 8, 2, 128),
])
def test_prefill_window_one_returns_own_value(dev, dtype, S, L, H, Hkv, D):
    """With a causal window of one key every query row sees only its own position, so its
    weight is exp(0) = 1 and the output is that key's V row, bit for bit."""
    say("prefill W=1 %s S=%d L=%d D=%d" % (dtype, S, L, D))
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 13 * S + D, S, L, H, Hkv, D, dtype)
    got = run_prefill(dev, q, k, v, True, 1, 0.0)
    G = H // Hkv
    for h in range(H):
        assert np.array_equal(got[:, h], v[L - S:, h // G]), h


def test_decode_window_one_returns_last_value(dev):
    """Decode with a window of one key: the output is the newest V row exactly (in f32)."""
    say("decode W=1")
    q, k, v = synth.decode_inputs(synth.seed_of(2) + 77, 32, 8, 128, 1000)
    got, _ = run_decode(dev, q, k, v, W=1)
    for h in range(32):
        assert np.array_equal(got[h], v[h // 4, -1].astype(np.float32)), h


# ---- chunked prefill against a cache whose length is read on the device -----------------

def run_prefill_dev_len(dev, q, kcap, vcap, L, causal, W=0, cap=0.0):
    S, H, D = q.shape
    qd, kd, vd = to_dev(q, dev), to_dev(kcap, dev), to_dev(vcap, dev)
    od = torch.empty_like(qd)
    kl = torch.tensor([L], dtype=torch.int32, device=dev)
    ta.attn_prefill_device_kv_len(qd, kd, vd, od, kl, causal=causal, scale=1 / math.sqrt(D),
                                  sliding_window=W, attn_softcap=cap)
    torch.cuda.synchronize()
    return od.cpu().numpy()


@pytest.mark.parametrize("dtype,D,W,cap", [
    ("f16", 64, 0, 0.0), ("f16", 128, 0, 0.0), ("f16", 256, 100, 50.0), ("f16", 128, 33, 0.0),
    ("f32", 64, 0, 0.0), ("f32", 128, 0, 20.0),
])
def test_prefill_device_kv_len(dev, dtype, D, W, cap):
    """A 77-query chunk against a 400-row cache at lengths 77 (no history), 250 and 400: the
    oracle on the first L keys, and bit-identical to attn_prefill with kv_len = L."""
    say("prefill device kv_len %s D=%d W=%d cap=%g" % (dtype, D, W, cap))
    S, Lmax, H, Hkv = 77, 400, 4, 2
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 31 + D, S, Lmax, H, Hkv, D, dtype)
    tol = TOL_F16 if dtype == "f16" else TOL_F32
    for L in (77, 250, 400):
        got = run_prefill_dev_len(dev, q, k, v, L, True, W, cap)
        want = oracle.attention(q[None], k[None, :L], v[None, :L], causal=True, window=W,
                                softcap=cap, scale=1 / math.sqrt(D))[0]
        assert np.all(np.isfinite(got))
        assert maxabs(got, want) < tol, L
        ref = run_prefill(dev, q, k[:L], v[:L], True, W, cap)
        assert np.array_equal(got, ref), L


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_prefill_device_kv_len_graph_replays(dev, dtype):
    """One captured launch replayed as the cache grows: every replay equals the eager call
    with that length (bitwise), including two replays at the same length."""
    say("prefill device kv_len graph replays %s" % dtype)
    S, Lmax, H, Hkv, D = 64, 1024, 8, 4, 128
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 41, S, Lmax, H, Hkv, D, dtype)
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    od = torch.empty_like(qd)
    kl = torch.tensor([Lmax], dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ta.attn_prefill_device_kv_len(qd, kd, vd, od, kl, causal=True, scale=1 / math.sqrt(D))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        ta.attn_prefill_device_kv_len(qd, kd, vd, od, kl, causal=True, scale=1 / math.sqrt(D))
    torch.cuda.synchronize()
    for L in (64, 300, 300, 1024, 700):
        kl.fill_(L)
        od.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = od.cpu().numpy()
        ref = run_prefill(dev, q, k[:L], v[:L], True)
        assert np.array_equal(got, ref), L
    rows = [0, 31, 63]
    want = prefill_oracle_rows(q, k[:700], v[:700], rows, True)
    assert maxabs(got[rows], want) < (TOL_F16 if dtype == "f16" else TOL_F32)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_prefill_device_kv_len_out_of_contract_gives_nan(dev, dtype):
    say("prefill device kv_len out of contract %s" % dtype)
    S, Lmax, H, Hkv, D = 40, 100, 2, 1, 64
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 51, S, Lmax, H, Hkv, D, dtype)
    for L in (39, 0, 101):
        got = run_prefill_dev_len(dev, q, k, v, L, True)
        assert np.all(np.isnan(got)), L
    got = run_prefill_dev_len(dev, q, k, v, 40, True)
    assert np.all(np.isfinite(got))


def test_prefill_softcap_is_applied(dev):
    say("prefill softcap sensitivity")
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 11, 160, 160, 2, 1, 128, "f16")
    q = (q.astype(np.float32) * 8).astype(np.float16)
    got = run_prefill(dev, q, k, v, True, 0, 5.0)
    capped = oracle.attention(q[None], k[None], v[None], causal=True, softcap=5.0,
                              scale=1 / math.sqrt(128))[0]
    plain = oracle.attention(q[None], k[None], v[None], causal=True, scale=1 / math.sqrt(128))[0]
    assert maxabs(capped, plain) > 30 * TOL_F16
    assert maxabs(got, capped) < TOL_F16


def test_prefill_window_row_equals_decode_slice(dev):
    """Causal + window prefill row i == decode over keys [i-W+1, i] (q f16 -> f32 exactly)."""
    say("prefill row == decode slice")
    S, H, Hkv, D, W = 300, 8, 2, 128, 64
    q, k, v = synth.prefill_inputs(synth.seed_of(3) + 21, S, S, H, Hkv, D, "f16")
    pre = run_prefill(dev, q, k, v, True, W)
    for i in (0, 5, 63, 64, 200, 299):
        lo = max(0, i - W + 1)
        kk = np.ascontiguousarray(np.transpose(k[lo:i + 1], (1, 0, 2)))
        vv = np.ascontiguousarray(np.transpose(v[lo:i + 1], (1, 0, 2)))
        dec, _ = run_decode(dev, q[i].astype(np.float32), kk, vv)
        assert maxabs(pre[i], dec) < 2 * TOL_F16


def run_vision(dev, q, k, v, scale):
    qd, kd, vd = to_dev(q, dev), to_dev(k, dev), to_dev(v, dev)
    od = torch.empty_like(qd)
    ta.attn_vision(qd, kd, vd, od, scale=scale)
    torch.cuda.synchronize()
    return od.cpu().numpy()


@pytest.mark.parametrize("H,P,D", [(2, 100, 64), (3, 257, 128), (1, 64, 256), (2, 1, 64)])
def test_vision_small(dev, H, P, D):
    say("vision H=%d P=%d D=%d" % (H, P, D))
    q, k, v = synth.vision_inputs(synth.seed_of(4) + P, P, H, D)
    got = run_vision(dev, q, k, v, 1 / math.sqrt(D))
    qt, kt, vt = (np.transpose(x, (1, 0, 2)) for x in (q, k, v))
    want = oracle.attention(qt[None], kt[None], vt[None], causal=False,
                            scale=1 / math.sqrt(D))[0]
    assert maxabs(np.transpose(got, (1, 0, 2)), want) < TOL_F16


def test_vision_full_workload_every_element(dev):
    """The 2304-patch, 16-head, head_dim 64 vision call, every output element against the
    oracle."""
    say("vision full workload, every element")
    q, k, v = synth.vision_inputs(synth.seed_of(4), 2304, 16, 64)
    got = run_vision(dev, q, k, v, 0.125)
    assert np.all(np.isfinite(got))
    qt, kt, vt = (np.transpose(x, (1, 0, 2)) for x in (q, k, v))
    want = oracle.attention(qt[None], kt[None], vt[None], causal=False, scale=0.125)[0]
    assert maxabs(np.transpose(got, (1, 0, 2)), want) < TOL_F16


@pytest.mark.parametrize("H,P,D", [(16, 1000, 64), (16, 1100, 128), (8, 777, 256)])
def test_vision_at_size_every_element(dev, H, P, D):
    """Vision grids of >= 256 workgroups with a ragged last key tile (1000 patches: ten
    96-key tiles and 40 keys; 1100: seventeen 64-key tiles and 12), every element."""
    say("vision at size H=%d P=%d D=%d" % (H, P, D))
    q, k, v = synth.vision_inputs(synth.seed_of(4) + 7 * P + D, P, H, D)
    got = run_vision(dev, q, k, v, 1 / math.sqrt(D))
    assert np.all(np.isfinite(got))
    qt, kt, vt = (np.transpose(x, (1, 0, 2)) for x in (q, k, v))
    want = oracle.attention(qt[None], kt[None], vt[None], causal=False, scale=1 / math.sqrt(D))[0]
    assert maxabs(np.transpose(got, (1, 0, 2)), want) < TOL_F16


def test_vision_equals_bidirectional_prefill(dev):
    say("vision == bidirectional prefill")
    q, k, v = synth.vision_inputs(synth.seed_of(4) + 3, 300, 4, 64)
    vis = run_vision(dev, q, k, v, 0.125)
    qt, kt, vt = (np.ascontiguousarray(np.transpose(x, (1, 0, 2))) for x in (q, k, v))
    pre = run_prefill(dev, qt, kt, vt, False, scale=0.125)
    assert np.array_equal(np.transpose(vis, (1, 0, 2)), pre)
