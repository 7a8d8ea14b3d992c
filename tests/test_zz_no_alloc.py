"""attn_decode_noalloc (the decode entry point that allocates nothing: its split partials
and arrival counters live in a library-owned device array) against attn_decode, through the
C ABI, on consecutive calls whose shapes shrink and grow again, so that whatever an earlier
call left in the shared array must not leak into a later one."""
import ctypes
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import transformer_attention_03_amd as ta  # noqa: E402

pytestmark = pytest.mark.gpu


def _call_both(L, dev, H, Hkv, D, Lk, W, cap, seed):
    q, k, v = synth.decode_inputs(seed, H, Hkv, D, Lk)
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    o_ref = torch.full((H, D), float("nan"), dtype=torch.float32, device=dev)
    o_na = torch.full((H, D), float("nan"), dtype=torch.float32, device=dev)
    ws = ta.decode_workspace(1, H, Hkv, D, Lk, dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    scale = 1.0 / math.sqrt(D)
    rc = L.attn_decode(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_ref.data_ptr(), H, Hkv, D,
                       Lk, W, cap, scale, ws.data_ptr(), ws.numel(), st)
    assert rc == ta.ATTN_OK, ta.attn_last_error()
    rc = L.attn_decode_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_na.data_ptr(), H, Hkv,
                               D, Lk, W, cap, scale, st)
    assert rc == ta.ATTN_OK, ta.attn_last_error()
    torch.cuda.synchronize()
    want = oracle.attention(q[None, None], np.transpose(k, (1, 0, 2))[None],
                            np.transpose(v, (1, 0, 2))[None], causal=True, window=W, softcap=cap,
                            scale=scale)[0, 0]
    return o_ref.cpu().numpy(), o_na.cpu().numpy(), want


def test_noalloc_equals_decode_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    L = ta.lib()
    # the 32/8-head 4096-token shape, then a smaller one (fewer splits and heads: the
    # counters now sit where the first call's partials were), then a large one with a cap
    for i, (H, Hkv, D, Lk, W, cap) in enumerate([(32, 8, 128, 4096, 0, 0.0),
                                                  (8, 2, 64, 700, 100, 0.0),
                                                  (16, 2, 256, 3000, 0, 50.0)]):
        print("noalloc call %d: H=%d Hkv=%d D=%d L=%d W=%d cap=%g" % (i, H, Hkv, D, Lk, W, cap), flush=True)
        ref, got, want = _call_both(L, dev, H, Hkv, D, Lk, W, cap, synth.seed_of(2) + 500 + i)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), i
        assert float(np.abs(got - want).max()) < 3e-3, i
