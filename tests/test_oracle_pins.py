"""Pins of the CPU oracle to facts that do not come from the oracle itself.

The pages print no numeric output, so the pins are: hand-derived closed forms
(tests/golden/closed_form.json), a deliberately different brute-force routine
on tiny shapes (extended precision, explicit additive -inf mask matrix, matrix
form), invariants of the definition, and special cases that reduce to a known
value.  Each pin is chosen so that a plausible slip in the oracle (a dropped
scale, the wrong KV head, an off-by-one in the window, a missing softcap, K and
V swapped) fails at least one of them; test_mutations_are_caught plants such
slips in a copy of the oracle and checks exactly that.
"""
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


# --------------------------------------------------------------------------------------------
# Independent brute force (long double, explicit mask matrix, matrix form)
# --------------------------------------------------------------------------------------------

def brute(q, k, v, kv_len, causal, window, softcap, scale):
    """q [B,S,H,D], k/v [B,L,Hkv,D] -> o [B,S,H,D] in np.longdouble.

    Builds, per (batch, head), the S x L score matrix, adds a mask matrix of 0 / -inf
    from the definition of the visible set, exponentiates after subtracting each row's
    maximum and normalises; KV heads are expanded with np.repeat (contiguous groups).
    """
    q = np.asarray(q, np.longdouble)
    k = np.asarray(k, np.longdouble)
    v = np.asarray(v, np.longdouble)
    B, S, H, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    G = H // Hkv
    o = np.zeros((B, S, H, D), np.longdouble)
    for b in range(B):
        Lb = int(kv_len[b])
        kk = np.repeat(k[b, :Lb], G, axis=1)   # [Lb, H, D]
        vv = np.repeat(v[b, :Lb], G, axis=1)
        mask = np.zeros((S, Lb), np.longdouble)
        for i in range(S):
            pos = Lb - S + i
            for j in range(Lb):
                if (causal and j > pos) or (window > 0 and pos - j >= window):
                    mask[i, j] = -np.inf
        for h in range(H):
            sc = (q[b, :, h, :] @ kk[:, h, :].T) * np.longdouble(scale)
            if softcap > 0:
                c = np.longdouble(softcap)
                sc = c * np.tanh(sc / c)
            sc = sc + mask
            mx = np.max(sc, axis=1, keepdims=True)
            e = np.exp(sc - mx)
            p = e / np.sum(e, axis=1, keepdims=True)
            o[b, :, h, :] = p @ vv[:, h, :]
    return o


def rand(rng, *shape):
    return rng.standard_normal(shape)


def test_brute_force_tiny_shapes():
    rng = np.random.default_rng(1234)
    n = 0
    for S in range(1, 6):
        for L in range(S, 6):
            for (H, Hkv) in [(1, 1), (2, 1), (2, 2), (4, 2), (4, 1)]:
                for D in (1, 3, 4):
                    causal = bool(rng.integers(0, 2))
                    window = int(rng.integers(0, 4))
                    softcap = [0.0, 0.5, 50.0][int(rng.integers(0, 3))]
                    scale = float(rng.uniform(0.2, 1.5))
                    B = 2
                    q = rand(rng, B, S, H, D) * 2
                    k = rand(rng, B, L, Hkv, D) * 2
                    v = rand(rng, B, L, Hkv, D)
                    kv_len = np.array([L, max(S, L - 1)], np.int32)
                    got = oracle.attention(q, k, v, kv_len=kv_len, causal=causal, window=window,
                                           softcap=softcap, scale=scale, threads=2)
                    want = brute(q, k, v, kv_len, causal, window, softcap, scale)
                    np.testing.assert_allclose(got, np.asarray(want, np.float64), rtol=0,
                                               atol=1e-12)
                    n += 1
    assert n == 225


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [0, 1, 2, 3])
@pytest.mark.parametrize("softcap", [0.0, 0.5, 50.0])
def test_brute_force_all_mask_softcap_combinations(causal, window, softcap):
    rng = np.random.default_rng(7 + window + int(causal) * 10 + int(softcap))
    q = rand(rng, 1, 5, 4, 3) * 3
    k = rand(rng, 1, 6, 2, 3) * 3
    v = rand(rng, 1, 6, 2, 3)
    got = oracle.attention(q, k, v, causal=causal, window=window, softcap=softcap, scale=0.7)
    want = brute(q, k, v, [6], causal, window, softcap, 0.7)
    np.testing.assert_allclose(got, np.asarray(want, np.float64), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------------
# Hand-derived fixtures
# --------------------------------------------------------------------------------------------

def _golden_cases():
    with open(os.path.join(HERE, "golden", "closed_form.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    q = np.array(case["q"], np.float64)[None]
    k = np.array(case["k"], np.float64)[None]
    v = np.array(case["v"], np.float64)[None]
    o = oracle.attention(q, k, v, causal=case["causal"], window=case["window"],
                         softcap=case["softcap"], scale=case["scale"])
    np.testing.assert_allclose(o[0], np.array(case["o"]), rtol=0, atol=case["tol"])


# --------------------------------------------------------------------------------------------
# Closed forms and special cases
# --------------------------------------------------------------------------------------------

def test_two_key_logistic_closed_form():
    """o = v0 + sigmoid(s1 - s0) (v1 - v0) for a row that sees exactly two keys."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        D = 4
        q = rand(rng, 1, 1, 1, D)
        k = rand(rng, 1, 2, 1, D)
        v = rand(rng, 1, 2, 1, D)
        sc = 0.37
        s0 = sc * float(q[0, 0, 0] @ k[0, 0, 0])
        s1 = sc * float(q[0, 0, 0] @ k[0, 1, 0])
        sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
        want = v[0, 0, 0] + sig * (v[0, 1, 0] - v[0, 0, 0])
        got = oracle.attention(q, k, v, scale=sc)[0, 0, 0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_one_key_rows_are_exact():
    """Causal row 0 returns v0 bit-exactly; with window 1 every row returns its own v_i."""
    rng = np.random.default_rng(4)
    q = rand(rng, 1, 7, 2, 5)
    k = rand(rng, 1, 7, 1, 5)
    v = rand(rng, 1, 7, 1, 5)
    o = oracle.attention(q, k, v, causal=True, scale=0.5)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], v[0, 0, 0])
    o = oracle.attention(q, k, v, causal=True, window=1, scale=0.5)
    for i in range(7):
        for h in range(2):
            assert np.array_equal(o[0, i, h], v[0, i, 0])


@pytest.mark.parametrize("causal,window,softcap", [(False, 0, 0.0), (True, 0, 0.0),
                                                   (True, 3, 50.0), (False, 2, 0.5)])
def test_uniform_v_returns_that_row(causal, window, softcap):
    rng = np.random.default_rng(5)
    q = rand(rng, 2, 6, 4, 8) * 3
    k = rand(rng, 2, 9, 2, 8) * 3
    u = rand(rng, 8)
    v = np.broadcast_to(u, (2, 9, 2, 8)).copy()
    o = oracle.attention(q, k, v, kv_len=[9, 7], causal=causal, window=window, softcap=softcap,
                         scale=0.3)
    np.testing.assert_allclose(o, np.broadcast_to(u, o.shape), rtol=0, atol=1e-15)


def test_one_hot_v_gives_softmax_weights():
    """With v_j = e_j the output row is the attention-weight row: sums to 1, equals a
    softmax computed by hand with math.exp."""
    rng = np.random.default_rng(6)
    L, D = 5, 6
    q = rand(rng, 1, 3, 1, D)
    k = rand(rng, 1, L, 1, D)
    v = np.zeros((1, L, 1, D))
    for j in range(L):
        v[0, j, 0, j] = 1.0
    sc = 0.8
    o = oracle.attention(q, k, v, causal=True, scale=sc)
    for i in range(3):
        pos = L - 3 + i
        s = [sc * float(q[0, i, 0] @ k[0, j, 0]) for j in range(pos + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        want = [x / tot for x in w] + [0.0] * (D - pos - 1)
        np.testing.assert_allclose(o[0, i, 0], want, rtol=0, atol=1e-15)
        assert abs(o[0, i, 0].sum() - 1.0) < 1e-15


def test_softcap_log_ratio_closed_form():
    """Two keys, one-hot V: ln(o_0 / o_1) = c tanh(s0/c) - c tanh(s1/c)."""
    rng = np.random.default_rng(8)
    for c in (0.5, 5.0, 50.0):
        q = rand(rng, 1, 1, 1, 3) * 4
        k = rand(rng, 1, 2, 1, 3) * 4
        v = np.zeros((1, 2, 1, 3))
        v[0, 0, 0, 0] = 1.0
        v[0, 1, 0, 1] = 1.0
        sc = 1.3
        s0 = sc * float(q[0, 0, 0] @ k[0, 0, 0])
        s1 = sc * float(q[0, 0, 0] @ k[0, 1, 0])
        o = oracle.attention(q, k, v, softcap=c, scale=sc)[0, 0, 0]
        want = c * math.tanh(s0 / c) - c * math.tanh(s1 / c)
        assert abs(math.log(o[0] / o[1]) - want) < 1e-12
        # and the cap matters: the uncapped gap differs
        assert abs((s0 - s1) - want) > 1e-6


def test_window_at_least_kv_len_equals_no_window():
    rng = np.random.default_rng(9)
    q = rand(rng, 1, 6, 2, 4)
    k = rand(rng, 1, 6, 2, 4)
    v = rand(rng, 1, 6, 2, 4)
    a = oracle.attention(q, k, v, causal=True, window=0, scale=0.5)
    for w in (6, 7, 100):
        assert np.array_equal(a, oracle.attention(q, k, v, causal=True, window=w, scale=0.5))
    b = oracle.attention(q, k, v, causal=True, window=5, scale=0.5)
    assert not np.array_equal(a, b)   # row 5 loses key 0


def test_windowed_prefill_row_equals_decode_on_slice():
    """Causal + window W, prefill row i == one-query attention over keys [max(0,i-W+1), i]."""
    rng = np.random.default_rng(10)
    S, H, Hkv, D, W = 9, 4, 2, 5, 3
    q = rand(rng, 1, S, H, D)
    k = rand(rng, 1, S, Hkv, D)
    v = rand(rng, 1, S, Hkv, D)
    full = oracle.attention(q, k, v, causal=True, window=W, softcap=2.0, scale=0.6)
    for i in range(S):
        lo = max(0, i - W + 1)
        one = oracle.attention(q[:, i:i + 1], k[:, lo:i + 1], v[:, lo:i + 1], causal=False,
                               softcap=2.0, scale=0.6)
        np.testing.assert_allclose(full[:, i:i + 1], one, rtol=0, atol=1e-15)


def test_query_block_at_end_of_cache():
    """seq_len < kv_len: the S queries are the last S positions (startPos = kv_len - S)."""
    rng = np.random.default_rng(11)
    L, S, D = 8, 3, 4
    q = rand(rng, 1, L, 2, D)
    k = rand(rng, 1, L, 1, D)
    v = rand(rng, 1, L, 1, D)
    full = oracle.attention(q, k, v, causal=True, window=4, scale=0.5)
    tail = oracle.attention(q[:, L - S:], k, v, causal=True, window=4, scale=0.5)
    np.testing.assert_allclose(tail, full[:, L - S:], rtol=0, atol=1e-15)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(12)
    H, Hkv = 8, 2
    q = rand(rng, 2, 4, H, 3)
    k = rand(rng, 2, 6, Hkv, 3)
    v = rand(rng, 2, 6, Hkv, 3)
    a = oracle.attention(q, k, v, kv_len=[6, 5], causal=True, window=2, scale=0.4)
    # contiguous groups: query head h uses KV head h // (H / Hkv)
    kr = np.repeat(k, H // Hkv, axis=2)
    vr = np.repeat(v, H // Hkv, axis=2)
    b = oracle.attention(q, kr, vr, kv_len=[6, 5], causal=True, window=2, scale=0.4)
    assert np.array_equal(a, b)
    # and a distinguishable interleaved map would differ
    ki = np.tile(k, (1, 1, H // Hkv, 1))
    vi = np.tile(v, (1, 1, H // Hkv, 1))
    c = oracle.attention(q, ki, vi, kv_len=[6, 5], causal=True, window=2, scale=0.4)
    assert not np.allclose(a, c)


def test_scale_power_of_two_exchange_is_exact():
    rng = np.random.default_rng(13)
    q = rand(rng, 1, 4, 2, 6)
    k = rand(rng, 1, 4, 2, 6)
    v = rand(rng, 1, 4, 2, 6)
    a = oracle.attention(q, k, v, causal=True, scale=0.375)
    b = oracle.attention(q * 4.0, k, v, causal=True, scale=0.375 / 4.0)
    assert np.array_equal(a, b)


def test_bidirectional_is_key_permutation_invariant():
    rng = np.random.default_rng(14)
    q = rand(rng, 1, 5, 2, 4)
    k = rand(rng, 1, 7, 2, 4)
    v = rand(rng, 1, 7, 2, 4)
    perm = rng.permutation(7)
    a = oracle.attention(q, k, v, scale=0.5)
    b = oracle.attention(q, k[:, perm], v[:, perm], scale=0.5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


def test_rows_are_independent_of_batching():
    """Multiple threads / rows give the same result as single rows one at a time."""
    rng = np.random.default_rng(15)
    q = rand(rng, 2, 5, 4, 8)
    k = rand(rng, 2, 9, 2, 8)
    v = rand(rng, 2, 9, 2, 8)
    a = oracle.attention(q, k, v, kv_len=[9, 6], causal=True, scale=0.3, threads=4)
    b = oracle.attention(q, k, v, kv_len=[9, 6], causal=True, scale=0.3, threads=1)
    assert np.array_equal(a, b)


def test_rejects_bad_arguments():
    z = np.zeros((1, 2, 3, 4))
    kz = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        oracle.attention(z, kz, kz)      # H % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 3, 2, 4)), kz, kz)   # S > kv_len


# --------------------------------------------------------------------------------------------
# int8 dequantisation
# --------------------------------------------------------------------------------------------

def test_dequant_known_values():
    q8 = np.array([[127, -127, 0, 1], [5, -3, 2, -1]], np.int8)
    sc = np.array([0.5, 0.25], np.float32)
    out = oracle.dequant_i8(q8, sc)
    assert np.array_equal(out, [[63.5, -63.5, 0.0, 0.5], [1.25, -0.75, 0.5, -0.25]])


def test_quantised_round_trip_error_bound():
    """|dequant(quant(x)) - x| <= scale/2 per element (plus f32 rounding)."""
    x = synth.normal_f32(99, (64, 8, 32))
    q8, sc = synth.quantize_i8(x)
    back = oracle.dequant_i8(q8, sc)
    err = np.abs(back - x.astype(np.float64))
    assert np.all(err <= sc[..., None].astype(np.float64) * 0.5 * (1 + 1e-6))
    assert q8.min() >= -127


# --------------------------------------------------------------------------------------------
# Planted mistakes in a copy of the oracle must be caught by the pins
# --------------------------------------------------------------------------------------------

MUTATIONS = {
    "dropped_scale": ("double s = J->scale * dot;", "double s = dot;"),
    "interleaved_kv_heads": ("const int kvh = h / G;", "const int kvh = h % J->Hkv;"),
    "window_off_by_one": ("p - j >= J->window", "p - j > J->window"),
    "no_softcap": ("if (J->softcap > 0.0) s =", "if (J->softcap < 0.0) s ="),
    "v_is_k": ("const double *vrow = J->v + (((long)b", "const double *vrow = J->k + (((long)b"),
    "causal_strict": ("if (J->causal && j > p)", "if (J->causal && j >= p)"),
    "query_at_start": ("const long p = (long)L - J->S + i;", "const long p = i;"),
    "no_normalise": ("for (int d = 0; d < J->D; ++d) orow[d] /= l;",
                     "for (int d = 0; d < J->D; ++d) orow[d] /= 1.0;"),
}


def _pin_suite(attn):
    """A compact pin suite over an attention callable; returns the first failure or None."""
    cases = _golden_cases()
    for case in cases:
        q = np.array(case["q"], np.float64)[None]
        k = np.array(case["k"], np.float64)[None]
        v = np.array(case["v"], np.float64)[None]
        o = attn(q, k, v, causal=case["causal"], window=case["window"],
                 softcap=case["softcap"], scale=case["scale"])
        if not np.allclose(o[0], np.array(case["o"]), rtol=0, atol=1e-12):
            return case["name"]
    rng = np.random.default_rng(77)
    for causal, window, softcap in [(True, 2, 0.0), (False, 0, 0.5), (True, 0, 0.0)]:
        q = rand(rng, 1, 3, 4, 3) * 2
        k = rand(rng, 1, 5, 2, 3) * 2
        v = rand(rng, 1, 5, 2, 3)
        o = attn(q, k, v, causal=causal, window=window, softcap=softcap, scale=0.8)
        if not np.allclose(o, np.asarray(brute(q, k, v, [5], causal, window, softcap, 0.8),
                                         np.float64), rtol=0, atol=1e-12):
            return "brute(%s,%s,%s)" % (causal, window, softcap)
    return None


def test_pin_suite_passes_on_oracle():
    assert _pin_suite(oracle.attention) is None


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutations_are_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, old
    (tmp_path / "oracle").mkdir()
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "__init__.py"),
                tmp_path / "oracle" / "__init__.py")
    import importlib.util
    spec = importlib.util.spec_from_file_location("mutant_oracle_" + name,
                                                  tmp_path / "oracle" / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    assert _pin_suite(mod.attention) is not None, "mutation %s went unnoticed" % name
