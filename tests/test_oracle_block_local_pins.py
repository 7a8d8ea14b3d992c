"""Pins of the block-local (Conformer) oracle to facts that do not come from the oracle.

The pages give the call of block_local_attention_chained (rullama 0.5.0,
src/backend/dispatch/attention.rs) and no numbers.  The pins: hand-derived cases
(tests/golden/block_local.json), a deliberately different brute force (extended
precision, full score and additive -inf mask matrices over every row of k_padded, the
position term gathered through an explicit offset matrix), the reduction to the core
attention oracle when the position term is zero, invariants of the definition, and
planted slips in a copy of the oracle that these pins must catch.

What stays "parity unpinned" against the pages is the reading itself of how pos_proj
enters the score (row j of pos_proj is the key offset j - max_past, added as q.pos to
q.k): the pages name the projection but not its indexing.  The pins hold the oracle to
that stated reading.
"""
import importlib.util
import json
import math
import os
import shutil

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    return json.load(open(os.path.join(HERE, "golden", "block_local.json")))["cases"]


def brute(q, k, v, pos, seq, max_past, max_future, pad_left, cap):
    """Matrix form over all kv rows, np.longdouble.  For every head: content scores
    Q K^T over every row r of k_padded (position r - pad_left), a position term built by
    gathering q.pos[offset + max_past] through the offset matrix (r - pad_left) - i, an
    additive mask of 0 / -inf, row max subtraction, exp, normalisation."""
    q, k, v, pos = (np.asarray(x, np.longdouble) for x in (q, k, v, pos))
    P, H, D = q.shape
    R = k.shape[0]
    out = np.zeros((P, H, D), np.longdouble)
    offs = (np.arange(R)[None, :] - pad_left) - np.arange(P)[:, None]          # [P, R]
    keypos = np.arange(R)[None, :] - pad_left + np.zeros((P, 1), int)
    vis = (offs >= -max_past) & (offs <= max_future) & (keypos >= 0) & (keypos < seq)
    for h in range(H):
        content = q[:, h, :] @ k[:, h, :].T                                     # [P, R]
        qp = q[:, h, :] @ pos[:, h, :].T                                        # [P, span]
        idx = np.clip(offs + max_past, 0, pos.shape[0] - 1)
        position = np.take_along_axis(qp, idx, axis=1)
        s = content + position
        if cap > 0:
            s = cap * np.tanh(s / cap)
        mask = np.where(vis, np.longdouble(0), np.longdouble(-np.inf))
        s = s + mask
        for i in range(P):
            if not vis[i].any():
                continue
            row = s[i] - s[i][vis[i]].max()
            w = np.exp(row)
            out[i, h] = (w[:, None] * v[:, h, :]).sum(0) / w.sum()
    return out


def run(fn, c):
    return fn(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), np.array(c["pos"]),
              seq=c["seq"], chunk_size=c["chunk_size"], max_past=c["max_past"],
              max_future=c["max_future"], logit_cap=c["logit_cap"],
              context_size=c["context_size"], max_span=c["max_span"], pad_left=c["pad_left"])


@pytest.mark.parametrize("case", golden(), ids=lambda c: c["name"])
def test_golden_hand_derived(case):
    o = run(oracle.block_local, case)
    assert np.allclose(o, np.array(case["o"]), rtol=0, atol=case["tol"])


def rand_case(rng, seq, chunk, past, future, H=2, D=5, scale=1.0):
    P = -(-seq // chunk) * chunk
    R = past + P + future
    q = rng.standard_normal((P, H, D)) * scale
    k = rng.standard_normal((R, H, D)) * scale
    v = rng.standard_normal((R, H, D))
    pos = rng.standard_normal((past + future + 1, H, D)) * scale
    # padding rows of k and v hold zeros, as the pages' buffers do
    k[:past] = 0
    v[:past] = 0
    k[past + seq:] = 0
    v[past + seq:] = 0
    return q, k, v, pos, P


@pytest.mark.parametrize("seq,chunk,past,future,cap", [
    (1, 1, 0, 0, 0.0), (5, 2, 1, 0, 0.0), (7, 3, 2, 1, 0.0), (9, 4, 3, 2, 1.5),
    (12, 12, 12, 0, 50.0), (13, 12, 12, 0, 0.0), (6, 2, 0, 3, 0.7), (4, 8, 5, 5, 0.0),
])
def test_brute_force(seq, chunk, past, future, cap):
    rng = np.random.default_rng(seq * 131 + chunk * 17 + past * 5 + future)
    q, k, v, pos, P = rand_case(rng, seq, chunk, past, future, scale=1.3)
    got = oracle.block_local(q, k, v, pos, seq=seq, chunk_size=chunk, max_past=past,
                             max_future=future, logit_cap=cap)
    want = np.asarray(brute(q, k, v, pos, seq, past, future, past, cap), np.float64)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_zero_position_term_reduces_to_core_attention():
    """pos_proj = 0, no cap: query i is plain (bidirectional, unscaled) attention over the
    key slice [max(0, i - max_past), min(seq - 1, i + max_future)], which the core oracle
    (pinned on its own) computes."""
    rng = np.random.default_rng(5)
    seq, chunk, past, future = 11, 4, 3, 2
    q, k, v, pos, P = rand_case(rng, seq, chunk, past, future)
    pos[:] = 0
    got = oracle.block_local(q, k, v, pos, seq=seq, chunk_size=chunk, max_past=past,
                             max_future=future)
    for i in range(seq):
        lo, hi = max(0, i - past), min(seq - 1, i + future)
        ks, vs = k[past + lo:past + hi + 1], v[past + lo:past + hi + 1]
        want = oracle.attention(q[None, i:i + 1], ks[None], vs[None], causal=False, scale=1.0)[0, 0]
        assert np.allclose(got[i], want, rtol=0, atol=1e-13), i


def test_constant_position_rows_change_nothing_without_cap():
    """Every pos_proj row equal to u adds q.u to every score of a row: the softmax does
    not move."""
    rng = np.random.default_rng(6)
    q, k, v, pos, P = rand_case(rng, 10, 5, 2, 2)
    base = oracle.block_local(q, k, v, np.zeros_like(pos), seq=10, chunk_size=5, max_past=2,
                              max_future=2)
    pos[:] = rng.standard_normal(pos.shape[1:])[None]
    got = oracle.block_local(q, k, v, pos, seq=10, chunk_size=5, max_past=2, max_future=2)
    assert np.allclose(got, base, rtol=0, atol=1e-13)


def test_position_term_alone_gives_softmax_of_q_dot_pos():
    """K = 0 and one-hot V: output row i is the weight row, softmax over the visible
    offsets of q_i . pos[offset + max_past] -- checked on a row whose window is whole."""
    rng = np.random.default_rng(7)
    seq, past, future, D = 8, 2, 1, 16
    P = seq
    q = rng.standard_normal((P, 1, D))
    k = np.zeros((past + P + future, 1, D))
    v = np.zeros_like(k)
    for t in range(seq):
        v[past + t, 0, t] = 1.0
    pos = rng.standard_normal((past + future + 1, 1, D))
    got = oracle.block_local(q, k, v, pos, seq=seq, chunk_size=1, max_past=past, max_future=future)
    i = 4
    s = np.array([q[i, 0] @ pos[j, 0] for j in range(past + future + 1)])
    w = np.exp(s - s.max())
    w /= w.sum()
    want = np.zeros(D)
    want[i - past:i + future + 1] = w
    assert np.allclose(got[i, 0], want, rtol=0, atol=1e-14)


def test_uniform_v_and_empty_padding_rows():
    """Uniform V rows give that row wherever a key is visible; a padding query whose window
    holds no key of [0, seq) is written as zeros."""
    rng = np.random.default_rng(8)
    seq, chunk, past = 1, 8, 2
    q, k, v, pos, P = rand_case(rng, seq, chunk, past, 0)
    u = rng.standard_normal(5)
    v[past:past + seq] = u
    got = oracle.block_local(q, k, v, pos, seq=seq, chunk_size=chunk, max_past=past,
                             max_future=0, logit_cap=3.0)
    for i in range(P):
        if i - past <= seq - 1:
            assert np.allclose(got[i], u, rtol=0, atol=1e-14), i
        else:
            assert np.all(got[i] == 0), i


def test_chunk_size_does_not_change_the_result():
    """With the consistent geometry the chunking only decides which rows a kernel stages."""
    rng = np.random.default_rng(9)
    seq, past, future = 20, 3, 2
    q, k, v, pos, P = rand_case(rng, seq, 1, past, future)
    ref = oracle.block_local(q, k, v, pos, seq=seq, chunk_size=1, max_past=past,
                             max_future=future, logit_cap=4.0)
    for chunk in (2, 4, 5, 10, 20):
        got = oracle.block_local(q, k, v, pos, seq=seq, chunk_size=chunk, max_past=past,
                                 max_future=future, logit_cap=4.0)
        assert np.array_equal(got, ref), chunk


@pytest.mark.parametrize("bad", [
    dict(context_size=5), dict(max_span=2), dict(pad_left=0), dict(chunk_size=3),
])
def test_rejects_inconsistent_geometry(bad):
    rng = np.random.default_rng(10)
    q, k, v, pos, P = rand_case(rng, 8, 4, 1, 1)
    kw = dict(seq=8, chunk_size=4, max_past=1, max_future=1)
    kw.update(bad)
    if "max_span" in bad:
        pos = pos[:bad["max_span"]]
    with pytest.raises(ValueError):
        oracle.block_local(q, k, v, pos, **kw)


# --------------------------------------------------------------------------------------------
# Planted slips in a copy of the oracle must be caught
# --------------------------------------------------------------------------------------------

MUTATIONS = {
    "pos_reversed": ("const double *prow = J->pos + ((long)j * H + h) * D;",
                     "const double *prow = J->pos + ((long)(span - 1 - j) * H + h) * D;"),
    "no_position_term": ("double s = content + position;", "double s = content;"),
    "no_logit_cap": ("if (J->cap > 0.0) s = J->cap * tanh(s / J->cap);",
                     "if (J->cap < 0.0) s = J->cap * tanh(s / J->cap);"),
    "padding_keys_visible": ("if (t < 0 || t >= J->seq) { score[j] = NAN; continue; }",
                             "if (t < 0) { score[j] = NAN; continue; }"),
    "left_padding_visible": ("if (t < 0 || t >= J->seq) { score[j] = NAN; continue; }",
                             "if (t < -J->pad_left || t >= J->seq) { score[j] = NAN; continue; }"),
    "pad_left_ignored": ("const double *krow = J->k + ((t + J->pad_left) * H + h) * D;",
                         "const double *krow = J->k + ((t) * H + h) * D;"),
    "v_is_k": ("const double *vrow = J->v + ((t + J->pad_left) * H + h) * D;",
               "const double *vrow = J->k + ((t + J->pad_left) * H + h) * D;"),
    "first_head_only": ("const double *krow = J->k + ((t + J->pad_left) * H + h) * D;",
                        "const double *krow = J->k + ((t + J->pad_left) * H + 0) * D;"),
}


def _pin_suite(fn):
    for c in golden():
        if not np.allclose(run(fn, c), np.array(c["o"]), rtol=0, atol=c["tol"]):
            return c["name"]
    rng = np.random.default_rng(99)
    for seq, chunk, past, future, cap in [(7, 3, 2, 1, 0.0), (9, 4, 3, 2, 1.5)]:
        q, k, v, pos, P = rand_case(rng, seq, chunk, past, future, scale=1.3)
        # non-zero padding rows make a stray read visible
        k[:past] += 0.5
        v[:past] += 0.5
        got = fn(q, k, v, pos, seq=seq, chunk_size=chunk, max_past=past, max_future=future,
                 logit_cap=cap)
        want = np.asarray(brute(q, k, v, pos, seq, past, future, past, cap), np.float64)
        if not np.allclose(got, want, rtol=0, atol=1e-12):
            return "brute(%d,%d,%d,%d)" % (seq, chunk, past, future)
    return None


def test_pin_suite_passes_on_oracle():
    assert _pin_suite(oracle.block_local) is None


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
    spec = importlib.util.spec_from_file_location("mutant_bl_oracle_" + name,
                                                  tmp_path / "oracle" / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    assert _pin_suite(mod.block_local) is not None, "mutation %s went unnoticed" % name
