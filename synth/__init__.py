"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the attention arithmetic.  It draws numbers, rounds
them to the storage dtypes, quantises KV rows to int8 (the cache format the
kernels consume) and lays them out, contiguous or paged.  Both the HIP path and
the oracle read what it produces; neither computes anything here.

Generator (counter based, so any slice can be drawn independently):
  * SplitMix64: output i of stream ``seed`` is mix64(seed + (i + 1) * 0x9E3779B97F4A7C15)
    with mix64(z) = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
    z *= 0x94D049BB133111EB; z ^= z >> 31   (Steele, Lea, Flood 2014).
  * uniform u = (x >> 11) * 2**-53 in [0, 1).
  * standard normals by Box-Muller on the pair (u_{2i}, u_{2i+1}):
    r = sqrt(-2 ln(1 - u_{2i})), n_{2i} = r cos(2 pi u_{2i+1}), n_{2i+1} = r sin(2 pi u_{2i+1}).
  * values are drawn in float64, rounded to float32, then to float16 with
    round-to-nearest-even where a tensor is stored in f16.
  * stream seed = seed_c * 256 + tensor_id, with tensor ids Q=1, K=2, V=3,
    kv lengths=4, page permutation=5, alternative permutation=6, hot-tier K=7, hot-tier V=8,
    positional projection=9.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

TID_Q, TID_K, TID_V, TID_KVLEN, TID_PERM, TID_PERM_ALT = 1, 2, 3, 4, 5, 6
TID_HOT_K, TID_HOT_V = 7, 8
PAGE = 16


def stream_seed(seed_c: int, tensor_id: int) -> int:
    return (int(seed_c) * 256 + int(tensor_id)) & 0xFFFFFFFFFFFFFFFF


def splitmix64(seed: int, start: int, n: int) -> np.ndarray:
    """Outputs start .. start+n-1 of the SplitMix64 stream `seed` (uint64)."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed) + idx * GAMMA
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    return (splitmix64(seed, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


_HERE = os.path.dirname(os.path.abspath(__file__))
_CLIB = os.path.join(_HERE, "libsynth.so")
_clib = None


def build(force: bool = True) -> str:
    """Compile synth.c (the threaded generator loop) with gcc into libsynth.so."""
    if force or not os.path.exists(_CLIB):
        tmp = _CLIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp,
                               os.path.join(_HERE, "synth.c"), "-lm", "-lpthread"])
        os.replace(tmp, _CLIB)
    return _CLIB


def _c():
    global _clib
    if _clib is None:
        if not os.path.exists(_CLIB):
            build(force=True)
        L = ctypes.CDLL(_CLIB)
        L.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_int]
        L.synth_normal_f32.restype = None
        L.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_void_p]
        L.synth_uniform.restype = None
        _clib = L
    return _clib


def _threads() -> int:
    return max(1, min(32, len(os.sched_getaffinity(0))))


def normal_f32_stream(seed: int, start: int, n: int) -> np.ndarray:
    """Normals with stream indices start .. start+n-1, rounded to float32 (C loop)."""
    out = np.empty(int(n), dtype=np.float32)
    if n:
        _c().synth_normal_f32(int(seed) & 0xFFFFFFFFFFFFFFFF, int(start), int(n),
                              out.ctypes.data, _threads())
    return out


def normal_numpy(seed: int, n: int) -> np.ndarray:
    """The same normals in float64, evaluated with numpy (a cross-check of the C loop)."""
    out = np.empty(n, dtype=np.float64)
    npair = (n + 1) // 2
    for p0 in range(0, npair, _CHUNK):
        p1 = min(npair, p0 + _CHUNK)
        u = uniform(seed, 2 * (p1 - p0), start=2 * p0)
        r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
        th = (2.0 * math.pi) * u[1::2]
        pair = np.empty(2 * (p1 - p0), dtype=np.float64)
        pair[0::2] = r * np.cos(th)
        pair[1::2] = r * np.sin(th)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = pair[: hi - lo]
    return out


def normal_f32(seed: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return normal_f32_stream(seed, 0, n).reshape(shape)


def normal_f16(seed: int, shape) -> np.ndarray:
    return normal_f32(seed, shape).astype(np.float16)


def quantize_i8(x: np.ndarray):
    """Symmetric int8 with one float32 scale per row of the last axis.

    scale = max|x| / 127 (float32), q = clamp(rint(x / scale), -127, 127) with
    round-half-even; an all-zero row gets scale 1.  -128 is never produced
    (it is reserved for poison).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale = np.where(amax > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(x / scale[..., None]).astype(np.float32)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, scale


def fisher_yates(seed: int, n: int) -> np.ndarray:
    """Permutation of range(n): for i = n-1 .. 1, swap a[i] with a[floor(u * (i + 1))]."""
    a = np.arange(n, dtype=np.int64)
    if n < 2:
        return a
    u = uniform(seed, n - 1)
    js = np.minimum((u * np.arange(n, 1, -1, dtype=np.float64)).astype(np.int64),
                    np.arange(n - 1, 0, -1, dtype=np.int64))
    for step, i in enumerate(range(n - 1, 0, -1)):
        j = int(js[step])
        a[i], a[j] = a[j], a[i]
    return a


# --------------------------------------------------------------------------------------------
# Paged int8 cache
# --------------------------------------------------------------------------------------------

def ragged_normal_f32(seed: int, kv_lens, hkv: int, d: int):
    """Per-sequence [L_b, hkv, d] float32 normals, drawn as one row-major ragged stream."""
    out, start = [], 0
    for L in kv_lens:
        n = int(L) * hkv * d
        out.append(normal_f32_stream(seed, start, n).reshape(int(L), hkv, d))
        start += n
    return out


def build_pages(k_q, k_s, v_q, v_s, seed_perm: int, n_poison: int = 64, max_pages=None):
    """Scatter per-sequence int8 rows into 16-token pages placed by a seeded permutation.

    k_q[b] : int8 [L_b, hkv, d]; k_s[b] : float32 [L_b, hkv]  (same for v).
    Returns (k_pages, v_pages, k_scales, v_scales, page_table):
      pages  int8    [n_pages, hkv, 16, d]  (head-major within a page)
      scales float32 [n_pages, hkv, 16]
      page_table int32 [B, max_pages]; entries past a sequence's last page are -1.
    Unreferenced pages and slots past kv_len in a last partial page hold int8 -128
    with scale NaN (poison), so a stray read turns an output row to NaN.
    """
    B = len(k_q)
    hkv, d = k_q[0].shape[1], k_q[0].shape[2]
    n_live = [(q.shape[0] + PAGE - 1) // PAGE for q in k_q]
    P = sum(n_live)
    n_pages = P + n_poison
    if max_pages is None:
        max_pages = max(n_live)
    perm = fisher_yates(seed_perm, n_pages)
    k_pages = np.full((n_pages, hkv, PAGE, d), -128, dtype=np.int8)
    v_pages = np.full((n_pages, hkv, PAGE, d), -128, dtype=np.int8)
    k_scales = np.full((n_pages, hkv, PAGE), np.nan, dtype=np.float32)
    v_scales = np.full((n_pages, hkv, PAGE), np.nan, dtype=np.float32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    g = 0
    for b in range(B):
        L = k_q[b].shape[0]
        phys = perm[g: g + n_live[b]]
        table[b, : n_live[b]] = phys
        full = L // PAGE
        if full:
            pf = phys[:full]
            k_pages[pf] = k_q[b][: full * PAGE].reshape(full, PAGE, hkv, d).transpose(0, 2, 1, 3)
            v_pages[pf] = v_q[b][: full * PAGE].reshape(full, PAGE, hkv, d).transpose(0, 2, 1, 3)
            k_scales[pf] = k_s[b][: full * PAGE].reshape(full, PAGE, hkv).transpose(0, 2, 1)
            v_scales[pf] = v_s[b][: full * PAGE].reshape(full, PAGE, hkv).transpose(0, 2, 1)
        rem = L - full * PAGE
        if rem:
            pl = phys[full]
            k_pages[pl, :, :rem] = k_q[b][full * PAGE:].transpose(1, 0, 2)
            v_pages[pl, :, :rem] = v_q[b][full * PAGE:].transpose(1, 0, 2)
            k_scales[pl, :, :rem] = k_s[b][full * PAGE:].T
            v_scales[pl, :, :rem] = v_s[b][full * PAGE:].T
        g += n_live[b]
    return k_pages, v_pages, k_scales, v_scales, table


# --------------------------------------------------------------------------------------------
# The five workloads (shapes and value recipes)
# --------------------------------------------------------------------------------------------

def seed_of(cfg: int) -> int:
    return 20261200 + int(cfg)


def prefill_inputs(seed_c, seq_len, kv_len, h, hkv, d, dtype):
    """Token-major Q [seq_len, h, d], K/V [kv_len, hkv, d], N(0,1) in `dtype`."""
    mk = normal_f16 if dtype == "f16" else normal_f32
    q = mk(stream_seed(seed_c, TID_Q), (seq_len, h, d))
    k = mk(stream_seed(seed_c, TID_K), (kv_len, hkv, d))
    v = mk(stream_seed(seed_c, TID_V), (kv_len, hkv, d))
    return q, k, v


def vision_inputs(seed_c, n_patches, h, d):
    """Head-major Q/K/V [h, n_patches, d] in f16."""
    q = normal_f16(stream_seed(seed_c, TID_Q), (h, n_patches, d))
    k = normal_f16(stream_seed(seed_c, TID_K), (h, n_patches, d))
    v = normal_f16(stream_seed(seed_c, TID_V), (h, n_patches, d))
    return q, k, v


def decode_inputs(seed_c, h, hkv, d, kv_len):
    """q f32 [h, d]; K/V f16 head-major [hkv, kv_len, d]."""
    q = normal_f32(stream_seed(seed_c, TID_Q), (h, d))
    k = normal_f16(stream_seed(seed_c, TID_K), (hkv, kv_len, d))
    v = normal_f16(stream_seed(seed_c, TID_V), (hkv, kv_len, d))
    return q, k, v


def paged_kv_lens(seed_c, batch, lo, hi):
    """kv_len_b = lo + floor(u * (hi - lo + 1)), uniform integers over [lo, hi]."""
    u = uniform(stream_seed(seed_c, TID_KVLEN), batch)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64).clip(lo, hi).astype(np.int32)


def paged_inputs(seed_c, batch, h, hkv, d, kv_lens, n_poison=64, alt_perm=False,
                 max_pages=None):
    """Batched paged int8 decode inputs.

    Returns a dict with q f32 [B, h, d], the logical int8 rows and scales per
    sequence (before paging), the pages, scales, page table and kv_lens.
    """
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    q = normal_f32(stream_seed(seed_c, TID_Q), (batch, h, d))
    kf = ragged_normal_f32(stream_seed(seed_c, TID_K), kv_lens, hkv, d)
    vf = ragged_normal_f32(stream_seed(seed_c, TID_V), kv_lens, hkv, d)
    kq, ks, vq, vs = [], [], [], []
    for b in range(batch):
        a, s = quantize_i8(kf[b]); kq.append(a); ks.append(s)
        a, s = quantize_i8(vf[b]); vq.append(a); vs.append(s)
    del kf, vf
    tid = TID_PERM_ALT if alt_perm else TID_PERM
    kp, vp, ksp, vsp, table = build_pages(kq, ks, vq, vs, stream_seed(seed_c, tid),
                                          n_poison=n_poison, max_pages=max_pages)
    return dict(q=q, k_q=kq, k_s=ks, v_q=vq, v_s=vs, k_pages=kp, v_pages=vp,
                k_scales=ksp, v_scales=vsp, page_table=table, kv_lens=kv_lens)


def tiered_inputs(seed_c, h, hkv, d, cold_len, hot_len, hot_window, hot_start, n_poison=16):
    """One sequence of a tiered cache.  Positions [0, cold_len) are the cold tier: drawn,
    quantised to int8 and paged exactly as paged_inputs does for a batch of one (an empty
    tier is one poison page).  Positions [cold_len, cold_len + hot_len) are the hot tier:
    f16 rows [hot_len, hkv, d] (token-major), laid into rings [hkv, hot_window, d] with
    position p at row (hot_start + p - cold_len) % hot_window; rows holding no position are
    NaN.  q is f32 [h, d]."""
    if cold_len > 0:
        cold = paged_inputs(seed_c, 1, h, hkv, d, [cold_len], n_poison=n_poison)
    else:
        cold = dict(q=normal_f32(stream_seed(seed_c, TID_Q), (1, h, d)),
                    k_q=[np.zeros((0, hkv, d), np.int8)], k_s=[np.zeros((0, hkv), np.float32)],
                    v_q=[np.zeros((0, hkv, d), np.int8)], v_s=[np.zeros((0, hkv), np.float32)],
                    k_pages=np.full((1, hkv, PAGE, d), -128, np.int8),
                    v_pages=np.full((1, hkv, PAGE, d), -128, np.int8),
                    k_scales=np.full((1, hkv, PAGE), np.nan, np.float32),
                    v_scales=np.full((1, hkv, PAGE), np.nan, np.float32),
                    page_table=np.zeros((1, 1), np.int32), kv_lens=np.zeros(1, np.int32))
    hot_k = normal_f16(stream_seed(seed_c, TID_HOT_K), (hot_len, hkv, d))
    hot_v = normal_f16(stream_seed(seed_c, TID_HOT_V), (hot_len, hkv, d))
    ring_k = np.full((hkv, hot_window, d), np.nan, np.float16)
    ring_v = np.full((hkv, hot_window, d), np.nan, np.float16)
    rows = (hot_start + np.arange(hot_len)) % hot_window
    ring_k[:, rows] = np.transpose(hot_k, (1, 0, 2))
    ring_v[:, rows] = np.transpose(hot_v, (1, 0, 2))
    return dict(q=cold["q"][0], cold=cold, hot_k=hot_k, hot_v=hot_v, ring_k=ring_k, ring_v=ring_v,
                cold_len=int(cold_len), hot_len=int(hot_len), hot_start=int(hot_start))



def build_pages_f16(rows, seed_perm: int, n_poison: int = 16, max_pages=None):
    """Scatter one sequence's f16 rows [L, hkv, d] into 16-token pages [n_pages, hkv, 16, d]
    (head-major within a page) placed by a seeded permutation; page table int32 [max_pages]
    (entries past the last page -1).  Unreferenced pages and the slots past L of a last
    partial page hold NaN."""
    L, hkv, d = rows.shape
    n_live = (L + PAGE - 1) // PAGE
    n_pages = max(1, n_live + n_poison)
    if max_pages is None:
        max_pages = max(1, n_live)
    perm = fisher_yates(seed_perm, n_pages)
    pages = np.full((n_pages, hkv, PAGE, d), np.nan, dtype=np.float16)
    table = np.full(max_pages, -1, dtype=np.int32)
    phys = perm[:n_live]
    table[:n_live] = phys
    for i, pg in enumerate(phys):
        blk = rows[i * PAGE:(i + 1) * PAGE]
        pages[pg, :, :blk.shape[0]] = np.transpose(blk, (1, 0, 2))
    return pages, table


def tiered_f16_inputs(seed_c, h, hkv, d, cold_len, hot_len, hot_window, hot_start, paged,
                      capacity=None, n_poison=16):
    """A tiered cache with an f16 cold tier.  The hot tier and q are those of tiered_inputs
    (same streams); the cold tier holds f16 rows [cold_len, hkv, d] drawn N(0, 1) from the K
    and V streams, either paged (build_pages_f16, seeded permutation) or contiguous
    [hkv, capacity, d] with NaN in the rows past cold_len (capacity defaults to cold_len + 16)."""
    t = tiered_inputs(seed_c, h, hkv, d, 0, hot_len, hot_window, hot_start, n_poison=1)
    ck = normal_f16(stream_seed(seed_c, TID_K), (cold_len, hkv, d))
    cv = normal_f16(stream_seed(seed_c, TID_V), (cold_len, hkv, d))
    t["cold_k"], t["cold_v"] = ck, cv
    t["cold_len"] = int(cold_len)
    if paged:
        t["cold_k_pages"], t["cold_page_table"] = build_pages_f16(ck, stream_seed(seed_c, TID_PERM), n_poison)
        t["cold_v_pages"], _ = build_pages_f16(cv, stream_seed(seed_c, TID_PERM), n_poison)
    else:
        cap = cold_len + 16 if capacity is None else capacity
        kk = np.full((hkv, cap, d), np.nan, np.float16)
        vv = np.full((hkv, cap, d), np.nan, np.float16)
        kk[:, :cold_len] = np.transpose(ck, (1, 0, 2))
        vv[:, :cold_len] = np.transpose(cv, (1, 0, 2))
        t["cold_k_contig"], t["cold_v_contig"] = kk, vv
    return t


def tiered_packed_inputs(seed_c, h, hkv, d, cold_len, hot_len, hot_window, hot_start,
                         capacity=None):
    """tiered_inputs with the int8 cold tier laid out contiguously instead of in pages:
    cold K/V int8 [hkv, capacity, d] and scales float32 [hkv, capacity]; rows past cold_len
    hold int8 -128 with scale NaN (capacity defaults to cold_len + 16)."""
    t = tiered_inputs(seed_c, h, hkv, d, cold_len, hot_len, hot_window, hot_start, n_poison=1)
    c = t["cold"]
    cap = cold_len + 16 if capacity is None else capacity
    out = {}
    for name, qq, ss in (("k", c["k_q"][0], c["k_s"][0]), ("v", c["v_q"][0], c["v_s"][0])):
        a = np.full((hkv, cap, d), -128, np.int8)
        sc = np.full((hkv, cap), np.nan, np.float32)
        a[:, :cold_len] = np.transpose(qq, (1, 0, 2))
        sc[:, :cold_len] = ss.T
        out[name], out[name + "_s"] = a, sc
    t["packed_k"], t["packed_v"] = out["k"], out["v"]
    t["packed_k_scales"], t["packed_v_scales"] = out["k_s"], out["v_s"]
    return t


TID_POS = 9


def block_local_inputs(seed_c, seq, chunk_size, max_past, max_future, h, d=128,
                       q_scale=None):
    """Conformer block-local inputs, float32.

    q_pad [padded_len, h, d] with padded_len = seq rounded up to a multiple of chunk_size;
    k_padded, v_padded [max_past + padded_len + max_future, h, d] (row r is position
    r - max_past; the rows of positions outside [0, seq) are zeros, as in the pages'
    zero-padded buffers); pos_proj [max_past + max_future + 1, h, d].  Values N(0, 1),
    except q, drawn N(0, 1) and multiplied by q_scale (default 1/sqrt(d): the pages' q_pad
    arrives already scaled per dimension), so that the scores have unit order.  Stream ids:
    Q 1, K 2, V 3, pos 9.
    """
    P = -(-seq // chunk_size) * chunk_size
    R = max_past + P + max_future
    span = max_past + max_future + 1
    qs = np.float32(1.0 / math.sqrt(d) if q_scale is None else q_scale)
    q = normal_f32(stream_seed(seed_c, TID_Q), (P, h, d)) * qs
    k = np.zeros((R, h, d), dtype=np.float32)
    v = np.zeros((R, h, d), dtype=np.float32)
    k[max_past:max_past + seq] = normal_f32(stream_seed(seed_c, TID_K), (seq, h, d))
    v[max_past:max_past + seq] = normal_f32(stream_seed(seed_c, TID_V), (seq, h, d))
    pos = normal_f32(stream_seed(seed_c, TID_POS), (span, h, d))
    return {"q": q, "k": k, "v": v, "pos": pos, "padded_len": P, "kv_rows": R}
