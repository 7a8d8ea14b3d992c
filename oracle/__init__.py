"""CPU oracle for softmax attention, in float64.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product library.  It
shares no code with the HIP path; the two meet only in the seeded input
generator, which holds none of the attention arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, double, two passes over a fully
materialised score row).  This module only marshals numpy arrays into the
canonical layouts that file documents and calls it.

Every function here has pins in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_block_local_pins.py``.  One part of ``block_local`` is a reading with no
anchor on the pages: which row of the positional projection belongs to which key (the pages
name the projection, not its indexing); the pins fix the oracle to that stated reading, not
to the pages, so that term is "parity unpinned" against the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC,
             "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.oracle_attention_f64.argtypes = [
            dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ip, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            ctypes.c_double, ctypes.c_int]
        lib.oracle_attention_f64.restype = ctypes.c_int
        lib.oracle_dequant_i8.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_int, dp]
        lib.oracle_dequant_i8.restype = None
        lib.oracle_block_local_f64.argtypes = [
            dp, dp, dp, dp, dp] + [ctypes.c_int] * 11 + [ctypes.c_double, ctypes.c_int]
        lib.oracle_block_local_f64.restype = ctypes.c_int
        lib.oracle_threads_used.argtypes = []
        lib.oracle_threads_used.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def attention(q, k, v, *, kv_len=None, causal=False, window=0, softcap=0.0, scale=None,
              threads=None):
    """Softmax attention in float64.

    q : [B, S, H, D];  k, v : [B, Lmax, Hkv, D]   (any real dtype; read as float64)
    kv_len : per-batch key count (default Lmax for every batch entry).
    Query row i of batch b sits at position kv_len[b] - S + i.
    Returns o : [B, S, H, D] float64.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,S,H,D] and k, v [B,L,Hkv,D]")
    B, S, H, D = q.shape
    Bk, L, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("batch / head_dim mismatch")
    if kv_len is None:
        kv_len = np.full(B, L, dtype=np.int32)
    kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros((B, S, H, D), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_attention_f64(
        q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp), o.ctypes.data_as(dp),
        B, S, L, kv_len.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), H, Hkv, D,
        1 if causal else 0, int(window), float(softcap), float(scale),
        int(threads if threads else default_threads()))
    if rc != 0:
        raise ValueError("oracle_attention_f64 rejected its arguments")
    return o


def block_local(q, k, v, pos, *, seq, chunk_size, max_past, max_future, logit_cap=0.0,
                context_size=None, max_span=None, pad_left=None, threads=None):
    """Conformer block-local attention with a relative-position term, in float64.

    q : [padded_len, H, D]; k, v : [kv_rows, H, D] with row r holding position r - pad_left;
    pos : [max_span, H, D], row j the relative offset j - max_past.  context_size, max_span
    and pad_left default to the consistent geometry (chunk + past + future, past + future +
    1, past); other values are passed through so that the oracle's checks see them.
    Returns o : [padded_len, H, D] float64 (rows past seq included).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.float64)
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or pos.ndim != 3:
        raise ValueError("q [P,H,D], k/v [R,H,D], pos [span,H,D]")
    P, H, D = q.shape
    R = k.shape[0]
    if k.shape[1:] != (H, D) or pos.shape[1:] != (H, D):
        raise ValueError("head / head_dim mismatch")
    if context_size is None:
        context_size = chunk_size + max_past + max_future
    if max_span is None:
        max_span = max_past + max_future + 1
    if pad_left is None:
        pad_left = max_past
    if pos.shape[0] != max_span:
        raise ValueError("pos must have max_span rows")
    o = np.zeros((P, H, D), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_block_local_f64(
        q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp), pos.ctypes.data_as(dp),
        o.ctypes.data_as(dp), int(seq), P, R, H, D, int(chunk_size), int(context_size),
        int(max_span), int(max_past), int(max_future), int(pad_left), float(logit_cap),
        int(threads if threads else default_threads()))
    if rc != 0:
        raise ValueError("oracle_block_local_f64 rejected its arguments")
    return o


def threads_used() -> int:
    """Threads that computed at least one row in the last attention() call."""
    return int(_load().oracle_threads_used())


def dequant_i8(q8, scales):
    """x = q8 * scale with one scale per row of the last axis; float64 result."""
    q8 = np.ascontiguousarray(q8, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    D = q8.shape[-1]
    rows = q8.size // D
    if scales.size != rows:
        raise ValueError("one scale per row of the last axis")
    out = np.empty(q8.shape, dtype=np.float64)
    _load().oracle_dequant_i8(q8.ctypes.data, scales.ctypes.data, rows, D,
                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out
