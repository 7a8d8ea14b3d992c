"""Softmax attention with online softmax for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libattn.so``: each function has the name of the C
entry point it calls (``include/attn.h``) and only marshals arguments (shapes,
device pointers, the current HIP stream).  Every step of the computation runs
in the library's HIP kernels; there is no fallback of any kind, and a missing
library is an error.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "AttnError", "lib", "attn_prefill", "attn_prefill_device_kv_len", "attn_vision", "attn_decode",
    "attn_decode_noalloc", "attn_decode_ring", "attn_decode_paged_q8", "attn_decode_tiered_q8",
    "attn_block_local", "attn_decode_tiered_q8_packed", "attn_decode_tiered_f16",
    "ATTN_COLD_CONTIGUOUS", "ATTN_COLD_PAGED",
    "attn_decode_workspace_bytes", "attn_set_decode_split", "attn_last_error", "decode_workspace",
    "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_WORKSPACE",
    "ATTN_ERR_LAUNCH", "ATTN_F32", "ATTN_F16", "LIB_PATH",
]

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_LAUNCH = 0, -1, -2, -3, -4
ATTN_F32, ATTN_F16 = 0, 1
ATTN_COLD_CONTIGUOUS, ATTN_COLD_PAGED = 0, 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
_lib = None


class AttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("attn error %d: %s" % (code, message))
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libattn.so is not built (%s); run `python -m "
                               "transformer_attention_03_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.attn_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, f, vp]
        L.attn_prefill_device_kv_len.argtypes = [vp, vp, vp, vp, i, i, i, vp, i, i, i, i, i, f, f, vp]
        L.attn_vision.argtypes = [vp, vp, vp, vp, i, i, i, f, vp]
        L.attn_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, f, vp, sz, vp]
        L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, f, vp]
        L.attn_decode_ring.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, f, vp, sz, vp]
        L.attn_decode_paged_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                           f, f, vp, sz, vp]
        L.attn_decode_tiered_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                            i, i, i, f, f, vp, sz, vp]
        L.attn_decode_tiered_q8_packed.argtypes = [vp] * 8 + [i] * 9 + [f, f, vp, sz, vp]
        L.attn_decode_tiered_f16.argtypes = [vp] * 7 + [i] * 12 + [f, f, vp, sz, vp]
        L.attn_block_local.argtypes = [vp, vp, vp, vp, vp] + [i] * 11 + [f, vp]
        L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
        L.attn_decode_workspace_bytes.restype = sz
        L.attn_set_decode_split.argtypes = [i]
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        for name in ("attn_prefill", "attn_prefill_device_kv_len", "attn_vision", "attn_decode",
                     "attn_decode_noalloc", "attn_decode_ring", "attn_block_local",
                     "attn_decode_tiered_q8_packed", "attn_decode_tiered_f16", "attn_decode_paged_q8", "attn_decode_tiered_q8",
                     "attn_set_decode_split"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def attn_last_error() -> str:
    return lib().attn_last_error().decode()


def _check(rc: int):
    if rc != ATTN_OK:
        raise AttnError(rc, attn_last_error())


def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dname(t):
    """The dtype name of a tensor ("float32", "float16", ...), for _need."""
    return str(getattr(t, "dtype", "?")).replace("torch.", "")


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.float16:
        return ATTN_F16
    raise TypeError("q/k/v/o must be float32 or float16, got %s" % t.dtype)


def _need_contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _need(what, **named):
    """Dtype and device checks before anything reaches the library: every tensor named
    here must have the dtype given with it and live on the same GPU as the first one.
    named: name -> (tensor, dtype name or tuple of dtype names).  A tensor of the wrong
    dtype would be read with the wrong element size, and a host tensor would hand the
    kernels a host pointer, so both are refused."""
    import torch
    dev = None
    for name, (t, want) in named.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: %s must be a torch.Tensor" % (what, name))
        wants = want if isinstance(want, tuple) else (want,)
        if not any(t.dtype == getattr(torch, w) for w in wants):
            raise ValueError("%s: %s must be %s, got %s" % (what, name, " or ".join(wants),
                                                            str(t.dtype).replace("torch.", "")))
    for name, (t, _) in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s: %s must be on a GPU, got %s" % (what, name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s: %s is on %s, the other tensors on %s" % (what, name, t.device, dev))


def attn_prefill(q, k, v, o, *, causal: bool, scale: float, sliding_window: int = 0,
                 attn_softcap: float = 0.0, stream=None):
    """q, o: [seq_len, num_heads, head_dim]; k, v: [kv_len, num_kv_heads, head_dim]."""
    _need("attn_prefill", q=(q, ("float32", "float16")), k=(k, _dname(q)), v=(v, _dname(q)),
          o=(o, _dname(q)))
    _need_contig(q, k, v, o)
    S, H, D = q.shape
    L, Hkv, Dk = k.shape
    if Dk != D or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    _check(lib().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(q), S, L, H, Hkv,
                              D, 1 if causal else 0, int(sliding_window), float(attn_softcap),
                              float(scale), _stream(q, stream)))


def attn_prefill_device_kv_len(q, k, v, o, kv_len, *, causal: bool, scale: float,
                               sliding_window: int = 0, attn_softcap: float = 0.0, stream=None):
    """q, o: [seq_len, num_heads, head_dim]; k, v: [max_kv_len, num_kv_heads, head_dim];
    kv_len: int32 device tensor of one element, read when the kernel runs."""
    _need("attn_prefill_device_kv_len", q=(q, ("float32", "float16")), k=(k, _dname(q)),
          v=(v, _dname(q)), o=(o, _dname(q)), kv_len=(kv_len, "int32"))
    _need_contig(q, k, v, o)
    S, H, D = q.shape
    Lmax, Hkv, Dk = k.shape
    if Dk != D or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if kv_len.numel() != 1:
        raise ValueError("kv_len must be one int32 element on the device of q")
    _check(lib().attn_prefill_device_kv_len(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(q), S,
                                            Lmax, _ptr(kv_len), H, Hkv, D, 1 if causal else 0,
                                            int(sliding_window), float(attn_softcap), float(scale),
                                            _stream(q, stream)))


def attn_vision(q, k, v, o, *, scale: float, stream=None):
    """q, k, v, o: float16 [num_heads, num_patches, head_dim]."""
    _need("attn_vision", q=(q, "float16"), k=(k, "float16"), v=(v, "float16"), o=(o, "float16"))
    _need_contig(q, k, v, o)
    H, P, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    _check(lib().attn_vision(_ptr(q), _ptr(k), _ptr(v), _ptr(o), P, H, D, float(scale),
                             _stream(q, stream)))


def attn_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_kv_len) -> int:
    return int(lib().attn_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim,
                                                 max_kv_len))


def attn_set_decode_split(tokens_per_split: int):
    _check(lib().attn_set_decode_split(int(tokens_per_split)))


def decode_workspace(batch, num_heads, num_kv_heads, head_dim, max_kv_len, device):
    """A zero-filled workspace of the required size, allocated by torch."""
    import torch
    n = attn_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_kv_len)
    if n == 0:
        raise ValueError("invalid decode shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def attn_decode(q, k, v, o, workspace, *, scale: float, sliding_window: int = 0,
                attn_softcap: float = 0.0, stream=None):
    """q, o: float32 [num_heads, head_dim]; k, v: float16 [num_kv_heads, kv_len, head_dim]."""
    _need("attn_decode", q=(q, "float32"), k=(k, "float16"), v=(v, "float16"), o=(o, "float32"),
          workspace=(workspace, "uint8"))
    _need_contig(q, k, v, o)
    H, D = q.shape
    Hkv, L, Dk = k.shape
    if Dk != D or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), H, Hkv, D, L,
                             int(sliding_window), float(attn_softcap), float(scale),
                             _ptr(workspace), ws_bytes, _stream(q, stream)))


def attn_decode_noalloc(q, k, v, o, *, scale: float, sliding_window: int = 0,
                        attn_softcap: float = 0.0, stream=None):
    """attn_decode without a workspace: the library's own per-GPU scratch holds the split
    partials.  Calls that overlap on one GPU race; see include/attn.h."""
    _need("attn_decode_noalloc", q=(q, "float32"), k=(k, "float16"), v=(v, "float16"),
          o=(o, "float32"))
    _need_contig(q, k, v, o)
    H, D = q.shape
    Hkv, L, Dk = k.shape
    if Dk != D or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    _check(lib().attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), H, Hkv, D, L,
                                     int(sliding_window), float(attn_softcap), float(scale),
                                     _stream(q, stream)))


def attn_decode_ring(q, k, v, o, workspace, *, total_len: int, scale: float,
                     sliding_window: int = 0, attn_softcap: float = 0.0, stream=None):
    """q, o: float32 [num_heads, head_dim]; k, v: float16 ring [num_kv_heads, ring_len,
    head_dim] holding position t at row t % ring_len; total_len tokens seen so far."""
    _need("attn_decode_ring", q=(q, "float32"), k=(k, "float16"), v=(v, "float16"),
          o=(o, "float32"), workspace=(workspace, "uint8"))
    _need_contig(q, k, v, o)
    H, D = q.shape
    Hkv, R, Dk = k.shape
    if Dk != D or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().attn_decode_ring(_ptr(q), _ptr(k), _ptr(v), _ptr(o), H, Hkv, D, R, int(total_len),
                                  int(sliding_window), float(attn_softcap), float(scale),
                                  _ptr(workspace), ws_bytes, _stream(q, stream)))


def attn_decode_paged_q8(q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens, o,
                         workspace, *, scale: float, sliding_window: int = 0,
                         attn_softcap: float = 0.0, stream=None):
    """q, o: float32 [batch, num_heads, head_dim]; pages int8 [num_pages, num_kv_heads, 16,
    head_dim]; scales float32 [num_pages, num_kv_heads, 16]; page_table int32
    [batch, max_pages]; kv_lens int32 [batch] (device)."""
    _need("attn_decode_paged_q8", q=(q, "float32"), k_pages=(k_pages, "int8"),
          v_pages=(v_pages, "int8"), k_scales=(k_scales, "float32"), v_scales=(v_scales, "float32"),
          page_table=(page_table, "int32"), kv_lens=(kv_lens, "int32"), o=(o, "float32"),
          workspace=(workspace, "uint8"))
    _need_contig(q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens, o)
    B, H, D = q.shape
    P, Hkv, ps, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if k_scales.shape != (P, Hkv, ps) or v_scales.shape != (P, Hkv, ps):
        raise ValueError("scales must be [num_pages, num_kv_heads, page_size]")
    if page_table.shape[0] != B or kv_lens.shape != (B,):
        raise ValueError("page_table must be [batch, max_pages] and kv_lens [batch]")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().attn_decode_paged_q8(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), _ptr(page_table),
        _ptr(kv_lens), _ptr(o), B, H, Hkv, D, ps, P, page_table.shape[1], int(sliding_window),
        float(attn_softcap), float(scale), _ptr(workspace), ws_bytes, _stream(q, stream)))


def attn_decode_tiered_q8(q, hot_k, hot_v, cold_k_pages, cold_v_pages, cold_k_scales,
                          cold_v_scales, cold_page_table, o, workspace, *, cold_len: int,
                          hot_len: int, hot_start: int, scale: float, sliding_window: int = 0,
                          attn_softcap: float = 0.0, stream=None):
    """q, o: float32 [num_heads, head_dim]; hot_k, hot_v: float16 ring [num_kv_heads,
    hot_window, head_dim] holding position p >= cold_len at row (hot_start + p - cold_len) %
    hot_window; cold pages int8 [num_pages, num_kv_heads, 16, head_dim], scales float32
    [num_pages, num_kv_heads, 16], page table int32 [max_pages] for positions < cold_len."""
    _need("attn_decode_tiered_q8", q=(q, "float32"), hot_k=(hot_k, "float16"),
          hot_v=(hot_v, "float16"), cold_k_pages=(cold_k_pages, "int8"),
          cold_v_pages=(cold_v_pages, "int8"), cold_k_scales=(cold_k_scales, "float32"),
          cold_v_scales=(cold_v_scales, "float32"), cold_page_table=(cold_page_table, "int32"),
          o=(o, "float32"), workspace=(workspace, "uint8"))
    _need_contig(q, hot_k, hot_v, cold_k_pages, cold_v_pages, cold_k_scales, cold_v_scales,
                 cold_page_table, o)
    H, D = q.shape
    Hkv, R, Dk = hot_k.shape
    P, Hkv2, ps, Dc = cold_k_pages.shape
    if Dk != D or Dc != D or Hkv2 != Hkv or hot_v.shape != hot_k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if cold_v_pages.shape != cold_k_pages.shape or cold_k_scales.shape != (P, Hkv, ps) or \
            cold_v_scales.shape != (P, Hkv, ps) or cold_page_table.dim() != 1:
        raise ValueError("cold tier: pages [P, Hkv, 16, D], scales [P, Hkv, 16], table [max_pages]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().attn_decode_tiered_q8(
        _ptr(q), _ptr(hot_k), _ptr(hot_v), _ptr(cold_k_pages), _ptr(cold_v_pages),
        _ptr(cold_k_scales), _ptr(cold_v_scales), _ptr(cold_page_table), _ptr(o), H, Hkv, D,
        int(cold_len), int(hot_len), R, int(hot_start), ps, P, cold_page_table.shape[0],
        int(sliding_window), float(attn_softcap), float(scale), _ptr(workspace), ws_bytes,
        _stream(q, stream)))



def attn_decode_tiered_q8_packed(q, hot_k, hot_v, cold_k, cold_v, cold_k_scales, cold_v_scales, o,
                                 workspace, *, cold_len: int, hot_len: int, hot_start: int,
                                 scale: float, sliding_window: int = 0, attn_softcap: float = 0.0,
                                 stream=None):
    """As attn_decode_tiered_q8 with a contiguous int8 cold tier: cold_k, cold_v int8
    [num_kv_heads, cold_capacity, head_dim], scales float32 [num_kv_heads, cold_capacity]."""
    _need("attn_decode_tiered_q8_packed", q=(q, "float32"), hot_k=(hot_k, "float16"),
          hot_v=(hot_v, "float16"), cold_k=(cold_k, "int8"), cold_v=(cold_v, "int8"),
          cold_k_scales=(cold_k_scales, "float32"), cold_v_scales=(cold_v_scales, "float32"),
          o=(o, "float32"), workspace=(workspace, "uint8"))
    _need_contig(q, hot_k, hot_v, cold_k, cold_v, cold_k_scales, cold_v_scales, o)
    H, D = q.shape
    Hkv, R, Dk = hot_k.shape
    Hc, C, Dc = cold_k.shape
    if Dk != D or Dc != D or Hc != Hkv or hot_v.shape != hot_k.shape or o.shape != q.shape or \
            cold_v.shape != cold_k.shape or cold_k_scales.shape != (Hkv, C) or \
            cold_v_scales.shape != (Hkv, C):
        raise ValueError("shape mismatch")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().attn_decode_tiered_q8_packed(
        _ptr(q), _ptr(hot_k), _ptr(hot_v), _ptr(cold_k), _ptr(cold_v), _ptr(cold_k_scales),
        _ptr(cold_v_scales), _ptr(o), H, Hkv, D, int(cold_len), int(hot_len), R, int(hot_start), C,
        int(sliding_window), float(attn_softcap), float(scale), _ptr(workspace), ws_bytes,
        _stream(q, stream)))


def attn_decode_tiered_f16(q, hot_k, hot_v, cold_k, cold_v, cold_page_table, o, workspace, *,
                           cold_len: int, hot_len: int, hot_start: int, scale: float,
                           sliding_window: int = 0, attn_softcap: float = 0.0, stream=None):
    """Tiered decode with an f16 cold tier.  Paged when cold_page_table is given: cold_k,
    cold_v float16 [num_pages, num_kv_heads, 16, head_dim], page table int32 [max_pages];
    contiguous when it is None: cold_k, cold_v float16 [num_kv_heads, cold_capacity, head_dim]."""
    _need("attn_decode_tiered_f16", q=(q, "float32"), hot_k=(hot_k, "float16"),
          hot_v=(hot_v, "float16"), cold_k=(cold_k, "float16"), cold_v=(cold_v, "float16"),
          cold_page_table=(cold_page_table, "int32"), o=(o, "float32"),
          workspace=(workspace, "uint8"))
    _need_contig(q, hot_k, hot_v, cold_k, cold_v, o)
    H, D = q.shape
    Hkv, R, Dk = hot_k.shape
    if Dk != D or hot_v.shape != hot_k.shape or o.shape != q.shape or cold_v.shape != cold_k.shape:
        raise ValueError("shape mismatch")
    if cold_page_table is not None:
        _need_contig(cold_page_table)
        P, Hc, ps, Dc = cold_k.shape
        if Hc != Hkv or Dc != D or cold_page_table.dim() != 1:
            raise ValueError("paged cold tier: pages [P, Hkv, 16, D], table [max_pages]")
        layout, cap, npages = ATTN_COLD_PAGED, cold_page_table.shape[0] * ps, P
    else:
        Hc, C, Dc = cold_k.shape
        if Hc != Hkv or Dc != D:
            raise ValueError("contiguous cold tier: [Hkv, cold_capacity, D]")
        layout, cap, ps, npages = ATTN_COLD_CONTIGUOUS, C, 0, 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().attn_decode_tiered_f16(
        _ptr(q), _ptr(hot_k), _ptr(hot_v), _ptr(cold_k), _ptr(cold_v), _ptr(cold_page_table),
        _ptr(o), H, Hkv, D, int(cold_len), int(hot_len), R, int(hot_start), layout, cap, ps, npages,
        int(sliding_window), float(attn_softcap), float(scale), _ptr(workspace), ws_bytes,
        _stream(q, stream)))


def attn_block_local(q_pad, k_padded, v_padded, pos_proj, attn_out, *, seq: int, chunk_size: int,
                     max_past: int, max_future: int, logit_cap: float = 0.0, context_size=None,
                     max_span=None, pad_left=None, stream=None):
    """Conformer block-local attention, float32.  q_pad, attn_out: [padded_len, H, 128];
    k_padded, v_padded: [kv_rows, H, 128] with row r at position r - pad_left; pos_proj:
    [max_span, H, 128].  context_size, max_span and pad_left default to chunk + past +
    future, past + future + 1 and past."""
    _need("attn_block_local", q_pad=(q_pad, "float32"), k_padded=(k_padded, "float32"),
          v_padded=(v_padded, "float32"), pos_proj=(pos_proj, "float32"),
          attn_out=(attn_out, "float32"))
    _need_contig(q_pad, k_padded, v_padded, pos_proj, attn_out)
    P, H, D = q_pad.shape
    R = k_padded.shape[0]
    if k_padded.shape[1:] != (H, D) or v_padded.shape != k_padded.shape or \
            pos_proj.shape[1:] != (H, D) or attn_out.shape != q_pad.shape:
        raise ValueError("shape mismatch")
    if context_size is None:
        context_size = chunk_size + max_past + max_future
    if max_span is None:
        max_span = max_past + max_future + 1
    if pad_left is None:
        pad_left = max_past
    if pos_proj.shape[0] != max_span:
        raise ValueError("pos_proj must have max_span rows")
    _check(lib().attn_block_local(_ptr(q_pad), _ptr(k_padded), _ptr(v_padded), _ptr(pos_proj),
                                  _ptr(attn_out), int(seq), P, R, H, D, int(chunk_size),
                                  int(context_size), int(max_span), int(max_past),
                                  int(max_future), int(pad_left), float(logit_cap),
                                  _stream(q_pad, stream)))
