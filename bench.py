"""Throughput of the attention hot path on one MI355X, against the roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_f16]
                    [--only-headline] [--no-cpu-baseline]

A step is one call of the workload's entry point over one batch of synthetic input
(inputs already resident in HBM).  The headline workload is single-token decode over a
contiguous f16 KV cache (32 query / 8 KV heads, head_dim 128, kv_len 4096); the other
workloads (f32 causal prefill, f16 windowed+softcapped GQA prefill, f16 vision, batched
paged int8 decode, f16 chunked prefill against a cache whose length is read on the device,
f16 decode over a ring-buffer cache, tiered decode over an int8 or f16 cold tier, paged or
contiguous, plus an f16 ring hot tier, and Conformer block-local attention) are measured on
the same JSON line under "workloads".  `--floors` times the memory-system floors of the
decode workloads (libattn_floors.so) beside the decode kernels instead.

Timing: W untimed steps, then K steps between HIP events recorded on the stream the
kernels run on, after a device synchronisation on both sides; the median of 5 such timed
replays is reported.  The K launches are captured into HIP graphs; untimed replays (at
least 20 ms of device work, so that the clocks have settled) come before the timed ones.
Every workload rotates over enough independent input copies (>= 1 GiB in total), in order
across replays, that each step reads its operands from HBM, not from the 256 MB Infinity
Cache.

The cpu_baseline leg times the float64 oracle (test infrastructure) on the host cores,
on the same workload, repeated for about ten seconds.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (prefill/vision) and KV GB/s (decode), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0     # dense f16 MFMA, TFLOP/s
F32_PEAK_TFS = 157.3           # f32 (vector and matrix), TFLOP/s
SETTLE_MS = 20.0               # untimed graph replays before the timed one, ms of device work
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_f16",
                    choices=["decode_f16", "prefill_f32", "prefill_f16", "vision_f16",
                             "decode_paged_q8", "prefill_chunk_f16", "decode_ring_f16",
                             "decode_tiered_q8", "decode_tiered_f16", "decode_tiered_q8_packed",
                             "decode_tiered_f16_contig", "block_local_f32", "all"])
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed replays; the median is reported")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from the host instead of replaying a HIP graph")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many steps of the selected workload(s), for profilers")
    ap.add_argument("--floors", action="store_true",
                    help="time the memory-system floors of the decode workloads (libattn_floors.so) "
                         "beside the decode kernels, one JSON line")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="with --profile-steps: also run a plain elementwise copy of this many "
                         "bytes per step (calibrates the HBM byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------------------------

class Workload:
    name = ""
    kind = ""            # "hbm" or "mfma" or "f32"
    desc = {}

    def units(self):
        """(algorithmic amount per step, unit): bytes for HBM-bound, FLOPs otherwise."""
        raise NotImplementedError


def n_copies(bytes_per_copy):
    """Input copies that together hold >= 1 GiB, rounded up to a multiple of 16 (a power of
    two below 16), so that few graphs of K launches cover a whole number of rounds through
    the copies for the usual K; at most 512."""
    n = max(2, int(math.ceil(ROTATE_BYTES / max(1, bytes_per_copy))))
    n = 1 << (n - 1).bit_length() if n < 16 else (n + 15) // 16 * 16
    return min(512, n)


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class DecodeF16(Workload):
    name = "decode_f16"
    kind = "hbm"
    kernel = "decode_split_kernel<128, 4, false, false, false>"

    def __init__(self, dev, H=32, Hkv=8, D=128, L=4096):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        self.H, self.Hkv, self.D, self.L = H, Hkv, D, L
        self.q_np, self.k_np, self.v_np = synth.decode_inputs(synth.seed_of(2), H, Hkv, D, L)
        kv_bytes = 2 * Hkv * L * D * 2
        self.nc = n_copies(kv_bytes)
        k = torch.from_numpy(self.k_np).to(dev)
        v = torch.from_numpy(self.v_np).to(dev)
        self.q = torch.from_numpy(self.q_np).to(dev)
        self.ks = [k.clone() for _ in range(self.nc)]
        self.vs = [v.clone() for _ in range(self.nc)]
        self.o = torch.empty((H, D), dtype=torch.float32, device=dev)
        self.ws = ta.decode_workspace(1, H, Hkv, D, L, dev)
        self.scale = 1.0 / math.sqrt(D)
        self.desc = {"workload": "single-token decode, f16 KV cache [8, 4096, 128], f32 q "
                                 "[32, 128], GQA 32/8, scale 1/sqrt(128)",
                     "batch": 1, "num_heads": H, "num_kv_heads": Hkv, "head_dim": D,
                     "kv_len": L, "kv_dtype": "f16", "q_dtype": "f32", "input_copies": self.nc}

    def step(self, i):
        j = i % self.nc
        self.ta.attn_decode(self.q, self.ks[j], self.vs[j], self.o, self.ws, scale=self.scale)

    def units(self):
        b = 2 * self.Hkv * self.L * self.D * 2 + 2 * self.H * self.D * 4
        return b, "bytes"

    def check(self):
        import numpy as np

        import oracle
        self.step(0)
        self.torch.cuda.synchronize()
        want = oracle.attention(self.q_np[None, None], np.transpose(self.k_np, (1, 0, 2))[None],
                                np.transpose(self.v_np, (1, 0, 2))[None], causal=True,
                                scale=self.scale)[0, 0]
        return float(np.abs(self.o.cpu().numpy() - want).max())

    def cpu_run(self, threads):
        import numpy as np

        import oracle
        return oracle.attention(self.q_np[None, None], np.transpose(self.k_np, (1, 0, 2))[None],
                                np.transpose(self.v_np, (1, 0, 2))[None], causal=True,
                                scale=self.scale, threads=threads)


class DecodeRing(DecodeF16):
    """Decode over a ring-buffer cache: a 4096-row ring holding the newest 4096 of 10000
    tokens (position t at row t % 4096), the same bytes as the contiguous decode."""
    name = "decode_ring_f16"
    kernel = "decode_split_kernel<128, 4, false, false, true>"

    def __init__(self, dev, total=10000):
        super().__init__(dev)
        import numpy as np
        import torch
        self.T = total
        shift = (total - self.L) % self.L     # visible token j sits at row (T - R + j) % R
        k = torch.from_numpy(np.ascontiguousarray(np.roll(self.k_np, shift, axis=1))).to(dev)
        v = torch.from_numpy(np.ascontiguousarray(np.roll(self.v_np, shift, axis=1))).to(dev)
        self.ks = [k.clone() for _ in range(self.nc)]
        self.vs = [v.clone() for _ in range(self.nc)]
        self.desc = dict(self.desc)
        self.desc["workload"] = ("single-token decode over a ring-buffer f16 cache [8, 4096, 128] "
                                 "holding the newest 4096 of 10000 tokens (row t mod 4096), f32 q "
                                 "[32, 128], GQA 32/8, scale 1/sqrt(128)")
        self.desc["ring_len"], self.desc["total_len"] = self.L, total

    def step(self, i):
        j = i % self.nc
        self.ta.attn_decode_ring(self.q, self.ks[j], self.vs[j], self.o, self.ws, total_len=self.T,
                                 scale=self.scale)


class PagedQ8(Workload):
    name = "decode_paged_q8"
    kind = "hbm"
    kernel = "decode_split_kernel<128, 4, true, false, false>"

    def __init__(self, dev):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        c = synth.seed_of(5)
        self.lens = synth.paged_kv_lens(c, 8, 16384, 32768)
        d = synth.paged_inputs(c, 8, 32, 8, 128, self.lens, n_poison=64, max_pages=2048)
        self.d = d
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.q = t(d["q"])
        self.kl = t(d["kv_lens"])
        self.pt = t(d["page_table"])
        per = d["k_pages"].nbytes * 2 + d["k_scales"].nbytes * 2
        self.nc = n_copies(per)
        kp, vp, ks, vs = t(d["k_pages"]), t(d["v_pages"]), t(d["k_scales"]), t(d["v_scales"])
        self.copies = [(kp, vp, ks, vs)] + [(kp.clone(), vp.clone(), ks.clone(), vs.clone())
                                            for _ in range(self.nc - 1)]
        self.o = torch.empty((8, 32, 128), dtype=torch.float32, device=dev)
        self.ws = ta.decode_workspace(8, 32, 8, 128, 2048 * 16, dev)
        self.desc = {"workload": "batched paged int8 decode, batch 8, kv_len ~ U[16384, 32768] "
                                 "(seeded), 16-token pages placed by a seeded permutation, f32 q, "
                                 "GQA 32/8, head_dim 128",
                     "batch": 8, "num_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                     "kv_lens": [int(x) for x in self.lens], "page_size": 16,
                     "kv_dtype": "int8", "q_dtype": "f32", "input_copies": self.nc}

    def step(self, i):
        kp, vp, ks, vs = self.copies[i % self.nc]
        self.ta.attn_decode_paged_q8(self.q, kp, vp, ks, vs, self.pt, self.kl, self.o, self.ws,
                                     scale=1 / math.sqrt(128))

    def units(self):
        tok = int(sum(int(x) for x in self.lens))
        pages = sum((int(x) + 15) // 16 for x in self.lens)
        b = tok * 8 * (128 + 128 + 4 + 4) + pages * 4 + 2 * 8 * 32 * 128 * 4
        return b, "bytes"

    def check(self):
        import numpy as np

        import oracle
        self.step(0)
        self.torch.cuda.synchronize()
        got = self.o.cpu().numpy()
        err = 0.0
        for b in range(8):
            want = self._oracle_b(b, None)
            err = max(err, float(np.abs(got[b] - want).max()))
        return err

    def _oracle_b(self, b, threads):
        import oracle
        d = self.d
        k = oracle.dequant_i8(d["k_q"][b], d["k_s"][b])[None]
        v = oracle.dequant_i8(d["v_q"][b], d["v_s"][b])[None]
        return oracle.attention(d["q"][b][None, None], k, v, causal=True,
                                scale=1 / math.sqrt(128), threads=threads)[0, 0]

    def cpu_run(self, threads):
        return [self._oracle_b(b, threads) for b in range(8)]


class Tiered(Workload):
    """Tiered decode of one sequence: 28672 old positions in an int8 paged cold tier
    (16-token pages placed by a seeded permutation) and the newest 4096 in a 4096-row f16
    ring (hot tier, seeded start row), 32/8 heads, head_dim 128."""
    name = "decode_tiered_q8"
    kind = "hbm"
    kernel = "decode_tiered_kernel<128, 4, 0, false>"

    def __init__(self, dev, cold=28672, hot=4096, R=4096, hot_start=1234):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        self.cold, self.hot = cold, hot
        t = synth.tiered_inputs(synth.seed_of(6), 32, 8, 128, cold, hot, R, hot_start, n_poison=64)
        self.t = t
        c = t["cold"]
        dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.q, self.pt = dv(t["q"]), dv(c["page_table"][0])
        per = c["k_pages"].nbytes * 2 + c["k_scales"].nbytes * 2 + t["ring_k"].nbytes * 2
        self.nc = n_copies(per)
        first = tuple(dv(x) for x in (t["ring_k"], t["ring_v"], c["k_pages"], c["v_pages"],
                                       c["k_scales"], c["v_scales"]))
        self.copies = [first] + [tuple(x.clone() for x in first) for _ in range(self.nc - 1)]
        self.o = torch.empty((32, 128), dtype=torch.float32, device=dev)
        self.ws = ta.decode_workspace(1, 32, 8, 128, cold + hot, dev)
        self.hot_start = hot_start
        self.desc = {"workload": "tiered single-token decode: 28672 positions in an int8 paged cold "
                                 "tier (16-token pages, seeded permutation) + the newest 4096 in an "
                                 "f16 ring [8, 4096, 128], f32 q [32, 128], GQA 32/8, scale 1/sqrt(128)",
                     "batch": 1, "num_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                     "cold_len": cold, "hot_len": hot, "hot_window": R, "hot_start": hot_start,
                     "cold_dtype": "int8", "hot_dtype": "f16", "q_dtype": "f32",
                     "input_copies": self.nc}

    def step(self, i):
        hk, hv, kp, vp, ks, vs = self.copies[i % self.nc]
        self.ta.attn_decode_tiered_q8(self.q, hk, hv, kp, vp, ks, vs, self.pt, self.o, self.ws,
                                      cold_len=self.cold, hot_len=self.hot, hot_start=self.hot_start,
                                      scale=1 / math.sqrt(128))

    def units(self):
        b = (self.cold * 8 * (128 + 128 + 4 + 4) + ((self.cold + 15) // 16) * 4
             + self.hot * 8 * 128 * 2 * 2 + 2 * 32 * 128 * 4)
        return b, "bytes"

    def _oracle(self, threads):
        import numpy as np

        import oracle
        t, c = self.t, self.t["cold"]
        k = np.concatenate([oracle.dequant_i8(c["k_q"][0], c["k_s"][0]), t["hot_k"].astype(np.float64)])
        v = np.concatenate([oracle.dequant_i8(c["v_q"][0], c["v_s"][0]), t["hot_v"].astype(np.float64)])
        return oracle.attention(t["q"][None, None], k[None], v[None], causal=True,
                                scale=1 / math.sqrt(128), threads=threads)[0, 0]

    def check(self):
        import numpy as np
        self.step(0)
        self.torch.cuda.synchronize()
        return float(np.abs(self.o.cpu().numpy() - self._oracle(None)).max())

    def cpu_run(self, threads):
        return self._oracle(threads)


class TieredF16(Tiered):
    """Tiered decode with an f16 cold tier in 16-token pages: 28672 old positions (seeded page
    placement) plus the newest 4096 in a 4096-row f16 ring, 32/8 heads, head_dim 128."""
    name = "decode_tiered_f16"
    kernel = "decode_tiered_kernel<128, 4, 2, false>"

    def __init__(self, dev, cold=28672, hot=4096, R=4096, hot_start=1234):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        self.cold, self.hot = cold, hot
        t = synth.tiered_f16_inputs(synth.seed_of(6) + 1, 32, 8, 128, cold, hot, R, hot_start, True,
                                    n_poison=64)
        self.t = t
        dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.q, self.pt = dv(t["q"]), dv(t["cold_page_table"])
        first = tuple(dv(x) for x in (t["ring_k"], t["ring_v"], t["cold_k_pages"], t["cold_v_pages"]))
        self.nc = n_copies(sum(x.nbytes for x in first))
        self.copies = [first] + [tuple(x.clone() for x in first) for _ in range(self.nc - 1)]
        self.o = torch.empty((32, 128), dtype=torch.float32, device=dev)
        self.ws = ta.decode_workspace(1, 32, 8, 128, cold + hot, dev)
        self.hot_start = hot_start
        self.desc = {"workload": "tiered single-token decode with an f16 cold tier: 28672 positions in "
                                 "16-token f16 pages (seeded permutation) + the newest 4096 in an f16 "
                                 "ring [8, 4096, 128], f32 q [32, 128], GQA 32/8, scale 1/sqrt(128)",
                     "batch": 1, "num_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                     "cold_len": cold, "hot_len": hot, "hot_window": R, "hot_start": hot_start,
                     "cold_dtype": "f16", "cold_layout": "paged", "hot_dtype": "f16", "q_dtype": "f32",
                     "input_copies": self.nc}

    def step(self, i):
        hk, hv, kp, vp = self.copies[i % self.nc]
        self.ta.attn_decode_tiered_f16(self.q, hk, hv, kp, vp, self.pt, self.o, self.ws,
                                       cold_len=self.cold, hot_len=self.hot, hot_start=self.hot_start,
                                       scale=1 / math.sqrt(128))

    def units(self):
        b = ((self.cold + self.hot) * 8 * 128 * 2 * 2 + ((self.cold + 15) // 16) * 4
             + 2 * 32 * 128 * 4)
        return b, "bytes"

    def _oracle(self, threads):
        import numpy as np

        import oracle
        t = self.t
        k = np.concatenate([t["cold_k"], t["hot_k"]]).astype(np.float64)
        v = np.concatenate([t["cold_v"], t["hot_v"]]).astype(np.float64)
        return oracle.attention(t["q"][None, None], k[None], v[None], causal=True,
                                scale=1 / math.sqrt(128), threads=threads)[0, 0]


class TieredPacked(Tiered):
    """Tiered decode whose int8 cold tier is one contiguous array per KV head (no page
    table): the same 28672 cold rows and scales as the paged int8 tier, plus the newest 4096
    in a 4096-row f16 ring, 32/8 heads, head_dim 128."""
    name = "decode_tiered_q8_packed"
    kernel = "decode_tiered_kernel<128, 4, 1, false>"

    def __init__(self, dev, cold=28672, hot=4096, R=4096, hot_start=1234):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        self.cold, self.hot = cold, hot
        t = synth.tiered_packed_inputs(synth.seed_of(6), 32, 8, 128, cold, hot, R, hot_start, capacity=cold)
        self.t = t
        dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.q = dv(t["q"])
        first = tuple(dv(t[x]) for x in ("ring_k", "ring_v", "packed_k", "packed_v", "packed_k_scales",
                                           "packed_v_scales"))
        self.nc = n_copies(sum(x.nbytes for x in first))
        self.copies = [first] + [tuple(x.clone() for x in first) for _ in range(self.nc - 1)]
        self.o = torch.empty((32, 128), dtype=torch.float32, device=dev)
        self.ws = ta.decode_workspace(1, 32, 8, 128, cold + hot, dev)
        self.hot_start = hot_start
        self.desc = {"workload": "tiered single-token decode with a packed int8 cold tier: 28672 "
                                 "positions in int8 [8, 28672, 128] with per-token scales (no page "
                                 "table) + the newest 4096 in an f16 ring [8, 4096, 128], f32 q "
                                 "[32, 128], GQA 32/8, scale 1/sqrt(128)",
                     "batch": 1, "num_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                     "cold_len": cold, "hot_len": hot, "hot_window": R, "hot_start": hot_start,
                     "cold_dtype": "int8", "cold_layout": "contiguous", "hot_dtype": "f16",
                     "q_dtype": "f32", "input_copies": self.nc}

    def step(self, i):
        hk, hv, kc, vc, ks, vs = self.copies[i % self.nc]
        self.ta.attn_decode_tiered_q8_packed(self.q, hk, hv, kc, vc, ks, vs, self.o, self.ws,
                                             cold_len=self.cold, hot_len=self.hot,
                                             hot_start=self.hot_start, scale=1 / math.sqrt(128))

    def units(self):
        b = self.cold * 8 * (128 + 128 + 4 + 4) + self.hot * 8 * 128 * 2 * 2 + 2 * 32 * 128 * 4
        return b, "bytes"


class TieredF16Contig(TieredF16):
    """Tiered decode with a contiguous f16 cold tier [8, 28672, 128] (no page table) plus the
    newest 4096 in a 4096-row f16 ring, 32/8 heads, head_dim 128."""
    name = "decode_tiered_f16_contig"
    kernel = "decode_tiered_kernel<128, 4, 3, false>"

    def __init__(self, dev, cold=28672, hot=4096, R=4096, hot_start=1234):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        self.cold, self.hot = cold, hot
        t = synth.tiered_f16_inputs(synth.seed_of(6) + 1, 32, 8, 128, cold, hot, R, hot_start, False,
                                    capacity=cold)
        self.t = t
        dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        self.q, self.pt = dv(t["q"]), None
        first = tuple(dv(t[x]) for x in ("ring_k", "ring_v", "cold_k_contig", "cold_v_contig"))
        self.nc = n_copies(sum(x.nbytes for x in first))
        self.copies = [first] + [tuple(x.clone() for x in first) for _ in range(self.nc - 1)]
        self.o = torch.empty((32, 128), dtype=torch.float32, device=dev)
        self.ws = ta.decode_workspace(1, 32, 8, 128, cold + hot, dev)
        self.hot_start = hot_start
        self.desc = {"workload": "tiered single-token decode with a contiguous f16 cold tier: 28672 "
                                 "positions in f16 [8, 28672, 128] + the newest 4096 in an f16 ring "
                                 "[8, 4096, 128], f32 q [32, 128], GQA 32/8, scale 1/sqrt(128)",
                     "batch": 1, "num_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                     "cold_len": cold, "hot_len": hot, "hot_window": R, "hot_start": hot_start,
                     "cold_dtype": "f16", "cold_layout": "contiguous", "hot_dtype": "f16",
                     "q_dtype": "f32", "input_copies": self.nc}

    def units(self):
        b = (self.cold + self.hot) * 8 * 128 * 2 * 2 + 2 * 32 * 128 * 4
        return b, "bytes"


class BlockLocal(Workload):
    """Conformer block-local attention (audio encoder): 3000 frames, 8 heads of 128, chunks
    of 12 frames attending over 12 frames of past and none of future, logit cap 50, f32."""
    name = "block_local_f32"
    kind = "hbm"
    kernel = "block_local_kernel<32, true>"

    def __init__(self, dev, seq=3000, H=8, chunk=12, past=12, future=0, cap=50.0):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch = ta, torch
        self.seq, self.H, self.chunk, self.past, self.future, self.cap = seq, H, chunk, past, future, cap
        d = synth.block_local_inputs(synth.seed_of(7), seq, chunk, past, future, H)
        self.d = d
        dv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        first = tuple(dv(d[x]) for x in ("q", "k", "v", "pos"))
        per = sum(x.nbytes for x in first)
        self.nc = n_copies(per)
        self.copies = [first] + [tuple(x.clone() for x in first) for _ in range(self.nc - 1)]
        self.o = torch.empty_like(first[0])
        self.desc = {"workload": "Conformer block-local attention, f32, 3000 frames, 8 heads x "
                                 "head_dim 128, chunk 12, max_past 12, max_future 0, logit cap 50, "
                                 "relative-position projection [13, 1024]",
                     "seq": seq, "num_heads": H, "head_dim": 128, "chunk_size": chunk,
                     "max_past": past, "max_future": future, "logit_cap": cap,
                     "input_copies": self.nc}

    def step(self, i):
        q, k, v, pos = self.copies[i % self.nc]
        self.ta.attn_block_local(q, k, v, pos, self.o, seq=self.seq, chunk_size=self.chunk,
                                 max_past=self.past, max_future=self.future, logit_cap=self.cap)

    def units(self):
        D, span = 128, self.past + self.future + 1
        P = self.d["padded_len"]
        b = 4 * self.H * D * (2 * P + 2 * self.seq + span)     # q, o, k and v rows of [0, seq), pos
        return b, "bytes"

    def _oracle(self, threads):
        import oracle
        d = self.d
        return oracle.block_local(d["q"], d["k"], d["v"], d["pos"], seq=self.seq,
                                  chunk_size=self.chunk, max_past=self.past,
                                  max_future=self.future, logit_cap=self.cap, threads=threads)

    def check(self):
        import numpy as np
        self.step(0)
        self.torch.cuda.synchronize()
        return float(np.abs(self.o.cpu().numpy() - self._oracle(None)).max())

    def cpu_run(self, threads):
        return self._oracle(threads)


class Forward(Workload):
    """Prefill (token-major) or vision (head-major) forward."""

    def __init__(self, dev, name):
        import numpy as np
        import torch

        import synth
        import transformer_attention_03_amd as ta
        self.ta, self.torch, self.name = ta, torch, name
        if name == "prefill_f32":
            self.S, self.H, self.Hkv, self.D, self.causal, self.W, self.cap = 128, 1, 1, 64, True, 0, 0.0
            q, k, v = synth.prefill_inputs(synth.seed_of(1), 128, 128, 1, 1, 64, "f32")
            self.kind = "f32"
            self.kernel = "fwd_f32_kernel<64, false, true>"
            self.desc = {"workload": "causal prefill, f32, 1 sequence, 1 head, seq_len 128, "
                                     "head_dim 64, scale 1/8"}
        elif name == "prefill_f16":
            self.S, self.H, self.Hkv, self.D, self.causal, self.W, self.cap = 2048, 16, 8, 256, True, 512, 50.0
            q, k, v = synth.prefill_inputs(synth.seed_of(3), 2048, 2048, 16, 8, 256, "f16")
            self.kind = "mfma"
            self.kernel = "fwd_f16_kernel<256, 1, 8, 2, 64, 1, 1>"
            self.desc = {"workload": "causal GQA prefill, f16, 2048 tokens, 16/8 heads, head_dim "
                                     "256, sliding window 512, softcap 50, scale 1/16"}
        elif name == "prefill_chunk_f16":
            self.S, self.H, self.Hkv, self.D, self.causal, self.W, self.cap = 512, 16, 8, 128, True, 0, 0.0
            self.L = 4096
            q, k, v = synth.prefill_inputs(synth.seed_of(3) + 61, 512, 4096, 16, 8, 128, "f16")
            self.kind = "mfma"
            self.kernel = "fwd_f16_kernel<128, 1, 8, 2, 32, 4, 0>"
            self.desc = {"workload": "chunked causal prefill against a cache, f16, 512 new tokens "
                                     "after 3584 cached (kv length 4096 read on the device), "
                                     "16/8 heads, head_dim 128, scale 1/sqrt(128)"}
        else:
            self.S, self.H, self.Hkv, self.D, self.causal, self.W, self.cap = 2304, 16, 16, 64, False, 0, 0.0
            q, k, v = synth.vision_inputs(synth.seed_of(4), 2304, 16, 64)
            self.kind = "mfma"
            self.kernel = "fwd_f16_kernel<64, 1, 3, 2, 96, 1, 0>"
            self.desc = {"workload": "bidirectional vision attention, f16 [16, 2304, 64] "
                                     "head-major, scale 1/8"}
        self.vision = name == "vision_f16"
        self.chunk = name == "prefill_chunk_f16"
        if not self.chunk:
            self.L = self.S
        self.scale = 1.0 / math.sqrt(self.D)
        self.np_in = (q, k, v)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
        per = tq.nbytes + tk.nbytes + tv.nbytes
        self.nc = n_copies(per)
        self.copies = [(tq, tk, tv)] + [(tq.clone(), tk.clone(), tv.clone())
                                        for _ in range(self.nc - 1)]
        self.o = torch.empty_like(tq)
        self.kv_len = torch.tensor([self.L], dtype=torch.int32, device=dev)
        self.desc["input_copies"] = self.nc

    def live_pairs(self):
        S, L = self.S, self.L
        if not self.causal:
            return S * L
        tot = 0
        for i in range(S):
            p = L - S + i
            lo = max(0, p - self.W + 1) if self.W > 0 else 0
            tot += p + 1 - lo
        return tot

    def step(self, i):
        q, k, v = self.copies[i % self.nc]
        if self.vision:
            self.ta.attn_vision(q, k, v, self.o, scale=self.scale)
        elif self.chunk:
            self.ta.attn_prefill_device_kv_len(q, k, v, self.o, self.kv_len, causal=self.causal,
                                               scale=self.scale, sliding_window=self.W,
                                               attn_softcap=self.cap)
        else:
            self.ta.attn_prefill(q, k, v, self.o, causal=self.causal, scale=self.scale,
                                 sliding_window=self.W, attn_softcap=self.cap)

    def units(self):
        return 4 * self.D * self.live_pairs() * self.H, "flops"

    def _oracle_rows(self, rows, threads):
        import numpy as np

        import oracle
        q, k, v = self.np_in
        if self.vision:
            q, k, v = (np.transpose(x, (1, 0, 2)) for x in (q, k, v))
        out = []
        for i in rows:
            hi = self.L - self.S + i + 1 if self.causal else k.shape[0]
            out.append(oracle.attention(q[None, i:i + 1], k[None, :hi], v[None, :hi],
                                        causal=self.causal, window=self.W, softcap=self.cap,
                                        scale=self.scale, threads=threads)[0, 0])
        return np.stack(out)

    def check(self):
        import numpy as np
        self.step(0)
        self.torch.cuda.synchronize()
        got = self.o.cpu().numpy().astype(np.float64)
        if self.vision:
            got = np.transpose(got, (1, 0, 2))
        rows = sorted(set([0, 1, self.S // 3, self.S // 2, self.S - 2, self.S - 1]))
        return float(np.abs(got[rows] - self._oracle_rows(rows, None)).max())

    def cpu_rows(self):
        """A bounded sample of query rows (spread over the sequence) for the CPU baseline."""
        n = min(self.S, 64)
        return [int(round(i * (self.S - 1) / max(1, n - 1))) for i in range(n)]

    def cpu_run(self, threads):
        return self._oracle_rows(self.cpu_rows(), threads)


ALL = ["decode_f16", "prefill_f32", "prefill_f16", "vision_f16", "decode_paged_q8", "prefill_chunk_f16",
       "decode_ring_f16", "decode_tiered_q8", "decode_tiered_f16", "decode_tiered_q8_packed",
       "decode_tiered_f16_contig", "block_local_f32"]


def make(name, dev):
    if name == "decode_f16":
        return DecodeF16(dev)
    if name == "decode_paged_q8":
        return PagedQ8(dev)
    if name == "decode_ring_f16":
        return DecodeRing(dev)
    if name == "decode_tiered_q8":
        return Tiered(dev)
    if name == "block_local_f32":
        return BlockLocal(dev)
    if name == "decode_tiered_f16":
        return TieredF16(dev)
    if name == "decode_tiered_q8_packed":
        return TieredPacked(dev)
    if name == "decode_tiered_f16_contig":
        return TieredF16Contig(dev)
    return Forward(dev, name)


# ---------------------------------------------------------------------------------------------
# measurement
# ---------------------------------------------------------------------------------------------

def time_steps(wl, steps, warmup, graph=True, repeats=5):
    """ms per step and the per-replay times: K steps between HIP events on the launch stream,
    median over `repeats` timed replays.  With graph=True the steps are captured into HIP
    graphs and replayed, so host-side launch cost does not pace the GPU.

    Input copies: step s of the run uses copy s mod nc.  The steps are captured as G graphs
    of K launches, graph g holding steps gK .. gK + K - 1, with G = nc / gcd(nc, K), and the
    graphs are replayed in turn; so the launch sequence runs through the copies in order
    whatever K is, and a copy is read again only after every other copy (>= 1 GiB of inputs
    in total) has been streamed: no replay finds its operands in the 256 MB Infinity Cache.
    (G is capped at 64; only workloads whose copies all fit the cache anyway, the 128-token
    f32 prefill, reach the cap.)"""
    import torch
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    times = []
    if graph:
        nc = max(1, getattr(wl, "nc", 1))
        n_graphs = min(64, nc // math.gcd(nc, steps))
        side = torch.cuda.Stream()
        side.wait_stream(st)
        graphs = []
        for g in range(n_graphs):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                for i in range(steps):
                    wl.step(g * steps + i)
            graphs.append(gr)
        torch.cuda.synchronize()
        # untimed replays until the device has run >= 20 ms of this work (clocks settle;
        # a single short replay left the first timed one 5-10% slow), at least one round of
        # every graph, at most 200 replays
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        spent, r = 0.0, 0
        while r < 200 and (spent < SETTLE_MS or r < n_graphs):
            w0.record(st)
            graphs[r % n_graphs].replay()
            w1.record(st)
            torch.cuda.synchronize()
            spent += w0.elapsed_time(w1)
            r += 1
        for _ in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            graphs[r % n_graphs].replay()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
            r += 1
        del graphs
    else:
        base = warmup
        for _ in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            for i in range(steps):
                wl.step(base + i)
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
            base += steps
    med = sorted(times)[len(times) // 2]
    return med / steps, [t / steps for t in times]      # ms per step


def summarize(wl, ms):
    amount, unit = wl.units()
    sec = ms * 1e-3
    if unit == "bytes":
        gbs = amount / sec / 1e9
        return {"value": gbs, "unit": "GB/s", "bound": "hbm", "achieved": gbs,
                "peak": HBM_PEAK_GBS, "peak_unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": amount, "us_per_call": ms * 1e3}
    tfs = amount / sec / 1e12
    peak = F32_PEAK_TFS if wl.kind == "f32" else MFMA_F16_PEAK_TFS
    return {"value": tfs, "unit": "TFLOP/s", "bound": "mfma", "achieved": tfs, "peak": peak,
            "peak_unit": "TFLOP/s", "frac": tfs / peak, "algorithmic_flops": amount,
            "us_per_call": ms * 1e3}


def kernel_source(wl):
    """The source file of a workload's kernel."""
    if wl.kernel.startswith("block_local"):
        return "block_local.hip"
    return "decode.hip" if wl.kind == "hbm" else "fwd.hip"


def traffic_for(kernel_src, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except Exception:
        return None
    if not rec:
        return None
    h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    if rec.get("source_sha256_16") != h:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, budget_s=10.0):
    import oracle
    threads = oracle.default_threads()
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        wl.cpu_run(threads)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and time.perf_counter() - t_start > budget_s:
            break
        if len(times) >= 5000:            # the time budget normally ends the loop first
            break
    used = oracle.threads_used()          # threads that computed rows in the last call
    times.sort()
    med = times[len(times) // 2]
    amount, unit = wl.units()
    if isinstance(wl, Forward):
        frac = len(wl.cpu_rows()) / wl.S        # rows sampled; work scales with visible keys
        rows = wl.cpu_rows()
        if wl.causal:
            full = wl.live_pairs()
            part = 0
            for i in rows:
                lo = max(0, i - wl.W + 1) if wl.W > 0 else 0
                part += i + 1 - lo
            frac = part / full
        amount = amount * frac
        sample = "%d of %d query rows, all %d heads, %d repeats" % (len(rows), wl.S, wl.H,
                                                                    len(times))
    else:
        sample = "the full workload, %d repeats" % len(times)
    val = amount / med / (1e9 if unit == "bytes" else 1e12)
    return {"value": val, "unit": "GB/s" if unit == "bytes" else "TFLOP/s", "cores": used,
            "threads_started": threads,
            "kind": "oracle", "sample": sample + " (median %.3f s per repeat)" % med}



# ---------------------------------------------------------------------------------------------
# memory-system floors (--floors): probes from libattn_floors.so, timed like the workloads
# ---------------------------------------------------------------------------------------------

def floors_lib():
    import ctypes
    path = os.path.join(ROOT, "transformer_attention_03_amd", "libattn_floors.so")
    if not os.path.exists(path):
        raise RuntimeError("libattn_floors.so is not built; run python -m transformer_attention_03_amd.build")
    L = ctypes.CDLL(path)
    vp, i, l = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
    L.floor_empty.argtypes = [i, vp]
    L.floor_stream.argtypes = [vp, l, i, vp, vp]
    L.floor_stream_merge.argtypes = [vp, l, i, i, vp, vp, vp, vp]
    L.floor_gather.argtypes = [vp, vp, vp, i, i, l, vp, vp]
    L.floor_lds_read.argtypes = [i, i, i, vp, vp]
    L.floor_lds_read64.argtypes = [i, i, i, vp, vp]
    for f in (L.floor_empty, L.floor_stream, L.floor_stream_merge, L.floor_gather, L.floor_lds_read,
              L.floor_lds_read64):
        f.restype = i
    return L


class Floor(Workload):
    kind = "floor"

    def __init__(self, dev, lib):
        import torch
        self.torch, self.lib, self.dev = torch, lib, dev

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def call(self, rc):
        if rc != 0:
            raise RuntimeError("%s: the probe refused its arguments (%d)" % (self.name, rc))


class FloorEmpty(Floor):
    """Launches of `grid` workgroups of 512 threads that do nothing."""

    def __init__(self, dev, lib, grid):
        super().__init__(dev, lib)
        self.grid, self.nbytes = grid, 0
        self.name = "empty_%dx512" % grid

    def step(self, i):
        self.call(self.lib.floor_empty(self.grid, self.stream()))


class FloorStream(Floor):
    """A plain read of `nbytes` (16-byte loads, workgroup w reads the w-th of `grid` equal
    ranges), over input copies as the workloads rotate them; with merge=(splits, groups), the
    read is followed by one split-KV-shaped merge per group."""

    def __init__(self, dev, lib, nbytes, grid=None, merge=None):
        super().__init__(dev, lib)
        torch = self.torch
        self.nbytes, self.merge = nbytes, merge
        self.grid = merge[0] * merge[1] if merge else grid
        self.nc = n_copies(nbytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        self.srcs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=g)
                     for _ in range(self.nc)]
        self.sink = torch.zeros(self.grid * 8, dtype=torch.float32, device=dev)
        if merge:
            sp, gr = merge
            self.part = torch.zeros(gr * sp * 520, dtype=torch.float32, device=dev)
            self.tickets = torch.zeros(gr, dtype=torch.int32, device=dev)
            self.out = torch.zeros(gr * 520, dtype=torch.float32, device=dev)
            self.name = "stream_merge_%dx%d" % (sp, gr)
        else:
            self.name = "stream_%dx512" % self.grid

    def step(self, i):
        src = self.srcs[i % self.nc].data_ptr()
        if self.merge:
            sp, gr = self.merge
            self.call(self.lib.floor_stream_merge(src, self.nbytes, sp, gr, self.part.data_ptr(),
                                                  self.tickets.data_ptr(), self.out.data_ptr(), self.stream()))
        else:
            self.call(self.lib.floor_stream(src, self.nbytes, self.grid, self.sink.data_ptr(), self.stream()))


class FloorLds(Floor):
    """LDS reads only: `grid` workgroups of `threads` threads, 4 * iters 16-byte reads per
    lane after filling 64 KB of LDS; nbytes counts the bytes read from LDS."""

    def __init__(self, dev, lib, grid, threads, iters=4000):
        super().__init__(dev, lib)
        self.grid, self.threads, self.iters = grid, threads, iters
        self.nbytes = grid * threads * 16 * 4 * iters
        self.out = self.torch.zeros(grid * threads, dtype=self.torch.int32, device=dev)
        self.name = "lds_read_%dx%d" % (grid, threads)

    def step(self, i):
        self.call(self.lib.floor_lds_read(self.grid, self.threads, self.iters, self.out.data_ptr(), self.stream()))


class FloorLds64(Floor):
    """LDS reads of 8 bytes per lane, plain or transposing (the V^T operand reads of the
    forward kernels): `grid` workgroups of 512 threads, 4 * iters reads per lane."""

    def __init__(self, dev, lib, grid, tr, iters=4000):
        super().__init__(dev, lib)
        self.grid, self.tr, self.iters, self.threads = grid, tr, iters, 512
        self.nbytes = grid * 512 * 8 * 4 * iters
        self.out = self.torch.zeros(grid * 512, dtype=self.torch.int32, device=dev)
        self.name = "lds_read%s_b64_%dx512" % ("_tr16" if tr else "", grid)

    def step(self, i):
        self.call(self.lib.floor_lds_read64(self.grid, self.tr, self.iters, self.out.data_ptr(), self.stream()))


class FloorGather(Floor):
    """The paged int8 workload's K and V blocks (2 KB: 16 tokens of one KV head) read through
    its page table with plain 16-byte loads, in the order (sequence, KV head, page); workgroup
    w reads `per_wg` consecutive blocks of K and the matching V blocks."""

    def __init__(self, dev, lib, per_wg):
        super().__init__(dev, lib)
        import numpy as np
        import synth
        torch = self.torch
        c = synth.seed_of(5)
        lens = synth.paged_kv_lens(c, 8, 16384, 32768)
        d = synth.paged_inputs(c, 8, 32, 8, 128, lens, n_poison=64, max_pages=2048)
        P, Hkv = d["k_pages"].shape[0], d["k_pages"].shape[1]
        ids = []
        for b in range(8):
            n_pages = (int(lens[b]) + 15) // 16
            phys = d["page_table"][b, :n_pages].astype(np.int64)
            for h in range(Hkv):
                ids.append(phys * Hkv + h)
        ids = np.concatenate(ids).astype(np.uint32)
        self.n, self.per_wg, self.pool = len(ids), per_wg, P * Hkv
        self.blocks = torch.from_numpy(ids).to(dev)
        kp = torch.from_numpy(np.ascontiguousarray(d["k_pages"])).to(dev)
        vp = torch.from_numpy(np.ascontiguousarray(d["v_pages"])).to(dev)
        self.nbytes = 2 * 2048 * self.n
        self.nc = n_copies(2 * kp.numel())
        self.copies = [(kp, vp)] + [(kp.clone(), vp.clone()) for _ in range(self.nc - 1)]
        self.grid = (self.n + per_wg - 1) // per_wg
        self.sink = torch.zeros(self.grid * 8, dtype=torch.float32, device=dev)
        self.name = "gather_paged_%d_per_wg" % per_wg

    def step(self, i):
        kp, vp = self.copies[i % self.nc]
        self.call(self.lib.floor_gather(kp.data_ptr(), vp.data_ptr(), self.blocks.data_ptr(), self.n,
                                        self.per_wg, self.pool, self.sink.data_ptr(), self.stream()))


def run_floors(dev, a):
    """Times the floors with the workloads' method and prints one JSON line beside the
    decode kernels' own times."""
    import torch
    lib = floors_lib()
    kv = 2 * 8 * 4096 * 128 * 2          # the headline decode's K and V bytes
    probes = [lambda: FloorEmpty(dev, lib, 128), lambda: FloorEmpty(dev, lib, 1024),
              lambda: FloorStream(dev, lib, kv, grid=128), lambda: FloorStream(dev, lib, kv, grid=256),
              lambda: FloorStream(dev, lib, kv, grid=1024),
              lambda: FloorStream(dev, lib, kv, merge=(16, 8)), lambda: FloorStream(dev, lib, kv, merge=(32, 8)),
              lambda: FloorGather(dev, lib, 256), lambda: FloorGather(dev, lib, 128),
              lambda: FloorGather(dev, lib, 64), lambda: FloorLds(dev, lib, 256, 512),
              lambda: FloorLds(dev, lib, 256, 1024), lambda: FloorLds(dev, lib, 512, 512),
              lambda: FloorLds64(dev, lib, 256, 0), lambda: FloorLds64(dev, lib, 256, 1)]
    rows = []
    for mk in probes:
        f = mk()
        log("floor %s" % f.name)
        ms, per = time_steps(f, a.steps, a.warmup, graph=True, repeats=a.repeats)
        us = ms * 1e3
        row = {"probe": f.name, "grid": f.grid, "bytes_per_launch": f.nbytes,
               "us_per_launch": round(us, 3),
               "TB_per_s": round(f.nbytes / (us * 1e-6) / 1e12, 3) if f.nbytes else None,
               "us_each_replay": [round(x * 1e3, 3) for x in per]}
        if isinstance(f, (FloorLds, FloorLds64)):     # bytes per clock per compute unit at 2.4 GHz
            row["B_per_clk_per_CU"] = round(f.nbytes / (us * 1e-6) / 2.4e9 / 256, 1)
        rows.append(row)
        del f
        torch.cuda.empty_cache()
    kernels = {}
    for name in ("decode_f16", "decode_paged_q8"):
        wl = make(name, dev)
        log("kernel %s" % name)
        ms, _ = time_steps(wl, a.steps if name == "decode_f16" else max(20, a.steps // 4), a.warmup,
                           graph=True, repeats=a.repeats)
        b, _u = wl.units()
        kernels[name] = {"us_per_call": round(ms * 1e3, 3), "algorithmic_bytes": b,
                         "TB_per_s": round(b / (ms * 1e-3) / 1e12, 3)}
        del wl
        torch.cuda.empty_cache()
    print(json.dumps({"floors": rows, "kernels": kernels, "steps": a.steps, "repeats": a.repeats,
                      "timing": "median of timed graph replays, as the workloads"}))

def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the hot path "
              "shards by head, query block or sequence with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import transformer_attention_03_amd as ta
    if not os.path.exists(ta.LIB_PATH):
        from transformer_attention_03_amd import build as b
        b.build()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if a.floors:
        run_floors(dev, a)
        return

    if a.profile_steps:
        names = ALL if a.workload == "all" else [a.workload]
        for name in names:
            log("profiling %s: %d steps" % (name, a.profile_steps))
            wl = make(name, dev)
            for i in range(a.profile_steps):
                wl.step(i)
            torch.cuda.synchronize()
            del wl
            torch.cuda.empty_cache()
        if a.copy_bytes:
            # a plain elementwise copy kernel (reads n*4 bytes, writes n*4 bytes) whose
            # source is far larger than L2 + MALL: calibrates FETCH_SIZE / WRITE_SIZE
            n = a.copy_bytes // 4
            src = torch.ones(n, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            for _ in range(a.profile_steps):
                torch.neg(src, out=dst)
            torch.cuda.synchronize()
        print(json.dumps({"profiled_workloads": names, "steps": a.profile_steps,
                          "copy_bytes": a.copy_bytes}))
        return

    if a.workload == "all":
        a.workload = "decode_f16"
    log("preparing %s" % a.workload)
    head = make(a.workload, dev)
    err = head.check()
    log("%s max-abs error vs oracle %.3g; timing %d steps" % (head.name, err, a.steps))
    ms, per_replay = time_steps(head, a.steps, a.warmup, graph=not a.no_graph, repeats=a.repeats)
    s = summarize(head, ms)
    src = os.path.join(ROOT, "transformer_attention_03_amd", "csrc", kernel_source(head))
    roof = {"bound": s["bound"], "achieved": round(s["achieved"], 3), "peak": s["peak"],
            "unit": s["peak_unit"], "frac": round(s["frac"], 4),
            "traffic": traffic_for(src, head.kernel), "kernel": head.kernel}
    out = {"metric": METRIC, "value": round(s["value"], 3), "unit": s["unit"], "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32" if head.kind != "mfma" else "f16",
           "data": "synthetic (seeded SplitMix64 + Box-Muller, N(0,1))",
           "config": dict(head.desc), "roofline": roof, "max_abs_err_vs_oracle": err,
           "timing": ("median of %d timed replays, HIP events around each replay of a HIP graph "
                      "holding the %d launches (graphs rotate over the input copies), after "
                      "untimed replays of >= %g ms of device work" % (a.repeats, a.steps, SETTLE_MS))
           if not a.no_graph else "median of %d runs of %d host launches" % (a.repeats, a.steps),
           "timed_replays": a.repeats,
           "us_per_step_each_replay": [round(x * 1e3, 3) for x in per_replay]}
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(head)
    if not a.only_headline:
        others = {}
        for name in ALL:
            if name == head.name:
                continue
            log("preparing %s" % name)
            wl = make(name, dev)
            e = wl.check()
            log("%s max-abs error vs oracle %.3g" % (name, e))
            ms_w, _ = time_steps(wl, max(20, a.steps // 4), a.warmup, graph=not a.no_graph,
                                 repeats=a.repeats)
            sw = summarize(wl, ms_w)
            others[name] = {"config": wl.desc, "us_per_call": round(sw["us_per_call"], 3),
                            "value": round(sw["value"], 3), "unit": sw["unit"],
                            "roofline": {"bound": sw["bound"], "achieved": round(sw["achieved"], 3),
                                         "peak": sw["peak"], "unit": sw["peak_unit"],
                                         "frac": round(sw["frac"], 4), "kernel": wl.kernel,
                                         "traffic": traffic_for(os.path.join(
                                             ROOT, "transformer_attention_03_amd", "csrc",
                                             kernel_source(wl)), wl.kernel)},
                            "max_abs_err_vs_oracle": e}
            del wl
            torch.cuda.empty_cache()
        out["workloads"] = others
    print(json.dumps(out))


if __name__ == "__main__":
    main()
