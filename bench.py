#!/usr/bin/env python
"""Throughput of the CSA2 decode hot path on one MI355X.

One step = one decode token for every row of the batch through the whole hot
path: append the token's FP4 entry to the cache (kv_compress_quantize), refresh
the block summary it falls in (index_block_summary), score + select with the
indexer (indexer_topk; hierarchical at 1M context), then the joint sparse +
window attention (sparse_attn_decode).  Inputs are seeded synthetic data,
resident in HBM before the timed region; several independent input sets are
rotated so the working set exceeds the 256 MB Infinity Cache.

The timed region replays captured HIP graphs that each hold four consecutive
steps (one per input set), as the graph of a model step holds the hot path of
many layers; the same steps replayed as one graph per step are timed as well
and reported beside it (each graph launch adds a few microseconds).
(Running the cache append on a second stream, joined before the attention,
was measured slower inside the graph: about 13 us per step more for 3-5 us
of overlapped work.)  An equal eager pass afterwards times the dominant
kernel (the coarse indexer scan) with HIP events recorded by the library on
the kernel's own stream; that duration gives the roofline line.  The
cpu_baseline leg times the oracle on a bounded sample of the same workload.

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fp4_kv_cache_indexer_amd import csa2 as C  # noqa: E402
from fp4_kv_cache_indexer_amd import schedule as SCH  # noqa: E402
from fp4_kv_cache_indexer_amd import synth  # noqa: E402

METRIC = "decode sparse-attn queries/sec at 1M ctx; indexer HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0     # dense bf16/fp16

WORKLOADS = {
    # the configuration the metric is quoted on
    "c3": dict(desc="hierarchical indexer at 1M context, batch 8: 1,048,576 FP4 entries/seq, "
                    "8-position block summaries, keep 2048 blocks -> 16384-position pool, top-512, "
                    "64 heads x 512 bf16 queries, SWA 128 fp8",
               B=8, N=1 << 20, H=64, k=512, keep=2048, hier=True, m=1, dist="normal"),
    "c2": dict(desc="flat indexer, batch 32: 65,536 FP4 entries/seq (131,072 tokens pooled at m=2), "
                    "top-512, 64 heads, SWA 128 fp8, Student-t(3) latents",
               B=32, N=1 << 16, H=64, k=512, keep=0, hier=False, m=2, dist="t3"),
    "c1": dict(desc="single decode query, 4,096 FP4 entries, top-512, 16 heads, SWA 128 fp8",
               B=1, N=4096, H=16, k=512, keep=0, hier=False, m=1, dist="normal"),
    # layer groups: one query = one token through all the group's layers
    "c4": dict(desc="layer group, batch 64: 262,144 FP4 entries/seq; Full (flat indexer, top-512) + "
                    "3 Reuse + Reindex (flat, new indexer queries) + 3 Reuse; 64 heads, SWA 128 fp8, "
                    "fresh queries and windows per layer",
               B=64, N=262144, H=64, k=512, keep=0, hier=False, m=1, dist="normal",
               layers=("full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse")),
    "c4pool": dict(desc="layer group, batch 64: 262,144 FP4 entries/seq; Full (hierarchical, keep 2048 "
                        "blocks -> 16384-position pool, top-512) + 3 Reuse + Reindex restricted to the "
                        "Full layer's pool + 3 Reuse; 64 heads, SWA 128 fp8, fresh queries per layer",
                   B=64, N=262144, H=64, k=512, keep=2048, hier=True, m=1, dist="normal", pool=True,
                   layers=("full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse")),
}
# the same workloads with FP4 index keys (64 code bytes + 4 E4M3 group scales per entry)
for _name in ("c3", "c4"):
    WORKLOADS[_name + "fp4"] = dict(WORKLOADS[_name], key="fp4",
                                    desc=WORKLOADS[_name]["desc"] + "; FP4 index keys (68 B/entry)")


# the full 40-layer decode step of the CSA2 schedule
WORKLOADS["sched40"] = dict(
    desc="40-layer CSA2 decode step at 1M context, batch 8: 2 window-only layers; 3 encoder groups "
         "(Full + 5 Reuse) on m=2 caches of 524,288 FP4 entries; 5 decoder groups on one m=1 cache of "
         "1,048,576 FP4 entries (Full + 3 Reuse, then Reindex within the Full layer's 16384-position pool "
         "+ 3 Reuse); hierarchical indexers keep 2048 blocks; per token: append to all four caches and "
         "all 40 windows; 64 heads, top-512, 128-token FP8 windows",
    B=8, T=1 << 20, H=64, k=512, keep=2048, sched=True, N=1 << 20, hier=True, m=1)
WORKLOADS["sched40fp4"] = dict(WORKLOADS["sched40"], key="fp4",
                               desc=WORKLOADS["sched40"]["desc"] + "; FP4 index keys (the 890 B/token layout)")


def layers_of(w):
    return w.get("layers", ("full",))


class InputSet:
    """One batch of caches and queries, all device-resident."""

    def __init__(self, w, set_id, seed=0):
        B, N, H, m = w["B"], w["N"], w["H"], w["m"]
        g = torch.Generator(device="cuda")
        g.manual_seed(1_000_003 * seed + 7919 * set_id + 17)
        self.codes = torch.empty((B, N, 256), dtype=torch.uint8, device="cuda")
        self.scales = torch.empty((B, N, 32), dtype=torch.uint8, device="cuda")
        for b in range(B):
            x = synth.latent_dev((1, N * m, 512), g, w["dist"]).to(torch.bfloat16)
            z = torch.randn((1, N * m, 512), generator=g, device="cuda").to(torch.bfloat16) if m > 1 else None
            C.kv_compress_quantize(x, m, gate=z, codes=self.codes[b:b + 1], scales=self.scales[b:b + 1])
            if b == 0 and set_id == 0:
                self.x0 = x[0]                       # kept for the oracle baseline
                self.z0 = None if z is None else z[0]
            del x, z
        self.fp4 = w.get("key") == "fp4"
        if self.fp4:
            self.keys = torch.empty((B, N, 64), dtype=torch.uint8, device="cuda")
            self.kscales = torch.empty((B, N, 4), dtype=torch.uint8, device="cuda")
            for b in range(B):
                kb = torch.randn((1, N, 128), generator=g, device="cuda").to(torch.bfloat16)
                C.index_key_quantize(kb, codes=self.keys[b:b + 1], scales=self.kscales[b:b + 1])
                del kb
            self.summ = C.index_block_summary_fp4(self.keys, self.kscales) if w["hier"] else None
        else:
            self.keys = torch.empty((B, N, 128), dtype=torch.uint8, device="cuda")
            for b in range(B):
                self.keys[b] = synth.to_e4m3(torch.randn((N, 128), generator=g, device="cuda"))
            self.kscales = None
            self.summ = C.index_block_summary(self.keys) if w["hier"] else None
        layers = layers_of(w)
        nl = len(layers)
        # every layer's window ring, one tensor [layers, B, 128, 512]
        self.rings = synth.to_e4m3(synth.latent_dev((nl * B, 128, 512), g, w["dist"])).view(nl, B, 128, 512)
        self.swa = self.rings[0]
        self.swa_len = torch.full((B,), 128, dtype=torch.int32, device="cuda")
        self.q_idx = synth.to_e4m3(torch.randn((B, 32, 128), generator=g, device="cuda"))
        self.q = torch.randn((B, H, 512), generator=g, device="cuda").to(torch.bfloat16)
        # the new token: its latent (and gate logits), its index key, its
        # position (sets alternate the parity, so m=2 caches alternately
        # complete the last entry and hold a pending token)
        self.x_tok = synth.latent_dev((B, 512), g, w["dist"]).to(torch.bfloat16)
        self.z_tok = torch.randn((B, 512), generator=g, device="cuda").to(torch.bfloat16) if m > 1 else None
        self.k_tok = torch.randn((B, 128), generator=g, device="cuda").to(torch.bfloat16)
        self.pos = torch.full((B,), N * m - 1 - (set_id % 2 if m > 1 else 0), dtype=torch.int64, device="cuda")
        self.pend_x = torch.zeros((B, m - 1, 512), dtype=torch.bfloat16, device="cuda") if m > 1 else None
        self.pend_z = torch.zeros((B, m - 1, 512), dtype=torch.bfloat16, device="cuda") if m > 1 else None
        # the other layers' windows take their own new tokens
        self.ring_rows = torch.tensor([li * B + b for li in range(1, nl) for b in range(B)], dtype=torch.int32,
                                      device="cuda")
        self.ring_pos = torch.full(((nl - 1) * B,), N * m - 1, dtype=torch.int64, device="cuda")
        self.ring_x = synth.latent_dev(((nl - 1) * B, 512), g, w["dist"]).to(torch.bfloat16) if nl > 1 else None
        # per-layer queries and windows (layer 0 uses the tensors above)
        self.lq, self.lq_idx, self.lswa = [self.q], [self.q_idx], [self.swa]
        for L in range(1, nl):
            self.lq_idx.append(synth.to_e4m3(torch.randn((B, 32, 128), generator=g, device="cuda"))
                               if layers[L] == "reindex" else None)
            self.lq.append(torch.randn((B, H, 512), generator=g, device="cuda").to(torch.bfloat16))
            self.lswa.append(self.rings[L])
        self.pool = w.get("pool", False)
        self.blocks = torch.empty((B, w["keep"]), dtype=torch.int32, device="cuda") if self.pool else None
        self.idx2 = torch.empty((B, w["k"]), dtype=torch.int32, device="cuda")
        self.ws_idx2 = torch.zeros(max(256, C.indexer_topk_workspace(
            self.q_idx, self.keys, w["k"], block_keys=None if self.pool else self.summ,
            keep_blocks=w["keep"] or 2048, cand_blocks=self.blocks, key_scales=self.kscales)),
            dtype=torch.uint8, device="cuda")
        self.idx = torch.empty((B, w["k"]), dtype=torch.int32, device="cuda")
        self.out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        self.ws_idx = torch.zeros(max(256, C.indexer_topk_workspace(
            self.q_idx, self.keys, w["k"], block_keys=self.summ, keep_blocks=w["keep"] or 2048,
            key_scales=self.kscales)),
            dtype=torch.uint8, device="cuda")
        need = C.sparse_attn_workspace(self.q, self.idx, swa=self.swa, swa_len=self.swa_len, codes=self.codes)
        self.ws_attn = torch.empty(max(256, need), dtype=torch.uint8, device="cuda")


def step(w, s):
    """One decode step for the whole batch (all hot-path rows)."""
    # the windows of the group's other layers take the new token
    if s.ring_x is not None:
        C.window_append(s.ring_x, s.ring_pos, s.rings.view(-1, 128, 512), row_seq=s.ring_rows)
    idx = None
    for L, mode in enumerate(layers_of(w)):
        # a0-a3: the Full layer appends the new token -- the window of layer
        # 0, the last entry (m tokens pooled; m = 1 in the decoder layers)
        # with its index key and the summary of its block -- and selects with
        # the indexer (coarse-to-fine at 1M context), in one library call
        # (hierarchical: the append runs inside the coarse scan's launch); a7:
        # Reuse layers keep the selection, Reindex layers select anew (within
        # the Full layer's pool when the workload says so)
        if mode == "full":
            C.append_indexer_topk(s.x_tok, s.pos, s.codes, s.scales, s.k_tok, s.lq_idx[L], s.keys, w["k"], s.summ,
                                  m=w["m"], gate=s.z_tok, pend_x=s.pend_x, pend_gate=s.pend_z,
                                  key_scales=s.kscales, swa=s.rings[0], keep_blocks=w["keep"] or 2048,
                                  out_idx=s.idx, out_blocks=s.blocks, workspace=s.ws_idx)
            idx = s.idx
        elif mode == "reindex":
            if s.pool:
                C.indexer_topk(s.lq_idx[L], s.keys, w["k"], cand_blocks=s.blocks, out_idx=s.idx2,
                               workspace=s.ws_idx2, key_scales=s.kscales)
            else:
                C.indexer_topk(s.lq_idx[L], s.keys, w["k"], block_keys=s.summ, keep_blocks=w["keep"] or 2048,
                               out_idx=s.idx2, workspace=s.ws_idx2, key_scales=s.kscales)
            idx = s.idx2
        # a4-a6: gather + dequant + joint sparse/window attention
        C.sparse_attn_decode(s.lq[L], s.codes, s.scales, idx, swa=s.lswa[L], swa_len=s.swa_len, out=s.out,
                             lse=s.lse, workspace=s.ws_attn)


class SchedSet:
    """One batch of the 40-layer schedule's caches, windows and per-layer
    queries, all device-resident.  Sets alternate the new token's position
    parity so the m=2 caches alternately complete an entry and hold a
    pending token."""

    def __init__(self, w, set_id, seed=0):
        B, T, H, k = w["B"], w["T"], w["H"], w["k"]
        g = torch.Generator(device="cuda")
        g.manual_seed(1_000_003 * seed + 7919 * set_id + 29)
        self.layers = SCH.csa2_layers()
        self.fp4 = w.get("key") == "fp4"
        bf = dict(dtype=torch.bfloat16, device="cuda")
        u8 = dict(dtype=torch.uint8, device="cuda")
        self.caches = []
        for m in SCH.cache_ratios(self.layers):
            N = T // m
            c = dict(m=m, N=N, hier=N > 8 * w["keep"])
            c["codes"] = torch.empty((B, N, 256), **u8)
            c["scales"] = torch.empty((B, N, 32), **u8)
            c["keys"] = torch.empty((B, N, 64 if self.fp4 else 128), **u8)
            c["key_scales"] = torch.empty((B, N, 4), **u8) if self.fp4 else None
            for b in range(B):
                x = synth.latent_dev((1, N * m, 512), g, "normal").to(torch.bfloat16)
                z = torch.randn((1, N * m, 512), generator=g, device="cuda").to(torch.bfloat16) if m > 1 else None
                C.kv_compress_quantize(x, m, gate=z, codes=c["codes"][b:b + 1], scales=c["scales"][b:b + 1])
                del x, z
                kb = torch.randn((1, N, 128), generator=g, device="cuda")
                if self.fp4:
                    C.index_key_quantize(kb.to(torch.bfloat16), codes=c["keys"][b:b + 1],
                                         scales=c["key_scales"][b:b + 1])
                else:
                    c["keys"][b] = synth.to_e4m3(kb[0])
                del kb
            c["summ"] = ((C.index_block_summary_fp4(c["keys"], c["key_scales"]) if self.fp4
                          else C.index_block_summary(c["keys"])) if c["hier"] else None)
            c["pend_x"] = torch.zeros((B, m - 1, 512), **bf) if m > 1 else None
            c["pend_z"] = torch.zeros((B, m - 1, 512), **bf) if m > 1 else None
            c["x_new"] = synth.latent_dev((B, 512), g, "normal").to(torch.bfloat16)
            c["z_new"] = torch.randn((B, 512), generator=g, device="cuda").to(torch.bfloat16) if m > 1 else None
            c["k_new"] = torch.randn((B, 128), generator=g, device="cuda").to(torch.bfloat16)
            self.caches.append(c)
        L = len(self.layers)
        self.rings = synth.to_e4m3(synth.latent_dev((L * B, SCH.WINDOW, 512), g, "normal")).view(L, B, SCH.WINDOW, 512)
        self.swa_len = torch.full((B,), SCH.WINDOW, dtype=torch.int32, device="cuda")
        p = T - 1 - (set_id % 2)
        self.pos = torch.full((B,), p, dtype=torch.int64, device="cuda")
        self.full_layer = {ly.cache: ly.index for ly in self.layers if ly.mode == "full"}
        ring_layers = [ly.index for ly in self.layers if ly.index not in self.full_layer.values()]
        self.ring_rows = torch.tensor([li * B + b for li in ring_layers for b in range(B)], dtype=torch.int32,
                                      device="cuda")
        self.ring_pos = torch.full((len(ring_layers) * B,), p, dtype=torch.int64, device="cuda")
        self.ring_x = synth.latent_dev((len(ring_layers) * B, 512), g, "normal").to(torch.bfloat16)
        self.q = [torch.randn((B, H, 512), generator=g, device="cuda").to(torch.bfloat16) for _ in self.layers]
        self.q_idx = {ly.index: synth.to_e4m3(torch.randn((B, 32, 128), generator=g, device="cuda"))
                      for ly in self.layers if ly.mode in ("full", "reindex")}
        groups = sorted({ly.group for ly in self.layers if ly.group >= 0})
        self.gidx = {gr: torch.empty((B, k), dtype=torch.int32, device="cuda") for gr in groups}
        dec = self.caches[3]
        # kept blocks of every hierarchical Full layer (the decoder's is its Reindex layers' pool)
        self.blocks_by_cache = {ci: torch.empty((B, w["keep"]), dtype=torch.int32, device="cuda")
                                for ci, c in enumerate(self.caches) if c["hier"]}
        self.blocks = self.blocks_by_cache.get(3)
        self.ws_idx = {}
        for ci, c in enumerate(self.caches):
            self.ws_idx[ci] = torch.zeros(max(256, C.indexer_topk_workspace(
                self.q_idx[self.full_layer[ci]], c["keys"], k, block_keys=c["summ"], keep_blocks=w["keep"],
                key_scales=c["key_scales"])), **u8)
        self.ws_pool = torch.zeros(max(256, C.indexer_topk_workspace(
            self.q_idx[self.full_layer[3]], dec["keys"], k, cand_blocks=self.blocks, key_scales=dec["key_scales"])),
            **u8)
        self.out = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        idx0 = self.gidx[groups[0]]
        need = max(C.sparse_attn_workspace(self.q[0], idx0, swa=self.rings[0], swa_len=self.swa_len,
                                           codes=self.caches[0]["codes"]),
                   C.sparse_attn_workspace(self.q[0], None, swa=self.rings[0], swa_len=self.swa_len))
        self.ws_attn = torch.empty(max(256, need), **u8)
        self.idx = self.gidx[groups[-1]]       # compared across graph replays


def step_sched(w, s):
    """One token through all 40 layers: appends, then every layer's selection
    (Full / Reindex) and attention."""
    for ci, c in enumerate(s.caches):
        C.decode_append(c["x_new"], s.pos, c["codes"], c["scales"], c["k_new"], c["keys"], m=c["m"],
                        gate=c["z_new"], pend_x=c["pend_x"], pend_gate=c["pend_z"], key_scales=c["key_scales"],
                        block_keys=c["summ"], swa=s.rings[s.full_layer[ci]])
    C.window_append(s.ring_x, s.ring_pos, s.rings.view(-1, SCH.WINDOW, 512), row_seq=s.ring_rows)
    SCH.decode_layers(s.layers, s.caches, s.rings, s.swa_len, s.q, s.q_idx, w["k"], w["keep"],
                      out=[s.out] * len(s.layers), lse=[s.lse] * len(s.layers), sel=s.gidx,
                      blocks=s.blocks_by_cache, ws_idx=s.ws_idx, ws_pool={3: s.ws_pool},
                      ws_attn=s.ws_attn)


def sched_work(T, B=1, H=64, k=512, keep=2048, window=SCH.WINDOW, fp4=False):
    """Algorithmic work of one token of the 40-layer schedule at context T:
    indexer and attention flops (raw and weighted as the pages weigh
    operations: BF16 1, FP8 0.5, FP4 0.25 -- indexer products take their
    FP8 queries' weight, attention runs on bf16 operands), coarse-scan bytes
    and the coarse-scan launches."""
    layers = SCH.csa2_layers()
    ratios = SCH.cache_ratios(layers)
    idx_fl = attn_fl = 0
    coarse_bytes = 0
    coarse_launches = 0
    key_b = 68 if fp4 else 128
    for ly in layers:
        w_eff = min(window, T)
        if ly.mode == "swa_only":
            attn_fl += 4 * H * w_eff * 512
            continue
        N = T // ratios[ly.cache]
        nb = (N + 7) // 8
        if ly.mode == "full":
            if nb > keep:
                idx_fl += (nb + min(N, keep * 8)) * 8192
                coarse_bytes += nb * 128 + 32 * 128 + 32 * 4
                coarse_launches += 1
            else:
                idx_fl += N * 8192
        elif ly.mode == "reindex":
            idx_fl += min(N, keep * 8) * 8192
        attn_fl += 4 * H * (min(k, N) + w_eff) * 512
    return dict(idx_flops=B * idx_fl, attn_flops=B * attn_fl,
                weighted=B * (0.5 * idx_fl + 1.0 * attn_fl),
                coarse_bytes=B * coarse_bytes, coarse_launches=coarse_launches, key_bytes=key_b)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_score_coarse_c3_traffic.md")
# the sources that define the scan kernel (its traffic is re-measured when they change)
SCAN_SOURCES = [os.path.join(ROOT, "fp4_kv_cache_indexer_amd", "csrc", f)
                for f in ("score.hip", "items.h", "csa2_dev.h", "csa2_launch.h")]


def scan_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed
    FETCH_SIZE/WRITE_SIZE summary, or None when there is none for this
    workload or the kernel source has changed since the counters were taken."""
    import re
    if workload != "c3" or not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    mb = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)\s*$", text, re.M)
    mh = re.search(r"^source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not mb or not mh:
        return None
    if scan_source_sha256() != mh.group(1):
        return None
    return float(mb.group(1))


def _time_us(fn, reps=8, skip=2):
    """Mean of reps - skip event-timed calls of fn on the current stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev[skip:]]
    return sum(t) / len(t)


def run_probe(which):
    """The diagnostic probes behind the kernels' designs: the block-summary
    scan's read shape, the overlap of a wave's vector work with its MFMA
    chain, and the attention gather's read shape."""
    st = torch.cuda.current_stream()
    if which == "scan":
        rows, n = 8, 131072                     # the C3 coarse scan: 8 rows x 131,072 summaries
        sets = [torch.randint(0, 256, (rows, n, 128), dtype=torch.uint8, device="cuda") for _ in range(4)]
        nbytes = rows * n * 128
        print("| workgroups per row | chunk | load shape | us | TB/s |\n|---:|---:|---|---:|---:|")
        for per_row in (64, 96, 128, 192):
            chunk = ((n + per_row - 1) // per_row + 15) // 16 * 16
            for full, nt in ((False, False), (False, True), (True, False), (True, True)):
                k = [0]
                def fn():
                    C.probe_scan_read(sets[k[0] % 4], chunk, full, nt, stream=st)
                    k[0] += 1
                us = _time_us(fn, reps=12, skip=4)
                shape = ("whole lines" if full else "half lines") + (", non-temporal" if nt else "")
                print(f"| {per_row} | {chunk} | {shape} | {us:.2f} | {nbytes / us / 1e6:.2f} |")
    elif which == "mfma-valu":
        iters, n_wg = 2048, 256
        print("| waves per SIMD | FMAs per MFMA | us | ns per MFMA per SIMD |\n|---:|---:|---:|---:|")
        for threads in (256, 512):
            for nv in (0, 4, 8, 12, 16):
                us = _time_us(lambda: C.probe_mfma_valu(nv, threads, iters, n_wg, stream=st))
                per_simd = iters * 8 * (threads // 64) / 4
                print(f"| {threads // 256} | {nv} | {us:.1f} | {us * 1e3 / per_simd:.2f} |")
    else:
        n_ent, rows = 524288, 4096              # the C5 attention: 4096 rows x 512 entries
        codes = torch.randint(0, 256, (n_ent, 256), dtype=torch.uint8, device="cuda")
        scales = torch.randint(0, 256, (n_ent, 32), dtype=torch.uint8, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(1)
        ids = torch.randint(0, n_ent, (rows, 512), dtype=torch.int32, device="cuda", generator=g)
        nbytes = rows * 512 * (256 + 32)
        print("| lane mapping | us | TB/s |\n|---|---:|---:|")
        for whole in (False, True):
            us = _time_us(lambda: C.probe_gather(codes, scales, ids, 256, whole, stream=st))
            name = "whole lines (16 lanes per entry)" if whole else "attention kernels' (4 x 16 B per quarter entry)"
            print(f"| {name} | {us:.1f} | {nbytes / us / 1e6:.2f} |")


def prof_summary(d):
    """Markdown tables from the rocprofv3 CSV output under directory d:
    kernel durations (*_kernel_stats.csv) and mean counter values per
    dispatch (*_counter_collection.csv), for this library's kernels and the
    copy kernel of --copy-probe-mib."""
    import csv
    import glob
    from collections import defaultdict

    def short(name):
        return name if len(name) <= 90 else name[:87] + "..."

    keep = ("csa2::", "neg_kernel")
    for f in sorted(glob.glob(os.path.join(d, "**", "*_kernel_trace.csv"), recursive=True)):
        durs = defaultdict(list)
        for r in csv.DictReader(open(f)):
            if any(k in r["Kernel_Name"] for k in keep):
                durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"kernel durations ({os.path.relpath(f, d)}; the median is the steady-state step, "
              f"the maximum includes building the caches)\n")
        print("| kernel | launches | median us | mean us | min us | max us |")
        print("|---|---:|---:|---:|---:|---:|")
        for k, v in sorted(durs.items(), key=lambda kv: -float(np.median(kv[1]))):
            print(f"| {short(k)} | {len(v)} | {np.median(v):.2f} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        print()
    for f in sorted(glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True)):
        agg = defaultdict(lambda: defaultdict(list))
        grid = {}
        for r in csv.DictReader(open(f)):
            if any(k in r["Kernel_Name"] for k in keep):
                agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
                grid[r["Kernel_Name"]] = r.get("Grid_Size", "")
        print(f"counters, mean per dispatch ({os.path.relpath(f, d)})\n")
        print("| kernel | grid | counter | dispatches | mean |")
        print("|---|---:|---|---:|---:|")
        for k, cs in agg.items():
            for c, v in sorted(cs.items()):
                print(f"| {short(k)} | {grid[k]} | {c} | {len(v)} | {sum(v) / len(v):.1f} |")
        print()
    print(f"source_sha256 of the scan kernel's sources ({', '.join(os.path.basename(f) for f in SCAN_SOURCES)}): "
          f"{scan_source_sha256()}")


def copy_probe(mib):
    """A plain copy-like kernel of known size for scaling the HBM counters:
    out = -in over `mib` MiB of float32 (reads and writes mib MiB each)."""
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: 3 x neg over {mib} MiB float32", file=sys.stderr, flush=True)


def scan_bytes(w):
    """Algorithmic HBM bytes of one launch of the dominant kernel (the
    indexer scan): the key rows it must read plus queries and weights.  The
    coarse scan reads E4M3 block keys (128 B); a flat scan reads E4M3 keys or
    FP4 keys (64 code bytes + 4 scale bytes)."""
    if w.get("sched"):
        sw = sched_work(w["T"], w["B"], w["H"], w["k"], w["keep"], fp4=w.get("key") == "fp4")
        return sw["coarse_bytes"] // max(1, sw["coarse_launches"])      # per coarse launch
    B, N = w["B"], w["N"]
    rows = (N + 7) // 8 if w["hier"] else N
    row_bytes = 68 if (w.get("key") == "fp4" and not w["hier"]) else 128
    return B * (rows * row_bytes + 32 * 128 + 32 * 4)


def attn_flops(w):
    """Algorithmic flops of one attention launch: QK^T and PV over the
    selected entries and the window, 2 * 2 * H * (k + 128) * 512 per query."""
    if w.get("sched"):
        return sched_work(w["T"], w["B"], w["H"], w["k"], w["keep"])["attn_flops"] // len(SCH.csa2_layers())
    return w["B"] * 4 * w["H"] * (w["k"] + 128) * 512


def stall_calibrate(seconds):
    """Cycles for torch.cuda._sleep that keep the stream busy for about
    `seconds` (measured once with events)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cyc = 1 << 20
    torch.cuda._sleep(cyc)
    e0.record()
    torch.cuda._sleep(cyc)
    e1.record()
    torch.cuda.synchronize()
    per_s = cyc / (e0.elapsed_time(e1) / 1e3)
    return max(1, int(per_s * seconds))


def cpu_baseline(w, s, seconds):
    """Time the oracle on a bounded sample: decode steps of sequence 0 of the
    first input set (every layer of the workload's group), with fresh seeded
    queries, until `seconds` elapse."""
    from threadpoolctl import threadpool_info

    from oracle import csa2 as O

    N, H, k, m = w["N"], w["H"], w["k"], w["m"]
    layers = layers_of(w)
    keys = s.keys[0].cpu().numpy()
    if s.fp4:
        keys = O.Fp4Keys(keys, s.kscales[0].cpu().numpy())
    x0 = s.x0.view(torch.int16).cpu().numpy().view(np.uint16)
    z0 = None if s.z0 is None else s.z0.view(torch.int16).cpu().numpy().view(np.uint16)
    swa = s.swa[0].cpu().numpy()
    summ = O.block_summary(keys) if w["hier"] else None          # cache state (untimed)
    g = np.random.default_rng(0)
    n = 0
    el = 0.0
    while True:
        q_idx = [synth.to_e4m3(g.standard_normal((32, 128)).astype(np.float32)) for _ in layers]
        q = [torch.from_numpy(g.standard_normal((H, 512)).astype(np.float32)).to(torch.bfloat16)
             .view(torch.int16).numpy().view(np.uint16) for _ in layers]
        k_new = synth.to_bf16_bits(g.standard_normal((1, 128)).astype(np.float32)) if s.fp4 else None
        ts = time.perf_counter()
        O.kv_compress_quantize(x0[-m:], None if z0 is None else z0[-m:], m)   # a0: the new entry
        if s.fp4:
            O.index_key_quantize_fp4(k_new)                             # ... and its index key
        if w["hier"]:
            O.block_summary(keys[(N - 1) // 8 * 8:])                   # a1: its block
        idx = kept = None
        for L, mode in enumerate(layers):
            if mode == "full" or (mode == "reindex" and not w.get("pool")):
                if w["hier"]:
                    idx, kept_l = O.indexer_topk_hier(q_idx[L], None, keys, summ, k, N, w["keep"])
                    kept = kept_l if mode == "full" else kept
                else:
                    idx = O.indexer_topk_flat(q_idx[L], None, keys, k, N)
            elif mode == "reindex":
                idx = O.indexer_topk_pool(q_idx[L], None, keys, O.pool_positions(kept, N), k, N)
            if mode != "reuse":
                sel = idx[idx >= 0]
                tok = (sel[:, None] * m + np.arange(m)[None, :]).reshape(-1)
                codes, scales = O.kv_compress_quantize(x0[tok], None if z0 is None else z0[tok], m)
            O.sparse_attn(q[L], codes, scales, np.arange(len(sel)), swa, O.swa_slots(0, 128, 128))
        el += time.perf_counter() - ts
        n += 1
        if el >= seconds:
            break
    threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": n / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode queries{f' ({len(layers)}-layer group each)' if len(layers) > 1 else ''} "
                      f"on sequence 0 of the {w['N']}-entry cache "
                      f"(fresh seeded queries; oracle float64, NumPy/BLAS on {threads} threads"
                      f"{', ' + model if model else ''}; {el:.1f} s)"}


def cpu_baseline_sched(w, seconds):
    """Time the oracle on a bounded sample of the 40-layer step: one
    sequence, seeded host inputs of the workload's shapes (index keys and
    summaries of every cache built once, untimed), fresh queries per token;
    per token the append of every cache (pooling, quantisation, index key,
    block summary) and every layer's selection and attention, the attended
    entries quantised from seeded tokens by the oracle."""
    from threadpoolctl import threadpool_info

    from oracle import csa2 as O

    T, H, k, keep = w["T"], w["H"], w["k"], w["keep"]
    fp4 = w.get("key") == "fp4"
    layers = SCH.csa2_layers()
    ratios = SCH.cache_ratios(layers)
    g = np.random.default_rng(1)
    caches = []
    for m in ratios:
        N = T // m
        kb = synth.to_bf16_bits(g.standard_normal((N, 128)).astype(np.float32))
        keys = O.Fp4Keys(*O.index_key_quantize_fp4(kb)) if fp4 else synth.to_e4m3(F64(kb))
        summ = O.block_summary(keys) if (N + 7) // 8 > keep else None
        caches.append(dict(m=m, N=N, keys=keys, summ=summ))
    swa = synth.to_e4m3(g.standard_normal((SCH.WINDOW, 512)).astype(np.float32))
    slots = O.swa_slots(0, SCH.WINDOW, SCH.WINDOW)

    def bf16(shape):
        return synth.to_bf16_bits(g.standard_normal(shape).astype(np.float32))

    n, el = 0, 0.0
    while el < seconds:
        q = [bf16((H, 512)) for _ in layers]
        q_idx = {ly.index: synth.to_e4m3(g.standard_normal((32, 128)).astype(np.float32))
                 for ly in layers if ly.mode in ("full", "reindex")}
        toks = {ci: bf16((c["m"], 512)) for ci, c in enumerate(caches)}
        gates = {ci: bf16((c["m"], 512)) for ci, c in enumerate(caches)}
        knew = bf16((1, 128))
        sel_tok = bf16((k, 512))                        # the attended entries' tokens (m = 1 view)
        ts = time.perf_counter()
        for ci, c in enumerate(caches):                 # appends
            O.kv_compress_quantize(toks[ci], gates[ci] if c["m"] > 1 else None, c["m"])
            kq = O.Fp4Keys(*O.index_key_quantize_fp4(knew)) if fp4 else synth.to_e4m3(F64(knew))
            blk = c["keys"][(c["N"] - 1) // 8 * 8:]
            O.block_summary(blk)
            del kq
        sel, pool = {}, None
        for ly in layers:
            if ly.mode == "swa_only":
                O.sparse_attn(q[ly.index], np.zeros((0, 256), np.uint8), np.zeros((0, 32), np.uint8),
                              np.zeros(0, np.int64), swa, slots)
                continue
            c = caches[ly.cache]
            if ly.mode == "full":
                if c["summ"] is not None:
                    idx, kept = O.indexer_topk_hier(q_idx[ly.index], None, c["keys"], c["summ"], k, c["N"], keep)
                    if ly.cache == 3:
                        pool = O.pool_positions(kept, c["N"])
                else:
                    idx = O.indexer_topk_flat(q_idx[ly.index], None, c["keys"], k, c["N"])
                sel[ly.group] = idx
            elif ly.mode == "reindex":
                if pool is not None:
                    sel[ly.group] = O.indexer_topk_pool(q_idx[ly.index], None, c["keys"], pool, k, c["N"])
                else:
                    sel[ly.group] = O.indexer_topk_flat(q_idx[ly.index], None, c["keys"], k, c["N"])
            if ly.mode in ("full", "reindex"):
                ne = int((sel[ly.group] >= 0).sum())
                codes, scales = O.kv_compress_quantize(sel_tok[:ne], None, 1)
            O.sparse_attn(q[ly.index], codes, scales, np.arange(ne), swa, slots)
        el += time.perf_counter() - ts
        n += 1
    threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    return {"value": n / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} tokens of one sequence through the 40-layer step at {T} tokens of context "
                      f"(seeded host inputs; oracle float64, NumPy/BLAS on {threads} threads; {el:.1f} s)"}


def F64(bits):
    """bf16 bits -> float32 values (exact) for the E4M3 rounding of synth."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def sweep(args, w0):
    """The 40-layer step across contexts: time per token step next to the
    schedule's algorithmic work per token."""
    print("| context tokens | us/step (batch %d) | tokens/s | indexer GFLOP/token | attention GFLOP/token "
          "| weighted GFLOP/token | global KV bytes/token |" % w0["B"])
    print("|---:|---:|---:|---:|---:|---:|---:|")
    base = None
    for T in (4096, 16384, 65536, 262144, 1 << 20):
        w = dict(w0, T=T, N=T)
        sets = [SchedSet(w, i) for i in range(2)]
        for i in range(3):
            step_sched(w, sets[i % 2])
        torch.cuda.synchronize()
        graphs = []
        for st in sets:
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                step_sched(w, st)
            graphs.append(gph)
        for i in range(4):
            graphs[i % 2].replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            graphs[i % 2].replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        sw = sched_work(T, 1, w["H"], w["k"], w["keep"], fp4=w.get("key") == "fp4")
        base = base or sw["weighted"]
        kvb = SCH.global_bytes_per_token(SCH.csa2_layers(), 288, sw["key_bytes"])
        print(f"| {T} | {us:.1f} | {w['B'] * 1e6 / us:.0f} | {sw['idx_flops'] / 1e9:.3f} | "
              f"{sw['attn_flops'] / 1e9:.3f} | {sw['weighted'] / 1e9:.3f} ({sw['weighted'] / base:.2f}x) | {kvb:g} |",
              flush=True)
        del sets, graphs
        torch.cuda.empty_cache()


PREFILL_C5 = dict(
    desc="prefill chunk at 1M context: 1,048,576 bf16 tokens (512-dim, gate logits) pooled at m=2 into "
         "524,288 FP4 entries (the cache write), then 4,096 queries at positions [T-4096, T), each a flat "
         "causal top-512 over its ~523K visible E4M3 index keys (32 x 128) and joint attention over its "
         "512 entries + 128-token FP8 window; 64 heads x 512 bf16",
    T=1 << 20, m=2, R=4096, H=64, k=512, W=128)


def cpu_baseline_prefill(w, xb, zb, kb, qi, hw, qb, sw, base, seconds, write_stride=32, row_stride=64):
    """Time the oracle on a bounded sample of the prefill step: the cache
    write of every `write_stride`-th group of m tokens (scaled by the stride)
    and the indexer + attention of rows 0, row_stride, 2*row_stride, ... until
    `seconds` elapse (at least 2 rows; scaled to all rows).  Host arrays:
    tokens and gate logits as bf16 bits [T, 512], index keys E4M3 [N, 128],
    index queries E4M3 [R, 32, 128], head weights [R, 32], queries as bf16
    bits [R, H, 512] and the window tokens E4M3 [T - base, 512] from token
    `base` on."""
    from threadpoolctl import threadpool_info

    from oracle import csa2 as O

    T, m, R, k, W = w["T"], w["m"], w["R"], w["k"], w["W"]
    N = T // m
    groups = np.arange(0, N, write_stride)
    tok = (groups[:, None] * m + np.arange(m)[None, :]).reshape(-1)
    ts = time.perf_counter()
    O.kv_compress_quantize(xb[tok], zb[tok], m)
    t_write = (time.perf_counter() - ts) * (N / len(groups))
    n, t_rows = 0, 0.0
    for r in range(0, R, row_stride):
        ts = time.perf_counter()
        nv, lo, ln = O.prefill_row_view(T - R + r, m, W)
        idx = O.indexer_topk_flat(qi[r], hw[r], kb, k, nv)
        sel = idx[idx >= 0]
        tk = (sel[:, None] * m + np.arange(m)[None, :]).reshape(-1)
        codes, scales = O.kv_compress_quantize(xb[tk], zb[tk], m)
        O.sparse_attn(qb[r], codes, scales, np.arange(len(sel)), sw, O.swa_slots(lo - base, ln, sw.shape[0]))
        t_rows += time.perf_counter() - ts
        n += 1
        if n >= 2 and t_rows >= seconds:
            break
    t_step = t_write + t_rows / n * R
    threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    return {"value": R / t_step, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"cache write of 1 in {write_stride} entries ({len(groups)} entries, {t_write / (N / len(groups)):.1f} s, "
                      f"scaled x{N / len(groups):.0f}) + indexer and attention of {n} rows strided by {row_stride} "
                      f"({t_rows:.1f} s, scaled to {R} rows); oracle float64, NumPy/BLAS on {threads} threads; "
                      f"estimated step {t_step:.0f} s"}


def run_prefill(args):
    """One step = the C5 prefill chunk: the cache write of the whole 1M-token
    context, the 4096-row causal indexer and the 4096-row attention.  Each
    part is timed with HIP events (kernels on one stream, back to back);
    value = rows of the chunk per second of the whole step."""
    w = PREFILL_C5
    T, m, R, H, k, W = w["T"], w["m"], w["R"], w["H"], w["k"], w["W"]
    N = T // m
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = synth.latent_dev((1, T, 512), g, "normal").to(torch.bfloat16)
    z = torch.randn((1, T, 512), generator=g, device="cuda").to(torch.bfloat16)
    codes = torch.empty((1, N, 256), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, N, 32), dtype=torch.uint8, device="cuda")
    keys = synth.to_e4m3(torch.randn((1, N, 128), generator=g, device="cuda"))
    pos = torch.arange(T - R, T, device="cuda", dtype=torch.int64)
    n_valid = ((pos + 1) // m).to(torch.int32)
    row_seq = torch.zeros(R, dtype=torch.int32, device="cuda")
    q_idx = synth.to_e4m3(torch.randn((R, 32, 128), generator=g, device="cuda"))
    head_w = torch.rand((R, 32), generator=g, device="cuda") * 0.75 + 0.25
    q = torch.randn((R, H, 512), generator=g, device="cuda").to(torch.bfloat16)
    base = T - R - (W - 1)                       # the window tokens of the chunk, in FP8
    swa = synth.to_e4m3(x[:, base:].float())
    lo = (pos - (W - 1)).clamp(min=0)
    swa_start = (lo - base).to(torch.int32)
    swa_len = (pos - lo + 1).to(torch.int32)
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    out = torch.empty((R, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    ws_i = torch.zeros(C.indexer_topk_workspace(q_idx, keys, k), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, C.sparse_attn_workspace(q, idx, swa=swa, swa_len=swa_len, codes=codes, swa_max=W)),
                       dtype=torch.uint8, device="cuda")
    parts = [
        ("cache_write", lambda: C.kv_compress_quantize(x, m, gate=z, codes=codes, scales=scales)),
        ("indexer", lambda: C.indexer_topk(q_idx, keys, k, head_w=head_w, row_seq=row_seq, n_valid=n_valid,
                                           out_idx=idx, workspace=ws_i)),
        ("attention", lambda: C.sparse_attn_decode(q, codes, scales, idx, swa=swa, swa_start=swa_start,
                                                   swa_len=swa_len, row_seq=row_seq, out=out, lse=lse,
                                                   workspace=ws_a, swa_max=W)),
    ]
    print(f"[bench] workload c5: {w['desc']}", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        for _, f in parts:
            f()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
    tot = [0.0] * len(parts)
    for _ in range(args.steps):
        ev[0].record()
        for i, (_, f) in enumerate(parts):
            f()
            ev[i + 1].record()
        torch.cuda.synchronize()
        for i in range(len(parts)):
            tot[i] += ev[i].elapsed_time(ev[i + 1])
    ms = [t / args.steps for t in tot]
    ms_step = sum(ms)
    for (name, _), t in zip(parts, ms):
        print(f"[bench] {name}: {t * 1e3:.1f} us", file=sys.stderr, flush=True)
    write_bytes = 2 * T * 512 * 2 + N * (256 + 32)             # x + gate read, FP4 entries written
    idx_flops = float(n_valid.double().sum().item()) * 8192     # 32 heads x 128 per visible entry
    attn_fl = 4.0 * H * (k + W) * 512 * R
    res = {
        "metric": METRIC, "value": round(R / (ms_step / 1e3), 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8/fp4 storage; fp16+bf16 MFMA, fp32 accumulation",
        "data": "synthetic (seeded, device-generated)",
        "config": {"workload": "c5: " + w["desc"], "tokens": T, "m": m, "entries": N, "rows": R,
                   "heads": H, "top_k": k, "swa_window": W, "timed": "eager, HIP events per part"},
        "parts_ms": {name: round(t, 4) for (name, _), t in zip(parts, ms)},
        "roofline": {"bound": "mfma", "achieved": round(idx_flops / (ms[1] / 1e3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(idx_flops / (ms[1] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                     "kernel": "indexer (fp16 MFMA scan of every visible key + top-512 per row)",
                     "flops_per_launch": idx_flops},
        "roofline_attn": {"bound": "mfma", "achieved": round(attn_fl / (ms[2] / 1e3) / 1e12, 2),
                          "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                          "frac": round(attn_fl / (ms[2] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                          "kernel": "sparse attention, 4096 rows x 64 heads", "flops_per_launch": attn_fl},
        "roofline_cache_write": {"bound": "hbm", "achieved": round(write_bytes / (ms[0] / 1e3) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(write_bytes / (ms[0] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "bytes_per_launch": write_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        h16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        res["cpu_baseline"] = cpu_baseline_prefill(
            w, h16(x[0]), h16(z[0]), keys[0].cpu().numpy(), q_idx.cpu().numpy(),
            head_w.cpu().numpy().astype(np.float64), h16(q), swa[0].cpu().numpy(), base, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS) + ["c5"])
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sites", action="store_true",
                    help="also print the event-timed average duration of every launch site")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--graph-steps", type=int, default=4,
                    help="steps per replayed graph in the timed region (1: one graph launch per step; "
                         "with more, the same steps with one launch each are timed too and reported)")
    ap.add_argument("--attn-plan", metavar="HPW,NS", default=None,
                    help="pin the attention geometry: heads per workgroup (16 or 64) and key splits")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a copy kernel of this size (for scaling rocprofv3 HBM counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="40-layer step across contexts 4K..1M (workload sched40 or sched40fp4); prints a table")
    ap.add_argument("--probe", choices=["scan", "mfma-valu", "gather"], default=None,
                    help="time one of the library's diagnostic probes and print its table")
    ap.add_argument("--prof-summary", metavar="DIR",
                    help="print markdown summaries of the rocprofv3 CSV output under DIR and exit")
    args = ap.parse_args()
    if args.prof_summary:
        prof_summary(args.prof_summary)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    C.lib()
    if args.probe:
        run_probe(args.probe)
        return
    if args.attn_plan:
        hpw, ns = (int(v) for v in args.attn_plan.split(","))
        C.attn_plan_override(hpw, ns)
        print(f"[bench] attention plan pinned: {hpw} heads per workgroup, {ns} key splits", file=sys.stderr)
    if args.workload == "c5":
        run_prefill(args)
        return
    w = WORKLOADS[args.workload]
    if args.sweep:
        if not w.get("sched"):
            sys.exit("bench.py: --sweep runs the 40-layer schedule (--workload sched40 or sched40fp4)")
        sweep(args, w)
        return
    print(f"[bench] workload {args.workload}: {w['desc']}", file=sys.stderr, flush=True)
    t = time.perf_counter()
    make_set, step_fn = (SchedSet, step_sched) if w.get("sched") else (InputSet, step)
    sets = [make_set(w, i) for i in range(args.sets)]
    torch.cuda.synchronize()
    print(f"[bench] {args.sets} input sets ready in {time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)

    for i in range(max(1, args.warmup)):
        step_fn(w, sets[i % len(sets)])
    torch.cuda.synchronize()

    graphs = None
    if not args.no_graph:
        for s in sets:                 # every set's eager result, the reference for its graph
            step_fn(w, s)
        torch.cuda.synchronize()
        ref = [(s.idx.clone(), s.out.clone()) for s in sets]
        graphs = []
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_fn(w, s)
            graphs.append(g)
        # every replay must reproduce the eager step exactly
        for _ in range(2):
            for g, s, (ri, ro) in zip(graphs, sets, ref):
                g.replay()
                torch.cuda.synchronize()
                if not (torch.equal(s.idx, ri) and torch.equal(s.out, ro)):
                    raise RuntimeError("graph replay differs from the eager step")
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
    # --graph-steps G: the timed region replays graphs that each hold G
    # consecutive steps (over the input sets in turn), as a model step's
    # graph holds the hot path of many layers; G = 1 launches one graph per
    # step.  K steps are floor(K / G) replays of the G-step graph and K mod G
    # replays of single-step graphs.
    gsteps = max(1, args.graph_steps) if graphs else 1
    multi = None
    if gsteps > 1:
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi):
            for j in range(gsteps):
                step_fn(w, sets[j % len(sets)])
        for _ in range(2):
            multi.replay()
        torch.cuda.synchronize()
        for s, (ri, ro) in zip(sets, ref):          # the last step of each set still matches its eager step
            if not (torch.equal(s.idx, ri) and torch.equal(s.out, ro)):
                raise RuntimeError("multi-step graph replay differs from the eager step")

    def timed_steps(g_steps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        if g_steps > 1:
            for i in range(args.steps // g_steps):
                multi.replay()
        for i in range(args.steps % g_steps if g_steps > 1 else args.steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                step_fn(w, sets[i % len(sets)])
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1)

    one_graph = None
    if gsteps > 1:                     # the same K steps, one graph launch each, for reference
        ms1 = timed_steps(1)
        one_graph = {"ms_per_step": round(ms1 / args.steps, 5),
                     "value": round(w["B"] * args.steps / (ms1 / 1e3), 1)}
        print(f"[bench] one graph per step: {ms1 / args.steps * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    ms = timed_steps(gsteps)
    ms_step = ms / args.steps
    qps = w["B"] * args.steps / (ms / 1e3)
    print(f"[bench] timed {args.steps} steps ({gsteps} per graph): {ms_step * 1e3:.1f} us/step, {qps:.0f} queries/s",
          file=sys.stderr, flush=True)

    # the distribution of single steps (a separate pass: an event pair around
    # each step, so the block above stays free of per-step events)
    per = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i, (a0, a1) in enumerate(evs):
        a0.record()
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step_fn(w, sets[i % len(sets)])
        a1.record()
    torch.cuda.synchronize()
    per = np.array([a0.elapsed_time(a1) * 1e3 for a0, a1 in evs])
    step_dist = {"p10": round(float(np.percentile(per, 10)), 2), "median": round(float(np.median(per)), 2),
                 "p90": round(float(np.percentile(per, 90)), 2)}
    print(f"[bench] single steps: median {step_dist['median']} us (p10 {step_dist['p10']}, p90 {step_dist['p90']})",
          file=sys.stderr, flush=True)

    # per-kernel durations from HIP events recorded around one launch site.
    # Eager steps follow a stall kernel on the same stream, so the launches
    # are queued before the GPU reaches them and the events see the kernel,
    # not the host's launch gaps.
    stall_cycles = stall_calibrate(300e-6)

    def time_site(site):
        C.kernel_timer_start(site, args.steps * (len(SCH.csa2_layers()) if w.get("sched") else len(layers_of(w))))
        for i in range(args.steps):
            torch.cuda._sleep(stall_cycles)
            step_fn(w, sets[i % len(sets)])
        n_l, tot_ms = C.kernel_timer_stop()
        return n_l, tot_ms / max(1, n_l) / 1e3

    # dominant kernel: the indexer scan (coarse stage when hierarchical)
    site = "score_coarse" if w["hier"] else "score_flat"
    n_l, avg_s = time_site(site)
    achieved = scan_bytes(w) / avg_s / 1e9
    print(f"[bench] {site}: {n_l} launches, avg {avg_s * 1e6:.2f} us, {achieved:.0f} GB/s algorithmic",
          file=sys.stderr, flush=True)
    # the attention contraction against the bf16 MFMA peak
    n_a, avg_a = time_site("attn")
    attn_tf = attn_flops(w) / avg_a / 1e12
    print(f"[bench] attn: {n_a} launches, avg {avg_a * 1e6:.2f} us, {attn_tf:.1f} TFLOP/s algorithmic",
          file=sys.stderr, flush=True)

    if args.sites:
        for name in C.SITES:
            n_x, avg_x = time_site(name)
            if n_x:
                print(f"[bench] site {name}: {n_x} launches, avg {avg_x * 1e6:.2f} us", file=sys.stderr, flush=True)

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)

    traffic = measured_traffic(args.workload)
    res = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "step_us": step_dist,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8/fp4 storage; fp16+bf16 MFMA, fp32 accumulation",
        "data": "synthetic (seeded, device-generated)",
        "config": {"workload": f"{args.workload}: {w['desc']}", "batch": w["B"],
                   "entries_per_seq": w["N"], "heads": w["H"], "top_k": w["k"],
                   "keep_blocks": w["keep"], "swa_window": 128, "input_sets_rotated": len(sets),
                   "layers": ("40-layer CSA2 schedule" if w.get("sched") else "/".join(layers_of(w))),
                   "timed": (f"graph replays, {gsteps} steps per graph" if graphs else "eager launches")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"index_score_kernel ({site})", "avg_us": round(avg_s * 1e6, 3),
                     "bytes_per_launch": scan_bytes(w)},
        "roofline_attn": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": MFMA_BF16_PEAK_TFS,
                          "unit": "TFLOP/s", "frac": round(attn_tf / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                          "kernel": "sparse attention (launch site attn: the narrow kernel at few rows, the wide one otherwise)", "avg_us": round(avg_a * 1e6, 3),
                          "flops_per_launch": attn_flops(w)},
        "cpu_baseline": None,
    }
    if one_graph is not None:
        res["one_graph_per_step"] = one_graph
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = (cpu_baseline_sched(w, args.cpu_seconds) if w.get("sched")
                               else cpu_baseline(w, sets[0], args.cpu_seconds))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
