#!/usr/bin/env python
"""Throughput of the CSA2 decode hot path on one MI355X.

One step = one decode token for every row of the batch through the whole hot
path: append the token's FP4 entry to the cache (kv_compress_quantize), refresh
the block summary it falls in (index_block_summary), score + select with the
indexer (indexer_topk; hierarchical at 1M context), then the joint sparse +
window attention (sparse_attn_decode).  Inputs are seeded synthetic data,
resident in HBM before the timed region; several independent input sets are
rotated so the working set exceeds the 256 MB Infinity Cache.

The timed region replays one captured HIP graph per input set (the form a
serving loop would run).  (Running the cache append on a second stream,
joined before the attention, was measured slower inside the graph: about
13 us per step more for 3-5 us of overlapped work.)  An equal eager pass afterwards times the dominant
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
            self.k_new = torch.randn((B, 1, 128), generator=g, device="cuda").to(torch.bfloat16)
            self.summ = C.index_block_summary_fp4(self.keys, self.kscales) if w["hier"] else None
        else:
            self.keys = torch.empty((B, N, 128), dtype=torch.uint8, device="cuda")
            for b in range(B):
                self.keys[b] = synth.to_e4m3(torch.randn((N, 128), generator=g, device="cuda"))
            self.kscales = None
            self.summ = C.index_block_summary(self.keys) if w["hier"] else None
        self.swa = synth.to_e4m3(synth.latent_dev((B, 128, 512), g, w["dist"]))
        self.swa_len = torch.full((B,), 128, dtype=torch.int32, device="cuda")
        self.q_idx = synth.to_e4m3(torch.randn((B, 32, 128), generator=g, device="cuda"))
        self.q = torch.randn((B, H, 512), generator=g, device="cuda").to(torch.bfloat16)
        self.x_new = synth.latent_dev((B, m, 512), g, w["dist"]).to(torch.bfloat16)
        self.z_new = torch.randn((B, m, 512), generator=g, device="cuda").to(torch.bfloat16) if m > 1 else None
        # per-layer queries and windows (layer 0 uses the tensors above)
        layers = layers_of(w)
        self.lq, self.lq_idx, self.lswa = [self.q], [self.q_idx], [self.swa]
        for L in range(1, len(layers)):
            self.lq_idx.append(synth.to_e4m3(torch.randn((B, 32, 128), generator=g, device="cuda"))
                               if layers[L] == "reindex" else None)
            self.lq.append(torch.randn((B, H, 512), generator=g, device="cuda").to(torch.bfloat16))
            self.lswa.append(synth.to_e4m3(synth.latent_dev((B, 128, 512), g, w["dist"])))
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
    N = w["N"]
    # a0: the newest entry (m tokens pooled; m = 1 in the decoder layers)
    C.kv_compress_quantize(s.x_new, w["m"], gate=s.z_new, codes=s.codes[:, N - 1:],
                           scales=s.scales[:, N - 1:], out_seq_stride=N)
    if s.fp4:                  # ... and its index key, quantized to FP4
        C.index_key_quantize(s.k_new, codes=s.keys[:, N - 1:], scales=s.kscales[:, N - 1:], out_seq_stride=N)
    # a1: refresh the summary of the block holding that entry
    if w["hier"]:
        b = (N - 1) // 8
        if s.fp4:
            C.index_block_summary_fp4(s.keys, s.kscales, summ=s.summ, blk_begin=b, blk_end=b + 1)
        else:
            C.index_block_summary(s.keys, summ=s.summ, blk_begin=b, blk_end=b + 1)
    idx = None
    for L, mode in enumerate(layers_of(w)):
        # a2-a3: indexer scores + top-k (coarse-to-fine at 1M context); a7:
        # Reuse layers keep the selection, Reindex layers select anew (within
        # the Full layer's pool when the workload says so)
        if mode == "full":
            C.indexer_topk(s.lq_idx[L], s.keys, w["k"], block_keys=s.summ, keep_blocks=w["keep"] or 2048,
                           out_idx=s.idx, out_blocks=s.blocks, workspace=s.ws_idx, key_scales=s.kscales)
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
    B, N = w["B"], w["N"]
    rows = (N + 7) // 8 if w["hier"] else N
    row_bytes = 68 if (w.get("key") == "fp4" and not w["hier"]) else 128
    return B * (rows * row_bytes + 32 * 128 + 32 * 4)


def attn_flops(w):
    """Algorithmic flops of one attention launch: QK^T and PV over the
    selected entries and the window, 2 * 2 * H * (k + 128) * 512 per query."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a copy kernel of this size (for scaling rocprofv3 HBM counters)")
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
    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    C.lib()
    print(f"[bench] workload {args.workload}: {w['desc']}", file=sys.stderr, flush=True)
    t = time.perf_counter()
    sets = [InputSet(w, i) for i in range(args.sets)]
    torch.cuda.synchronize()
    print(f"[bench] {args.sets} input sets ready in {time.perf_counter() - t:.1f} s", file=sys.stderr, flush=True)

    for i in range(max(1, args.warmup)):
        step(w, sets[i % len(sets)])
    torch.cuda.synchronize()

    graphs = None
    if not args.no_graph:
        for s in sets:                 # every set's eager result, the reference for its graph
            step(w, s)
        torch.cuda.synchronize()
        ref = [(s.idx.clone(), s.out.clone()) for s in sets]
        graphs = []
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(w, s)
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

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(w, sets[i % len(sets)])
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    qps = w["B"] * args.steps / (ms / 1e3)
    print(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.1f} us/step, {qps:.0f} queries/s",
          file=sys.stderr, flush=True)

    # per-kernel durations from HIP events recorded around one launch site.
    # Eager steps follow a stall kernel on the same stream, so the launches
    # are queued before the GPU reaches them and the events see the kernel,
    # not the host's launch gaps.
    stall_cycles = stall_calibrate(300e-6)

    def time_site(site):
        C.kernel_timer_start(site, args.steps * len(layers_of(w)))
        for i in range(args.steps):
            torch.cuda._sleep(stall_cycles)
            step(w, sets[i % len(sets)])
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

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)

    traffic = measured_traffic(args.workload)
    res = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8/fp4 storage; fp16+bf16 MFMA, fp32 accumulation",
        "data": "synthetic (seeded, device-generated)",
        "config": {"workload": f"{args.workload}: {w['desc']}", "batch": w["B"],
                   "entries_per_seq": w["N"], "heads": w["H"], "top_k": w["k"],
                   "keep_blocks": w["keep"], "swa_window": 128, "input_sets_rotated": len(sets),
                   "layers": "/".join(layers_of(w)),
                   "timed": "graph replays" if graphs else "eager launches"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"index_score_kernel ({site})", "avg_us": round(avg_s * 1e6, 3),
                     "bytes_per_launch": scan_bytes(w)},
        "roofline_attn": {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": MFMA_BF16_PEAK_TFS,
                          "unit": "TFLOP/s", "frac": round(attn_tf / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                          "kernel": "sparse_attn_kernel", "avg_us": round(avg_a * 1e6, 3),
                          "flops_per_launch": attn_flops(w)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, sets[0], args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
