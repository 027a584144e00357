#!/usr/bin/env python3
"""Decode-step benchmark of the fused exponent-coded KV attention on one MI355X.

Workload: a Qwen3-8B-shaped decode step at 8192-token context - 36 layers, batch 16, 32 query /
8 KV heads, head_dim 128, 16-token pages; per sequence 511 compressed pages plus the 16-token BF16
tail page (the page that completes in this step).  Seeded synthetic KV: per-channel scale 2^u,
u ~ U[-5, 5], 5% of blocks with a forced out-of-window element; queries ~ N(0, 1).

One step = the whole hot path once: fused decode attention for all 36 layers (each layer reads
its own buffers, so no layer is served from cache), then page completion - the tail page of every
(layer, sequence, KV head, K|V) is encoded into the slot pool - then those runs are freed again so
every step sees the same pool state.  The step is replayed from HIP graphs.

Printed (one JSON line): effective BF16-equivalent KV GB/s of the whole step (value), ms per step,
the roofline of the attention call (algorithmic bytes per layer launch / its mean duration from
HIP events on the launch stream; HBM traffic from the committed counter summary), the
uncompressed BF16 baseline timed in the same run, a labelled variant with compressible data
(u ~ U[-3, 3], 8 layers), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step + effective KV GB/s (fraction of HBM peak) at 8K ctx"
HBM_PEAK_GBPS = 8000.0

B, HQ, HKV, LAYERS, CTX = 16, 32, 8, 36, 8192
N_COMP = 511
TAIL = 16
U_MAX = 5.0
FORCED = 0.05
SEED = 2
VARIANT_LAYERS, VARIANT_U_MAX = 8, 3.0
# The other workload shapes, timed as labelled extras (not the headline): name, batch, query
# heads, KV heads, compressed pages per sequence (no tail page), distinct layers, u_max, forced
# fraction, seed, stress values.
OTHER_CONFIGS = [
    ("llama2k", 32, 32, 8, 128, 32, 3.0, 0.05, 1, False),
    ("single131k", 1, 32, 8, 8192, 4, 3.0, 0.10, 4, True),
    # a ragged batch: one 32K-token sequence among 15 of 2K tokens (automatic split count 2, so
    # the long sequence's many pieces are merged inside the attention kernel)
    ("ragged32k", 16, 32, 8, [2048] + [128] * 15, 8, 3.0, 0.05, 5, False),
]
BREAKDOWN_LAYERS = 8
GAAC_LAYERS = 8
FP8_LAYERS = 8
N_PHYS = B * N_COMP
SCALE = 1.0 / math.sqrt(128.0)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_qwen8k_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_kvz_amd", "csrc", f)
                  for f in ("attention.hip", "kvz_internal.h", "gaac_internal.h", "fp8_internal.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def exponent_entropy(pages) -> dict:
    """Shannon entropy in bits of the BF16 exponent field (bits 14..7) over the K values, the V
    values and both, of pages [..., 2, Hkv, 16, 128] (the measure of the GAAC page, "Compression
    Effectiveness and Generality", and the ExANS page, "Entropy and effective alphabet size")."""
    import torch
    e = (pages.contiguous().view(torch.int16).to(torch.int32) >> 7) & 0xFF
    res = {}
    for name, sel in (("k", e.select(-4, 0)), ("v", e.select(-4, 1)), ("kv", e)):
        c = torch.bincount(sel.reshape(-1), minlength=256).double()
        pr = c[c > 0] / c.sum()
        res[name] = round(float(-(pr * torch.log2(pr)).sum()), 3)
    return res


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def alg_bytes_per_layer(record_bytes: float) -> float:
    """Bytes one attention launch must move: every group record + 16 B metadata per (page, KV
    head) + 4 B block-table entry per page + tail + q + out."""
    return (record_bytes + N_PHYS * HKV * 16 + N_PHYS * 4 + B * 2 * HKV * 16 * 128 * 2
            + B * HQ * 128 * 2 + B * HQ * 128 * 4)


def baseline_bytes_per_layer() -> float:
    return (N_PHYS * HKV * 4096 * 2 + N_PHYS * 4 + B * 2 * HKV * 16 * 128 * 2
            + B * HQ * 128 * 2 + B * HQ * 128 * 4)


def build_layers(arena, n_layers, u_max, seed, with_baseline, dev, encode_us=None, entropy=None):
    """Encode n_layers layers of the workload into `arena` (the prompt's pages, in bulk); return
    per-layer device buffers.  encode_us, if a list, receives each layer's kvz_encode_pages time
    (HIP events around the call; item records already on the device); entropy, if a dict,
    receives the exponent entropy of layer 0's pages."""
    import torch
    from decode_attention_kvz_amd import kvz, paged, synth
    rng = np.random.default_rng(seed)
    layers = []
    t0 = time.time()
    for layer in range(n_layers):
        pages = synth.kv_pages(B, N_COMP + 1, HKV, seed=seed, layer=layer, u_max=u_max,
                               forced_frac=FORCED, device=dev)
        if entropy is not None and layer == 0:
            entropy.update(exponent_entropy(pages))
        block_table = rng.permutation(N_PHYS).reshape(B, N_COMP).astype(np.int32)
        meta = paged.new_meta_table(N_PHYS, HKV, device=dev)
        items = paged.page_items(pages, [(b, p) for b in range(B) for p in range(N_COMP)], meta,
                                 block_table.reshape(-1))
        d_items = torch.from_numpy(np.ascontiguousarray(items)).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvz.kvz_encode_pages(arena.pool, d_items, N_PHYS * HKV * 2, 0)
        e1.record()
        store = None
        if with_baseline:
            inv = torch.as_tensor(np.argsort(block_table.reshape(-1)), device=dev)
            store = paged.pack_bf16_pages(pages[:, :N_COMP].reshape(N_PHYS, 2, HKV, 16, 128)[inv])
        layers.append(dict(meta=meta, block_table=torch.from_numpy(block_table).to(dev),
                           tail=pages[:, N_COMP].contiguous(), store=store,
                           q=synth.queries(B, HQ, seed=seed * 1000 + layer, device=dev),
                           out=torch.empty((B, HQ, 128), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        if encode_us is not None:
            encode_us.append(e0.elapsed_time(e1) * 1e3)
        del d_items, pages
        if layer % 6 == 5 or layer == n_layers - 1:
            log(f"setup: {layer + 1}/{n_layers} layers encoded (u_max {u_max}, "
                f"{time.time() - t0:.1f}s)")
    return layers


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--layers", type=int, default=LAYERS,
                    help="layers per step (the workload has 36; fewer is for quick checks only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-all-cores", action="store_true",
                    help=argparse.SUPPRESS)   # the child process of the all-cores oracle timing
    ap.add_argument("--no-baseline", action="store_true")
    ap.add_argument("--no-variant", action="store_true")
    ap.add_argument("--no-gaac", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-online", action="store_true",
                    help="skip the online page-completion leg (64 sequences, 32 layers)")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other workload shapes (2K batch of 32, one 131K sequence)")
    ap.add_argument("--breakdown", action="store_true",
                    help="only the attention time breakdown (loads / restore / computation, and "
                         "the BF16 and decompress-first pipelines) at the 8K and 2K shapes")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for hardware-counter runs: one layer of fused and baseline attention "
                         "(3 launches each) and a 1 GiB device copy as a traffic reference")
    ap.add_argument("--pmc-shape", default="qwen8k", choices=["qwen8k", "llama2k", "single131k"],
                    help="the layer shape of --pmc-probe (qwen8k: the workload, with the other "
                         "formats; llama2k, single131k: the other shapes, fused and BF16 only)")
    args = ap.parse_args()
    if args.cpu_all_cores:        # child process: host only, never touches the GPU
        print(json.dumps(cpu_all_cores()), flush=True)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (its (sequence, "
              "KV head) units are independent, so a multi-GPU version would place KV heads, or "
              "page ranges of long sequences, on different GPUs).", file=sys.stderr)
        sys.exit(2)

    # the all-cores oracle timing runs in a child process started now, before this process
    # touches the GPU; it waits for a line on its stdin before working
    all_cores_child = None
    if not args.no_cpu_baseline and not args.pmc_probe:
        import subprocess
        all_cores_child = subprocess.Popen(
            [sys.executable, "-u", os.path.abspath(__file__), "--cpu-all-cores"],
            stdin=subprocess.PIPE, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)

    import torch
    from decode_attention_kvz_amd import kvz, paged

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvz.kvz_device_check(0)
    if args.pmc_probe:
        if args.pmc_shape == "qwen8k":
            pmc_probe(args, dev)
        else:
            pmc_probe_other(args, dev, next(c for c in OTHER_CONFIGS if c[0] == args.pmc_shape))
        return
    if args.breakdown:
        print(json.dumps({"breakdown": breakdown(args, dev)}), flush=True)
        return
    n_layers = args.layers

    # ---------------- setup --------------------------------------------------------------
    arena = paged.SlotArena(n_layers * (N_PHYS + B) * HKV * 2 * 4096 + (16 << 20), device=dev)
    enc_layer_us = []
    entropy = {}
    layers = build_layers(arena, n_layers, U_MAX, SEED, not args.no_baseline, dev, enc_layer_us,
                          entropy)
    seq_lens = torch.full((B,), CTX, dtype=torch.int32, device=dev)
    n_comp = torch.full((B,), N_COMP, dtype=torch.int32, device=dev)
    ws = paged.workspace(B, HQ, HKV, N_COMP, args.splits, device=dev)

    # page completion: the tail page of every (layer, sequence, KV head, K|V) this step
    comp_meta = paged.new_meta_table(n_layers * B, HKV, device=dev)
    src, dst, kinds = [], [], []
    for layer, L in enumerate(layers):
        t = L["tail"]
        for b in range(B):
            for h in range(HKV):
                for kind in range(2):
                    src.append(t.data_ptr() + (((b * 2 + kind) * HKV + h) * 2048) * 2)
                    dst.append(comp_meta.data_ptr() + (((layer * B + b) * HKV + h) * 2 + kind) * 8)
                    kinds.append(kind)
    n_comp_items = len(src)
    comp_items = torch.from_numpy(kvz.encode_items(src, dst, 128, kinds)).to(dev)
    comp_ptrs = torch.from_numpy(np.asarray(dst, dtype=np.int64)).to(dev)

    stats = arena.stats()
    rec_bytes = stats["live_granules"] * 256 / n_layers
    raw_frac = stats["live_raw_blocks"] / (stats["live_runs"] * 4)
    bf16_kv_layer = B * CTX * HKV * 128 * 2 * 2
    alg_bytes = alg_bytes_per_layer(rec_bytes)
    log(f"raw block fraction {raw_frac:.3f}, records {rec_bytes / 1e6:.1f} MB/layer vs BF16 "
        f"{N_PHYS * HKV * 4096 * 2 / 1e6:.1f} MB")

    def attention(L, fused=True):
        if fused:
            kvz.kvz_decode_attention(L["q"], L["out"], arena.arena, L["meta"], L["block_table"],
                                     seq_lens, n_comp, L["tail"], SCALE, ws, args.splits)
        else:
            kvz.kvz_bf16_decode_attention(L["q"], L["out"], L["store"], L["block_table"], seq_lens,
                                          n_comp, L["tail"], SCALE, ws, HKV, args.splits)

    def complete_pages():
        # one launch: free the records the previous step stored (steady state), encode this
        # step's completed pages into them
        kvz.kvz_complete_pages(arena.pool, comp_ptrs, comp_items, n_comp_items)

    def capture(fn):
        """Eager warm-up calls, then a HIP graph of fn (host launch overhead cannot starve the
        GPU between layers when the step is replayed)."""
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    g_attn = capture(lambda: [attention(L) for L in layers])
    eager_out = layers[-1]["out"].clone()

    def step_body():
        for L in layers:
            attention(L)
        complete_pages()
    # the whole decode step (36 attention calls, then the page completion) as one graph, as an
    # engine would capture its step; g_attn (and the completion below) time the parts on their own
    g_step = capture(step_body)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        """Mean ms per call from HIP events on the launch stream around `reps` calls."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def whole_step():
        g_step.replay()

    for _ in range(args.warmup):
        whole_step()
    torch.cuda.synchronize()
    assert torch.equal(layers[-1]["out"], eager_out), "graph replay differs from the eager call"
    t0 = time.perf_counter()
    for _ in range(args.steps):
        whole_step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the attention call alone (attention kernel + split merge), per layer, per step
    attn_ms = np.asarray([timed(g_attn.replay, 1) / n_layers for _ in range(args.steps)])
    us_layer = float(np.median(attn_ms)) * 1e3
    us_layer_mean = float(np.mean(attn_ms)) * 1e3
    # the same samples as 5 consecutive runs: median us/step of each, then their mean and sd
    run_medians = [float(np.median(c)) * 1e3 * n_layers for c in np.array_split(attn_ms, 5) if len(c)]
    achieved = alg_bytes / (us_layer_mean * 1e-6) / 1e9
    # the completion on its own: eight steady-state calls per graph (each frees the records the
    # previous one stored and encodes the same pages again), as inside the step's graph; a graph
    # of one call would add a graph launch to every call
    enc_us = graph_us_per_layer(lambda: [complete_pages() for _ in range(8)], 8, args)
    log(f"fused: {ms_step:.3f} ms/step, attention {us_layer:.1f} us/layer (median), "
        f"{achieved:.0f} GB/s algorithmic; encode+free {enc_us:.1f} us/step")

    baseline = None
    if not args.no_baseline:
        g_base = capture(lambda: [attention(L, fused=False) for L in layers])
        b_ms = np.asarray([timed(g_base.replay, 1) / n_layers for _ in range(args.steps)])
        b_us, b_mean = float(np.median(b_ms)) * 1e3, float(np.mean(b_ms)) * 1e3
        b_gbps = baseline_bytes_per_layer() / (b_mean * 1e-6) / 1e9
        baseline = {"us_per_layer": round(b_us, 2), "us_per_step_attention": round(b_mean * n_layers, 1),
                    "achieved_GBps": round(b_gbps, 1), "hbm_frac": round(b_gbps / HBM_PEAK_GBPS, 4)}
        log(f"bf16 baseline: {b_us:.1f} us/layer, {b_gbps:.0f} GB/s")
        del g_base

    for L in layers:
        L.pop("store", None)          # the baseline's stores are no longer needed
    dfirst = decompress_first(args, arena, layers, seq_lens, n_comp, ws, N_PHYS, HKV)
    traffic = committed_traffic()
    read_peak = stream_read_peak(timed)
    variant = None if args.no_variant else compressible_variant(args, dev, seq_lens, n_comp, ws)
    others = None if args.no_other else {c[0]: other_config(args, dev, *c) for c in OTHER_CONFIGS}
    online = None if args.no_online else online_completion(args, dev)
    gaac_leg = None if args.no_gaac else gaac_format(args, dev, seq_lens, n_comp, ws)
    fp8_leg = None if args.no_fp8 else {name: fp8_format(args, dev, seq_lens, n_comp, ws, fmt)
                                        for name, fmt in (("e4m3", 0), ("e5m2", 1))}
    del g_attn, g_step
    bdown = None if args.no_breakdown else breakdown(args, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(layers, all_cores_child)

    value = bf16_kv_layer * n_layers / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; per-channel scale 2^U[-5,5], 5% forced-raw blocks)",
        "config": {"workload": "qwen3-8b-shaped decode step at 8192-token context",
                   "layers": n_layers, "batch": B, "q_heads": HQ, "kv_heads": HKV,
                   "head_dim": 128, "page_tokens": 16, "context": CTX,
                   "compressed_pages": N_COMP, "tail_tokens": TAIL,
                   "splits": args.splits or "auto", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "measured_read_peak": read_peak["GBps"],
                     "frac_of_measured_read_peak": round(achieved / read_peak["GBps"], 4)},
        "cpu_baseline": cpu,
        "attention_us_per_layer": round(us_layer, 2),
        "attention_us_per_step": round(us_layer_mean * n_layers, 1),
        "attention_us_per_step_runs": {"medians": [round(x, 1) for x in run_medians],
                                       "mean": round(float(np.mean(run_medians)), 1),
                                       "sd": round(float(np.std(run_medians, ddof=1)), 1)
                                       if len(run_medians) > 1 else 0.0},
        "stream_read_reference": read_peak,
        "algorithmic_bytes_per_launch": int(alg_bytes),
        "encode_free_us_per_step": round(enc_us, 1),
        "effective_attention_GBps": round(bf16_kv_layer / (us_layer_mean * 1e-6) / 1e9, 1),
        "raw_block_fraction": round(raw_frac, 4),
        "exponent_entropy_bits": entropy,
        "record_bytes_per_layer": int(rec_bytes),
        "bf16_kv_bytes_per_layer": int(bf16_kv_layer),
        "baseline_bf16": baseline,
        "speedup_vs_bf16_kernel": (round(baseline["us_per_layer"] / us_layer, 4) if baseline else None),
        "decompress_first": dfirst,
        "fused_speedup_vs_decompress_first": round(dfirst["us_per_layer"] / us_layer, 3),
        "prefill_encode": {"groups_per_layer": N_PHYS * HKV * 2,
                           "us_per_layer_median": round(float(np.median(enc_layer_us)), 1),
                           "input_GBps": round(N_PHYS * HKV * 2 * 4096 /
                                               (float(np.median(enc_layer_us)) * 1e-6) / 1e9, 1)},
        "compressible_variant": variant,
        "other_configs": others,
        "online_completion": online,
        "gaac_format": gaac_leg,
        "fp8_formats": fp8_leg,
        "breakdown": bdown,
    }
    print(json.dumps(line), flush=True)
    arena.close()


def stream_read_peak(timed):
    """Practical HBM read ceiling on this device: the library's streaming-read reference kernel
    (16-byte non-temporal loads, as the page loads) over a 4 GiB buffer, best of a sweep of
    workgroup counts."""
    import torch
    from decode_attention_kvz_amd import kvz
    buf = torch.ones(1 << 32, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    best, best_wg, sweep = 0.0, 0, {}
    for per_cu in (1, 2, 4, 8, 16):
        wg = per_cu * n_cu
        kvz.kvz_stream_read(buf, sink, wg)
        ms = timed(lambda: kvz.kvz_stream_read(buf, sink, wg), 10)
        gbps = buf.numel() / (ms * 1e-3) / 1e9
        sweep[str(per_cu)] = round(gbps, 1)
        if gbps > best:
            best, best_wg = gbps, per_cu
    del buf
    log(f"stream read reference: {best:.0f} GB/s ({best_wg} workgroups per CU)")
    return {"GBps": round(best, 1), "bytes": 1 << 32, "workgroups_per_cu": best_wg,
            "sweep_GBps_by_workgroups_per_cu": sweep}


def build_gaac_layers(arena, n_layers, dev, encode_us=None):
    """Layers of the headline workload (u~U[-5,5], 5% forced) in the group-adaptive format, each
    with bases calibrated on another sample of the same layer; plus the BF16 page store.  The
    bulk encode of each layer is timed into encode_us (events around the call, item records
    already on the device)."""
    import torch
    from decode_attention_kvz_amd import kvz, paged, synth
    rng = np.random.default_rng(SEED)
    layers = []
    for layer in range(n_layers):
        cal = synth.kv_pages(4, 32, HKV, seed=SEED, layer=layer, u_max=U_MAX, forced_frac=FORCED,
                             sample=1, device=dev)
        bases = paged.gaac_calibrate(cal)
        del cal
        pages = synth.kv_pages(B, N_COMP + 1, HKV, seed=SEED, layer=layer, u_max=U_MAX,
                               forced_frac=FORCED, device=dev)
        block_table = rng.permutation(N_PHYS).reshape(B, N_COMP).astype(np.int32)
        meta = paged.new_meta_table(N_PHYS, HKV, device=dev)
        items = paged.gaac_page_items(pages, [(b, p) for b in range(B) for p in range(N_COMP)],
                                      meta, block_table.reshape(-1), bases)
        d_items = torch.from_numpy(np.ascontiguousarray(items)).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvz.kvz_gaac_encode_pages(arena.pool, d_items, items.size // kvz.GAAC_ITEM_DTYPE.itemsize)
        e1.record()
        inv = torch.as_tensor(np.argsort(block_table.reshape(-1)), device=dev)
        store = paged.pack_bf16_pages(pages[:, :N_COMP].reshape(N_PHYS, 2, HKV, 16, 128)[inv])
        layers.append(dict(meta=meta, bases=bases, store=store,
                           block_table=torch.from_numpy(block_table).to(dev),
                           tail=pages[:, N_COMP].contiguous(),
                           q=synth.queries(B, HQ, seed=SEED * 1000 + layer, device=dev),
                           out=torch.empty((B, HQ, 128), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        if encode_us is not None:
            encode_us.append(e0.elapsed_time(e1) * 1e3)
        del d_items, pages
    return layers


def gaac_format(args, dev, seq_lens, n_comp, ws):
    """The second page format (group-adaptive additive code) on the headline workload's shape
    and data model (u~U[-5,5], 5% forced), 8 layers, each with bases calibrated on another
    sample of the same layer: fused attention vs the uncompressed kernel and vs
    decompress-first, and the storage ratio."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    arena = paged.SlotArena(GAAC_LAYERS * (N_PHYS + B) * HKV * 2 * 4096 + (16 << 20), device=dev)
    enc_us = []
    layers = build_gaac_layers(arena, GAAC_LAYERS, dev, enc_us)
    st = arena.stats()
    rec = st["live_granules"] * 256 / GAAC_LAYERS
    raw_tiles = st["live_raw_blocks"] / 4 / st["live_runs"]
    res = {}
    for mode in ("gaac", "bf16"):
        def run():
            for L in layers:
                if mode == "gaac":
                    kvz.kvz_gaac_decode_attention(L["q"], L["out"], arena.arena, L["meta"], L["bases"],
                                                  L["block_table"], seq_lens, n_comp, L["tail"],
                                                  SCALE, ws, args.splits)
                else:
                    kvz.kvz_bf16_decode_attention(L["q"], L["out"], L["store"], L["block_table"],
                                                  seq_lens, n_comp, L["tail"], SCALE, ws, HKV,
                                                  args.splits)
        res[mode] = graph_us_per_layer(run, GAAC_LAYERS, args)
    # same split count -> the same arithmetic on the same values: bit-identical outputs
    L = layers[-1]
    same = [torch.empty_like(L["out"]) for _ in range(2)]
    ws16 = paged.workspace(B, HQ, HKV, N_COMP, 16, device=dev)
    kvz.kvz_gaac_decode_attention(L["q"], same[0], arena.arena, L["meta"], L["bases"],
                                  L["block_table"], seq_lens, n_comp, L["tail"], SCALE, ws16, 16)
    kvz.kvz_bf16_decode_attention(L["q"], same[1], L["store"], L["block_table"], seq_lens, n_comp,
                                  L["tail"], SCALE, ws16, HKV, 16)
    torch.cuda.synchronize()
    assert torch.equal(same[0], same[1]), "GAAC attention differs from the BF16 kernel"
    for L in layers:
        del L["store"]
    scratch = torch.empty((N_PHYS, 2, HKV, 4, 1024), dtype=torch.uint8, device=dev)

    def dfirst():
        for L in layers:
            paged.gaac_decompress_pages(arena, L["meta"], L["bases"], scratch)
            kvz.kvz_bf16_decode_attention(L["q"], L["out"], scratch, L["block_table"], seq_lens,
                                          n_comp, L["tail"], SCALE, ws, HKV, args.splits)
    dfirst_us = graph_us_per_layer(dfirst, GAAC_LAYERS, args)
    arena.close()
    alg = alg_bytes_per_layer(rec) + HKV * 512      # + the layer's bases
    out = {"label": "group-adaptive additive code (second format), headline shape and data model, "
                    "8 layers, per-layer bases calibrated on another sample of the layer",
           "record_bytes_per_layer": int(rec),
           "storage_ratio_vs_bf16": round(N_PHYS * HKV * 2 * 4096 / rec, 4),
           "raw_tile_fraction": round(raw_tiles, 4),
           "fused_us_per_layer": round(res["gaac"], 2),
           "fused_achieved_GBps": round(alg / (res["gaac"] * 1e-6) / 1e9, 1),
           "bf16_us_per_layer": round(res["bf16"], 2),
           "speedup_vs_bf16_kernel": round(res["bf16"] / res["gaac"], 4),
           "prefill_encode_us_per_layer": round(float(np.median(enc_us)), 1),
           "decompress_first_us_per_layer": round(dfirst_us, 2)}
    log(f"gaac format: fused {res['gaac']:.1f} us/layer vs bf16 {res['bf16']:.1f} "
        f"(storage ratio {out['storage_ratio_vs_bf16']}, raw tiles {raw_tiles:.4f}); "
        f"bulk encode {out['prefill_encode_us_per_layer']:.1f} us/layer")
    return out


def build_fp8_layers(arena, n_layers, dev, fmt, encode_us=None):
    """Layers of the headline shape in FP8 (fmt 0 = E4M3, 1 = E5M2) for the FP8 tiles: KV from the
    BF16 data model with u~U[-3,3] and 5% forced blocks converted to FP8, bases calibrated on
    another sample of the layer; plus the uncompressed FP8 page store.  The bulk encode of each
    layer is timed into encode_us (events around the call, item records on the device)."""
    import torch
    from decode_attention_kvz_amd import kvz, paged, synth
    rng = np.random.default_rng(SEED + 7)
    layers = []
    for layer in range(n_layers):
        cal = synth.fp8_kv_pages(4, 32, HKV, seed=SEED, fmt=fmt, layer=layer, u_max=3.0,
                                 forced_frac=FORCED, sample=1, device=dev)
        bases = paged.fp8_calibrate(cal, fmt)
        del cal
        pages = synth.fp8_kv_pages(B, N_COMP + 1, HKV, seed=SEED, fmt=fmt, layer=layer, u_max=3.0,
                                   forced_frac=FORCED, device=dev)
        block_table = rng.permutation(N_PHYS).reshape(B, N_COMP).astype(np.int32)
        meta = paged.new_meta_table(N_PHYS, HKV, device=dev)
        items = paged.fp8_page_items(pages, [(b, p) for b in range(B) for p in range(N_COMP)],
                                     meta, block_table.reshape(-1), bases)
        d_items = torch.from_numpy(np.ascontiguousarray(items)).to(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvz.kvz_fp8_encode_pages(arena.pool, d_items, items.size // kvz.FP8_ITEM_DTYPE.itemsize, fmt)
        e1.record()
        inv = torch.as_tensor(np.argsort(block_table.reshape(-1)), device=dev)
        store = paged.pack_fp8_pages(pages[:, :N_COMP].reshape(N_PHYS, 2, HKV, 16, 128)[inv])
        layers.append(dict(meta=meta, bases=bases, store=store,
                           block_table=torch.from_numpy(block_table).to(dev),
                           tail=pages[:, N_COMP].contiguous(),
                           q=synth.queries(B, HQ, seed=SEED * 1000 + layer, device=dev),
                           out=torch.empty((B, HQ, 128), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        if encode_us is not None:
            encode_us.append(e0.elapsed_time(e1) * 1e3)
        del d_items, pages
    return layers


def fp8_format(args, dev, seq_lens, n_comp, ws, fmt):
    """The third page format (the exponent code on FP8 KV) on the headline shape, 8 layers: KV
    from the BF16 data model with u~U[-3,3] (so every value lies inside E4M3's range) and 5%
    forced blocks, converted to FP8; bases per layer calibrated on another sample of the layer.
    Fused attention over the coded tiles vs the uncompressed FP8 kernel (checked bit-identical at
    equal split counts) vs decompress-first, and the storage ratios."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    name = ("e4m3", "e5m2")[fmt]
    arena = paged.SlotArena(FP8_LAYERS * (N_PHYS + B) * HKV * 2 * 2048 + (16 << 20), device=dev,
                            fp8=True)
    enc_us = []
    layers = build_fp8_layers(arena, FP8_LAYERS, dev, fmt, enc_us)
    st = arena.stats()
    rec = st["live_granules"] * 128 / FP8_LAYERS
    # a compressed tile takes 15 (E4M3) or 13 (E5M2) granules of 128 bytes, an uncompressed 16
    comp_gran = 15 if fmt == 0 else 13
    raw_tiles = (st["live_granules"] - comp_gran * st["live_runs"]) / (16 - comp_gran) / st["live_runs"]

    ws16 = paged.workspace(B, HQ, HKV, N_COMP, 16, device=dev)

    def call(L, fused, out, splits):
        w = ws16 if splits == 16 else ws
        if fused:
            kvz.kvz_fp8_decode_attention(L["q"], out, fmt, arena.arena, L["meta"], L["bases"],
                                         L["block_table"], seq_lens, n_comp, L["tail"], SCALE,
                                         1.0, 1.0, w, splits)
        else:
            kvz.kvz_fp8_raw_decode_attention(L["q"], out, fmt, L["store"], L["block_table"],
                                             seq_lens, n_comp, L["tail"], SCALE, 1.0, 1.0, w,
                                             HKV, splits)
    res = {}
    for mode in ("fused", "fp8"):
        res[mode] = graph_us_per_layer(
            lambda: [call(L, mode == "fused", L["out"], args.splits) for L in layers],
            FP8_LAYERS, args)
    L = layers[-1]
    same = [torch.empty_like(L["out"]) for _ in range(2)]
    call(L, True, same[0], 16)
    call(L, False, same[1], 16)
    torch.cuda.synchronize()
    assert torch.equal(same[0], same[1]), "FP8 fused attention differs from the FP8 kernel"
    for L in layers:
        del L["store"]
    scratch = torch.empty((N_PHYS, 2, HKV, 2048), dtype=torch.uint8, device=dev)

    def dfirst():
        for L in layers:
            paged.fp8_decompress_pages(arena, L["meta"], L["bases"], fmt, scratch)
            kvz.kvz_fp8_raw_decode_attention(L["q"], L["out"], fmt, scratch, L["block_table"],
                                             seq_lens, n_comp, L["tail"], SCALE, 1.0, 1.0, ws,
                                             HKV, args.splits)
    dfirst_us = graph_us_per_layer(dfirst, FP8_LAYERS, args)
    arena.close()
    small = N_PHYS * 4 + B * 2 * HKV * 16 * 128 + B * HQ * 128 * 2 + B * HQ * 128 * 4
    alg = rec + N_PHYS * HKV * 16 + HKV * 512 + small
    alg_fp8 = N_PHYS * HKV * 2 * 2048 + small
    fp8_bytes = N_PHYS * HKV * 2 * 2048
    out = {"label": f"exponent code on FP8 {name.upper()} KV (third format), headline shape, KV "
                    "data model u~U[-3,3] with 5% forced blocks converted to FP8, 8 layers, "
                    "per-layer bases calibrated on another sample of the layer",
           "record_bytes_per_layer": int(rec),
           "storage_ratio_vs_fp8": round(fp8_bytes / rec, 4),
           "storage_ratio_vs_bf16": round(2 * fp8_bytes / rec, 4),
           "raw_tile_fraction": round(raw_tiles, 4),
           "fused_us_per_layer": round(res["fused"], 2),
           "prefill_encode_us_per_layer": round(float(np.median(enc_us)), 1),
           "fused_achieved_GBps": round(alg / (res["fused"] * 1e-6) / 1e9, 1),
           "fp8_kernel_us_per_layer": round(res["fp8"], 2),
           "fp8_kernel_achieved_GBps": round(alg_fp8 / (res["fp8"] * 1e-6) / 1e9, 1),
           "speedup_vs_fp8_kernel": round(res["fp8"] / res["fused"], 4),
           "decompress_first_us_per_layer": round(dfirst_us, 2)}
    log(f"fp8 {name}: fused {res['fused']:.1f} us/layer vs fp8 kernel {res['fp8']:.1f} "
        f"(storage ratio vs FP8 {out['storage_ratio_vs_fp8']}, raw tiles {raw_tiles:.4f}); "
        f"bulk encode {out['prefill_encode_us_per_layer']:.1f} us/layer")
    return out


def graph_us_per_layer(run, n_layers, args):
    """Warm up `run` (a pass over n_layers layers), capture it in a HIP graph and return the
    median over replays of the event time per layer (us)."""
    import torch
    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(max(args.steps // 5, 3)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / n_layers)
    del g
    return float(np.median(ts))


def decompress_first(args, arena, layers, seq_lens, n_comp, ws, n_phys, hkv):
    """The pipeline fused attention replaces: per layer, decompress every page of the layer into
    one reused uncompressed store (kvz_decompress_pages), then the uncompressed attention over
    it.  Also times the decompression alone."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    scratch = torch.empty((n_phys, 2, hkv, 4, 1024), dtype=torch.uint8, device="cuda")

    def both():
        for L in layers:
            paged.decompress_pages(arena, L["meta"], scratch)
            kvz.kvz_bf16_decode_attention(L["q"], L["out"], scratch, L["block_table"], seq_lens,
                                          n_comp, L.get("tail"), SCALE, ws, hkv, args.splits)

    def decomp_only():
        for L in layers:
            paged.decompress_pages(arena, L["meta"], scratch)

    n = len(layers)
    total = graph_us_per_layer(both, n, args)
    dec = graph_us_per_layer(decomp_only, n, args)
    del scratch
    log(f"decompress-first: {total:.1f} us/layer (decompress {dec:.1f})")
    return {"us_per_layer": round(total, 2), "decompress_us_per_layer": round(dec, 2)}


def committed_traffic():
    """HBM bytes per attention call (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy) from the
    committed counter summary - only while the kernel source still matches it."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        log("traffic: kernel source changed since the counters were taken -> null")
        return None
    return rec.get("hbm_bytes_per_call")


def compressible_variant(args, dev, seq_lens, n_comp, ws):
    """The same shape with u ~ U[-3, 3] (most blocks compress), 8 layers, fused vs baseline."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    arena = paged.SlotArena(VARIANT_LAYERS * (N_PHYS + B) * HKV * 2 * 4096 + (16 << 20), device=dev)
    layers = build_layers(arena, VARIANT_LAYERS, VARIANT_U_MAX, SEED + 100, True, dev)
    st = arena.stats()
    rec = st["live_granules"] * 256 / VARIANT_LAYERS
    res = {}
    for fused in (True, False):
        def run():
            for L in layers:
                if fused:
                    kvz.kvz_decode_attention(L["q"], L["out"], arena.arena, L["meta"],
                                             L["block_table"], seq_lens, n_comp, L["tail"], SCALE,
                                             ws, args.splits)
                else:
                    kvz.kvz_bf16_decode_attention(L["q"], L["out"], L["store"], L["block_table"],
                                                  seq_lens, n_comp, L["tail"], SCALE, ws, HKV,
                                                  args.splits)
        res[fused] = graph_us_per_layer(run, VARIANT_LAYERS, args)
    for L in layers:
        del L["store"]
    dfirst = decompress_first(args, arena, layers, seq_lens, n_comp, ws, N_PHYS, HKV)
    arena.close()
    out = {"label": "same shape, u~U[-3,3] per-channel scale (compressible), 8 layers",
           "raw_block_fraction": round(st["live_raw_blocks"] / (st["live_runs"] * 4), 4),
           "record_bytes_per_layer": int(rec),
           "fused_us_per_layer": round(res[True], 2),
           "fused_achieved_GBps": round(alg_bytes_per_layer(rec) / (res[True] * 1e-6) / 1e9, 1),
           "bf16_us_per_layer": round(res[False], 2),
           "decompress_first": dfirst,
           "fused_speedup_vs_decompress_first": round(dfirst["us_per_layer"] / res[True], 3),
           "speedup_vs_bf16_kernel": round(res[False] / res[True], 4)}
    log(f"compressible variant: fused {res[True]:.1f} us/layer vs bf16 {res[False]:.1f} "
        f"(raw fraction {out['raw_block_fraction']})")
    return out


def online_completion(args, dev):
    """Online page completion at the 64-sequence, 32-layer, 8-KV-head shape with staggered
    phases: every step 4 sequences complete a page, so 4 x 32 layers x 8 heads x K|V = 2,048
    groups are encoded and, in steady state, as many are freed.  One graph per step holding one
    kvz_complete_pages launch: free the 2,048 groups the previous step stored, then encode the new
    ones into the same metadata (the freed runs are reused, deterministic in item order).
    Forced-raw fraction 0 / 10 / 50 %."""
    import torch
    from decode_attention_kvz_amd import kvz, paged, synth
    n_seq, n_layers, hkv = 4, 32, 8
    res = {}
    for forced in (0.0, 0.10, 0.50):
        # the completing pages: sequence s, "page" = layer (one 16-token page per layer)
        pages = synth.kv_pages(n_seq, n_layers, hkv, seed=31, u_max=3.0, forced_frac=forced,
                               device=dev)
        arena = paged.SlotArena(64 << 20, device=dev)
        meta = paged.new_meta_table(n_seq * n_layers, hkv, device=dev)
        ids = [(s, l) for s in range(n_seq) for l in range(n_layers)]
        items = paged.page_items(pages, ids, meta, list(range(len(ids))))
        n = items.size // kvz.ENCODE_ITEM_DTYPE.itemsize
        d_items = torch.from_numpy(np.ascontiguousarray(items)).to(dev)
        ptrs = torch.from_numpy(meta.data_ptr() + np.arange(n, dtype=np.int64) * 8).to(dev)
        kvz.kvz_encode_pages(arena.pool, d_items, n)

        def step():
            kvz.kvz_complete_pages(arena.pool, ptrs, d_items, n)
        # eight steps per graph, as inside a captured decode step (not the launch of a
        # one-node graph per step)
        us = graph_us_per_layer(lambda: [step() for _ in range(8)], 8, args)
        st = arena.stats()
        rec = st["live_granules"] * 256
        raw = st["live_raw_blocks"] / max(st["live_runs"] * 4, 1)
        res[f"forced_{int(forced * 100)}pct"] = {
            "groups_per_step": n, "us_per_step": round(us, 1),
            "raw_block_fraction": round(raw, 4),
            "bytes_read": n * 4096, "bytes_written": int(rec + n * 8),
            "GBps": round((n * 4096 + rec + n * 8) / (us * 1e-6) / 1e9, 1)}
        log(f"online completion, {n} groups/step, forced {forced:.0%}: {us:.1f} us/step "
            f"(raw fraction {raw:.3f})")
        del arena
    return res


def other_layers(dev, bsz, hq, hkv, n_comp, n_layers, u_max, forced, seed, stress, entropy=None):
    """n_layers distinct layers of bsz sequences with n_comp compressed pages each (an int, or a
    list per sequence; no tail page), encoded into one arena in random physical order, with the
    BF16 baseline's pages.  Returns the arena, the layers and the per-sequence page counts."""
    import torch
    from decode_attention_kvz_amd import kvz, paged, synth
    counts = list(n_comp) if isinstance(n_comp, (list, tuple)) else [n_comp] * bsz
    n_phys, max_pages = sum(counts), max(counts)
    arena = paged.SlotArena(n_layers * n_phys * hkv * 2 * 4096 + (16 << 20), device=dev)
    rng = np.random.default_rng(seed)
    ids = [(b, p) for b in range(bsz) for p in range(counts[b])]
    layers = []
    for layer in range(n_layers):
        pages = synth.kv_pages(bsz, max_pages, hkv, seed=seed, layer=layer, u_max=u_max,
                               forced_frac=forced, stress=stress, device=dev)
        if entropy is not None and layer == 0:
            sel = torch.cat([pages[b, :counts[b]] for b in range(bsz)])
            entropy.update(exponent_entropy(sel))
            del sel
        perm = rng.permutation(n_phys).astype(np.int32)
        bt = np.zeros((bsz, max_pages), dtype=np.int32)
        k = 0
        for b in range(bsz):
            bt[b, :counts[b]] = perm[k:k + counts[b]]
            k += counts[b]
        meta = paged.new_meta_table(n_phys, hkv, device=dev)
        items = paged.page_items(pages, ids, meta, perm)
        kvz.kvz_encode_pages(arena.pool, torch.from_numpy(np.ascontiguousarray(items)).to(dev),
                             n_phys * hkv * 2, 0)
        nat = torch.stack([pages[b, p] for b, p in ids])          # [n_phys, 2, Hkv, 16, 128]
        store = paged.pack_bf16_pages(nat[torch.as_tensor(np.argsort(perm), device=dev)])
        layers.append(dict(meta=meta, block_table=torch.from_numpy(bt).to(dev), store=store,
                           q=synth.queries(bsz, hq, seed=seed * 1000 + layer, device=dev),
                           out=torch.empty((bsz, hq, 128), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        del pages, items, nat
    return arena, layers, counts


def other_config(args, dev, name, bsz, hq, hkv, n_comp, n_layers, u_max, forced, seed, stress):
    """Another workload shape: n_layers distinct layers of bsz sequences of n_comp compressed
    pages each (no tail page), fused attention vs the BF16 kernel and vs decompress-first, per
    layer (graph replays over the layers, so no layer is served from cache)."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    entropy = {}
    arena, layers, counts = other_layers(dev, bsz, hq, hkv, n_comp, n_layers, u_max, forced, seed,
                                         stress, entropy)
    n_phys, max_pages = sum(counts), max(counts)
    st = arena.stats()
    rec = st["live_granules"] * 256 / n_layers
    seq_lens = torch.as_tensor([16 * c for c in counts], dtype=torch.int32, device=dev)
    ncomp = torch.as_tensor(counts, dtype=torch.int32, device=dev)
    ws = paged.workspace(bsz, hq, hkv, max_pages, args.splits, device=dev)
    res = {}
    for fused in (True, False):
        def run():
            for L in layers:
                if fused:
                    kvz.kvz_decode_attention(L["q"], L["out"], arena.arena, L["meta"],
                                             L["block_table"], seq_lens, ncomp, None, SCALE, ws,
                                             args.splits)
                else:
                    kvz.kvz_bf16_decode_attention(L["q"], L["out"], L["store"], L["block_table"],
                                                  seq_lens, ncomp, None, SCALE, ws, hkv, args.splits)
        res[fused] = graph_us_per_layer(run, n_layers, args)
    for L in layers:
        del L["store"]
    dfirst = decompress_first(args, arena, layers, seq_lens, ncomp, ws, n_phys, hkv)
    io = n_phys * (hkv * 16 + 4) + bsz * hq * 128 * (2 + 4)   # metadata, block table, q, out
    alg = rec + io
    alg_bf16 = n_phys * hkv * 2 * 4096 + io
    shape = (f"{bsz} sequence(s) x {16 * counts[0]} tokens" if len(set(counts)) == 1 else
             f"{bsz} sequences: " + ", ".join(f"{counts.count(c)} x {16 * c}" for c in sorted(set(counts), reverse=True))
             + " tokens")
    out = {"label": f"{shape}, {hq}/{hkv} heads, {n_layers} distinct layers, "
                    f"u~U[-{u_max:g},{u_max:g}], {forced:.0%} forced-raw blocks"
                    + (", stress values" if stress else ""),
           "record_bytes_per_layer": int(rec),
           "raw_block_fraction": round(st["live_raw_blocks"] / (st["live_runs"] * 4), 4),
           "exponent_entropy_bits": entropy,
           "fused_us_per_layer": round(res[True], 2),
           "fused_achieved_GBps": round(alg / (res[True] * 1e-6) / 1e9, 1),
           "fused_hbm_frac": round(alg / (res[True] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "bf16_us_per_layer": round(res[False], 2),
           "bf16_hbm_frac": round(alg_bf16 / (res[False] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "speedup_vs_bf16_kernel": round(res[False] / res[True], 4),
           "decompress_first": dfirst,
           "fused_speedup_vs_decompress_first": round(dfirst["us_per_layer"] / res[True], 3)}
    arena.close()
    log(f"{name}: fused {res[True]:.1f} us/layer ({out['fused_hbm_frac']:.1%} of HBM peak) vs "
        f"bf16 {res[False]:.1f} ({out['bf16_hbm_frac']:.1%}), decompress-first "
        f"{dfirst['us_per_layer']:.1f}")
    return out


def breakdown(args, dev):
    """The attention time split into KV loading, exponent decoding and computation (GAAC page,
    "Attention Time Breakdown", Table 5), at the 8K workload, the 2K batch shape (8 distinct
    layers each) and the single 131K-token sequence (4 layers).  The library's compile-time variants of the attention kernel time the page loads
    alone (KVZ_PART_LOAD) and the loads with the in-register restore (KVZ_PART_LOAD_RESTORE);
    decoding = (loads + restore) - loads, computation = full call - (loads + restore) (scores,
    softmax, products, tail page, merge).  The uncompressed kernel gives its own loading and
    computation, and decompress-first adds the standalone decompression of every page."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    res = {}
    # the 8K workload: the first BREAKDOWN_LAYERS layers, with its tail pages
    arena = paged.SlotArena(BREAKDOWN_LAYERS * (N_PHYS + B) * HKV * 2 * 4096 + (16 << 20), device=dev)
    layers = build_layers(arena, BREAKDOWN_LAYERS, U_MAX, SEED, True, dev)
    lens = torch.full((B,), CTX, dtype=torch.int32, device=dev)
    ncomp = torch.full((B,), N_COMP, dtype=torch.int32, device=dev)
    ws = paged.workspace(B, HQ, HKV, N_COMP, args.splits, device=dev)
    res["qwen8k"] = _breakdown_shape(args, arena, layers, lens, ncomp, ws, N_PHYS, HKV,
                                     "16 sequences x 8192 tokens (511 pages + 16-token tail), "
                                     "32/8 heads, u~U[-5,5], 5% forced-raw blocks")
    arena.close()
    del layers
    torch.cuda.empty_cache()
    for name, bsz, hq, hkv, n_comp, n_layers, u_max, forced, seed, stress in OTHER_CONFIGS[:2]:
        arena, layers, counts = other_layers(dev, bsz, hq, hkv, n_comp,
                                             min(n_layers, BREAKDOWN_LAYERS), u_max, forced, seed,
                                             stress)
        lens = torch.as_tensor([16 * c for c in counts], dtype=torch.int32, device=dev)
        ncomp = torch.as_tensor(counts, dtype=torch.int32, device=dev)
        ws = paged.workspace(bsz, hq, hkv, max(counts), args.splits, device=dev)
        res[name] = _breakdown_shape(args, arena, layers, lens, ncomp, ws, sum(counts), hkv,
                                     f"{bsz} sequence(s) x {16 * n_comp} tokens, {hq}/{hkv} heads, "
                                     f"u~U[-{u_max:g},{u_max:g}], {forced:.0%} forced-raw blocks"
                                     + (", stress values" if stress else ""))
        arena.close()
        del layers
        torch.cuda.empty_cache()
    return res


def _breakdown_shape(args, arena, layers, lens, ncomp, ws, n_phys, hkv, label):
    import torch
    from decode_attention_kvz_amd import kvz, paged
    n = len(layers)

    def fused(part):
        def run():
            for L in layers:
                kvz.kvz_decode_attention_part(L["q"], L["out"], arena.arena, L["meta"],
                                              L["block_table"], lens, ncomp, L.get("tail"), SCALE,
                                              ws, part, args.splits)
        return graph_us_per_layer(run, n, args)

    def bf16(part):
        def run():
            for L in layers:
                kvz.kvz_bf16_decode_attention_part(L["q"], L["out"], L["store"], L["block_table"],
                                                   lens, ncomp, L.get("tail"), SCALE, ws, hkv,
                                                   part, args.splits)
        return graph_us_per_layer(run, n, args)

    t_full, t_load, t_rest = fused(kvz.KVZ_PART_ALL), fused(kvz.KVZ_PART_LOAD), fused(kvz.KVZ_PART_LOAD_RESTORE)
    b_full, b_load = bf16(kvz.KVZ_PART_ALL), bf16(kvz.KVZ_PART_LOAD)
    for L in layers:
        del L["store"]
    df = decompress_first(args, arena, layers, lens, ncomp, ws, n_phys, hkv)
    r2 = lambda x: round(x, 2)
    out = {"label": label + f", {n} distinct layers; us per layer",
           "bf16_kernel": {"kv_loading": r2(b_load), "computation": r2(b_full - b_load),
                           "measured_total": r2(b_full)},
           "decompress_first": {"kv_loading": r2(b_load),
                                "exponent_decoding": r2(df["decompress_us_per_layer"]),
                                "computation": r2(b_full - b_load),
                                "measured_total": r2(df["us_per_layer"])},
           "fused": {"kv_loading": r2(t_load), "exponent_decoding": r2(t_rest - t_load),
                     "computation": r2(t_full - t_rest), "measured_total": r2(t_full)}}
    log(f"breakdown {label[:40]}...: fused load {t_load:.1f} + decode {t_rest - t_load:.1f} + "
        f"compute {t_full - t_rest:.1f} = {t_full:.1f}; bf16 load {b_load:.1f} + compute "
        f"{b_full - b_load:.1f} = {b_full:.1f}; decompress-first {df['us_per_layer']:.1f}")
    return out


def pmc_probe(args, dev):
    """Launches for a counter run: a 1 GiB device-to-device copy (reads and writes exactly
    1 GiB; the reference that scales FETCH_SIZE / WRITE_SIZE), then 3 fused and 3 baseline
    attention calls on layer 0 of the workload, then 3 calls over the same layer in the
    group-adaptive format, then 3 fused and 3 uncompressed calls over an FP8 E4M3 layer."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    arena = paged.SlotArena((N_PHYS + B) * HKV * 2 * 4096 + (16 << 20), device=dev)
    L = build_layers(arena, 1, U_MAX, SEED, True, dev)[0]
    seq_lens = torch.full((B,), CTX, dtype=torch.int32, device=dev)
    n_comp = torch.full((B,), N_COMP, dtype=torch.int32, device=dev)
    ws = paged.workspace(B, HQ, HKV, N_COMP, args.splits, device=dev)
    for _ in range(3):
        kvz.kvz_decode_attention(L["q"], L["out"], arena.arena, L["meta"], L["block_table"],
                                 seq_lens, n_comp, L["tail"], SCALE, ws, args.splits)
    for _ in range(3):
        kvz.kvz_bf16_decode_attention(L["q"], L["out"], L["store"], L["block_table"], seq_lens,
                                      n_comp, L["tail"], SCALE, ws, HKV, args.splits)
    torch.cuda.synchronize()
    st = arena.stats()
    garena = paged.SlotArena((N_PHYS + B) * HKV * 2 * 4096 + (16 << 20), device=dev)
    G = build_gaac_layers(garena, 1, dev)[0]
    for _ in range(3):
        kvz.kvz_gaac_decode_attention(G["q"], G["out"], garena.arena, G["meta"], G["bases"],
                                      G["block_table"], seq_lens, n_comp, G["tail"], SCALE, ws,
                                      args.splits)
    torch.cuda.synchronize()
    log(f"pmc probe: GAAC layer {garena.stats()['live_granules'] * 256} record bytes")
    garena.close()
    farena = paged.SlotArena((N_PHYS + B) * HKV * 2 * 2048 + (16 << 20), device=dev, fp8=True)
    F8 = build_fp8_layers(farena, 1, dev, 0)[0]
    for _ in range(3):
        kvz.kvz_fp8_decode_attention(F8["q"], F8["out"], 0, farena.arena, F8["meta"], F8["bases"],
                                     F8["block_table"], seq_lens, n_comp, F8["tail"], SCALE, 1.0,
                                     1.0, ws, args.splits)
    for _ in range(3):
        kvz.kvz_fp8_raw_decode_attention(F8["q"], F8["out"], 0, F8["store"], F8["block_table"],
                                         seq_lens, n_comp, F8["tail"], SCALE, 1.0, 1.0, ws, HKV,
                                         args.splits)
    torch.cuda.synchronize()
    log(f"pmc probe: FP8 E4M3 layer {farena.stats()['live_granules'] * 128} record bytes")
    farena.close()
    log(f"pmc probe done: {st['live_granules'] * 256} record bytes in the layer, algorithmic "
        f"{alg_bytes_per_layer(st['live_granules'] * 256):.0f} bytes per call; kernel source "
        f"sha256 {kernel_source_sha()}")
    arena.close()


def pmc_probe_other(args, dev, cfg):
    """Counter-run launches for another shape: the 1 GiB device copy (the byte counters' scale
    reference), then 3 fused and 3 BF16 attention calls over one layer of the shape."""
    import torch
    from decode_attention_kvz_amd import kvz, paged
    name, bsz, hq, hkv, n_comp, _, u_max, forced, seed, stress = cfg
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    arena, layers, counts = other_layers(dev, bsz, hq, hkv, n_comp, 1, u_max, forced, seed, stress)
    L = layers[0]
    lens = torch.as_tensor([16 * c for c in counts], dtype=torch.int32, device=dev)
    ncomp = torch.as_tensor(counts, dtype=torch.int32, device=dev)
    ws = paged.workspace(bsz, hq, hkv, max(counts), args.splits, device=dev)
    for _ in range(3):
        kvz.kvz_decode_attention(L["q"], L["out"], arena.arena, L["meta"], L["block_table"], lens,
                                 ncomp, None, SCALE, ws, args.splits)
    for _ in range(3):
        kvz.kvz_bf16_decode_attention(L["q"], L["out"], L["store"], L["block_table"], lens, ncomp,
                                      None, SCALE, ws, hkv, args.splits)
    torch.cuda.synchronize()
    rec = arena.stats()["live_granules"] * 256
    n_phys = sum(counts)
    io = n_phys * (hkv * 16 + 4) + bsz * hq * 128 * (2 + 4)
    log(f"pmc probe done: {rec} record bytes in the layer, algorithmic {rec + io} bytes per call "
        f"(bf16 {n_phys * hkv * 2 * 4096 + io}); shape {name}; kernel source sha256 "
        f"{kernel_source_sha()}")
    arena.close()


def cpu_baseline(layers, all_cores_child=None):
    """The oracle on a bounded sample: decode + fp64 attention of layer 0 (all 16 sequences, all
    KV heads, 8192 tokens each), inputs encoded by the oracle itself outside the timed region."""
    import contextlib
    from decode_attention_kvz_amd import synth
    from oracle import attention
    from oracle.cache import OracleCache
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:   # pragma: no cover
        threadpool_limits = None

    # regenerate layer 0 (the same seeded pages) and hand the host copy to the oracle
    pages = synth.kv_pages(B, N_COMP + 1, HKV, seed=SEED, layer=0, u_max=U_MAX, forced_frac=FORCED,
                           device="cuda")
    nat = synth.bits(pages)                         # [B, 512, 2, Hkv, 16, 128]
    del pages
    q = synth.bits(layers[0]["q"])
    oc = OracleCache((B * N_COMP * HKV * 2 + 16) * 4096)
    flat = nat[:, :N_COMP].transpose(0, 1, 3, 2, 4, 5).reshape(-1, 16, 128)   # (b, p, h, K/V)
    def one_thread():   # a fresh limiter per timed block (it applies its limit when made)
        return threadpool_limits(limits=1) if threadpool_limits is not None else contextlib.nullcontext()

    with one_thread():
        t0 = time.perf_counter()
        metas = oc.encode(flat, [i % 2 for i in range(flat.shape[0])])
        dt_enc = time.perf_counter() - t0
    enc_bytes = flat.shape[0] * 16 * 128 * 2
    log(f"cpu baseline: oracle encode of the sample {dt_enc:.1f}s ({enc_bytes / dt_enc / 1e9:.4f} GB/s "
        f"of BF16 input)")
    meta_table = [[[metas[(pp * HKV + h) * 2 + k] for k in range(2)] for h in range(HKV)]
                  for pp in range(B * N_COMP)]
    block_table = np.arange(B * N_COMP, dtype=np.int64).reshape(B, N_COMP)
    tail = nat[:, N_COMP]
    with one_thread():
        t0 = time.perf_counter()
        attention.decode_attention(q, oc.arena, meta_table, block_table, [CTX] * B, [N_COMP] * B,
                                   tail, SCALE)
        dt = time.perf_counter() - t0
    bytes_eff = B * CTX * HKV * 128 * 2 * 2
    log(f"cpu baseline: {dt:.1f}s for one layer ({bytes_eff / dt / 1e9:.4f} GB/s)")
    all_cores = cpu_all_cores_result(all_cores_child)
    return {"value": round(bytes_eff / dt / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "all_cores": all_cores,
            "sample": "layer 0 of the workload (16 sequences x 8192 tokens, 8 KV / 32 query heads; "
                      "1/36 of a step's attention): oracle block decode + fp64 attention, "
                      "1 thread, inputs encoded by the oracle beforehand",
            "encode_GBps": round(enc_bytes / dt_enc / 1e9, 5),
            "encode_sample": "the oracle encode of the same layer's 130,816 groups, 1 thread "
                             "(GB/s of BF16 input)"}


def cpu_model() -> str | None:
    """The host CPU's model name (/proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_all_cores_result(child):
    """Release the all-cores child (started before the GPU was touched) and read its JSON line;
    None if there is none or it failed."""
    if child is None:
        return None
    try:
        out, _ = child.communicate("go\n", timeout=300)
        res = json.loads(out.strip().splitlines()[-1])
    except Exception as e:   # pragma: no cover - reported, not fatal
        child.kill()
        log(f"cpu baseline, all cores: failed ({e})")
        return None
    log(f"cpu baseline, all cores: {res['seconds']:.1f}s for one layer ({res['value']:.4f} GB/s, "
        f"{res['cores']} worker processes)")
    return res


_PAR = {}


def _par_encode(b):
    from oracle.cache import OracleCache
    flat = _PAR["nat"][b, :N_COMP].transpose(0, 2, 1, 3, 4).reshape(-1, 16, 128)   # (p, h, K/V)
    oc = OracleCache(_PAR["seq_arena"])
    metas = oc.encode(flat, [i % 2 for i in range(flat.shape[0])])
    return oc.arena, metas


def _par_attention(b):
    from oracle import attention
    with _one_thread():
        out = attention.decode_attention(_PAR["q"], _PAR["arena"], _PAR["meta_table"],
                                         _PAR["block_table"], [CTX] * B, [N_COMP] * B,
                                         _PAR["nat"][:, N_COMP], SCALE, batch_indices=[b])
    return out[b]


def _one_thread():
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except ImportError:   # pragma: no cover
        return contextlib.nullcontext()


def cpu_all_cores():
    """The oracle's decode + fp64 attention of one layer of the workload on the host's cores:
    forked worker processes, one sequence each at a time (up to 16, the host share of one GPU),
    one BLAS thread each.  The layer is regenerated here on the host with the same seeds (the
    host generator draws other values than the device one: the same shapes and distribution,
    not the same numbers); each sequence is encoded by the oracle into its own arena, in the
    workers, outside the timed region."""
    import multiprocessing as mp
    if sys.stdin.readline().strip() != "go":   # the parent ended or did not ask
        return None
    from decode_attention_kvz_amd import synth
    pages = synth.kv_pages(B, N_COMP + 1, HKV, seed=SEED, layer=0, u_max=U_MAX, forced_frac=FORCED)
    _PAR["nat"] = synth.bits(pages)                # [B, 512, 2, Hkv, 16, 128]
    del pages
    _PAR["q"] = synth.bits(synth.queries(B, HQ, seed=SEED * 1000))
    _PAR["seq_arena"] = (N_COMP * HKV * 2 + 16) * 4096
    workers = max(1, min(os.cpu_count() or 1, 16, B))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        enc = pool.map(_par_encode, range(B))
    # one arena: sequence b's records at b * seq_arena bytes; page (b, p) is physical page b*512+p
    _PAR["arena"] = np.concatenate([a for a, _ in enc])
    gran = _PAR["seq_arena"] // 256
    meta_table = []
    for b, (_, metas) in enumerate(enc):
        for pp in range(N_COMP):
            row = []
            for h in range(HKV):
                pair = []
                for k in range(2):
                    off, tags = metas[(pp * HKV + h) * 2 + k]
                    pair.append((off if off == 0xFFFFFFFF else off + b * gran, tags))
                row.append(pair)
            meta_table.append(row)
    _PAR["meta_table"] = meta_table
    _PAR["block_table"] = np.arange(B * N_COMP, dtype=np.int64).reshape(B, N_COMP)
    del enc
    with ctx.Pool(workers) as pool:
        t0 = time.perf_counter()
        pool.map(_par_attention, range(B))
        dt = time.perf_counter() - t0
    bytes_eff = B * CTX * HKV * 128 * 2 * 2
    return {"value": round(bytes_eff / dt / 1e9, 5), "unit": "GB/s", "cores": workers,
            "seconds": round(dt, 2),
            "sample": "layer 0 of the workload regenerated on the host (same seeds and shapes), "
                      "oracle block decode + fp64 attention, one sequence per worker process, "
                      "one BLAS thread each; oracle encode beforehand in the workers"}


if __name__ == "__main__":
    main()
