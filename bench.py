#!/usr/bin/env python3
"""Benchmark: NVFP4 decode attention over a paged NVFP4 KV cache on one MI355X.

A step is the whole decode-time path for every layer of the workload: the
split-K decode attention kernel, which also quantizes each sequence's new
token into the cache in place (RoPE, Hadamard-128, NVFP4, no separate append
pass), and the reduce kernel.
The default workload is three concurrent sequences of 330K/400K/470K cached
tokens, 16 layers, 24 query / 4 KV heads, head_dim 128, 64-token pages with a
randomly permuted page table; all inputs are seeded synthetic data resident in
HBM before the timed region starts.

Prints one JSON line.  `value` is the algorithmic KV bytes of a step (144
bytes per cached token per KV head per layer) divided by the step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="three_long")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0,
                    help="run only this many layers of the workload (0 = all); every layer's decode "
                         "launch is the same kernel on the same shape, so profiling runs use 1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the HBM copy-ceiling measurement")
    ap.add_argument("--quality", action="store_true",
                    help="report attention error against unquantized attention on the 600K-token "
                         "outlier workload, per rotation variant, instead of timing")
    ap.add_argument("--append", action="store_true",
                    help="time the prefill-style append of the workload's chunk per sequence instead "
                         "(batch64: 64 x 8192 tokens)")
    ap.add_argument("--spill", action="store_true",
                    help="time host spill and restore of the longest sequence's pages instead")
    ap.add_argument("--multi", type=int, default=0,
                    help="time multi-query decode instead: this many new query tokens per sequence")
    ap.add_argument("--v-format", type=int, default=0, choices=[0, 1],
                    help="1: time the decode step on a pool that keeps V in fp16 (the upstream "
                         "storage, 328 B per token per kv head) instead of NVFP4")
    return ap.parse_args()


def copy_ceiling_gbps(torch) -> float:
    """Achieved HBM bandwidth of a plain device copy of 4 GiB (read + write)."""
    n = 1 << 32
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def stream_read_ceiling_gbps(step, wl, torch, kv) -> float:
    """Achieved rate of nvfp4kv_stream_read over layer 0: every block a decode
    launch reads, with the decode kernel's loads, one wavefront per resident
    decode slot (8 per CU), no compute.  The measured ceiling of the decode
    access pattern on this device."""
    n_waves = torch.cuda.get_device_properties(0).multi_processor_count * 8
    words = torch.empty(n_waves, dtype=torch.int32, device="cuda")
    for _ in range(3):
        kv.nvfp4kv_stream_read(step.pool, 0, step.table, step.seq_lens, n_waves, words)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        kv.nvfp4kv_stream_read(step.pool, 0, step.table, step.seq_lens, n_waves, words)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return wl.decode_bytes_per_layer() / (ms * 1e-3) / 1e9


def traffic_from_profiles(kernel_tag: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source and headers (same hashes); else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    csrc = os.path.join(ROOT, "nvfp4_quantized_kv_amd", "csrc")
    want = dict(rec.get("header_sha256", {}))
    want[rec.get("source", "decode_attn.hip")] = rec.get("source_sha256")
    for name, digest in want.items():
        # the kernel's source and the headers it includes, as when counted
        if hashlib.sha256(open(os.path.join(csrc, name), "rb").read()).hexdigest() != digest:
            return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name, as lscpu reports it (/proc/cpuinfo if lscpu
    is missing)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(step, wl, torch, v_format=0):
    """Time the CPU oracle on a bounded sample of the same step: layer 0 of
    the workload, i.e. the append of every sequence's new token and decode
    attention of every sequence and query head over the layer's cache."""
    import numpy as np
    import oracle
    from nvfp4_quantized_kv_amd import workloads as W

    cores = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0)))))
    torch.cuda.synchronize()
    layer_bytes = step.pool.data.numel() // wl.layers
    pool0 = step.pool.data[:layer_bytes].cpu().numpy()       # layer 0 blocks (the layer is first)
    oc = os_ = None
    if wl.rotary_dim:
        oc, os_ = oracle.rope_table(wl.theta, wl.rotary_dim, wl.pos_scale, step.max_pos)
    k = step.k_new[0].float().cpu().numpy()
    v = step.v_new[0].float().cpu().numpy()
    q = step.q[0].float().cpu().numpy()
    slots = step.new_slots.cpu().numpy()
    pos = np.array(wl.cached, np.int32)
    t0 = time.perf_counter()
    oracle.append(pool0, step.pool.num_pages, wl.hkv, wl.rotary_dim, wl.hadamard, 0, k, v, slots, pos, oc, os_,
                  v_format=v_format)
    ref = oracle.decode_attention(pool0, step.pool.num_pages, wl.hkv, 0, wl.rotary_dim, wl.hadamard, q,
                                  pos, step.table_np, wl.seq_lens, W.sm_scale(), oc, os_, v_format=v_format)
    sec = time.perf_counter() - t0
    nbytes = wl.decode_bytes_per_layer(v_format)
    # the same layer on the GPU (new token quantized by the decode kernel), for a parity figure
    out = step.decode(0, fused=True).clone()
    torch.cuda.synchronize()
    err = float(np.abs(out.cpu().numpy().astype(np.float64) - ref).max())
    return {
        "value": nbytes / sec / 1e9, "unit": "GB/s", "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"layer 0 of {wl.layers}: append of {wl.n_seq} new tokens + fp64 decode attention "
                  f"for {wl.n_seq} sequences x {wl.hq} query heads over {sum(wl.seq_lens)} tokens "
                  f"({sec:.1f} s)",
        "seconds": sec,
    }, err


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("only one GPU is used: the attention path shards by kv head, sequence or context with no "
            "exchange inside the kernels, and a single GPU runs one shard at its real shape")
        sys.exit(2)
    import torch
    import nvfp4_quantized_kv_amd as kv
    from nvfp4_quantized_kv_amd import workloads as W
    from nvfp4_quantized_kv_amd.runner import DecodeStep

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.quality:
        return bench_quality(args, torch, kv, W, DecodeStep)
    if args.v_format and (args.multi or args.spill or args.append):
        log("--v-format applies to the decode step only")
        sys.exit(2)
    wl = W.config(args.workload)
    if args.layers:
        wl.layers = min(args.layers, wl.layers)
    log(f"workload {wl.name}: {wl.n_seq} seqs {wl.cached} cached, {wl.layers} layers, "
        f"hq {wl.hq} hkv {wl.hkv}, {kv.nvfp4kv_version()}")
    ceiling = None if args.no_ceiling else copy_ceiling_gbps(torch)
    if ceiling:
        log(f"plain copy ceiling {ceiling:.0f} GB/s")
    step = DecodeStep(wl, pages_per_split=args.pages_per_split, v_format=args.v_format)
    t0 = time.perf_counter()
    for layer in range(wl.layers):
        step.fill([layer])
        torch.cuda.synchronize()
        log(f"filled layer {layer + 1}/{wl.layers} ({time.perf_counter() - t0:.1f} s)")
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    if args.multi:
        return bench_multi(args, step, wl, torch, kv, W, ceiling)
    if args.spill:
        return bench_spill(args, step, wl, torch, kv)
    if args.append:
        return bench_append(args, step, wl, torch, kv, W)

    stream = torch.cuda.current_stream()
    # the timed steps: decode + reduce per layer, nothing else on the stream
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        for layer in range(wl.layers):
            step.decode_splits(layer, fused=True)
            step.decode_reduce(layer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    # then the same steps again with HIP events around every decode launch,
    # on the stream it runs on, for the decode kernel's own duration
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps * wl.layers)]
    i = 0
    for _ in range(args.steps):
        for layer in range(wl.layers):
            ev[i][0].record(stream)
            step.decode_splits(layer, fused=True)
            ev[i][1].record(stream)
            step.decode_reduce(layer)
            i += 1
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    avg_kernel_ms = sum(kern_ms) / len(kern_ms)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, decode kernel avg {avg_kernel_ms * 1e3:.1f} us")

    bytes_per_layer = wl.decode_bytes_per_layer(args.v_format)
    bytes_per_step = bytes_per_layer * wl.layers
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    tok_heads = sum(wl.seq_lens) * wl.hkv * wl.layers
    achieved = bytes_per_layer / (avg_kernel_ms * 1e-3) / 1e9
    # (the counters and the read probe cover the NVFP4 pool)
    traffic = traffic_from_profiles("decode_attn_splitk", wl.name) if args.v_format == 0 else None
    read_ceiling = (None if args.no_ceiling or args.v_format
                    else stream_read_ceiling_gbps(step, wl, torch, kv))
    if read_ceiling:
        log(f"stream-read ceiling of the same blocks {read_ceiling:.0f} GB/s")

    cpu = None
    parity_err = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on layer 0")
        cpu, parity_err = cpu_baseline(step, wl, torch, args.v_format)
        cpu.pop("seconds", None)
        log(f"oracle {cpu['value']:.3f} GB/s on {cpu['cores']} threads; max |gpu - oracle| = {parity_err:.2e}")

    rec = {
        "metric": "NVFP4 decode-attn achieved HBM GB/s (% peak) and KV tokens·heads/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.n_seq} sequences at {'/'.join(str(t) for t in wl.cached)} cached "
                        f"tokens + 1 appended, {wl.layers} layers, {wl.hq} query / {wl.hkv} KV heads, "
                        f"head_dim 128, 64-token pages, randomly permuted page table"
                        + (", V kept in fp16 (328 B per token per kv head)" if args.v_format else ""),
            "n_seq": wl.n_seq, "layers": wl.layers, "q_heads": wl.hq, "kv_heads": wl.hkv,
            "rotary_dim": wl.rotary_dim, "hadamard": wl.hadamard, "input_dtype": wl.dtype,
            "step": "per layer: decode_attn_splitk (new token quantized in place) + decode_reduce",
            "pages_per_split": args.pages_per_split or "auto",
            "v_format": args.v_format,
        },
        "pct_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "kv_token_heads_per_s": round(tok_heads / (ms_per_step * 1e-3), 1),
        "bytes_per_step": bytes_per_step,
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_attn_splitk_kernel" + (" (fp16 V)" if args.v_format else ""),
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_kernel_ms * 1e3, 2),
            "algo_bytes_per_launch": bytes_per_layer,
            "frac_of_stream_read_ceiling": round(achieved / read_ceiling, 4) if read_ceiling else None,
        },
        "stream_read_ceiling_gbps": round(read_ceiling, 1) if read_ceiling else None,
        "hbm_copy_ceiling_gbps": round(ceiling, 1) if ceiling else None,
        "cpu_baseline": cpu,
        "parity_max_abs_err_layer0": parity_err,
    }
    print(json.dumps(rec), flush=True)


def bench_multi(args, step, wl, torch, kv, W, ceiling):
    """Multi-query decode: every layer, n_qtok = args.multi new query tokens per
    sequence (already in the cache) attend causally over the cache, one call
    (a decode launch and its reduce per 48 // heads tokens)."""
    m = args.multi
    step.prepare_multi(m)
    for layer in range(wl.layers):
        step.append(layer)          # the newest token; the m query tokens are the last m cached ones
        step.decode_multi(layer)
    torch.cuda.synchronize()
    heads = wl.hq // wl.hkv
    per_launch = max(1, min(m, 48 // heads))      # a launch takes up to 48 query columns per kv head
    launches = -(-m // per_launch)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps * wl.layers)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    i = 0
    for _ in range(args.steps):
        for layer in range(wl.layers):
            ev[i][0].record(stream)
            step.decode_multi(layer)
            ev[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    call_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    bytes_per_layer = wl.decode_bytes_per_layer()
    qrows = wl.n_seq * m * wl.hq * wl.layers
    log(f"multi-query n_qtok {m}: {launches} decode launches per layer, {ms_per_step:.3f} ms/step, "
        f"{call_ms * 1e3:.1f} us per layer call")
    cpu = parity = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle (multi-query) on layer 0")
        gpu = step.decode_multi(0).cpu().numpy()
        pool = step.pool.data[:step.pool.data.numel() // wl.layers].cpu().numpy()   # layer 0 blocks
        oc, os_ = (oracle.rope_table(wl.theta, wl.rotary_dim, wl.pos_scale, step.max_pos)
                   if wl.rotary_dim else (None, None))
        t0 = time.perf_counter()
        ref = oracle.decode_attention_multi(pool, step.pool.num_pages, wl.hkv, 0, wl.rotary_dim, wl.hadamard,
                                            step.mq[0].float().cpu().numpy(), step.mq_pos.cpu().numpy(),
                                            step.table_np, wl.seq_lens, W.sm_scale(), oc, os_)
        secs = time.perf_counter() - t0
        parity = float(abs(gpu - ref).max())
        cpu = {"value": round(m * wl.n_seq * wl.hq / secs, 1), "unit": "query token·heads/s", "cores": int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0)))),
               "kind": "oracle", "sample": f"layer 0 of {wl.layers}: fp64 attention of {wl.n_seq} x {m} query tokens "
                                             f"x {wl.hq} heads ({secs:.1f} s)"}
        log(f"oracle {secs:.1f} s; max |gpu - oracle| = {parity:.2e}")
    rec = {
        "metric": "NVFP4 multi-query decode-attn query token·heads/s (speculative verification)",
        "value": round(qrows / (ms_per_step * 1e-3), 1),
        "unit": "query token·heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{wl.name} with {m} new query tokens per sequence (causal among them)",
                   "n_seq": wl.n_seq, "layers": wl.layers, "q_heads": wl.hq, "kv_heads": wl.hkv, "n_qtok": m,
                   "decode_launches_per_layer": launches,
                   "step": "per layer: nvfp4kv_decode_attn_multi (decode launch + reduce per "
                           f"{per_launch} tokens)"},
        "cache_gbps_per_call": round(bytes_per_layer / (call_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": "decode_attn_splitk_kernel (multi-query columns)",
                     "achieved": round(launches * bytes_per_layer / (call_ms * 1e-3) / 1e9, 2),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(launches * bytes_per_layer / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": None, "note": "per call: the cache read once per decode launch, reduces included"},
        "hbm_copy_ceiling_gbps": round(ceiling, 1) if ceiling else None,
        "cpu_baseline": cpu,
        "parity_max_abs_err_layer0": parity,
    }
    print(json.dumps(rec), flush=True)


def bench_quality(args, torch, kv, W, DecodeStep):
    """Attention error of the NVFP4 cache against fp64 attention on the raw
    (unquantized) rows: one sequence of 600,000 cached tokens + 1, RoPE over
    32 dims with linear scaling 2.3, N(0,1) bf16 inputs with 3 outlier
    channels (layer 0 of the workload), for no rotation, the Hadamard
    rotation and the randomized rotation (a drawn sign mask).  Outlier
    channels x32 (the workload as defined) scale Q and K alike, so scores
    spread by ~150 and the softmax is nearly one-hot: its error mostly says
    whether the top token changed.  Outliers x4 keep the softmax spread out.
    The GPU's decode output is compared with the reference; so is the
    oracle's fp64 NVFP4 attention on the GPU's own pool bytes, which
    separates the format's error from the kernel's.  The fp16-V variant
    (NVFP4 K with the Hadamard rotation, V kept in fp16: 328 bytes per token
    per kv head, the upstream storage) runs on the GPU through a v_format 1
    pool and is checked against the oracle on that pool."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(2026)
    mask = tuple(int(x) for x in rng.integers(0, 2 ** 32, 4, dtype=np.uint64))
    variants = [("none", 0, None), ("hadamard", 1, None), ("random_sign", 2, mask)]
    report = {}
    for outlier_scale in (32.0, 4.0):
        res = {}
        ref = None
        for name, had, signs in variants:
            wl = W.config("single600k")
            wl.layers, wl.hadamard, wl.outlier_scale = 1, had, outlier_scale
            step = DecodeStep(wl, signs=signs or (0, 0, 0, 0))
            step.fill([0])
            out = step.decode(0, fused=True).cpu().numpy()[0].astype(np.float64)
            T = wl.seq_lens[0]
            oc, os_ = oracle.rope_table(wl.theta, wl.rotary_dim, wl.pos_scale, step.max_pos)
            if ref is None:
                k = W.rows(wl, "k", 0, step.base[0], T, wl.hkv, "cuda").float().cpu().numpy()
                v = W.rows(wl, "v", 0, step.base[0], T, wl.hkv, "cuda").float().cpu().numpy()
                q = step.q[0][0].float().cpu().numpy()
                t0 = time.perf_counter()
                ref = oracle.reference_attention(q, wl.cached[0], k, v, np.arange(T), wl.rotary_dim,
                                                 W.sm_scale(), oc, os_)
                log(f"outliers x{outlier_scale:g}: reference attention over {T} tokens "
                    f"{time.perf_counter() - t0:.1f} s")
                del k, v
            npg = (T + 63) // 64
            pages = torch.from_numpy(step.table_np[0, :npg].astype(np.int64)).cuda()
            compact = step.pool.data.view(1, step.pool.num_pages, wl.hkv * 9216)[0].index_select(0, pages)
            orc = oracle.decode_attention(compact.contiguous().view(-1).cpu().numpy(), npg, wl.hkv, 0,
                                          wl.rotary_dim, had, step.q[0].float().cpu().numpy(), [wl.cached[0]],
                                          np.arange(npg, dtype=np.int32)[None], [T], W.sm_scale(), oc, os_,
                                          signs=np.array(signs, np.uint32) if signs else None)[0]
            rel = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
            res[name] = {"rel_l2_err": round(rel, 6), "max_abs_err": float(np.abs(out - ref).max()),
                         "median_head_rel_l2": round(float(np.median([np.linalg.norm(out[h] - ref[h]) /
                                                                      np.linalg.norm(ref[h])
                                                                      for h in range(wl.hq)])), 6),
                         "gpu_vs_oracle_max_abs": float(np.abs(out - orc).max())}
            log(f"outliers x{outlier_scale:g} {name}: rel L2 {rel:.4g}, median head "
                f"{res[name]['median_head_rel_l2']:.4g}, GPU vs oracle {res[name]['gpu_vs_oracle_max_abs']:.2g}")
            del step, compact
            torch.cuda.empty_cache()
            if name == "hadamard":
                # the upstream storage: NVFP4 K, V in fp16 (328 bytes per token per kv head), on the
                # GPU through the fp16-V pool format, checked against the oracle on its own pool
                step = DecodeStep(wl, v_format=1)
                step.fill([0])
                o16 = step.decode(0, fused=True).cpu().numpy()[0].astype(np.float64)
                bb = step.pool.block_bytes
                compact = step.pool.data.view(1, step.pool.num_pages, wl.hkv * bb)[0].index_select(0, pages)
                orc16 = oracle.decode_attention(compact.contiguous().view(-1).cpu().numpy(), npg, wl.hkv, 0,
                                                wl.rotary_dim, had, step.q[0].float().cpu().numpy(),
                                                [wl.cached[0]], np.arange(npg, dtype=np.int32)[None], [T],
                                                W.sm_scale(), oc, os_, v_format=1)[0]
                res["hadamard_fp16_v"] = {
                    "rel_l2_err": round(float(np.linalg.norm(o16 - ref) / np.linalg.norm(ref)), 6),
                    "max_abs_err": float(np.abs(o16 - ref).max()),
                    "median_head_rel_l2": round(float(np.median([np.linalg.norm(o16[h] - ref[h]) /
                                                                 np.linalg.norm(ref[h]) for h in range(wl.hq)])), 6),
                    "gpu_vs_oracle_max_abs": float(np.abs(o16 - orc16).max()),
                    "bytes_per_token_kv_head": 328,
                    "computed_by": "GPU (v_format 1 pool), checked against the oracle"}
                log(f"outliers x{outlier_scale:g} hadamard + fp16 V (GPU): rel L2 "
                    f"{res['hadamard_fp16_v']['rel_l2_err']:.4g}, GPU vs oracle "
                    f"{res['hadamard_fp16_v']['gpu_vs_oracle_max_abs']:.2g}")
                del step, compact
                torch.cuda.empty_cache()
        report[f"outliers_x{outlier_scale:g}"] = res
    rec = {
        "metric": "NVFP4 attention error vs unquantized fp64 attention (relative L2), per rotation",
        "value": report["outliers_x4"]["hadamard"]["rel_l2_err"], "unit": "relative L2",
        "n_gpus": 1, "steps": 1, "warmup": 0, "ms_per_step": None, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "single600k layer 0: 600,000 cached tokens + 1, 24 query / 4 KV heads, "
                               "RoPE 32 dims theta 1e7 scaling 2.3, bf16 N(0,1) with 3 outlier channels "
                               "(x32 as defined, and x4); value: outliers x4, Hadamard rotation"},
        "variants": report,
    }
    print(json.dumps(rec), flush=True)


PEAK_PCIE_GBPS = 64.0          # PCIe 5.0 x16 host link, per direction


def bench_append(args, step, wl, torch, kv, W):
    """Prefill-style append: every sequence's chunk of wl.prefill_chunk tokens
    (positions T+1 .. T+chunk, after the step's token) quantized into the
    pool in one nvfp4kv_append call on layer 0; inputs resident in HBM."""
    import numpy as np
    chunk = wl.prefill_chunk
    if chunk <= 0:
        raise SystemExit(f"workload {wl.name} has no prefill chunk")
    ks, vs, sl, ps = [], [], [], []
    for i, T in enumerate(wl.cached):
        first = T + 1
        ks.append(W.rows(wl, "k", 0, step.base[i] + first, chunk, wl.hkv, "cuda"))
        vs.append(W.rows(wl, "v", 0, step.base[i] + first, chunk, wl.hkv, "cuda"))
        pos = np.arange(first, first + chunk)
        sl.append(W.slots(step.table_np, i, pos))
        ps.append(pos.astype(np.int32))
    k = torch.cat(ks).contiguous()
    v = torch.cat(vs).contiguous()
    del ks, vs
    slots = torch.from_numpy(np.concatenate(sl)).cuda()
    pos = torch.from_numpy(np.concatenate(ps)).cuda()
    n_tok = k.shape[0]
    for _ in range(2):
        kv.nvfp4kv_append(step.pool, 0, k, v, slots, pos, step.rope_cos, step.rope_sin)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kv.nvfp4kv_append(step.pool, 0, k, v, slots, pos, step.rope_cos, step.rope_sin)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    t = sum(times) / len(times)
    in_bytes = 2 * n_tok * wl.hkv * 128 * k.element_size()
    out_bytes = 144 * n_tok * wl.hkv
    gbps = (in_bytes + out_bytes) / t / 1e9
    # sampled rows against the oracle's quantization of the same inputs
    cpu = None
    import oracle
    rng = np.random.default_rng(0)
    oc, os_ = oracle.rope_table(wl.theta, wl.rotary_dim, wl.pos_scale, step.max_pos) if wl.rotary_dim else (None, None)
    view = step.pool.data.view(wl.layers, step.pool.num_pages, wl.hkv * 9216)
    for j in rng.choice(n_tok, 16, replace=False):
        j = int(j)
        s_ = int(slots[j]); page, off = s_ // 64, s_ % 64
        blk = view[0, page].cpu().numpy()
        for g in range(wl.hkv):
            p_ = int(pos[j])
            kc, ksc = oracle.quant_row(k[j, g].float().cpu().numpy(), wl.rotary_dim,
                                       oc[p_] if oc is not None else None, os_[p_] if os_ is not None else None,
                                       int(wl.hadamard))
            gk = oracle.pool_read_row(blk, 1, wl.hkv, 0, off, g, 0)
            assert (gk[0] == kc).all() and (gk[1] == ksc).all(), f"appended K row {j} differs from the oracle"
    if not args.no_cpu_baseline:
        # a bounded sample: the first half of the call's tokens (up to 262,144),
        # about a second on 16 threads
        n = min(n_tok, 262144)
        kk, vv = k[:n].float().cpu().numpy(), v[:n].float().cpu().numpy()
        pool_h = np.zeros(oracle.pool_bytes(1, step.pool.num_pages, wl.hkv), np.uint8)
        t0 = time.perf_counter()
        oracle.append(pool_h, step.pool.num_pages, wl.hkv, wl.rotary_dim, int(wl.hadamard), 0, kk, vv,
                      slots[:n].cpu().numpy(), pos[:n].cpu().numpy(), oc, os_)
        secs = time.perf_counter() - t0
        cpu = {"value": round(n * wl.hkv * (2 * 128 * 2 + 144) / secs / 1e9, 4), "unit": "GB/s",
               "cores": int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0)))), "kind": "oracle",
               "sample": f"oracle append of the first {n} tokens x {wl.hkv} kv heads ({secs:.2f} s)"}
    log(f"append of {n_tok} tokens x {wl.hkv} kv heads: {t * 1e3:.3f} ms, {gbps:.1f} GB/s")
    rec = {
        "metric": "NVFP4 prefill append achieved HBM GB/s (tokens/s)",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 2,
        "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.n_seq} sequences x {chunk}-token chunk ({n_tok} tokens), "
                               f"{wl.hkv} kv heads, {wl.dtype} inputs, RoPE {wl.rotary_dim} dims, "
                               f"rotation {int(wl.hadamard)}",
                   "step": "one nvfp4kv_append call"},
        "tokens_per_s": round(n_tok / t, 1),
        "roofline": {"bound": "hbm", "kernel": "kv_quant_append_kernel", "achieved": round(gbps, 2),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_from_profiles("kv_quant_append", wl.name),
                     "algo_bytes_per_launch": in_bytes + out_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_spill(args, step, wl, torch, kv):
    """Host spill and restore: every page of the longest sequence (all layers
    and kv heads) to a pinned host arena and back into the same page ids."""
    import numpy as np
    seq = int(np.argmax(wl.seq_lens))
    npg = (wl.seq_lens[seq] + 63) // 64
    ids = torch.from_numpy(step.table_np[seq, :npg].copy()).to(step.pool.data.device)
    page_bytes = kv.nvfp4kv_page_bytes(step.pool)
    total = page_bytes * npg
    log(f"spill: {npg} pages of {page_bytes} bytes ({total / 1e9:.2f} GB) to pinned host memory")
    arena = torch.empty((npg, wl.layers, wl.hkv, 9216), dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream()
    kv.nvfp4kv_spill_pages(step.pool, ids, arena)
    kv.nvfp4kv_restore_pages(step.pool, ids, arena)
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    t_sp, t_re = [], []
    for _ in range(reps):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        kv.nvfp4kv_spill_pages(step.pool, ids, arena)
        e1.record(stream)
        kv.nvfp4kv_restore_pages(step.pool, ids, arena)
        e2.record(stream)
        torch.cuda.synchronize()
        t_sp.append(e0.elapsed_time(e1) * 1e-3)
        t_re.append(e1.elapsed_time(e2) * 1e-3)
    sp, re_ = sum(t_sp) / reps, sum(t_re) / reps
    # the arena holds the pool's bytes: sampled pages, every layer
    rng = np.random.default_rng(0)
    view = step.pool.data.view(wl.layers, step.pool.num_pages, wl.hkv * 9216)
    for i in rng.choice(npg, 8, replace=False):
        got = arena[int(i)].reshape(wl.layers, -1)
        want = view[:, int(ids[int(i)])].cpu()
        assert torch.equal(got, want), f"arena page {i} differs from the pool"
    log(f"spill {total / sp / 1e9:.2f} GB/s ({npg / sp:.0f} pages/s), restore {total / re_ / 1e9:.2f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = min(npg, 256)
        sub = view[:, ids[:n].long()].cpu().numpy()            # [layers][n][hkv*9216]: a pool of n pages
        t0 = time.perf_counter()
        reps_cpu = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.spill_pages(sub, wl.layers, n, wl.hkv, np.arange(n))
            reps_cpu += 1
        secs = (time.perf_counter() - t0) / reps_cpu
        cpu = {"value": round(n * page_bytes / secs / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"oracle spill_pages of {n} pages ({n * page_bytes / 1e6:.0f} MB) host to host, "
                         f"{reps_cpu} repetitions in ~10 s"}
    rec = {
        "metric": "NVFP4 page spill to pinned host memory, GB/s (pages/s)",
        "value": round(total / sp / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": reps, "warmup": 1, "ms_per_step": round((sp + re_) * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{wl.name}: the {wl.seq_lens[seq]}-token sequence's {npg} pages, "
                               f"{wl.layers} layers x {wl.hkv} kv heads ({page_bytes} bytes a page)",
                   "step": "nvfp4kv_spill_pages then nvfp4kv_restore_pages of the same page ids"},
        "pages_per_s": round(npg / sp, 1),
        "restore_gbps": round(total / re_ / 1e9, 2),
        "restore_pages_per_s": round(npg / re_, 1),
        "roofline": {"bound": "pcie", "kernel": "page_copy_kernel", "achieved": round(total / sp / 1e9, 2),
                     "peak": PEAK_PCIE_GBPS, "unit": "GB/s", "frac": round(total / sp / 1e9 / PEAK_PCIE_GBPS, 4),
                     "traffic": None, "restore_achieved": round(total / re_ / 1e9, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
