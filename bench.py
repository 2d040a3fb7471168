"""Benchmark of the attention layer on one MI355X.

One step = the whole prefill path of the layer (key/value preparation,
attention with the fused query prologue, output norm and gate) over the
Glimmer local-layer workload: batch 1, 32768 tokens, 32 query / 2 KV heads,
head width 128, causal window 2048, RoPE base 10000, multiplier 3.87.
`value` is that step's algorithmic throughput (4 * Hq * D FLOPs per visible
(query, key) pair) in TFLOP/s.  The same JSON line carries:
  roofline      - the attention kernel's duration from HIP events recorded
                  around it on the launch stream, against the bf16/f16 MFMA peak;
  cpu_baseline  - the fp64 oracle on a bounded sample of the same workload;
  decode        - the Spark decode step over a paged global-layer cache
                  (16 sequences, lengths uniform in [131072, 1048576]) and a
                  2048-entry ring, in GB/s of cached K/V read, against HBM peak;
  prefill_other - the other prefill workloads (one or two timed reps each).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn prefill TFLOP/s & decode KV GB/s on 1 MI355X (% of MFMA/HBM peak)"
MFMA_PEAK_TFLOPS = 2500.0      # dense bf16 / fp16
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent pairs through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "global_muse_rope_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ["prefill.hip", "kernels.h", "common.h"]
DECODE_SOURCES = ["decode.hip", "kernels.h", "common.h"]


def committed_traffic(name, digest):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


def timed_steps(fn, steps, warmup, events, torch):
    """Run warmup + steps; returns (wall ms per step, mean attention-kernel ms)."""
    import global_muse_rope_amd._capi as capi
    lib = capi.load()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    pairs = [(events.create(), events.create()) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in pairs:
        capi.check(lib.muse_profile_events(a, b))
        fn()
    capi.check(lib.muse_profile_events(None, None))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    kern = sum(events.elapsed_ms(a, b) for a, b in pairs) / steps
    for a, b in pairs:
        events.destroy(a)
        events.destroy(b)
    return wall, kern


def prefill_case(cfg, steps, warmup, events, torch, ma, keep=False):
    from synth.device import prefill_device_inputs
    from global_muse_rope_amd import accounting as acc
    L = cfg.layer
    lp = ma.LayerParams.from_layer(L)
    x = prefill_device_inputs(cfg)
    out = torch.empty((cfg.batch, cfg.seq, L.hq, L.d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ma.prefill_workspace_size(lp, cfg.batch, cfg.seq), dtype=torch.uint8, device="cuda")

    def step():
        ma.prefill(lp, x["q"], x["k"], x["v"], x["g"], out=out, workspace=ws)

    wall, kern = timed_steps(step, steps, warmup, events, torch)
    flops = acc.prefill_flops(L.hq, L.d, cfg.batch, cfg.seq, L.window)
    res = {"ms_per_step": wall, "tflops": flops / (wall * 1e-3) / 1e12, "kernel_ms": kern,
           "kernel_tflops": flops / (kern * 1e-3) / 1e12, "flops": flops}
    if keep:
        res["_tensors"] = (x, out)
    else:
        del x, out, ws
        torch.cuda.empty_cache()
    return res


def chunk_case(cfg, steps, warmup, events, torch, ma, draft=False):
    """Chunked prefill: the chunk after `start` cached positions.  Each step
    rewrites the chunk's own cache entries with the same values, so every
    step sees the same cache."""
    from synth.device import chunk_device_setup
    from global_muse_rope_amd import accounting as acc
    L = cfg.layer
    lp = ma.LayerParams.from_layer(L)
    s = chunk_device_setup(cfg)
    if s["kind"] == "ring":
        cache = ma.KvCache.ring(s["kc"], s["vc"])
    else:
        cache = ma.KvCache.paged(s["kc"], s["vc"], s["block_table"], s["page_tokens"])
    out = torch.empty((cfg.batch, cfg.seq, L.hq, L.d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ma.prefill_chunk_workspace_size(lp, cfg.batch, cfg.seq, cfg.start), dtype=torch.uint8,
                     device="cuda")

    fn = ma.draft_block if draft else ma.prefill_chunk

    def step():
        fn(lp, s["q"], s["k"], s["v"], s["g"], s["start"], cfg.start, cache, out=out, workspace=ws)

    wall, kern = timed_steps(step, steps, warmup, events, torch)
    pairs = (acc.block_pairs if draft else acc.chunk_pairs)(cfg.start, cfg.seq, L.window)
    flops = acc.flops_per_pair(L.hq, L.d) * cfg.batch * pairs
    res = {"ms_per_step": wall, "tflops": flops / (wall * 1e-3) / 1e12, "kernel_ms": kern,
           "kernel_tflops": flops / (kern * 1e-3) / 1e12, "flops": flops}
    del s, cache, out, ws
    torch.cuda.empty_cache()
    return res


def block_case(cfg, steps, warmup, events, torch, ma):
    """The attention half of a decoder block with seeded synthetic weights
    (bf16; the residual gate in fp32) on seeded N(0,1) hidden states."""
    from synth.device import block_device_setup
    from global_muse_rope_amd import accounting as acc
    L = cfg.layer
    s = block_device_setup(cfg)
    w = ma.BlockWeights(in_norm=s["in_norm"], w_qkvg=s["w_qkvg"], w_o=s["w_o"], residual_gate=s["residual_gate"],
                        post_norm=s["post_norm"])
    lp = ma.LayerParams.from_layer(L)
    x = s["x"]
    out = torch.empty_like(x)
    ws = torch.empty(ma.block_prefill_workspace_size(lp, w, cfg.batch, cfg.seq), dtype=torch.uint8, device="cuda")

    def step():
        ma.attention_block_prefill(lp, w, x, out=out, workspace=ws)

    wall, kern = timed_steps(step, steps, warmup, events, torch)
    flops = acc.block_flops(L.hq, L.hkv, L.d, cfg.hidden, cfg.batch, cfg.seq, L.window)
    res = {"ms_per_step": wall, "tflops": flops / (wall * 1e-3) / 1e12, "attn_kernel_ms": kern, "flops": flops}
    del s, w, x, out, ws
    torch.cuda.empty_cache()
    return res


def block_decode_case(cfg, steps, warmup, events, torch, ma, flush=False):
    """One new token per sequence of a decode workload through the attention half
    of a decoder block (hidden 8192, the seeded synthetic weights of the block
    workload) over that workload's cache."""
    from synth.device import decode_device_setup, block_device_setup
    from synth.workloads import SPARK_BLOCK_LOCAL, S_X
    from synth import normal_bf16_torch_tensor
    L = cfg.layer
    s = decode_device_setup(cfg)
    if s["kind"] == "ring":
        cache = ma.KvCache.ring(s["kc"], s["vc"])
    else:
        cache = ma.KvCache.paged(s["kc"], s["vc"], s["block_table"], s["page_tokens"])
    w = block_device_setup(SPARK_BLOCK_LOCAL)   # the weights depend on the head shape and width only
    wb = ma.BlockWeights(in_norm=w["in_norm"], w_qkvg=w["w_qkvg"], w_o=w["w_o"], residual_gate=w["residual_gate"],
                         post_norm=w["post_norm"])
    lp = ma.LayerParams.from_layer(L)
    x = normal_bf16_torch_tensor(cfg.seed, S_X, (cfg.batch, SPARK_BLOCK_LOCAL.hidden), "cuda")
    out = torch.empty_like(x)
    ws = torch.empty(ma.block_decode_workspace_size(lp, wb, cfg.batch, s["max_len"], cache), dtype=torch.uint8,
                     device="cuda")
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if flush else None

    def step():
        if scrub is not None:
            scrub.view(torch.int64).sum()   # evict the 256 MB last-level cache (a read: no dirty lines left)
        ma.attention_block_decode(lp, wb, x, s["kv_len"], s["max_len"], cache, out=out, workspace=ws)

    wall, kern = timed_steps(step, steps, warmup, events, torch)
    res = {"ms_per_step": wall, "decode_kernel_ms": kern}
    del s, cache, w, wb, x, out, ws, scrub
    torch.cuda.empty_cache()
    return res


def decode_case(cfg, steps, warmup, events, torch, ma, flush=False, fp8=False):
    from synth.device import decode_device_setup
    from global_muse_rope_amd import accounting as acc
    L = cfg.layer
    s = decode_device_setup(cfg, fp8=fp8)
    ks, vs = s.get("k_scale"), s.get("v_scale")
    if s["kind"] == "ring":
        s["cache"] = ma.KvCache.ring(s["kc"], s["vc"], ks, vs)
    else:
        s["cache"] = ma.KvCache.paged(s["kc"], s["vc"], s["block_table"], s["page_tokens"], ks, vs)
    lp = ma.LayerParams.from_layer(L)
    ws = torch.empty(ma.decode_workspace_size(lp, cfg.batch, s["max_len"], s["cache"]), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((cfg.batch, L.hq, L.d), dtype=torch.bfloat16, device="cuda")
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if flush else None

    def step():
        if scrub is not None:
            # evict the 256 MB last-level cache between steps with a 512 MB read: a write
            # would leave dirty lines whose write-back then competes with the step's reads
            scrub.view(torch.int64).sum()
        ma.decode(lp, s["q"], s["k"], s["v"], s["g"], s["kv_len"], s["max_len"], s["cache"], out=out, workspace=ws)

    wall, kern = timed_steps(step, steps, warmup, events, torch)
    eb = 1 if fp8 else 2
    kv_bytes = acc.decode_kv_bytes(L.hkv, L.d, s["lengths"], L.window, eb)
    if fp8:
        kv_bytes += acc.decode_scale_bytes(L.hkv, s["lengths"], L.window, s["page_tokens"])
    io = acc.decode_io_bytes(L.hq, L.hkv, L.d, cfg.batch, eb)
    res = {"kernel_ms": kern, "kv_bytes": kv_bytes, "gbs": (kv_bytes + io) / (kern * 1e-3) / 1e9,
           "ms_per_step": wall, "lengths_sum": int(sum(s["lengths"]))}
    del s, ws, out, scrub
    torch.cuda.empty_cache()
    return res


def copy_bandwidth(torch, events, nbytes=2 << 30, reps=5):
    """A plain device-to-device copy (the runtime's blit kernel) of `nbytes`:
    bytes read + written per second, the practical HBM ceiling the decode
    figures are also compared with."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = events.create(), events.create()
    stream = torch.cuda.current_stream().cuda_stream
    hip = events.hip
    hip.hipEventRecord(e0, stream)
    for _ in range(reps):
        b.copy_(a)
    hip.hipEventRecord(e1, stream)
    torch.cuda.synchronize()
    ms = events.elapsed_ms(e0, e1) / reps
    events.destroy(e0)
    events.destroy(e1)
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(cfg, gpu_out, budget_s=15.0):
    """The fp64 oracle, as it stands, on a bounded sample of rows of the same
    workload; returns its throughput in TFLOP/s and the GPU/oracle max-abs
    difference on those rows."""
    import numpy as np
    import oracle
    from global_muse_rope_amd import accounting as acc
    from synth.device import host_tokens, host_rows
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    L = cfg.layer
    T = cfg.seq
    k = host_tokens(cfg, "k", 0, 0, T)   # [T, Hkv, D] float64
    v = host_tokens(cfg, "v", 0, 0, T)
    rng = np.random.default_rng(1)
    order = np.concatenate([[0, 1, L.window - 2, L.window - 1, L.window, T - 1],
                            rng.permutation(T)]).astype(np.int64)
    gpu = gpu_out.float().cpu().numpy()[0] if gpu_out is not None else None
    t_start = time.perf_counter()
    done, flops, worst = 0, 0, 0.0
    elapsed = 0.0
    while done < len(order) and elapsed < budget_s:
        rows = order[done:done + 128]
        q = host_rows(cfg, "q", 0, rows)
        g = host_rows(cfg, "g", 0, rows)
        t0 = time.perf_counter()
        y = oracle.prefill(q, k[:rows.max() + 1], v[:rows.max() + 1], g, L, rows=rows)
        elapsed += time.perf_counter() - t0
        for r in rows:
            lo, hi = oracle.visible_range(int(r), L.window)
            flops += acc.flops_per_pair(L.hq, L.d) * (hi - lo + 1)
        if gpu is not None:
            worst = max(worst, float(np.max(np.abs(gpu[rows] - y))))
        done += len(rows)
    wall = time.perf_counter() - t_start
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} query rows (all {L.hq} heads) of {cfg.name}, chosen by a seeded permutation "
                      f"plus window-edge rows; {flops / 1e9:.1f} GFLOP in {elapsed:.1f} s of oracle time "
                      f"({wall:.1f} s with input regeneration)",
            "gpu_max_abs_err_on_sample": worst, "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pmc_pass(torch, ma, workload):
    """A short run for rocprofv3 counter passes: two steps of one workload
    (prefill or decode; default: the benchmark workload) and one plain 1 GiB
    device copy as the calibration of the byte counters."""
    from synth import workloads as wl
    cfgs = {c.name: c for c in wl.PREFILL + wl.DECODE}
    cfg = cfgs[workload]
    if cfg in wl.DECODE:
        decode_case(cfg, 1, 1, HipEvents(), torch, ma)
    else:
        prefill_case(cfg, 1, 1, HipEvents(), torch, ma)
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"pmc pass done: 2 steps of {workload} + 1 GiB copy")


def _counter_rows(path):
    """(kernel name, counter value) per dispatch from a rocprofv3 counter CSV."""
    import csv
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def traffic_summary(workload, kernel, fetch_csv, write_csv, commands):
    """HBM bytes per launch of `kernel` from one FETCH_SIZE and one WRITE_SIZE
    rocprofv3 pass over `bench.py --pmc-pass`, each scaled by what the same
    counter reads for the pass's plain 1 GiB copy; written next to the other
    profile summaries with the digest of the kernel sources it was taken on."""
    copy_bytes = float(1 << 30)
    res = {"workload": workload, "kernel": kernel, "commands": commands}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        kern = [v for n, v in rows if kernel in n]
        copy = [v for n, v in rows if "copyBuffer" in n]   # the runtime's blit kernel doing the 1 GiB copy
        if not kern or not copy:
            raise SystemExit(f"{path}: no {kernel} or copy dispatch found")
        kib = sum(kern) / len(kern)
        copy_kib = max(copy)
        factor = (copy_bytes / 1024) / copy_kib
        res[name] = {"kib_per_dispatch": kib, "dispatches": len(kern), "copy_kib": copy_kib,
                     "scale": round(factor, 4), "bytes_per_launch": kib * 1024 * factor}
        total += kib * 1024 * factor
    res["hbm_bytes_per_launch"] = total
    srcs = PREFILL_SOURCES if "prefill" in kernel else DECODE_SOURCES
    res["source_digest"] = source_digest(srcs)
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def only_case(name, steps, warmup, torch, ma):
    """Time one workload by itself (for a per-workload kernel trace)."""
    from synth import workloads as wl
    fp8 = name.endswith("_fp8")
    through_block = name.endswith("_block")
    base = name[:-4] if fp8 else name[:-6] if through_block else name
    cfg = {c.name: c for c in wl.PREFILL + wl.DECODE + wl.CHUNK + wl.DRAFT + wl.BLOCKS}[base]
    events = HipEvents()
    if through_block and cfg in wl.DECODE:
        r = block_decode_case(cfg, steps, warmup, events, torch, ma, flush=cfg.layer.window > 0)
        print(json.dumps({"workload": name, "ms_per_step": round(r["ms_per_step"], 4),
                          "decode_kernel_ms": round(r["decode_kernel_ms"], 4), "steps": steps, "warmup": warmup}),
              flush=True)
    elif cfg in wl.BLOCKS:
        r = block_case(cfg, steps, warmup, events, torch, ma)
        print(json.dumps({"workload": name, "ms_per_step": round(r["ms_per_step"], 4),
                          "step_TFLOP/s": round(r["tflops"], 2), "attn_kernel_ms": round(r["attn_kernel_ms"], 4),
                          "steps": steps, "warmup": warmup}), flush=True)
    elif cfg in wl.CHUNK or cfg in wl.DRAFT:
        r = chunk_case(cfg, steps, warmup, events, torch, ma, draft=cfg in wl.DRAFT)
        print(json.dumps({"workload": name, "kernel": "prefill_kernel", "kernel_ms": round(r["kernel_ms"], 4),
                          "kernel_TFLOP/s": round(r["kernel_tflops"], 2), "step_TFLOP/s": round(r["tflops"], 2),
                          "ms_per_step": round(r["ms_per_step"], 4), "steps": steps, "warmup": warmup}),
              flush=True)
    elif cfg in wl.DECODE:
        r = decode_case(cfg, steps, warmup, events, torch, ma, flush=cfg.layer.window > 0, fp8=fp8)
        print(json.dumps({"workload": name, "kernel": "decode_split_kernel", "kernel_ms": round(r["kernel_ms"], 4),
                          "GB/s": round(r["gbs"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                          "steps": steps, "warmup": warmup}), flush=True)
    else:
        r = prefill_case(cfg, steps, warmup, events, torch, ma)
        print(json.dumps({"workload": name, "kernel": "prefill_kernel", "kernel_ms": round(r["kernel_ms"], 4),
                          "kernel_TFLOP/s": round(r["kernel_tflops"], 2), "step_TFLOP/s": round(r["tflops"], 2),
                          "ms_per_step": round(r["ms_per_step"], 4), "steps": steps, "warmup": warmup}),
              flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="only the benchmark workload and the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--pmc-workload", default="glimmer_local_prefill_32k")
    ap.add_argument("--only", metavar="WORKLOAD", help="time one workload by itself and print its line")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("WORKLOAD", "KERNEL", "FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic summary of two counter passes (no GPU needed)")
    ap.add_argument("--commands", default="", help="the rocprofv3 commands, recorded in the summary")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.commands)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import global_muse_rope_amd as ma
    from synth import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ma._capi.load()   # fails loudly if the library is missing
    if args.pmc_pass:
        pmc_pass(torch, ma, args.pmc_workload)
        return
    if args.only:
        only_case(args.only, args.steps, args.warmup, torch, ma)
        return
    events = HipEvents()
    props = torch.cuda.get_device_properties(0)

    cfg = wl.GLIMMER_LOCAL
    log(f"prefill {cfg.name}: warmup {args.warmup}, steps {args.steps}")
    main_res = prefill_case(cfg, args.steps, args.warmup, events, torch, ma, keep=True)
    x, gpu_out = main_res.pop("_tensors")
    log(f"  {main_res['tflops']:.1f} TFLOP/s step, attention kernel {main_res['kernel_ms']:.3f} ms "
        f"({main_res['kernel_tflops']:.1f} TFLOP/s)")
    digest = source_digest(PREFILL_SOURCES)
    traffic = committed_traffic(f"prefill_kernel_{cfg.name}", digest)
    result = {
        "metric": METRIC,
        "value": round(main_res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seq, "q_heads": cfg.layer.hq,
                   "kv_heads": cfg.layer.hkv, "head_dim": cfg.layer.d, "window": cfg.layer.window,
                   "rope_theta": cfg.layer.theta, "qk_scale": cfg.layer.scale, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(main_res["kernel_tflops"], 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(main_res["kernel_tflops"] / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill_kernel", "kernel_ms": round(main_res["kernel_ms"], 4),
                     "flops_per_launch": main_res["flops"], "source_digest": digest},
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    if not args.no_cpu:
        log("cpu baseline (oracle, bounded sample)")
        result["cpu_baseline"] = cpu_baseline(cfg, gpu_out)
        log(f"  {result['cpu_baseline']['sample']}")
    del x, gpu_out
    torch.cuda.empty_cache()

    if not args.no_decode:
        copy_gbs = copy_bandwidth(torch, events)
        log(f"device copy {copy_gbs:.0f} GB/s (read + write)")
        result["hbm_copy_gbs"] = round(copy_gbs, 1)
        dec = {}
        for dcfg, steps, flush, fp8 in [(wl.SPARK_DECODE_GLOBAL, 10, False, False),
                                        (wl.SPARK_DECODE_LOCAL, 20, True, False),
                                        (wl.SPARK_DECODE_GLOBAL, 10, False, True)]:
            name = dcfg.name + ("_fp8" if fp8 else "")
            log(f"decode {name}")
            r = decode_case(dcfg, steps, 2, events, torch, ma, flush=flush, fp8=fp8)
            log(f"  {r['gbs']:.0f} GB/s, split kernel {r['kernel_ms']:.3f} ms")
            dec[name] = {"value": round(r["gbs"], 1), "unit": "GB/s", "kernel": "decode_split_kernel",
                         "cache_dtype": "e4m3" if fp8 else "bf16",
                         "kernel_ms": round(r["kernel_ms"], 4), "ms_per_step": round(r["ms_per_step"], 4),
                         "kv_bytes_per_step": r["kv_bytes"], "cache_flushed": flush,
                         "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                                      "frac_of_copy": round(r["gbs"] / copy_gbs, 4)}}
        result["decode"] = dec

    if not args.no_decode:
        chunks = {}
        for ccfg in wl.CHUNK:
            log(f"prefill chunk {ccfg.name}")
            r = chunk_case(ccfg, 5, 1, events, torch, ma)
            log(f"  {r['tflops']:.1f} TFLOP/s step, kernel {r['kernel_tflops']:.1f} TFLOP/s")
            chunks[ccfg.name] = {"tflops_step": round(r["tflops"], 2), "ms_per_step": round(r["ms_per_step"], 4),
                                 "kernel_tflops": round(r["kernel_tflops"], 2),
                                 "kernel_ms": round(r["kernel_ms"], 4),
                                 "frac_of_mfma_peak": round(r["kernel_tflops"] / MFMA_PEAK_TFLOPS, 4)}
        result["prefill_chunk"] = chunks
        draft = {}
        for bcfg in wl.DRAFT:
            log(f"draft block {bcfg.name}")
            r = chunk_case(bcfg, 20, 3, events, torch, ma, draft=True)
            log(f"  {r['ms_per_step'] * 1e3:.1f} us per step, kernel {r['kernel_tflops']:.1f} TFLOP/s")
            draft[bcfg.name] = {"us_per_step": round(r["ms_per_step"] * 1e3, 2),
                                "kernel_us": round(r["kernel_ms"] * 1e3, 2),
                                "tflops_step": round(r["tflops"], 2), "kernel_tflops": round(r["kernel_tflops"], 2)}
        result["draft_block"] = draft
        blocks = {}
        for kcfg in wl.BLOCKS:
            log(f"attention block {kcfg.name}")
            r = block_case(kcfg, 5, 1, events, torch, ma)
            log(f"  {r['ms_per_step']:.3f} ms per step, {r['tflops']:.1f} TFLOP/s")
            blocks[kcfg.name] = {"ms_per_step": round(r["ms_per_step"], 4), "tflops_step": round(r["tflops"], 2),
                                 "attn_kernel_ms": round(r["attn_kernel_ms"], 4)}
        result["attention_block"] = blocks
        block_dec = {}
        for dcfg in wl.DECODE:
            log(f"decode through the block: {dcfg.name}")
            r = block_decode_case(dcfg, 5, 1, events, torch, ma, flush=dcfg.layer.window > 0)
            log(f"  {r['ms_per_step']:.3f} ms per step (decode split kernel {r['decode_kernel_ms']:.3f} ms)")
            block_dec[dcfg.name] = {"ms_per_step": round(r["ms_per_step"], 4),
                                    "decode_kernel_ms": round(r["decode_kernel_ms"], 4),
                                    "cache_flushed": dcfg.layer.window > 0}
        result["attention_block_decode"] = block_dec

    if not args.quick:
        other = {}
        for pcfg in [wl.GLIMMER_GLOBAL, wl.SPARK_LOCAL, wl.SPARK_GLOBAL]:
            log(f"prefill {pcfg.name}")
            r = prefill_case(pcfg, 2, 1, events, torch, ma)
            log(f"  {r['tflops']:.1f} TFLOP/s step, kernel {r['kernel_tflops']:.1f} TFLOP/s")
            other[pcfg.name] = {"tflops_step": round(r["tflops"], 2), "ms_per_step": round(r["ms_per_step"], 3),
                                "kernel_tflops": round(r["kernel_tflops"], 2),
                                "frac_of_mfma_peak": round(r["kernel_tflops"] / MFMA_PEAK_TFLOPS, 4)}
        result["prefill_other"] = other

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
