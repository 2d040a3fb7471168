"""Benchmark of the attention layer on one MI355X.

One step = the whole prefill path of the layer (key/value preparation,
attention with the fused query prologue, output norm and gate) over the
Glimmer local-layer workload: batch 1, 32768 tokens, 32 query / 2 KV heads,
head width 128, causal window 2048, RoPE base 10000, multiplier 3.87.
`value` is that step's algorithmic throughput (4 * Hq * D FLOPs per visible
(query, key) pair) in TFLOP/s.  The same JSON line carries:
  roofline      - the attention kernel's duration from HIP events recorded
                  around it on the launch stream, against the bf16/f16 MFMA peak,
                  with the HBM bytes per launch from calibrated rocprofv3
                  counters when they were taken on the current kernel sources;
  cpu_baseline  - the fp64 oracle on a bounded sample of the same workload;
  one block per other workload, each with its own roofline, oracle baseline
  and median over timed reps:
    glimmer_global_prefill_128k - 131072 tokens, global NoPE layer;
    spark_prefill_256k          - 262144 tokens, one local and one global layer;
    spark_decode                - 16 sequences, lengths uniform in [131072,
                                  1048576], over a paged global-layer cache (bf16
                                  and E4M3) and a 2048-entry ring, in GB/s of
                                  cached K/V read against HBM peak;
  and the next rows: chunked prefill, the drafter block, the decoder block.

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
DRAFT_SOURCES = ["draft.hip", "draft.h", "kernels.h", "common.h"]


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


def timed_steps(fn, steps, warmup, events, torch, per_step=None):
    """Run warmup, then `steps` plain steps between two synchronizations (the
    wall time), then `steps` more with the library's HIP events recorded
    around its attention kernels on their stream (the kernel times: the
    per-step event calls are kept out of the wall time).  Returns (wall ms
    per step, mean attention-kernel ms); per_step (a list) receives each
    step's attention-kernel ms."""
    import global_muse_rope_amd._capi as capi
    lib = capi.load()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    pairs = [(events.create(), events.create()) for _ in range(steps)]
    for a, b in pairs:
        capi.check(lib.muse_profile_events(a, b))
        fn()
    capi.check(lib.muse_profile_events(None, None))
    torch.cuda.synchronize()
    each = [events.elapsed_ms(a, b) for a, b in pairs]
    if per_step is not None:
        per_step.extend(each)
    kern = sum(each) / steps
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

    each = []
    wall, kern = timed_steps(step, steps, warmup, events, torch, each)
    flops = acc.prefill_flops(L.hq, L.d, cfg.batch, cfg.seq, L.window)
    res = {"ms_per_step": wall, "tflops": flops / (wall * 1e-3) / 1e12, "kernel_ms": kern,
           "kernel_tflops": flops / (kern * 1e-3) / 1e12, "flops": flops, "kernel_ms_each": each}
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
    size_fn = ma.draft_block_workspace_size if draft else ma.prefill_chunk_workspace_size
    ws = torch.empty(size_fn(lp, cfg.batch, cfg.seq, cfg.start), dtype=torch.uint8, device="cuda")

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

    # pick the projection GEMMs' algorithms once, outside the timed region
    ma.attention_block_tune(lp, w, cfg.batch * cfg.seq, workspace=ws)
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

    tune_ws = torch.empty(ma.block_prefill_workspace_size(lp, wb, 1, cfg.batch), dtype=torch.uint8, device="cuda")
    ma.attention_block_tune(lp, wb, cfg.batch, workspace=tune_ws)
    del tune_ws

    wall, kern = timed_steps(step, steps, warmup, events, torch)
    res = {"ms_per_step": wall, "decode_kernel_ms": kern}
    del s, cache, w, wb, x, out, ws, scrub
    torch.cuda.empty_cache()
    return res


def decode_case(cfg, steps, warmup, events, torch, ma, flush=False, fp8=False, keep_out=False, plain_fill=False):
    from synth.device import decode_device_setup
    from global_muse_rope_amd import accounting as acc
    L = cfg.layer
    s = decode_device_setup(cfg, fp8=fp8, plain_fill=plain_fill)
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

    each = []
    wall, kern = timed_steps(step, steps, warmup, events, torch, each)
    eb = 1 if fp8 else 2
    kv_bytes = acc.decode_kv_bytes(L.hkv, L.d, s["lengths"], L.window, eb)
    if fp8:
        kv_bytes += acc.decode_scale_bytes(L.hkv, s["lengths"], L.window, s["page_tokens"])
    io = acc.decode_io_bytes(L.hq, L.hkv, L.d, cfg.batch, eb)
    res = {"kernel_ms": kern, "kv_bytes": kv_bytes, "io_bytes": io,
           "gbs": (kv_bytes + io) / (kern * 1e-3) / 1e9, "ms_per_step": wall,
           "lengths_sum": int(sum(s["lengths"])), "kernel_ms_each": each, "lengths": s["lengths"]}
    if keep_out:
        res["_out"] = out.float().cpu().numpy()
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


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def baseline_order(cfg, row_limit=None):
    """Query rows the oracle baseline takes, in order: the window-edge rows,
    then a seeded permutation of the rows below row_limit."""
    import numpy as np
    lim = min(cfg.seq, row_limit or cfg.seq)
    W = cfg.layer.window
    rng = np.random.default_rng(1)
    edge = [r for r in [0, 1, W - 2, W - 1, W, lim - 1] if 0 <= r < lim]
    return np.concatenate([edge, rng.permutation(lim)]).astype(np.int64), lim


BASELINE_ROWS = 8192   # GPU output rows kept on the host for the oracle baseline


def keep_baseline_rows(cfg, out, row_limit=None):
    """The GPU outputs of the first BASELINE_ROWS rows of the baseline order,
    copied to the host right after the timed run (bf16, [n, Hq, D])."""
    order, _ = baseline_order(cfg, row_limit)
    return out[0, torch_index(order[:BASELINE_ROWS])].cpu()


def cpu_baseline(cfg, gpu_rows, budget_s=15.0, row_limit=None, kv=None):
    """The fp64 oracle, as it stands, on a bounded sample of query rows of the
    same workload (baseline_order).  Returns its throughput in TFLOP/s, the
    full-workload oracle time extrapolated per visible pair, and the
    GPU/oracle max-abs difference on those rows (gpu_rows: the GPU's outputs
    of the first rows of that order).  kv: host (k, v) of tokens 0 ..
    row_limit - 1, if already regenerated."""
    import numpy as np
    import oracle
    from global_muse_rope_amd import accounting as acc
    from synth.device import host_tokens, host_rows
    L = cfg.layer
    T = cfg.seq
    order, lim = baseline_order(cfg, row_limit)
    order = order[:BASELINE_ROWS]
    if kv is None:
        kv = (host_tokens(cfg, "k", 0, 0, lim), host_tokens(cfg, "v", 0, 0, lim))   # [lim, Hkv, D] float64
    k, v = kv
    t_start = time.perf_counter()
    done, pairs, worst = 0, 0, 0.0
    elapsed = 0.0
    while done < len(order) and elapsed < budget_s:
        rows = order[done:done + 64]
        q = host_rows(cfg, "q", 0, rows)
        g = host_rows(cfg, "g", 0, rows)
        t0 = time.perf_counter()
        y = oracle.prefill(q, k[:rows.max() + 1], v[:rows.max() + 1], g, L, rows=rows)
        elapsed += time.perf_counter() - t0
        for r in rows:
            lo, hi = oracle.visible_range(int(r), L.window)
            pairs += hi - lo + 1
        if gpu_rows is not None:
            gy = gpu_rows[done:done + len(rows)].float().numpy()
            worst = max(worst, float(np.max(np.abs(gy - y))))
        done += len(rows)
    flops = acc.flops_per_pair(L.hq, L.d) * pairs
    wall = time.perf_counter() - t_start
    total_pairs = acc.visible_pairs(T, L.window) * cfg.batch
    where = "" if lim == T else f" among the first {lim} tokens"
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(_threads()), "kind": "oracle",
            "sample": f"{done} query rows{where} (all {L.hq} heads) of {cfg.name}, window-edge rows then a seeded "
                      f"permutation; {flops / 1e9:.1f} GFLOP in {elapsed:.1f} s of oracle time "
                      f"({wall:.1f} s with input regeneration)",
            "extrapolated_full_s": elapsed / pairs * total_pairs,
            "gpu_max_abs_err_on_sample": worst, "cpu_model": cpu_model()}


def torch_index(rows):
    import torch
    return torch.as_tensor(rows, dtype=torch.int64, device="cuda")


def cpu_baseline_decode(cfg, y_gpu, lengths, budget_s=10.0):
    """The fp64 oracle on the decode workload: (sequence, KV head) pairs,
    shortest sequences first, each one decode step over its whole history,
    streamed from the host regeneration of its cached entries, until budget_s
    of oracle time (or twice that of wall time) is spent.  Rate: cached K and
    V bytes the oracle reads per second; plus the GPU/oracle max-abs
    difference on those pairs."""
    import numpy as np
    import oracle
    from synth import device as sd
    L = cfg.layer
    G = L.group
    new = sd.new_token_host(cfg)
    lay = type(L)(hq=G, hkv=1, d=L.d, window=L.window, theta=L.theta, scale=L.scale, qk_eps=L.qk_eps,
                  out_norm=L.out_norm, out_eps=L.out_eps)
    elapsed, nbytes, worst, done, seqs = 0.0, 0, 0.0, 0, []
    t_start = time.perf_counter()
    for b in (int(i) for i in np.argsort(lengths, kind="stable")):
        Lb = int(lengths[b])
        p = Lb - 1
        lo, _ = oracle.visible_range(p, L.window)
        for hk in range(L.hkv):
            if elapsed >= budget_s or time.perf_counter() - t_start >= 2 * budget_s:
                break
            kh = sd.cache_values_host(cfg.seed, b, hk, L.hkv, "k", lo, p, L.d)[:, None, :]
            vh = sd.cache_values_host(cfg.seed, b, hk, L.hkv, "v", lo, p, L.d)[:, None, :]
            hs = slice(hk * G, (hk + 1) * G)
            t0 = time.perf_counter()
            ref = oracle.decode_one(new["q"][b, hs], new["k"][b, hk:hk + 1], new["v"][b, hk:hk + 1],
                                    new["g"][b, hs], kh, vh, lo, Lb, lay)
            elapsed += time.perf_counter() - t0
            nbytes += (p - lo) * 2 * L.d * 2
            worst = max(worst, float(np.max(np.abs(y_gpu[b, hs] - ref))))
            done += 1
            if not seqs or seqs[-1][0] != b:
                seqs.append((b, p - lo))
        else:
            continue
        break
    wall = time.perf_counter() - t_start
    span = ", ".join(f"{b} ({n} entries)" for b, n in seqs[:4]) + (", ..." if len(seqs) > 4 else "")
    return {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": int(_threads()), "kind": "oracle",
            "sample": f"{done} (sequence, KV head) pairs of {len(seqs)} sequence(s) of {cfg.name}, shortest first: "
                      f"{span}; each one decode step over the sequence's cached entries; {nbytes / 1e9:.2f} GB of "
                      f"bf16 K and V in {elapsed:.2f} s of oracle time ({wall:.1f} s with cache regeneration)",
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
    (prefill, decode or drafter block; default: the benchmark workload) and
    one plain 1 GiB device copy as the calibration of the byte counters."""
    from synth import workloads as wl
    cfgs = {c.name: c for c in wl.PREFILL + wl.DECODE + wl.DRAFT}
    fp8 = workload.endswith("_fp8")
    cfg = cfgs[workload[:-4] if fp8 else workload]
    if cfg in wl.DRAFT:
        chunk_case(cfg, 1, 1, HipEvents(), torch, ma, draft=True)
    elif cfg in wl.DECODE:
        # the byte counters do not depend on the cached values: one fill per pool (a few launches
        # instead of the seeded streams' thousands)
        decode_case(cfg, 1, 1, HipEvents(), torch, ma, flush=cfg.layer.window > 0, fp8=fp8, plain_fill=True)
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
    res = {"workload": workload, "kernel": kernel, "commands": [c for c in commands.split(" ;; ") if c]}
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
    srcs = PREFILL_SOURCES if "prefill" in kernel else DRAFT_SOURCES if "draft" in kernel else DECODE_SOURCES
    res["source_digest"] = source_digest(srcs)
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def _dispatch_durations(trace_csv, kernel):
    """Dispatch id -> duration (ns) of `kernel` from a rocprofv3 kernel-trace CSV."""
    import csv
    out = {}
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                out[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out


def counter_summary(workload, kernel, run_dirs, commands, cus=256, xcds=8):
    """Markdown summary of SQ/GRBM counter passes over `kernel` (one rocprofv3
    output directory per pass, each holding run_counter_collection.csv and
    run_kernel_trace.csv), per dispatch, averaged over the kernel's
    dispatches, with derived figures.  GRBM_GUI_ACTIVE is summed over the
    XCDs (its ratio to the kernel's duration is xcds times the shader clock);
    SQ_VALU_MFMA_BUSY_CYCLES counts SIMD cycles with a matrix instruction in
    flight; SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* count wave
    quad-cycles."""
    import csv
    import statistics
    vals, durs = {}, []
    for d in run_dirs:
        dd = _dispatch_durations(os.path.join(d, "run_kernel_trace.csv"), kernel)
        per = {}
        with open(os.path.join(d, "run_counter_collection.csv"), newline="") as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for disp, cs in per.items():
            for c, v in cs.items():
                vals.setdefault(c, []).append(v)
            if disp in dd and "GRBM_GUI_ACTIVE" in cs:
                durs.append((dd[disp], cs["GRBM_GUI_ACTIVE"]))
    mean = {c: statistics.fmean(v) for c, v in vals.items()}
    lines = [f"# `{kernel}` on `{workload}`: SQ and GRBM counters", "",
             "Counter passes (one rocprofv3 run each, counters per dispatch, with the kernel trace of the same run "
             "for the durations), then this summary:", "", "```", *commands, "```", "",
             "| counter | mean per dispatch | dispatches |", "|---|---|---|"]
    for c in sorted(mean):
        lines.append(f"| {c} | {mean[c]:.6g} | {len(vals[c])} |")
    lines += ["", "Derived (per dispatch):", ""]
    dur_ns = statistics.fmean(d for d, _ in durs) if durs else None
    grbm = mean.get("GRBM_GUI_ACTIVE")
    if dur_ns and durs:
        clk = statistics.fmean(g / xcds / d for d, g in durs)
        lines.append(f"- kernel duration in the counter runs: {dur_ns / 1e6:.4f} ms; shader clock "
                     f"GRBM_GUI_ACTIVE / {xcds} / duration = **{clk:.3f} GHz**")
    if grbm and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (grbm / xcds * cus * 4)
        lines.append(f"- matrix cores busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x {cus} CUs x 4 "
                     f"SIMDs) = **{100 * busy:.1f} %** of the cycles")
    if grbm and "SQ_BUSY_CU_CYCLES" in mean:
        lines.append(f"- CUs busy: SQ_BUSY_CU_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x {cus}) = "
                     f"{100 * mean['SQ_BUSY_CU_CYCLES'] / (grbm / xcds * cus):.1f} %")
    wc = mean.get("SQ_WAVE_CYCLES")
    for c, what in (("SQ_WAIT_ANY", "waiting at s_waitcnt"), ("SQ_WAIT_INST_ANY", "waiting to issue"),
                    ("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_ACTIVE_INST_VALU", "issuing vector-ALU work"),
                    ("SQ_ACTIVE_INST_LDS", "issuing LDS work"), ("SQ_WAIT_INST_LDS", "waiting to issue LDS work")):
        if wc and c in mean:
            lines.append(f"- share of wave time {what}: {c} / SQ_WAVE_CYCLES = {100 * mean[c] / wc:.1f} %")
    mf = mean.get("SQ_INSTS_MFMA")
    for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
        if mf and c in mean:
            lines.append(f"- {c} per matrix instruction: {mean[c] / mf:.2f}")
    if "SQ_INSTS_LDS" in mean and "SQ_LDS_BANK_CONFLICT" in mean:
        lines.append(f"- LDS bank-conflict cycles per LDS instruction: "
                     f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_INSTS_LDS']:.4f}")
    text = "\n".join(lines) + "\n"
    path = os.path.join(PROFILES, f"{kernel}_{workload}_sq_counters.md")
    with open(path, "w") as f:
        f.write(text)
    print(text)


def trace_summary(workload, kernel, stats_csv, bench_log, commands):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of
    `bench.py --only WORKLOAD`: the library's kernels and the largest others,
    with the HIP-event figure the same run printed, written next to the other
    profile summaries."""
    import csv
    with open(stats_csv, newline="") as f:
        rows = list(csv.DictReader(f))
    lib = [r for r in rows if "muse::" in r["Name"] or "copyBuffer" in r["Name"]]
    other = [r for r in rows if r not in lib][:3]
    lines = [f"# `{kernel}` on `{workload}`: rocprofv3 kernel trace", "", "Command (one MI355X):", "", "```",
             *commands, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in lib + other:
        name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    main = [r for r in rows if kernel in r["Name"]]
    if main:
        calls = sum(int(r["Calls"]) for r in main)
        avg = sum(float(r["TotalDurationNs"]) for r in main) / calls
        lines += ["", f"`{kernel}` average over the trace: {avg / 1e6:.4f} ms over {calls} launches "
                      "(warm-up launches included)."]
    with open(bench_log) as f:
        js = [ln for ln in f if ln.startswith("{")]
    if js:
        lines += ["", "The same run's line (HIP events recorded around the kernel on its launch stream, timed steps "
                      "only):", "", "```", js[-1].strip(), "```"]
    path = os.path.join(PROFILES, f"{kernel}_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
        kname = "draft_split_kernel + draft_combine_kernel" if cfg in wl.DRAFT else "prefill_kernel"
        print(json.dumps({"workload": name, "kernel": kname, "kernel_ms": round(r["kernel_ms"], 4),
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


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _prefill_roofline(r, cfg):
    digest = source_digest(PREFILL_SOURCES)
    med = _median(r["kernel_ms_each"])
    achieved = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
            "frac_at_median": round(r["flops"] / (med * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "traffic": committed_traffic(f"prefill_kernel_{cfg.name}", digest), "kernel": "prefill_kernel",
            "kernel_ms_median": round(med, 4), "kernel_ms_mean": round(r["kernel_ms"], 4),
            "flops_per_launch": r["flops"], "source_digest": digest}


def prefill_block(cfg, steps, warmup, events, torch, ma, cpu=True, row_limit=16384, kv=None):
    """One prefill workload timed on its own (median over `steps` reps of the
    attention kernel), with its roofline and the oracle on a row sample."""
    log(f"prefill {cfg.name}: warmup {warmup}, reps {steps}")
    r = prefill_case(cfg, steps, warmup, events, torch, ma, keep=True)
    x, out = r.pop("_tensors")
    block = {"workload": cfg.name, "value": round(r["tflops"], 2), "unit": "TFLOP/s",
             "ms_per_step": round(r["ms_per_step"], 4), "reps": steps, "warmup": warmup,
             "config": {"batch": cfg.batch, "seq_len": cfg.seq, "q_heads": cfg.layer.hq, "kv_heads": cfg.layer.hkv,
                        "head_dim": cfg.layer.d, "window": cfg.layer.window, "rope_theta": cfg.layer.theta,
                        "qk_scale": cfg.layer.scale, "out_norm": cfg.layer.out_norm},
             "roofline": _prefill_roofline(r, cfg)}
    log(f"  {r['tflops']:.1f} TFLOP/s step, kernel median {block['roofline']['kernel_ms_median']:.3f} ms "
        f"({block['roofline']['frac']:.3f} of MFMA peak)")
    if cpu:
        # the oracle runs after every GPU timing (its host threads would slow launch-bound steps)
        rows = keep_baseline_rows(cfg, out, row_limit)
        PENDING.append((block, "cpu_baseline",
                        lambda: cpu_baseline(cfg, rows, row_limit=row_limit, kv=kv() if callable(kv) else kv),
                        cfg.name))
    del x, out
    torch.cuda.empty_cache()
    return block


PENDING = []   # (block, key, oracle baseline to run once the GPU timings are done, label)


def run_pending():
    for block, key, fn, label in PENDING:
        log(f"cpu baseline (oracle) {label}")
        block[key] = fn()
        log(f"  {block[key]['sample']}")
    PENDING.clear()


def spark_prefill_block(events, torch, ma, cpu=True):
    """The Spark 262144-token workload: one local and one global layer (same
    seeded inputs), each timed and baselined on its own; `value` is the two
    layers' FLOPs over their summed step time."""
    from synth import workloads as wl
    from synth.device import host_tokens
    # host k, v of the first 16384 tokens, regenerated once when the first
    # baseline reads them (both layers draw the same seeded inputs)
    kv_cache = {}

    def kv():
        if "kv" not in kv_cache:
            lim = 16384
            kv_cache["kv"] = (host_tokens(wl.SPARK_LOCAL, "k", 0, 0, lim), host_tokens(wl.SPARK_LOCAL, "v", 0, 0, lim))
        return kv_cache["kv"]

    loc = prefill_block(wl.SPARK_LOCAL, 10, 3, events, torch, ma, cpu=cpu, kv=kv)
    glo = prefill_block(wl.SPARK_GLOBAL, 3, 2, events, torch, ma, cpu=cpu, kv=kv)
    flops = loc["roofline"]["flops_per_launch"] + glo["roofline"]["flops_per_launch"]
    ms = loc["ms_per_step"] + glo["ms_per_step"]
    return {"workload": "spark_prefill_256k (one local + one global layer)",
            "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 3),
            "local": loc, "global": glo}


def decode_block(events, torch, ma, copy_gbs, cpu=True):
    """The Spark decode step: paged global cache (bf16, and E4M3), 2048-entry
    ring (last-level cache evicted between steps); median split-kernel time
    over the reps against HBM peak, and the oracle streaming one sequence."""
    from synth import workloads as wl
    from global_muse_rope_amd import accounting as acc
    dec = {}
    digest = source_digest(DECODE_SOURCES)
    for dcfg, steps, flush, fp8 in [(wl.SPARK_DECODE_GLOBAL, 10, False, False),
                                    (wl.SPARK_DECODE_LOCAL, 20, True, False),
                                    (wl.SPARK_DECODE_GLOBAL, 10, False, True)]:
        name = dcfg.name + ("_fp8" if fp8 else "")
        log(f"decode {name}")
        base = not fp8   # the oracle baseline on both bf16 caches
        r = decode_case(dcfg, steps, 3, events, torch, ma, flush=flush, fp8=fp8, keep_out=base and cpu)
        med = _median(r["kernel_ms_each"])
        gbs = (r["kv_bytes"] + r["io_bytes"]) / (r["kernel_ms"] * 1e-3) / 1e9
        gbs_med = (r["kv_bytes"] + r["io_bytes"]) / (med * 1e-3) / 1e9
        log(f"  {gbs:.0f} GB/s, split kernel mean {r['kernel_ms']:.3f} ms, median {med:.3f} ms")
        dec[name] = {"value": round(gbs, 1), "unit": "GB/s", "kernel": "decode_split_kernel",
                     "cache_dtype": "e4m3" if fp8 else "bf16", "reps": steps, "warmup": 3,
                     "kernel_ms_median": round(med, 4), "kernel_ms_mean": round(r["kernel_ms"], 4),
                     "ms_per_step": round(r["ms_per_step"], 4), "kv_bytes_per_step": r["kv_bytes"],
                     "cache_flushed": flush,
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "frac_at_median": round(gbs_med / HBM_PEAK_GBS, 4),
                                  "frac_of_copy": round(gbs / copy_gbs, 4),
                                  "traffic": committed_traffic(f"decode_split_kernel_{name}", digest),
                                  "bytes_per_launch": r["kv_bytes"] + r["io_bytes"], "source_digest": digest}}
        if base and cpu:
            y_host, lengths = r["_out"], r["lengths"]
            PENDING.append((dec[name], "cpu_baseline",
                            lambda d=dcfg, y=y_host, ln=lengths: cpu_baseline_decode(d, y, ln), name))
    return dec


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
    ap.add_argument("--trace-summary", nargs=4, metavar=("WORKLOAD", "KERNEL", "STATS_CSV", "BENCH_LOG"),
                    help="summarize a rocprofv3 kernel-trace run of --only WORKLOAD (no GPU needed)")
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG",
                    help="WORKLOAD KERNEL RUN_DIR...: summarize SQ/GRBM counter passes (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.commands)
        return
    if args.counter_summary:
        wlname, kernel, *dirs = args.counter_summary
        counter_summary(wlname, kernel, dirs, [c for c in args.commands.split(" ;; ") if c])
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, [c for c in args.commands.split(" ;; ") if c])
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
        rows = keep_baseline_rows(cfg, gpu_out)
        PENDING.append((result, "cpu_baseline", lambda: cpu_baseline(cfg, rows), cfg.name))
    del x, gpu_out
    torch.cuda.empty_cache()

    if not args.quick:
        result["glimmer_global_prefill_128k"] = prefill_block(wl.GLIMMER_GLOBAL, 5, 2, events, torch, ma,
                                                              cpu=not args.no_cpu)
        result["spark_prefill_256k"] = spark_prefill_block(events, torch, ma, cpu=not args.no_cpu)

    if not args.no_decode:
        copy_gbs = copy_bandwidth(torch, events)
        log(f"device copy {copy_gbs:.0f} GB/s (read + write)")
        result["hbm_copy_gbs"] = round(copy_gbs, 1)
        result["spark_decode"] = decode_block(events, torch, ma, copy_gbs, cpu=not args.no_cpu)

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
        from global_muse_rope_amd import accounting as acc
        draft = {}
        ddigest = source_digest(DRAFT_SOURCES)
        for bcfg in wl.DRAFT:
            log(f"draft block {bcfg.name}")
            r = chunk_case(bcfg, 50, 5, events, torch, ma, draft=True)
            L = bcfg.layer
            nbytes = acc.draft_bytes(L.hq, L.hkv, L.d, bcfg.batch, bcfg.seq, bcfg.start, L.window)
            gbs = nbytes / (r["kernel_ms"] * 1e-3) / 1e9
            log(f"  {r['ms_per_step'] * 1e3:.1f} us per step, kernels {r['kernel_ms'] * 1e3:.1f} us, {gbs:.0f} GB/s")
            draft[bcfg.name] = {"us_per_step": round(r["ms_per_step"] * 1e3, 2),
                                "kernel_us": round(r["kernel_ms"] * 1e3, 2),
                                "tflops_step": round(r["tflops"], 2), "kernel_tflops": round(r["kernel_tflops"], 2),
                                "steps": 50, "warmup": 5,
                                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                             "traffic": committed_traffic(f"draft_split_kernel_{bcfg.name}", ddigest),
                                             "kernel": "draft_split_kernel + draft_combine_kernel",
                                             "bytes_per_launch": nbytes, "source_digest": ddigest}}
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

    run_pending()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
