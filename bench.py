"""Throughput of the SparseVILA decode and prefill hot paths on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode step of the whole batch through every layer: for each
layer, query-aware retrieval (relevance scan + top-k select) and sparse
decode attention over the selected visual entries plus the text entries
(split-K partials + combine), all in one launch per layer
(sv_retrieve_attend).  The headline workload is LLaVA-NeXT-7B shaped: 8
sequences, 32 layers x 32 heads, head dim 128, bf16, 1440 retained visual
tokens, k = 360, 256 text entries.  All caches are resident in HBM before
timing starts (7.1 GB, far above the 256 MB Infinity Cache, so every step
streams from HBM).  The step's launches are captured once in a HIP graph and
replayed.

Printed: one JSON line with steps/s (whole job), algorithmic HBM GB/s, the
roofline of the dominant kernel (the one-launch decode layer, timed live
with HIP events over the timed region on the stream it runs on), the same
step through the two-call path, and the CPU oracle timed on a bounded sample
of the same workload.  The same line carries, each with its own roofline and
oracle baseline:
  workloads.image576_fp32     576-token fp32 image, one layer (64 rotating replicas)
  workloads.qwen2_7b_video    Qwen2-7B GQA long video, batch 1, 28 layers, N = 25088
  workloads.multiturn_128k    4 x 131072 visual tokens, the 3-round x 128-step schedule
  salience                    SigLIP-shaped prefill salience, 256 frames x 729 tokens
  summary_salience            CLIP (one summary token) and RADIO (four) shapes,
                              rotating over >= 1 GB of encoder Q/K
  packed                      per-question retrieval + dense packing, decode over packed rows
  hbm_measured                1 GiB device copy and read: the bandwidth actually reachable
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

EXTRA_DECODE = ("image576_fp32", "qwen2_7b_video", "multiturn_128k")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llava_next_7b")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    p.add_argument("--no-salience", action="store_true")
    p.add_argument("--salience-only", action="store_true",
                   help="time only the prefill salience call (profiling runs); prints its object")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-pack", action="store_true")
    p.add_argument("--no-summary", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="time only the headline decode workload (no other decode workloads)")
    p.add_argument("--salience-long-only", action="store_true",
                   help="time only the long-frame (two-pass streaming) salience call")
    p.add_argument("--summary-only", action="store_true",
                   help="time only the summary-token salience calls (profiling runs); prints "
                        "their object")
    p.add_argument("--pack-only", action="store_true",
                   help="time only the per-question pack and the decode over packed rows "
                        "(profiling runs); prints its object")
    p.add_argument("--prefill-only", action="store_true",
                   help="time only the question prefill with fused retrieval (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="budget of each CPU oracle sample")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--profile-traffic", action="store_true",
                   help="no timing: run two one-launch decode steps and a 1 GiB device copy "
                        "(the calibration) for rocprofv3 counter passes")
    return p.parse_args()


def decode_bytes(w, T=None):
    """Algorithmic HBM bytes of one step, and of one layer of the whole batch
    (T text entries per sequence, w.T by default)."""
    T = w.T if T is None else T
    e = 2 if w.dtype.itemsize == 2 else 4
    row = w.Hkv * w.D * e
    q = w.Hq * w.D * e
    scan = w.N * row + q + w.N * 4                       # keys once, query, fp32 scores out
    select = w.N * 4 + w.k * 4                            # scores in, indices out
    attn = (w.k + T) * 2 * row + q + w.k * 4 + w.Hq * w.D * 4   # K,V of the attended rows
    per_seq_layer = scan + select + attn
    return per_seq_layer * w.B * w.L, per_seq_layer * w.B


# Sources of the one-launch decode layer's kernel (their hash keys the
# committed counter summaries).
FUSED_SOURCES = ("fused.hip", "fused_kernel.h", "fused_bf16.hip", "fused_bf16_long.hip",
                 "fused_f32.hip", "fused_f32_long.hip", "decode_items.h", "long_select.h",
                 "select.h", "common.h")


# Sources of the dense-packing kernel.
PACK_SOURCES = ("pack.hip", "pack.h", "common.h")


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "visual_token_sparsity_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


SALIENCE_SOURCES = ("salience.hip", "common.h")


def committed_mfma_ops(workload, src_hash):
    """MFMA flops one salience call executes, from the committed rocprofv3 counter
    summary (bf16 score MFMAs plus f16 column sums), if still current."""
    path = os.path.join(ROOT, "profiles", "salience_counters.json")
    try:
        with open(path) as f:
            t = json.load(f)[workload]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != src_hash:
        return None
    return (t["mfma_mops_bf16_per_call"] + t["mfma_mops_f16_per_call"]) * t["flops_per_mop"]


def committed_traffic(kernel_key, src_hash):
    """Per-launch HBM bytes from the committed rocprofv3 counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != src_hash:
        return None
    return t.get("bytes_per_launch")


def calibration_copy(torch, dev):
    """Two 1 GiB device-to-device copies: the known-size reference of the counter passes."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    return src.numel()


def gpu_time(fn, reps, stream):
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def capture(fn, stream):
    """Capture fn's launches (on ``stream``) into a HIP graph; returns the graph or None."""
    import torch
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g
    except Exception as e:  # capture unsupported: fall back to eager launches
        print(f"[bench] graph capture failed ({e}); timing eager launches", file=sys.stderr, flush=True)
        return None


def cpu_info():
    n = len(os.sched_getaffinity(0))
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def free(torch):
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    a = parse()
    a.deferred = []                         # CPU baselines, run after every GPU measurement
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        sys.exit(2)

    import torch

    import synthetic
    import visual_token_sparsity_amd as sv

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.load()
    stream = torch.cuda.Stream(device=dev)      # default priority
    def flush_baselines():
        for target, key, fn in a.deferred:
            target[key] = fn()
            free(torch)
        a.deferred.clear()

    if a.salience_only:
        out = {"salience": bench_salience(a, dev, stream)}
        flush_baselines()
        print(json.dumps(out), flush=True)
        return
    if a.summary_only:
        out = {"summary_salience": bench_summary(a, dev, stream)}
        flush_baselines()
        print(json.dumps(out), flush=True)
        return
    if a.salience_long_only:
        out = {"salience_long": bench_salience_long(a, dev, stream)}
        flush_baselines()
        print(json.dumps(out), flush=True)
        return
    w = synthetic.DECODE[a.workload]
    if a.pack_only:
        layers = make_layers(a, dev, w)
        res = bench_packed(a, dev, stream, w, layers)
        if res is not None:
            print(json.dumps({"packed": res}), flush=True)
        return
    if a.profile_traffic:
        profile_traffic(a, dev, w)
        return
    if a.prefill_only:
        layers = make_layers(a, dev, w)
        out = {"prefill_retrieve": bench_prefill(a, dev, stream, w, layers)}
        del layers
        free(torch)
        flush_baselines()
        print(json.dumps(out), flush=True)
        return

    # ------------------------------------------------------------ headline decode workload
    layers = make_layers(a, dev, w)
    head = bench_decode(a, dev, stream, w, layers, two_call=True)
    dtype = "bf16" if w.dtype == torch.bfloat16 else "f32"
    res = {
        "metric": "decode steps/s (retrieval + sparse attention, all layers, whole batch)",
        "value": head["value"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": head["timed_steps"],
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded Gaussian caches, 5% planted relevant tokens; no weights)",
        "config": dict(head["config"], parallelism="none (1 GPU)"),
    }
    for key in ("hbm_gbs_algorithmic", "hbm_frac_algorithmic", "step_bytes_algorithmic",
                "roofline", "two_call_path", "wall_s_timed"):
        if key in head:
            res[key] = head[key]

    # ------------------------------------------------------------ per-question dense packing
    if not a.no_pack and w.name != "multiturn_128k":
        res["packed"] = bench_packed(a, dev, stream, w, layers)
        res["packed"]["decode_speedup_vs_fused_step"] = round(
            res["packed"]["decode"]["steps_per_s"] / res["value"], 3)

    # ------------------------------------------------------------ question prefill + fused retrieval
    if not a.no_pack and w.name != "multiturn_128k":
        res["prefill_retrieve"] = bench_prefill(a, dev, stream, w, layers)

    # ------------------------------------------------------------ CPU oracle, headline workload
    if not a.no_cpu_baseline:
        defer_baseline(a, res, "cpu_baseline", lambda: decode_baseline_fresh(a, dev, w))
    del layers
    free(torch)

    # ------------------------------------------------------------ the other decode workloads
    if not a.no_extra:
        res["workloads"] = {}
        for name in EXTRA_DECODE:
            if name == w.name:
                continue
            wx = synthetic.DECODE[name]
            lx = make_layers(a, dev, wx)
            obj = bench_decode(a, dev, stream, wx, lx, two_call=False, full_schedule=True)
            if not a.no_cpu_baseline:
                defer_baseline(a, obj, "cpu_baseline",
                               lambda wx=wx: decode_baseline_fresh(a, dev, wx))
            res["workloads"][name] = obj
            del lx
            free(torch)

    # ------------------------------------------------------------ prefill salience
    if not a.no_salience:
        res["salience"] = bench_salience(a, dev, stream)
        free(torch)
    if not a.no_salience:
        res["salience_long"] = bench_salience_long(a, dev, stream)
        free(torch)
    if not a.no_summary:
        res["summary_salience"] = bench_summary(a, dev, stream)
        free(torch)

    res["hbm_measured"] = hbm_measured(dev, stream)

    # ------------------------------------------------------------ CPU oracle baselines, last
    flush_baselines()
    print(json.dumps(res), flush=True)


def replicas(w):
    """Independent input sets per timed unit: the one-layer fp32 image workload
    fits the last-level cache, so 64 replicas (1.3 GB) rotate through HBM."""
    return 64 if w.name == "image576_fp32" else w.L


def make_layers(a, dev, w):
    import synthetic
    n = replicas(w)
    say(f"workload {w.name}: B={w.B} L={w.L} Hq={w.Hq} Hkv={w.Hkv} D={w.D} N={w.N} k={w.k} "
        f"T={w.T} ({n} input sets)")
    return [synthetic.make_decode_layer(w, a.seed, layer=l, device=dev, gen_device="cuda")
            for l in range(n)]


def bench_decode(a, dev, stream, w, layers, two_call, full_schedule=False):
    """Time decode steps of workload w over its resident layers.

    One unit is a decode step through w.L layers; the fp32 image workload has
    one layer and rotates over its replicas (each replica one step).  The
    multi-turn workload times --steps steps of its round schedule, or the whole
    schedule with full_schedule."""
    import torch

    import synthetic
    import visual_token_sparsity_amd as sv
    L = len(layers)
    units_per_call = L // w.L                     # steps per pass over the input sets
    idx = [torch.empty((w.B, w.k), dtype=torch.int32, device=dev) for _ in range(L)]
    out = [torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev) for _ in range(L)]
    ws_f = sv.new_workspace(sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k, w.Tmax), dev)
    ws_r = sv.new_workspace(sv.retrieve_workspace_bytes(w.B, w.N, w.k), dev)
    ws_a = sv.new_workspace(sv.sparse_decode_attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.k, w.Tmax), dev)

    # Multi-turn workload: conversation rounds of decode steps over one reused
    # visual cache.  Step i takes a fresh query and the text length of its
    # place in the round schedule (partial eviction between rounds).
    sched = None
    if w.name == "multiturn_128k":
        lens = [t for rnd in synthetic.multiturn_text_lengths() for t in rnd]
        sched = {"lens": lens,
                 "txt": torch.tensor([[t] * w.B for t in lens], dtype=torch.int32, device=dev),
                 "q": (torch.randn((len(lens), w.B, 1, w.Hq, w.D), device=dev,
                                   generator=torch.Generator(device=dev).manual_seed(
                                       synthetic.stream_seed(a.seed, w.name, "q_per_step")))
                       .to(w.dtype)),
                 "i": 0}

    def step():
        for l, d in enumerate(layers):
            q, tl = d["q"], d["txt_len"]
            if sched is not None:
                j = sched["i"] % len(sched["lens"])
                q, tl = sched["q"][j], sched["txt"][j]
            sv.retrieve_attend(q, d["k_vis"], d["v_vis"], w.k, d["k_txt"], d["v_txt"],
                               tl, workspace=ws_f, out=out[l], idx_out=idx[l])
        if sched is not None:
            sched["i"] += 1

    def step_two_call():
        for l, d in enumerate(layers):
            q, tl = d["q"], d["txt_len"]
            if sched is not None:
                j = sched["i"] % len(sched["lens"])
                q, tl = sched["q"][j], sched["txt"][j]
            sv.retrieve(q, d["k_vis"], w.k, workspace=ws_r, out=idx[l])
            sv.sparse_decode_attn(q, d["k_vis"], d["v_vis"], idx[l], d["k_txt"], d["v_txt"],
                                  tl, workspace=ws_a, out=out[l])
        if sched is not None:
            sched["i"] += 1

    def vis_checksum():
        return [int(d[n].view(torch.int16).sum(dtype=torch.int64).item())
                for d in layers for n in ("k_vis", "v_vis")]

    calls = len(sched["lens"]) if (sched is not None and full_schedule) else a.steps
    sum_before = vis_checksum() if sched is not None else None
    with torch.cuda.stream(stream):
        for _ in range(max(1, a.warmup)):
            step()
            if two_call:
                step_two_call()
        torch.cuda.synchronize()
        # The multi-turn schedule changes the query and text length every step:
        # eager launches (each step is one ~0.8 ms kernel).
        eager = a.no_graph or sched is not None
        g_step = None if eager else capture(step, stream)
        g_two = None if (eager or not two_call) else capture(step_two_call, stream)
        run_step = g_step.replay if g_step is not None else step
        run_two = g_two.replay if g_two is not None else step_two_call
        for _ in range(a.warmup):
            run_step()
        # ---------------------------------------------------- timed region: exactly `calls` passes
        torch.cuda.synchronize()
        if sched is not None:
            sched["i"] = 0                       # the timed steps start the schedule
        t0 = time.perf_counter()
        secs = gpu_time(run_step, calls, stream)
        wall = time.perf_counter() - t0
        timed_lens = ([sched["lens"][i % len(sched["lens"])] for i in range(calls)]
                      if sched is not None else None)
        sv.workspace_status(ws_f)               # no in-kernel wait gave up
        two_secs = None
        if two_call:
            for _ in range(3):
                run_two()
            two_reps = max(5, a.steps // 2)
            two_secs = gpu_time(run_two, two_reps, stream) / two_reps

    steps = calls * units_per_call
    step_bytes, layer_bytes = decode_bytes(w)
    if timed_lens is not None:                   # mean over the timed steps' text lengths
        per = [decode_bytes(w, T) for T in timed_lens]
        step_bytes = sum(p[0] for p in per) // len(per)
        layer_bytes = sum(p[1] for p in per) // len(per)
    steps_per_s = steps / secs
    gbs = step_bytes * steps_per_s / 1e9
    # One launch per layer: the average launch duration over the timed region.
    layer_avg = secs / (calls * L)
    layer_gbs = layer_bytes / layer_avg / 1e9
    traffic = committed_traffic(f"fused_{w.name}", source_hash(*FUSED_SOURCES))
    res = {
        "value": round(steps_per_s, 2), "unit": "steps/s", "timed_steps": steps,
        "ms_per_step": round(secs / steps * 1e3, 4),
        "config": {"workload": w.name, "batch": w.B, "layers": w.L, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "visual_tokens": w.N, "k": w.k,
                   "text_tokens": w.T, "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
                   "launch": "hipgraph" if g_step is not None else "eager"},
        "hbm_gbs_algorithmic": round(gbs, 1),
        "hbm_frac_algorithmic": round(gbs / HBM_PEAK_GBS, 4),
        "step_bytes_algorithmic": step_bytes,
        "roofline": {"kernel": "fused_kernel (one decode layer of the whole batch per launch: "
                               "scan + select + sparse attention + combine)",
                     "bound": "hbm", "achieved": round(layer_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": layer_bytes,
                     "avg_launch_us": round(layer_avg * 1e6, 3)},
        "wall_s_timed": round(wall, 4),
    }
    if units_per_call > 1:
        res["config"]["input_sets"] = f"{L} replicas rotated, one step each (footprint >= 1 GB)"
    if two_secs is not None:
        res["two_call_path"] = {"ms_per_step": round(two_secs / units_per_call * 1e3, 4),
                                "value": round(units_per_call / two_secs, 2), "unit": "steps/s",
                                "launches_per_layer": 2}
    if sched is not None:
        if vis_checksum() != sum_before:
            raise RuntimeError("the visual cache changed during the multi-turn schedule")
        res["config"].update({
            "text_tokens": f"{min(timed_lens)}-{max(timed_lens)}",
            "schedule": "3 rounds x 128 decode steps, fresh query per step; text = 64 system + "
                        "64 question + step + 1, question and answer evicted between rounds; "
                        "the timed steps follow the schedule from its start",
            "visual_cache_unchanged": True})
    return res


def profile_traffic(a, dev, w):
    """Counter passes: the fused decode layer as timed, and a plain copy of known
    size whose counters give the scale factor of the counters."""
    import torch

    import visual_token_sparsity_amd as sv
    layers = make_layers(a, dev, w)
    ws_f = sv.new_workspace(sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k, w.Tmax), dev)
    for _ in range(2):
        for d in layers:
            sv.retrieve_attend(d["q"], d["k_vis"], d["v_vis"], w.k, d["k_txt"], d["v_txt"],
                               d["txt_len"], workspace=ws_f)
    torch.cuda.synchronize()
    nbytes = calibration_copy(torch, dev)
    print(json.dumps({"profile_traffic": w.name, "layer_bytes": decode_bytes(w)[1],
                      "copy_bytes": nbytes}), flush=True)


def bench_packed(a, dev, stream, w, layers):
    """Per-question retrieval + dense packing, then decode steps over the packed rows.

    One question (8 tokens) selects k visual tokens per sequence and layer;
    sv_pack_selected copies their K and V rows into contiguous buffers; a
    decode step then runs sv_sparse_decode_attn over the packed rows plus the
    text entries at every layer.  Timed: the packs of one question (every
    layer, whole batch; reported per launch) and the packed decode step (all
    layers).
    """
    import torch

    import synthetic
    import visual_token_sparsity_amd as sv
    e = 2 if w.dtype.itemsize == 2 else 4
    row = w.Hkv * w.D * e
    ws_r = sv.new_workspace(sv.retrieve_workspace_bytes(w.B, w.N, w.k), dev)
    ws_a = sv.new_workspace(sv.sparse_decode_attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.k, w.Tmax), dev)
    gq = torch.Generator(device=dev).manual_seed(synthetic.stream_seed(a.seed, w.name, "question"))
    question = torch.randn((w.B, 8, w.Hq, w.D), generator=gq, device=dev).to(w.dtype)
    idx = [sv.retrieve(question, d["k_vis"], w.k, workspace=ws_r) for d in layers]
    packs = [sv.pack_selected(d["k_vis"], d["v_vis"], i) for d, i in zip(layers, idx)]
    out = [torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev) for _ in layers]
    torch.cuda.synchronize()

    def pack_once():                       # every layer's pack for one question
        for l, d in enumerate(layers):
            sv.pack_selected(d["k_vis"], d["v_vis"], idx[l], out=packs[l])

    pack_bytes = w.B * w.k * (4 * row + 4)                 # K and V rows read and written, idx
    if a.profile_traffic:
        # Counter passes: the packs of two questions (eager), then the copy
        # calibration.
        for _ in range(2):
            pack_once()
        torch.cuda.synchronize()
        calibration_copy(torch, dev)
        print(json.dumps({"profile_traffic": f"pack_{w.name}", "launch_bytes": pack_bytes}),
              flush=True)
        return None

    def packed_step():
        for l, d in enumerate(layers):
            kp, vp = packs[l]
            # The packed rows are the selection: no index list (rows 0..k-1).
            sv.sparse_decode_attn(d["q"], kp, vp, w.k, d["k_txt"], d["v_txt"], d["txt_len"],
                                  workspace=ws_a, out=out[l])

    with torch.cuda.stream(stream):
        for _ in range(3):
            pack_once()
            packed_step()
        torch.cuda.synchronize()
        g_pack = None if a.no_graph else capture(pack_once, stream)
        g_step = None if a.no_graph else capture(packed_step, stream)
        run_pack = g_pack.replay if g_pack is not None else pack_once
        run_step = g_step.replay if g_step is not None else packed_step
        for _ in range(3):
            run_pack()
            run_step()
        reps = max(5, a.steps // 4)
        pack_secs = gpu_time(run_pack, reps, stream) / (reps * len(layers))
        step_secs = gpu_time(run_step, a.steps, stream) / a.steps
    q = w.Hq * w.D * e
    step_bytes = w.L * w.B * ((w.k + w.T) * 2 * row + q + w.Hq * w.D * 4)
    pack_gbs = pack_bytes / pack_secs / 1e9
    step_gbs = step_bytes / step_secs / 1e9
    return {"question_tokens": 8,
            "pack": {"kernel": "pack_kernel (one layer of the whole batch per launch)",
                     "us_per_launch": round(pack_secs * 1e6, 3), "bytes_per_launch": pack_bytes,
                     "roofline": {"bound": "hbm", "achieved": round(pack_gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(pack_gbs / HBM_PEAK_GBS, 4),
                                  "traffic": committed_traffic(f"pack_{w.name}",
                                                               source_hash(*PACK_SOURCES))},
                     "launches_per_question": w.L,
                     "ms_per_question": round(pack_secs * w.L * 1e3, 4)},
            "decode": {"what": "sv_sparse_decode_attn over packed rows 0..k-1 (no index list) plus text, every layer",
                       "steps_per_s": round(1.0 / step_secs, 2),
                       "ms_per_step": round(step_secs * 1e3, 4), "bytes_per_step": step_bytes,
                       "hbm_gbs_algorithmic": round(step_gbs, 1),
                       "hbm_frac_algorithmic": round(step_gbs / HBM_PEAK_GBS, 4),
                       "launch": "hipgraph" if g_step is not None else "eager"}}


def bench_prefill(a, dev, stream, w, layers, Tq=32):
    """A question of Tq tokens through every layer: causal prefill attention over the
    visual cache and the text (whose last Tq rows are the question's), with the
    query-aware retrieval of k tokens fused in (sv_prefill_attend_retrieve, one
    launch per layer plus its combine / select launches).  Next to it, the
    retrieval alone as a separate pass (sv_retrieve with the same Tq)."""
    import numpy as np
    import torch

    import synthetic
    import visual_token_sparsity_amd as sv
    gq = torch.Generator(device=dev).manual_seed(synthetic.stream_seed(a.seed, w.name, "prefill_q"))
    qs = [torch.randn((w.B, Tq, w.Hq, w.D), generator=gq, device=dev).to(w.dtype) for _ in layers]
    ws = sv.new_workspace(sv.prefill_attend_retrieve_workspace_bytes(w.B, Tq, w.Hq, w.Hkv, w.D, w.N,
                                                                     w.Tmax), dev)
    ws_r = sv.new_workspace(sv.retrieve_workspace_bytes(w.B, w.N, w.k), dev)
    out = [torch.empty((w.B, Tq, w.Hq, w.D), dtype=torch.float32, device=dev) for _ in layers]
    idx = [torch.empty((w.B, w.k), dtype=torch.int32, device=dev) for _ in layers]

    def fused():
        for l, d in enumerate(layers):
            sv.prefill_attend_retrieve(qs[l], d["k_vis"], d["v_vis"], d["k_txt"], d["v_txt"],
                                       d["txt_len"], w.k, workspace=ws, out=out[l], idx_out=idx[l])

    def retrieval_only():
        for l, d in enumerate(layers):
            sv.retrieve(qs[l], d["k_vis"], w.k, workspace=ws_r, out=idx[l])

    with torch.cuda.stream(stream):
        for _ in range(2):
            fused()
            retrieval_only()
        g1 = None if a.no_graph else capture(fused, stream)
        g2 = None if a.no_graph else capture(retrieval_only, stream)
        r1 = g1.replay if g1 is not None else fused
        r2 = g2.replay if g2 is not None else retrieval_only
        for _ in range(2):
            r1()
            r2()
        reps = max(5, a.steps // 10)
        t_fused = gpu_time(r1, reps, stream) / reps
        t_ret = gpu_time(r2, reps, stream) / reps
    e = 2 if w.dtype.itemsize == 2 else 4
    row = w.Hkv * w.D * e
    per_layer = w.B * ((w.N + w.T) * 2 * row + Tq * w.Hq * w.D * (e + 4) + w.N * 4 + w.k * 4)
    flops = 4.0 * w.B * Tq * w.Hq * (w.N + w.T) * w.D * len(layers)
    gbs = per_layer * len(layers) / t_fused / 1e9
    res = {"question_tokens": Tq, "layers": len(layers), "k": w.k,
           "ms_per_question": round(t_fused * 1e3, 4),
           "tokens_per_s": round(w.B * Tq / t_fused, 1),
           "roofline": {"kernel": "prefill_attn_kernel + combine + score sum + top-k, every layer",
                        "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "bytes_per_layer": per_layer,
                        "mfma_tflops": round(flops / t_fused / 1e12, 2)},
           "retrieval_alone_ms": round(t_ret * 1e3, 4),
           "what": "attention of the question (causal over the text, all visual tokens) and its "
                   "top-k retrieval from one pass; retrieval_alone is sv_retrieve with the same "
                   "question tokens (a separate pass over the visual keys)"}
    if not a.no_cpu_baseline:
        def prefill_baseline():
            import oracle
            lays = make_layers(a, dev, w)      # the same seeded inputs, generated again
            ncores, model = cpu_info()
            done, spent = 0, 0.0
            for l, d in enumerate(lays):
                for b in range(w.B):
                    h = {n: d[n][b:b + 1].cpu() for n in ("k_vis", "v_vis", "k_txt", "v_txt")}
                    qb = qs[l][b:b + 1].cpu()
                    tl = d["txt_len"][b:b + 1].cpu().numpy()
                    t0 = time.perf_counter()
                    oracle.prefill_attention(qb, h["k_vis"], h["v_vis"], h["k_txt"], h["v_txt"], tl)
                    oracle.retrieve(qb, h["k_vis"], w.k)
                    spent += time.perf_counter() - t0
                    done += 1
                    if spent >= a.cpu_seconds:
                        break
                if spent >= a.cpu_seconds:
                    break
            del lays
            per_q = spent / done * w.B * len(layers_n)
            return {"value": round(w.B * Tq / per_q, 2), "unit": "tokens/s",
                    "cores": blas_threads(), "host_cores_visible": ncores,
                    "cpu_model": model, "kind": "oracle",
                    "sample": f"{done} (layer, sequence) units of {w.B * len(layers_n)} "
                              f"(prefill attention + retrieval, fp64), {spent:.1f} s"}
        layers_n = list(range(len(layers)))
        defer_baseline(a, res, "cpu_baseline", prefill_baseline)
    return res


def bench_summary(a, dev, stream):
    """Summary-token salience and per-frame pruning: CLIP shape (one CLS token) and
    RADIO shape (4 summary tokens).  Each call takes the next of several Q/K sets
    (>= 1 GB of keys in all), so the keys stream from HBM, not the last-level cache."""
    import torch

    import synthetic
    import visual_token_sparsity_amd as sv
    res = {}
    for name, S in (("clip_l14_336_256f", 1), ("radio_1028_64f", 4)):
        sw = synthetic.SALIENCE[name]
        key_bytes = sw.F * sw.H * sw.N * sw.D * 2
        nsets = max(1, -(-(1 << 30) // key_bytes))
        sets = [synthetic.make_salience(sw, a.seed + i, device=dev, gen_device="cuda")
                for i in range(nsets)]
        sal = torch.empty((sw.F, sw.N), dtype=torch.float32, device=dev)
        keep = torch.empty((sw.F, sw.keep), dtype=torch.int32, device=dev)
        ws = sv.new_workspace(sv.summary_salience_prune_workspace_bytes(sw.F, sw.H, sw.N), dev)

        def once():                          # one call per set
            for Q, K in sets:
                sv.summary_salience_prune(Q, K, S, sw.keep, workspace=ws, salience_out=sal,
                                          idx_out=keep)

        with torch.cuda.stream(stream):
            for _ in range(2):
                once()
            g = None if a.no_graph else capture(once, stream)
            run = g.replay if g is not None else once
            for _ in range(2):
                run()
            reps = max(5, a.steps // 10)
            secs = gpu_time(run, reps, stream) / (reps * nsets)
        # keys once, the summary queries, per-head column values written and read
        # back, the salience written and read by the select, the kept indices
        nbytes = (sw.F * sw.H * sw.N * sw.D * 2 + sw.F * sw.H * S * sw.D * 2
                  + 2 * sw.F * sw.H * sw.N * 4 + 2 * sw.F * sw.N * 4 + sw.F * sw.keep * 4)
        gbs = nbytes / secs / 1e9
        res[name] = {"frames": sw.F, "tokens_per_frame": sw.N, "heads": sw.H,
                     "head_dim": sw.D, "summary_tokens": S, "keep": sw.keep,
                     "ms_per_call": round(secs * 1e3, 4),
                     "tokens_per_s": round(sw.F * sw.N / secs, 1),
                     "rotation": f"{nsets} Q/K sets, {nsets * key_bytes / 1e9:.2f} GB of keys",
                     "roofline": {"kernel": "summary_cols_kernel + summary_mean_kernel + "
                                            "per-frame top-k: whole call",
                                  "bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "bytes_algorithmic": nbytes}}
        if not a.no_cpu_baseline:
            import oracle
            Q0, K0 = sets[0]
            defer_baseline(a, res[name], "cpu_baseline",
                           lambda sw=sw, Q0=Q0, K0=K0, S=S: cpu_baseline_salience(
                               a, sw, Q0, K0, lambda q, k: oracle.summary_salience(q, k, S)))
        del sets
        free(torch)
    return res


def bench_salience(a, dev, stream):
    import torch

    import synthetic
    import visual_token_sparsity_amd as sv
    sw = synthetic.SALIENCE["siglip_256f"]
    Q, K = synthetic.make_salience(sw, a.seed, device=dev, gen_device="cuda")
    sal = torch.empty((sw.F, sw.N), dtype=torch.float32, device=dev)
    keep = torch.empty((sw.F, sw.keep), dtype=torch.int32, device=dev)
    ws = sv.new_workspace(sv.salience_prune_workspace_bytes(sw.F, sw.H, sw.N), dev)

    def once():
        sv.salience_prune(Q, K, sw.keep, workspace=ws, salience_out=sal, idx_out=keep)

    with torch.cuda.stream(stream):
        for _ in range(3):
            once()
        g = None if a.no_graph else capture(once, stream)
        run = g.replay if g is not None else once
        reps = max(5, a.steps // 4)
        secs = gpu_time(run, reps, stream) / reps
    flops = synthetic.flop_count_salience(sw)
    tflops = flops / secs / 1e12
    executed = committed_mfma_ops(sw.name, source_hash(*SALIENCE_SOURCES))
    res = {"workload": sw.name, "frames": sw.F, "tokens_per_frame": sw.N, "heads": sw.H,
           "head_dim": sw.D, "keep": sw.keep, "ms_per_call": round(secs * 1e3, 4),
           "tokens_per_s": round(sw.F * sw.N / secs, 1),
           "roofline": {"kernel": "salience_rows_kernel (+ flagged-item fp32 pass, head mean, per-frame top-k): whole call",
                        "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                        "flops_algorithmic": flops,
                        # MFMA work the call executes (padding of D and of the key
                        # tiles, column-sum MFMAs), from the committed counters
                        "flops_executed_counters": executed,
                        "executed_tflops": (round(executed / secs / 1e12, 2)
                                            if executed else None)}}
    if not a.no_cpu_baseline:
        import oracle
        defer_baseline(a, res, "cpu_baseline",
                       lambda: cpu_baseline_salience(a, sw, Q, K, oracle.salience))
    return res


def bench_salience_long(a, dev, stream):
    """Salience of a QwenVL-style long frame (16384 tokens in one attention, 16
    heads of 80): the two-pass streaming kernels, one graph-captured call."""
    import torch

    import synthetic
    import visual_token_sparsity_amd as sv
    sw = synthetic.SALIENCE["qwenvl_16k"]
    Q, K = synthetic.make_salience(sw, a.seed, device=dev, gen_device="cuda")
    sal = torch.empty((sw.F, sw.N), dtype=torch.float32, device=dev)
    keep = torch.empty((sw.F, sw.keep), dtype=torch.int32, device=dev)
    ws = sv.new_workspace(sv.salience_prune_workspace_bytes(sw.F, sw.H, sw.N), dev)

    def once():
        sv.salience_prune(Q, K, sw.keep, workspace=ws, salience_out=sal, idx_out=keep)

    with torch.cuda.stream(stream):
        for _ in range(2):
            once()
        g = None if a.no_graph else capture(once, stream)
        run = g.replay if g is not None else once
        reps = max(3, a.steps // 20)
        secs = gpu_time(run, reps, stream) / reps
    flops = synthetic.flop_count_salience(sw)        # one Q K^T per (frame, head)
    tflops = flops / secs / 1e12
    res = {"workload": sw.name, "frames": sw.F, "tokens_per_frame": sw.N, "heads": sw.H,
           "head_dim": sw.D, "keep": sw.keep, "ms_per_call": round(secs * 1e3, 4),
           "tokens_per_s": round(sw.F * sw.N / secs, 1),
           "roofline": {"kernel": "salience_rowstat_kernel + salience_colstream_kernel (two "
                                  "streaming passes) + head mean + per-frame top-k: whole call",
                        "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                        "flops_algorithmic": flops,
                        "frac_of_two_pass_work": round(2 * tflops / BF16_PEAK_TFLOPS, 4)}}
    if not a.no_cpu_baseline:
        def long_baseline():
            import oracle
            ncores, model = cpu_info()
            done, spent = 0, 0.0
            for h in range(sw.H):                # one head of the frame at a time
                q, k = Q[:, h:h + 1].cpu(), K[:, h:h + 1].cpu()
                t0 = time.perf_counter()
                oracle.salience(q, k)
                spent += time.perf_counter() - t0
                done += 1
                if spent >= a.cpu_seconds:
                    break
            per_call = spent / done * sw.H
            return {"value": round(sw.F * sw.N / per_call, 1), "unit": "tokens/s",
                    "cores": blas_threads(), "host_cores_visible": ncores,
                    "cpu_model": model, "kind": "oracle",
                    "ms_per_call_equivalent": round(per_call * 1e3, 1),
                    "sample": f"{done} of {sw.H} heads of the frame (materialised "
                              f"fp64 softmax), {spent:.1f} s, scaled to the call"}
        defer_baseline(a, res, "cpu_baseline", long_baseline)
    return res


def hbm_measured(dev, stream):
    """The bandwidth a plain streaming kernel reaches on this GPU: a 1 GiB
    device-to-device copy (read + write) and a 1 GiB reduction (read)."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    nbytes = src.numel() * 4
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
            torch.sum(src, dim=0, out=acc)
        copy_s = gpu_time(lambda: dst.copy_(src), 10, stream) / 10
        read_s = gpu_time(lambda: torch.sum(src, dim=0, out=acc), 10, stream) / 10
    return {"what": "torch device copy and sum over 1 GiB buffers (HIP events): what generic "
                    "streaming kernels reach, next to the 8 TB/s peak",
            "copy_gbs": round(2 * nbytes / copy_s / 1e9, 1),
            "read_gbs": round(nbytes / read_s / 1e9, 1),
            "peak_gbs": HBM_PEAK_GBS}


# ---------------------------------------------------------------- CPU oracle baselines
def defer_baseline(a, target, key, fn):
    """Queue a CPU-oracle baseline for after every GPU measurement: the oracle's
    BLAS threads would otherwise still be busy while the next workload's graph
    replays are launched from the host, and a starved launch thread leaves the
    GPU idle between replays."""
    a.deferred.append((target, key, fn))


def decode_baseline_fresh(a, dev, w):
    """cpu_baseline_decode on the workload's inputs generated again from the same
    seed (identical data), so no workload's caches stay resident meanwhile."""
    import torch
    layers = make_layers(a, dev, w)
    try:
        return cpu_baseline_decode(a, w, layers)
    finally:
        del layers
        free(torch)


def cpu_baseline_decode(a, w, layers):
    """The fp64 oracle on the host over whole (sequence, layer) units of the same
    decode inputs until the time budget is spent, scaled to steps/s.  Rows of the
    131072-token workload are scored in token chunks (every score depends on its
    own token only) so the fp64 copy of a sequence's keys fits in memory."""
    import numpy as np
    import torch

    import oracle
    ncores, model = cpu_info()
    units = [(l, b) for l in range(len(layers)) for b in range(w.B)]
    per_step = w.L * w.B                       # (layer, sequence) units per step
    done, spent = 0, 0.0
    for l, b in units:
        d = layers[l]
        q = d["q"][b:b + 1].cpu()
        kt, vt = d["k_txt"][b:b + 1].cpu(), d["v_txt"][b:b + 1].cpu()
        tl = d["txt_len"][b:b + 1].cpu()
        if w.N > 32768:
            chunks = [d["k_vis"][b:b + 1, t0:t0 + 16384].cpu() for t0 in range(0, w.N, 16384)]
            t0 = time.perf_counter()
            s = np.concatenate([oracle.retrieval_scores(q, c) for c in chunks], axis=1)
            idx = oracle.topk_ascending(s, w.k)
            spent += time.perf_counter() - t0
            sel = torch.from_numpy(idx[0]).to(d["k_vis"].device)
            kv, vv = d["k_vis"][b:b + 1, sel].cpu(), d["v_vis"][b:b + 1, sel].cpu()
            t0 = time.perf_counter()
            oracle.sparse_decode_attn(q, kv, vv, np.arange(w.k)[None], kt, vt, tl)
            spent += time.perf_counter() - t0
        else:
            kv, vv = d["k_vis"][b:b + 1].cpu(), d["v_vis"][b:b + 1].cpu()
            t0 = time.perf_counter()
            idx = oracle.retrieve(q, kv, w.k)
            oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
            spent += time.perf_counter() - t0
        done += 1
        if spent >= a.cpu_seconds:
            break
    steps_per_s = done / per_step / spent
    return {"value": round(steps_per_s, 6), "unit": "steps/s", "cores": blas_threads(),
            "host_cores_visible": ncores, "cpu_model": model, "kind": "oracle",
            "sample": f"{done} (layer, sequence) units, {per_step} per step (retrieve + sparse "
                      f"attention, fp64 NumPy, on the same inputs), {spent:.1f} s, scaled to "
                      f"whole steps"}


def cpu_baseline_salience(a, sw, Q, K, fn):
    """The fp64 oracle over whole frames until the time budget is spent, scaled to
    tokens/s."""
    ncores, model = cpu_info()
    done, spent = 0, 0.0
    for f in range(sw.F):
        q, k = Q[f:f + 1].cpu(), K[f:f + 1].cpu()
        t0 = time.perf_counter()
        fn(q, k)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= a.cpu_seconds:
            break
    tok_s = done * sw.N / spent
    return {"value": round(tok_s, 1), "unit": "tokens/s", "cores": blas_threads(),
            "host_cores_visible": ncores, "cpu_model": model, "kind": "oracle",
            "ms_per_call_equivalent": round(sw.F * sw.N / tok_s * 1e3, 1),
            "sample": f"{done} of {sw.F} frames ({sw.H} heads each, materialised fp64 softmax), "
                      f"{spent:.1f} s, scaled to tokens/s"}


if __name__ == "__main__":
    main()
