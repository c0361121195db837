"""Throughput of the Q4 x Q8 block-quantised matmul path on one MI355X.

Headline: Llama-3.2-1B-shaped decode at batch 1.  One step reads every Q4
weight of 16 layers once (Q, K, V, O 2048 x 2048 / 512 x 2048, gate/up
8192 x 2048, down 2048 x 8192).  Each layer has four synthetic fp32
activation rows x ~ N(0,1) (attention input, O input, FFN input, down input)
with their own norm weights g ~ N(1, 0.1); every row goes through the fused
RMSNorm * g -> Q8 prologue once and the products that share it read the same
codes.  The step is one grouped call: a prologue pass over the 64 rows, then
one streaming launch over the 112 products, captured in a HIP graph and
replayed back to back: value = algorithmic bytes per step / mean replay time
over the timed replays (two timing-only HIP events around them), where the
bytes are the
Q4 weights (18 B per 32), each matrix's Q8 activation (36 B per 32) and its
fp32 output.

Also reported in the same JSON line (not part of value):
  roofline      the streaming kernel alone (the dominant kernel), timed per
                launch with HIP events on its stream, against 8 TB/s; traffic
                is the calibrated FETCH_SIZE + WRITE_SIZE of the committed
                counter summary, or null when the kernel sources changed since;
  cpu_baseline  the multithreaded oracle on this host over the same step;
  chained       the same step as a real decoder would order it (per layer:
                Q/K/V group, O, gate/up group, down);
  unfused       one prologue launch per activation row and one launch per
                matrix (176 launches per step);
  decode_8b     Llama-3-8B-shaped decode (8 layers) at B = 1, 2, 4, 8;
  prefill       Llama-3-8B-shaped prefill GEMM (one layer) at T = 512, 2048,
                int8 TOPS against 5.0 POPS;
  moe           MUL_MAT_ID decode (64 experts, 16 tokens, top-8).

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--skip-extras]
       python bench.py --kernel-only 10      (launches for rocprofv3 runs)
       python bench.py --gemm-only 10        (prefill GEMM launches for rocprofv3 runs)
       python bench.py --moe-only 10         (routed MoE launches for rocprofv3 runs)
       python bench.py --moe-widths          (routed call time per pass width, the MoE schedule's window costs)
       python bench.py --q8-0-only 10        (Q8_0 weight launches for rocprofv3 runs)
       python bench.py --decode-8b-only B 10 (Llama-3-8B-shaped decode steps at batch B for rocprofv3 runs)
       python bench.py --pmc-summary FETCH_DIR WRITE_DIR [REQ_DIR]   (traffic summary)
       python bench.py --trace-summary DIR   (kernel durations of a --kernel-trace run)
       python bench.py --trace-calls DIR KERNEL ROLE [ROLE ...]   (one kernel's dispatches by role, in order)
       python bench.py --counter-summary KERNEL DIR [DIR ...]   (counters of --pmc runs)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
I8_PEAK_TOPS = 5000.0


def q4_bytes(M, K):
    return M * K * 9 // 16


def gemv_bytes(M, K, B):
    return q4_bytes(M, K) + B * K * 9 // 8 + B * M * 4


def capture(fn):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, steps, warmup):
    """Plain average over `steps` replays after `warmup`, bracketed by
    synchronisation on both sides (one process, so no barrier is needed)."""
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


class TimingEvents:
    """HIP events made for timing only, through the HIP runtime that torch
    loaded: created with hipEventDisableSystemFence, so that recording one
    does not write back and invalidate the caches between the steps it
    separates (a default event does, and that costs the next step several
    microseconds; the runtime documents the flag for timing events)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes

        import torch
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self._ct = ctypes
        self._hip = ctypes.CDLL(path)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self._hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def record(self, i, stream):
        rc = self._hip.hipEventRecord(self.ev[i], self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i, j):
        f = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(f), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def time_graph_replays(g, steps, warmup):
    """A captured step replayed back to back: `warmup` replays, a
    synchronisation, then `steps` replays between two timing-only HIP events
    on the current stream and a synchronisation (the timed region; its mean
    per replay is the step time).  A second pass of `steps` replays records
    an event after every replay as well, for the distribution of single
    replays (median, min, max; those extra events cost a few microseconds per
    replay, so the second pass is not the step time).  Returns (mean ms of the
    timed region, wall seconds of it, median ms, min ms, max ms of pass 2)."""
    import statistics

    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = TimingEvents(2)
    t0 = time.perf_counter()
    ev.record(0, stream)
    for _ in range(steps):
        g.replay()
    ev.record(1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = ev.elapsed_ms(0, 1) / steps
    ev.close()
    ev = TimingEvents(steps + 1)
    ev.record(0, stream)
    for i in range(steps):
        g.replay()
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    per = [ev.elapsed_ms(i, i + 1) for i in range(steps)]
    ev.close()
    return mean, wall, statistics.median(per), min(per), max(per)


def time_direct(fn, steps, warmup):
    """Average time of `steps` back-to-back calls of fn on the current stream
    after `warmup` calls, bracketed by synchronisation on both sides (one
    process, so no barrier is needed)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def gpu_clocks(busy=None):
    """Shader (sclk) and memory (mclk) clocks as rocm-smi reports them (a
    read-only query), taken while `busy` keeps the GPU loaded (it is called
    over and over until the query returns, at most 20 s); from the sysfs DPM
    tables (active level marked '*') if rocm-smi gives nothing.  Only values
    that carry a frequency unit are kept."""
    import glob
    import subprocess

    import torch
    out = {"sclk": None, "mclk": None, "source": None, "under_load": busy is not None}
    try:
        proc = subprocess.Popen(["rocm-smi", "--showclocks", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
        t0 = time.perf_counter()
        while busy is not None and proc.poll() is None and time.perf_counter() - t0 < 20:
            busy()
            torch.cuda.synchronize()
        stdout, _ = proc.communicate(timeout=20)
        data = json.loads(stdout)
        card = data[sorted(data)[0]]
        for k, v in card.items():
            kl, vs = k.lower(), str(v)
            if "hz" not in vs.lower():
                continue
            for key in ("sclk", "mclk"):
                if kl.startswith(key):
                    out[key] = vs
        out["source"] = "rocm-smi --showclocks"
    except Exception:
        pass
    if out["sclk"] is None:
        for key in ("sclk", "mclk"):
            for f in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{key}")):
                try:
                    with open(f) as fh:
                        act = [l.strip() for l in fh if "*" in l]
                    if act:
                        out[key] = act[0]
                        out["source"] = "sysfs pp_dpm_*"
                        break
                except OSError:
                    continue
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def per_launch_ms(fn, reps):
    """Average duration of one launch of fn: `reps` launches back to back on
    the current stream (the stream fn launches on), HIP events recorded on
    that stream before the first and after the last."""
    import torch
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def per_launch_graph_ms(fn, reps=20, replays=20):
    """Average GPU time of one launch of fn: `reps` calls captured back to
    back in one HIP graph, the graph replayed `replays` times between two
    HIP events (per_launch_ms over direct calls measures the host's call
    rate for launches this short)."""
    g = capture(lambda: [fn() for _ in range(reps)])
    ms, _ = time_graph(g, replays, 3)
    return ms / reps


class DecodeModel:
    """Quantised weights, activations and outputs of a decode workload."""

    def __init__(self, layer_shapes, n_layers, B, seed, dev):
        import torch

        import block_quantized_matmul_q8_amd as q
        import workloads as wl

        self.layer_shapes, self.n_layers, self.B = layer_shapes, n_layers, B
        self.mats = []      # per layer: list of dicts
        self.acts = []      # per layer: {slot: (x, g)}
        for l in range(n_layers):
            acts = {}
            for slot, K in wl.slot_k(layer_shapes).items():
                acts[slot] = (wl.activation_device(seed, l, slot, B, K, dev),
                              wl.norm_weight_device(seed, l, slot, K, dev))
            mats = []
            for mi, m in enumerate(layer_shapes):
                w = wl.weight_device(seed, l, mi, m.M, m.K, dev)
                qs, d = q.q4_quantize(w)
                del w
                mats.append({"name": m.name, "M": m.M, "K": m.K, "slot": m.slot, "qs": qs, "d": d,
                             "y": torch.zeros((B, m.M), dtype=torch.float32, device=dev)})
            self.mats.append(mats)
            self.acts.append(acts)
        torch.cuda.synchronize()
        self.step_bytes = n_layers * sum(gemv_bytes(m.M, m.K, B) for m in layer_shapes)

    def problems(self, layer, names=None):
        out = []
        for m in self.mats[layer]:
            if names is not None and m["name"] not in names:
                continue
            x, g = self.acts[layer][m["slot"]]
            out.append({"qs": m["qs"], "d": m["d"], "y": m["y"], "x": x, "g": g, "eps": 1e-5})
        return out


def decode_1b_groups(model):
    """The headline step (fp32 rows, prologue pass + streaming pass) and the
    same products over precomputed Q8 planes (the streaming pass alone)."""
    import block_quantized_matmul_q8_amd as q

    probs = []
    for l in range(model.n_layers):
        probs += model.problems(l)
    step = q.Group(probs, B=model.B)
    q8 = []
    for l in range(model.n_layers):
        planes = {s: q.q8_quantize_rmsnorm(x, g, 1e-5)[:2] for s, (x, g) in model.acts[l].items()}
        for m in model.mats[l]:
            xq, xd = planes[m["slot"]]
            q8.append({"qs": m["qs"], "d": m["d"], "y": m["y"], "xq": xq, "xd": xd})
    stream_only = q.Group(q8, B=model.B)
    return step, stream_only


KERNEL_SOURCES = ("block_quantized_matmul_q8_amd/csrc/gemv.hip", "block_quantized_matmul_q8_amd/csrc/gemv_dev.h",
                  "block_quantized_matmul_q8_amd/csrc/common.h", "block_quantized_matmul_q8_amd/csrc/prologue_dev.h")
TRAFFIC_SUMMARY = "profiles/gemv_stream_llama1b_decode_traffic.txt"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """Calibrated HBM bytes per launch of the streaming kernel from the
    committed counter summary, if it was taken on the current sources."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None, "no counter summary"
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("RESULT "):
                rec = json.loads(line[len("RESULT "):])
    if rec is None:
        return None, "counter summary without a RESULT line"
    if rec.get("source_hash") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    return rec["traffic_bytes_per_launch"], TRAFFIC_SUMMARY


def bench_decode_1b(args, dev, report):
    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    model = DecodeModel(wl.LLAMA_3_2_1B, 16, 1, 0, dev)
    step, stream_only = decode_1b_groups(model)
    # headline: the step captured in a HIP graph, replayed back to back
    g_step = capture(lambda: step())
    ms, wall, ms_med, ms_min, ms_max = time_graph_replays(g_step, args.steps, args.warmup)

    def busy():
        for _ in range(200):
            g_step.replay()
    clocks = gpu_clocks(busy)
    del g_step
    value = model.step_bytes / (ms * 1e-3) / 1e9
    # the same step launched directly, back to back (no graph)
    ms_direct, _ = time_direct(lambda: step(), args.steps, args.warmup)

    # dominant kernel: the streaming pass, the same launch as the step's second
    # kernel (same products, Q8 planes of the same values)
    dom_ms = per_launch_ms(lambda: stream_only(), max(args.steps, 10))
    dom_kernel = q.q4q8_last_kernel()
    dom_gbs = model.step_bytes / (dom_ms * 1e-3) / 1e9
    traffic, traffic_src = committed_traffic()

    extras = {}
    if not args.skip_extras:
        extras.update(decode_1b_extras(args, dev, model))

    report.update({
        "metric": "Q4xQ8 GEMV HBM GB/s at B=1 (Llama-3.2-1B-shaped decode step)",
        "value": round(value, 1),
        "unit": "GB/s",
        "ms_per_step": round(ms, 5),
        "wall_s_timed": round(wall, 4),
        "step_bytes": model.step_bytes,
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "launches_per_step": 2,
        "timing": (f"the step captured in a HIP graph; {args.warmup} warm-up replays and a synchronisation, "
                   f"then {args.steps} replays back to back between two HIP events (created with "
                   "hipEventDisableSystemFence, timing-only events) and a synchronisation; value and "
                   "ms_per_step from the mean replay time of that region"),
        "graph_replay_stats": {"median_ms": round(ms_med, 5), "min_ms": round(ms_min, 5), "max_ms": round(ms_max, 5),
                               "how": (f"a second pass of {args.steps} replays with an event after each one; "
                                       "those events add a few microseconds to every replay")},
        "direct_launches": {"GB/s": round(model.step_bytes / (ms_direct * 1e-3) / 1e9, 1),
                            "ms_per_step": round(ms_direct, 5),
                            "timing": "the same step launched directly, back to back, mean over the timed steps"},
        "gpu_clocks": clocks,
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": dom_kernel,
                     "launch": "the grouped streaming pass over the 112 products, on Q8 planes",
                     "bytes_per_launch": model.step_bytes, "avg_launch_ms": round(dom_ms, 5),
                     "timing": "back-to-back launches between two HIP events on the launch stream"},
    })
    report.update(extras)
    return model


def decode_1b_extras(args, dev, model):
    import torch

    import block_quantized_matmul_q8_amd as q

    extras = {}
    # chained: per layer Q/K/V group, O, gate/up group, down (each a prologue
    # pass and a streaming pass)
    chain = []
    for l in range(model.n_layers):
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            chain.append(q.Group(model.problems(l, names), B=1))
    g_chain = capture(lambda: [c() for c in chain])
    ms_c, _ = time_graph(g_chain, args.steps, args.warmup)
    extras["chained"] = {"GB/s": round(model.step_bytes / (ms_c * 1e-3) / 1e9, 1),
                         "ms_per_step": round(ms_c, 4), "launches_per_step": 8 * model.n_layers}
    # unfused: one prologue launch per activation row, one launch per matrix
    bufs = []
    for l in range(model.n_layers):
        per = {}
        for slot, (x, gw) in model.acts[l].items():
            K = x.shape[1]
            per[slot] = (x, gw, torch.empty((1, K), dtype=torch.int8, device=dev),
                         torch.empty((1, K // 32), dtype=torch.float32, device=dev))
        bufs.append(per)

    def unfused():
        for l in range(model.n_layers):
            for slot, (x, gw, xq, xd) in bufs[l].items():
                q.q8_quantize_rmsnorm(x, gw, 1e-5, xq=xq, xd=xd)
            for m in model.mats[l]:
                _, _, xq, xd = bufs[l][m["slot"]]
                q.mul_mat_q4q8(m["qs"], m["d"], xq, xd, y=m["y"])

    g_unf = capture(unfused)
    ms_u, _ = time_graph(g_unf, args.steps, args.warmup)
    extras["unfused"] = {"GB/s": round(model.step_bytes / (ms_u * 1e-3) / 1e9, 1),
                         "ms_per_step": round(ms_u, 4), "launches_per_step": 11 * model.n_layers}
    # folded: the prologue folded into every workgroup of the streaming kernel
    # (single-product entry point, one launch per matrix)
    def folded():
        for l in range(model.n_layers):
            for m in model.mats[l]:
                x, gw = model.acts[l][m["slot"]]
                q.mul_mat_q4q8_rmsnorm(m["qs"], m["d"], x, gw, 1e-5, y=m["y"])
    g_fold = capture(folded)
    ms_f, _ = time_graph(g_fold, args.steps, args.warmup)
    extras["folded_per_matrix"] = {"GB/s": round(model.step_bytes / (ms_f * 1e-3) / 1e9, 1),
                                   "ms_per_step": round(ms_f, 4), "launches_per_step": 7 * model.n_layers}
    del g_chain, g_unf, g_fold
    return extras


def kernel_only(n, dev):
    """Launch sequence for profiler runs: a calibration copy of 256 MiB, then
    n headline steps and n streaming passes."""
    import torch

    import workloads as wl

    model = DecodeModel(wl.LLAMA_3_2_1B, 16, 1, 0, dev)
    step, stream_only = decode_1b_groups(model)
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()
    for i in range(n):
        step()
        stream_only()
    torch.cuda.synchronize()
    print(f"[kernel-only] {n} copies of 256 MiB, {n} steps, {n} streaming passes; step_bytes {model.step_bytes}",
          flush=True)


def gemm_only(n, dev):
    """Launch sequence for profiler runs of the prefill GEMM: the Llama-3-8B
    layer's seven products as one grouped tiled launch over Q8 planes of
    T = 2048 tokens, n times."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    T = 2048
    layer = wl.LLAMA_3_8B
    probs = []
    planes = {}
    for slot, K in wl.slot_k(layer).items():
        x = wl.activation_device(2, 0, slot, T, K, dev)
        g = wl.norm_weight_device(2, 0, slot, K, dev)
        planes[slot] = q.q8_quantize_rmsnorm(x, g, 1e-5)[:2]
    for mi, m in enumerate(layer):
        w = wl.weight_device(2, 0, mi, m.M, m.K, dev)
        qs, d = q.q4_quantize(w)
        del w
        y = torch.empty((T, m.M), dtype=torch.float32, device=dev)
        probs.append({"qs": qs, "d": d, "y": y, "xq": planes[m.slot][0], "xd": planes[m.slot][1]})
    gemm = q.Group(probs, B=T)
    torch.cuda.synchronize()
    for _ in range(n):
        gemm()
    torch.cuda.synchronize()
    ops = 2 * T * sum(m.M * m.K for m in layer)
    print(f"[gemm-only] {n} grouped prefill launches, T={T}, {ops} int8 ops each", flush=True)


def q8_0_only(n, dev):
    """Launch sequence for profiler runs of the Q8_0 weight type: the
    Llama-3-8B layer shapes as Q8_0, 4 layers; n grouped streaming launches at
    B = 1 over the 28 products, then n grouped tiled launches at T = 2048 over
    one layer's seven products (all on Q8 planes)."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    layer = wl.LLAMA_3_8B
    mats = []
    for l in range(4):
        for mi, m in enumerate(layer):
            w = wl.weight_device(3, l, mi, m.M, m.K, dev)
            qw, d = q.q8_0_quantize(w)
            del w
            mats.append((m, qw, d))
    for B in (1, 2048):
        planes = {}
        for slot, K in wl.slot_k(layer).items():
            x = wl.activation_device(3, 0, slot, B, K, dev)
            g = wl.norm_weight_device(3, 0, slot, K, dev)
            planes[slot] = q.q8_quantize_rmsnorm(x, g, 1e-5)[:2]
        use = mats if B == 1 else mats[:7]
        ys = [torch.empty((B, m.M), dtype=torch.float32, device=dev) for m, _, _ in use]
        grp = q.Group([{"qw": qw, "d": d, "y": y, "xq": planes[m.slot][0], "xd": planes[m.slot][1]}
                       for (m, qw, d), y in zip(use, ys)], B=B)
        torch.cuda.synchronize()
        for _ in range(n):
            grp()
        torch.cuda.synchronize()
        if B == 1:
            nbytes = sum(q8_0_bytes(m.M, m.K) + m.K * 9 // 8 + m.M * 4 for m, _, _ in use)
            print(f"[q8_0-only] {n} grouped decode launches, B=1, {len(use)} products, {nbytes} bytes each",
                  flush=True)
        else:
            ops = 2 * B * sum(m.M * m.K for m in layer)
            print(f"[q8_0-only] {n} grouped prefill launches, T={B}, {ops} int8 ops each", flush=True)
        del grp, ys, planes


def moe_weight_copies(dev, n_copies=4):
    """n_copies independent sets of the MoE expert weights (stacked gate/up
    [E][2 x 1408][2048] and down [E][2048][1408], 311 MB per set): steps
    rotate over them, so the 256 MB last-level cache cannot serve a step from
    the previous one."""
    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    cfg = wl.MOE
    copies = []
    for c in range(n_copies):
        qsd = []
        for i, (M, K) in enumerate(((2 * cfg.ffn, cfg.hidden), (cfg.hidden, cfg.ffn))):
            w = wl.weight_device(3 + 16 * c, 0, i, cfg.E * M, K, dev)
            qs, d = q.q4_quantize(w)
            del w
            qsd.append((qs.view(cfg.E, M, K // 2), d.view(cfg.E, M, K // 32)))
        copies.append(qsd)
    return copies


def moe_widths(dev):
    """The measurements behind the routed schedule's window costs: one routed
    call with every expert of a 64-expert layer at exactly w pairs (token t
    selects experts 8t .. 8t + 7 mod 64, 8w tokens), for w = 1, 2, 3, 4, 5, 8,
    in the 1536 band (the down projection's shape, K = 1408, one row per
    (token, slot)) and the 2048 band (the stacked gate/up shape, 2816 rows,
    K = 2048, one row per token); GPU time per call from 10 calls captured in
    a HIP graph and replayed."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    E = 64
    for M, K, S in ((2048, 1408, 8), (2816, 2048, 1)):
        w = wl.weight_device(5, 0, 0, E * M, K, dev)
        qs, d = q.q4_quantize(w)
        del w
        qs, d = qs.view(E, M, K // 2), d.view(E, M, K // 32)
        times = []
        for width in (1, 2, 3, 4, 5, 8):
            T = 8 * width
            ids = torch.tensor([[(8 * t + j) % E for j in range(8)] for t in range(T)], dtype=torch.int32,
                               device=dev)
            x = wl.activation_device(5, 1, width, T * S, K, dev)
            g = wl.norm_weight_device(5, 1, 0, K, dev)
            xq, xd, _ = q.q8_quantize_rmsnorm(x, g, 1e-5)
            xq, xd = xq.view(T, S, K), xd.view(T, S, K // 32)
            y = torch.empty((T, 8, M), dtype=torch.float32, device=dev)
            ws = torch.empty(q.mul_mat_id_q4q8_workspace(E, T, 8), dtype=torch.uint8, device=dev)
            ms = per_launch_graph_ms(lambda: q.mul_mat_id_q4q8(qs, d, xq, xd, ids, y=y, ws=ws), reps=10, replays=10)
            times.append(f"{width} pairs {ms * 1e3:.1f} us")
        print(f"M = {M}, K = {K}: " + " | ".join(times), flush=True)


def moe_only(n, dev):
    """Launch sequence for profiler runs of the routed MoE step (stacked
    gate/up and down routed calls on the 64-expert, 16-token, top-8 shape),
    n times."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    cfg = wl.MOE
    ids = torch.from_numpy(wl.expert_ids(0, cfg.T, cfg.E, cfg.top_k)).to(dev)
    copies = moe_weight_copies(dev)
    calls = []
    for i, (M, K, S) in enumerate(((2 * cfg.ffn, cfg.hidden, 1), (cfg.hidden, cfg.ffn, cfg.top_k))):
        x = wl.activation_device(3, 0, i, cfg.T * S, K, dev)
        g = wl.norm_weight_device(3, 0, i, K, dev)
        xq, xd, _ = q.q8_quantize_rmsnorm(x, g, 1e-5)
        y = torch.empty((cfg.T, cfg.top_k, M), dtype=torch.float32, device=dev)
        ws = torch.empty(q.mul_mat_id_q4q8_workspace(cfg.E, cfg.T, cfg.top_k), dtype=torch.uint8, device=dev)
        calls.append((xq.view(cfg.T, S, K), xd.view(cfg.T, S, K // 32), y, ws))
    torch.cuda.synchronize()
    for step in range(n):
        for (qs, d), (xq, xd, y, ws) in zip(copies[step % len(copies)], calls):
            q.mul_mat_id_q4q8(qs, d, xq, xd, ids, y=y, ws=ws)
    torch.cuda.synchronize()
    print(f"[moe-only] {n} MoE steps (2 routed calls each, rotating {len(copies)} weight copies)", flush=True)


def decode_8b_only(B, n, dev):
    """Launch sequence for profiler runs of the Llama-3-8B-shaped decode group
    (8 layers x 7 Q4 matrices) at batch B: n grouped steps (prologue pass +
    streaming pass)."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    model = DecodeModel(wl.LLAMA_3_8B, 8, B, 1, dev)
    probs = []
    for l in range(8):
        probs += model.problems(l)
    grp = q.Group(probs, B=B)
    torch.cuda.synchronize()
    for _ in range(n):
        grp()
    torch.cuda.synchronize()
    print(f"[decode-8b-only] B={B}: {n} grouped steps, {model.step_bytes} algorithmic bytes each", flush=True)


def trace_summary(trace_dir):
    """Per-kernel duration table of a rocprofv3 --kernel-trace run (csv
    output): calls, mean, median, min and max in microseconds, plus the
    registers and LDS of each kernel of this library, sorted by total time."""
    import csv
    import glob
    import statistics

    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    dur, res = {}, {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("void ", "", 1).split("(")[0]
                if name.startswith("at::native::"):
                    name = "at::native:: (torch set-up kernels)"
                dur.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                if name.startswith("q4q8::"):
                    res[name] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["LDS_Block_Size"])
    print(f"{'kernel':58s} {'calls':>6s} {'mean us':>9s} {'median us':>10s} {'min us':>9s} {'max us':>9s}")
    for name, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        print(f"{name[:58]:58s} {len(v):6d} {statistics.fmean(v):9.2f} {statistics.median(v):10.2f} "
              f"{min(v):9.2f} {max(v):9.2f}")
    if res:
        print("\nresources per kernel instance, as the trace records them: VGPR_Count (on gfx950 half the\n"
              "compiler's per-lane VGPR count, e.g. 234 -> 120), accumulation VGPRs, SGPRs, LDS bytes:")
        for name, (v, a, sg, lds) in sorted(res.items()):
            print(f"  {name}: {v} / {a} / {sg} / {lds}")


def trace_calls(trace_dir, needle, roles):
    """Durations of the dispatches of the kernel whose name contains `needle`
    in a --kernel-trace run, in launch order, dispatch i counted for role
    roles[i % len(roles)] (e.g. the two routed calls of a MoE step, which
    launch the same kernel instance): calls, mean, median, min, max in us."""
    import csv
    import glob
    import statistics

    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if needle in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = {k: [] for k in roles}
    for i, r in enumerate(rows):
        per[roles[i % len(roles)]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"{'call':20s} {'calls':>6s} {'mean us':>9s} {'median us':>10s} {'min us':>9s} {'max us':>9s}")
    for k in roles:
        v = per[k]
        print(f"{k:20s} {len(v):6d} {statistics.fmean(v):9.2f} {statistics.median(v):10.2f} {min(v):9.2f} "
              f"{max(v):9.2f}")


def counter_summary(needle, dirs):
    """Per-dispatch medians of every counter that rocprofv3 --pmc runs (csv
    output, one directory per pass) collected for the kernels whose name
    contains `needle`; dispatch durations come from no counter, so none here."""
    import csv
    import glob
    import statistics

    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            per = {}
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if needle not in r["Kernel_Name"]:
                        continue
                    key = (r["Counter_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            for (c, _), v in per.items():
                vals.setdefault(c, []).append(v)
    for c in sorted(vals):
        print(f"  {c:30s} {statistics.median(vals[c]):.4e}   (median of {len(vals[c])} dispatches)")


def pmc_summary(fetch_dir, write_dir, req_dir=None):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the streaming kernel,
    scaled by what the same counters read for the 256 MiB copy; with req_dir
    (a pass over TCC_EA0_RDREQ_sum, TCC_EA0_RDREQ_32B_sum, TCC_EA0_RDREQ_64B_sum,
    TCC_EA0_RDREQ_128B_sum), the read bytes are also counted directly from the
    request sizes, which explains the fetch factor."""
    import csv
    import glob
    import statistics

    def read(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = {}
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] != counter:
                        continue
                    key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
                    rows[key] = rows.get(key, 0.0) + float(r["Counter_Value"])
        per = {}
        for (k, _), v in rows.items():
            per.setdefault(k, []).append(v)
        return per

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    copy_bytes = 256 << 20

    def pick(per, needle):
        ks = [k for k in per if needle in k]
        if not ks:
            raise SystemExit(f"no kernel matching {needle}: {sorted(per)[:8]}")
        return statistics.median(v for k in ks for v in per[k])

    copy_f, copy_w = pick(fetch, "copyBuffer") * 1024, pick(write, "copyBuffer") * 1024
    f_factor, w_factor = copy_bytes / copy_f, copy_bytes / copy_w
    gem_f, gem_w = pick(fetch, "gemv_kernel") * 1024, pick(write, "gemv_kernel") * 1024
    traffic = gem_f * f_factor + gem_w * w_factor
    import workloads as wl
    step_bytes = 16 * sum(gemv_bytes(m.M, m.K, 1) for m in wl.LLAMA_3_2_1B)
    lines = [
        "calibration: 256 MiB device copy (torch copy_, served by the runtime kernel __amd_rocclr_copyBuffer)",
        f"  FETCH_SIZE {copy_f / 1024:.0f} KiB per dispatch -> factor {f_factor:.4f}",
        f"  WRITE_SIZE {copy_w / 1024:.0f} KiB per dispatch -> factor {w_factor:.4f}",
        "streaming kernel (gemv_kernel, Llama-3.2-1B-shaped decode step, 112 products, median over dispatches)",
        f"  FETCH_SIZE raw {gem_f / 1024:.0f} KiB -> {gem_f * f_factor / 1e6:.2f} MB",
        f"  WRITE_SIZE raw {gem_w / 1024:.0f} KiB -> {gem_w * w_factor / 1e6:.3f} MB",
        f"  calibrated traffic {traffic / 1e6:.2f} MB per launch vs {step_bytes / 1e6:.2f} MB algorithmic "
        f"({traffic / step_bytes:.3f}x)",
    ]
    rec = {"traffic_bytes_per_launch": int(round(traffic)), "algorithmic_bytes": step_bytes,
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "source_hash": kernel_source_hash()}
    if req_dir:
        req = {c: read(req_dir, c) for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                                             "TCC_EA0_RDREQ_128B_sum")}

        def direct(needle):
            n = {c: pick(v, needle) for c, v in req.items()}
            b = 32 * n["TCC_EA0_RDREQ_32B_sum"] + 64 * n["TCC_EA0_RDREQ_64B_sum"] + 128 * n["TCC_EA0_RDREQ_128B_sum"]
            return b, n
        cb, cn = direct("copyBuffer")
        gb, gn = direct("gemv_kernel")
        lines += [
            "cross-check from the read-request sizes (bytes = 32 x 32B + 64 x 64B + 128 x 128B requests; no calibration):",
            f"  copy: requests {cn['TCC_EA0_RDREQ_sum']:.0f} (32B {cn['TCC_EA0_RDREQ_32B_sum']:.0f}, 64B "
            f"{cn['TCC_EA0_RDREQ_64B_sum']:.0f}, 128B {cn['TCC_EA0_RDREQ_128B_sum']:.0f}) -> {cb / 2**20:.1f} MiB "
            f"for 256 MiB read ({cb / copy_bytes:.4f}x)",
            f"  streaming kernel: requests {gn['TCC_EA0_RDREQ_sum']:.0f} (32B {gn['TCC_EA0_RDREQ_32B_sum']:.0f}, 64B "
            f"{gn['TCC_EA0_RDREQ_64B_sum']:.0f}, 128B {gn['TCC_EA0_RDREQ_128B_sum']:.0f}) -> {gb / 1e6:.2f} MB read "
            f"({(gb + gem_w * w_factor) / step_bytes:.3f}x algorithmic with the writes)",
            f"  raw FETCH_SIZE / (64 B x requests): copy {copy_f / (64 * cn['TCC_EA0_RDREQ_sum']):.4f}, streaming "
            f"kernel {gem_f / (64 * gn['TCC_EA0_RDREQ_sum']):.4f}: FETCH_SIZE's expression on this GPU counts a "
            "request as 64 B unless TCC_BUBBLE marks it 128 B, and nearly every read here is a 128-byte request, "
            "so the raw counter reads half the bytes; that is the copy's factor of 2",
        ]
        rec["direct_read_bytes_per_launch"] = int(round(gb))
        rec["copy_direct_over_moved"] = round(cb / copy_bytes, 4)
    print("\n".join(lines))
    print("RESULT " + json.dumps(rec))


def bench_decode_8b(args, dev):
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    out = {}
    n_layers = 8
    for B in (1, 2, 4, 8):
        model = DecodeModel(wl.LLAMA_3_8B, n_layers, B, 1, dev)
        probs = []
        for l in range(n_layers):
            probs += model.problems(l)
        grp = q.Group(probs, B=B)
        fn = lambda: grp()
        route = "grouped: prologue pass + streaming pass"
        ms, _ = time_direct(fn, max(5, args.steps // 2), 2)
        out[f"B={B}"] = {"GB/s": round(model.step_bytes / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms, 4),
                         "hbm_frac": round(model.step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "route": route}
        del grp, model
        torch.cuda.empty_cache()
    return {"layers": n_layers, **out}


def bench_prefill(args, dev):
    """Llama-3-8B-shaped prefill, one layer: the seven products as one grouped
    tiled launch.  `TOPS` times that launch over Q8 planes (the GEMM alone);
    `step` adds the prologue pass over the four fp32 activation inputs."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    out = {}
    layer = wl.LLAMA_3_8B
    mats = []
    for mi, m in enumerate(layer):
        w = wl.weight_device(2, 0, mi, m.M, m.K, dev)
        qs, d = q.q4_quantize(w)
        del w
        mats.append((m, qs, d))
    for T in (512, 2048):
        acts, planes = {}, {}
        for slot, K in wl.slot_k(layer).items():
            x = wl.activation_device(2, 0, slot, T, K, dev)
            gw = wl.norm_weight_device(2, 0, slot, K, dev)
            acts[slot] = (x, gw)
            planes[slot] = q.q8_quantize_rmsnorm(x, gw, 1e-5)[:2]
        ys = [torch.empty((T, m.M), dtype=torch.float32, device=dev) for m, _, _ in mats]
        gemm = q.Group([{"qs": qs, "d": d, "y": y, "xq": planes[m.slot][0], "xd": planes[m.slot][1]}
                        for (m, qs, d), y in zip(mats, ys)], B=T)
        step = q.Group([{"qs": qs, "d": d, "y": y, "x": acts[m.slot][0], "g": acts[m.slot][1], "eps": 1e-5}
                        for (m, qs, d), y in zip(mats, ys)], B=T)
        ms = per_launch_ms(lambda: gemm(), max(5, args.steps // 2))
        kernel = q.q4q8_last_kernel()
        ms_step, _ = time_direct(lambda: step(), max(5, args.steps // 2), 2)
        ops = 2 * T * sum(m.M * m.K for m in layer)
        tops = ops / (ms * 1e-3) / 1e12
        out[f"T={T}"] = {"TOPS": round(tops, 1), "frac_i8_peak": round(tops / I8_PEAK_TOPS, 4),
                         "ms_per_layer": round(ms, 4), "kernel": kernel,
                         "step_with_prologue": {"TOPS": round(ops / (ms_step * 1e-3) / 1e12, 1),
                                                "ms": round(ms_step, 4)},
                         "launch": "one grouped tiled launch over the 7 products"}
        del gemm, step
    return out


def q8_0_bytes(M, K):
    return M * K * 17 // 16  # 32 int8 codes + one fp16 scale per 32 weights


def bench_q8_0(args, dev):
    """Q8_0 weights on the Llama-3-8B layer shapes, 4 layers (about 0.93 GB of
    weights, past the on-die caches).  Decode at B = 1 and 8 over Q8 planes:
    one grouped streaming launch over the 28 products (`GB/s`, over weights +
    Q8 activations + fp32 outputs), and one launch per matrix captured in a
    HIP graph (`per_matrix`).  Prefill at T = 2048: one grouped tiled launch
    over the seven products of one layer."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    layer = wl.LLAMA_3_8B
    n_layers = 4
    mats = []
    for l in range(n_layers):
        for mi, m in enumerate(layer):
            w = wl.weight_device(3, l, mi, m.M, m.K, dev)
            qw, d = q.q8_0_quantize(w)
            del w
            mats.append((m, qw, d))
    torch.cuda.synchronize()
    out = {"layers": n_layers}
    reps = max(5, args.steps // 2)
    for B in (1, 8):
        planes = {}
        for slot, K in wl.slot_k(layer).items():
            x = wl.activation_device(3, 0, slot, B, K, dev)
            gw = wl.norm_weight_device(3, 0, slot, K, dev)
            planes[slot] = q.q8_quantize_rmsnorm(x, gw, 1e-5)[:2]
        ys = [torch.empty((B, m.M), dtype=torch.float32, device=dev) for m, _, _ in mats]
        nbytes = sum(q8_0_bytes(m.M, m.K) + B * m.K * 9 // 8 + B * m.M * 4 for m, _, _ in mats)
        grp = q.Group([{"qw": qw, "d": d, "y": y, "xq": planes[m.slot][0], "xd": planes[m.slot][1]}
                       for (m, qw, d), y in zip(mats, ys)], B=B)
        ms_grp = per_launch_ms(lambda: grp(), reps)

        def step():
            for (m, qw, d), y in zip(mats, ys):
                q.mul_mat_q8_0_q8(qw, d, planes[m.slot][0], planes[m.slot][1], y=y)

        g = capture(step)
        ms, _ = time_graph(g, reps, 2)
        out[f"B={B}"] = {"GB/s": round(nbytes / (ms_grp * 1e-3) / 1e9, 1), "ms_per_launch": round(ms_grp, 4),
                         "hbm_frac": round(nbytes / (ms_grp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "route": "one grouped streaming launch over the 28 products",
                         "per_matrix": {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4),
                                        "launches": len(mats)}}
        del g, grp, ys, planes
    T = 2048
    planes = {}
    for slot, K in wl.slot_k(layer).items():
        x = wl.activation_device(3, 0, slot, T, K, dev)
        gw = wl.norm_weight_device(3, 0, slot, K, dev)
        planes[slot] = q.q8_quantize_rmsnorm(x, gw, 1e-5)[:2]
        del x
    ys = [torch.empty((T, m.M), dtype=torch.float32, device=dev) for m, _, _ in mats[:7]]
    gemm = q.Group([{"qw": qw, "d": d, "y": y, "xq": planes[m.slot][0], "xd": planes[m.slot][1]}
                    for (m, qw, d), y in zip(mats[:7], ys)], B=T)
    ms = per_launch_ms(lambda: gemm(), reps)
    ops = 2 * T * sum(m.M * m.K for m in layer)
    tops = ops / (ms * 1e-3) / 1e12
    out[f"prefill_T={T}"] = {"TOPS": round(tops, 1), "frac_i8_peak": round(tops / I8_PEAK_TOPS, 4),
                             "ms_per_layer": round(ms, 4), "launch": "one grouped tiled launch over the 7 products"}
    del gemm, ys, planes, mats
    torch.cuda.empty_cache()
    return out


def bench_prologues(args, dev):
    """The standalone activation prologues on Llama-3-8B-shaped rows
    (K = 4096): RMS_NORM+MUL -> Q8 and RMS_NORM+MUL+ADD -> Q8 (one addend row
    per input row), GPU time per launch from graph replays.  Bytes: x (and the addend) read, g read once,
    codes and scales written."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    K = 4096
    out = {}
    for B in (1, 8):
        x = wl.activation_device(6, 0, 0, B, K, dev)
        a = wl.activation_device(6, 1, 0, B, K, dev)
        g = wl.norm_weight_device(6, 0, 0, K, dev)
        xq = torch.empty((B, K), dtype=torch.int8, device=dev)
        xd = torch.empty((B, K // 32), dtype=torch.float32, device=dev)
        ms_n = per_launch_graph_ms(lambda: q.q8_quantize_rmsnorm(x, g, wl.RMS_EPS, xq=xq, xd=xd))
        ms_a = per_launch_graph_ms(lambda: q.q8_quantize_rmsnorm_add(x, g, a, wl.RMS_EPS, xq=xq, xd=xd))
        b_n = B * K * 4 + K * 4 + B * K * 9 // 8
        b_a = b_n + B * K * 4
        out[f"B={B}"] = {"rmsnorm_mul_q8": {"us": round(ms_n * 1e3, 2), "GB/s": round(b_n / (ms_n * 1e-3) / 1e9, 1)},
                         "rmsnorm_mul_add_q8": {"us": round(ms_a * 1e3, 2),
                                                "GB/s": round(b_a / (ms_a * 1e-3) / 1e9, 1)}}
    # SwiGLU -> Q8 from a stacked gate|up buffer: the MoE down projection's
    # 16 x 8 slot rows of 1408, and one Llama-3-8B decode row of 14336
    for name, rows, F in (("swiglu_q8 moe 128x1408", 128, 1408), ("swiglu_q8 8b 1x14336", 1, 14336)):
        buf = wl.activation_device(7, 0, 0, rows, 2 * F, dev)
        xq = torch.empty((rows, F), dtype=torch.int8, device=dev)
        xd = torch.empty((rows, F // 32), dtype=torch.float32, device=dev)
        ms = per_launch_graph_ms(lambda: q.q8_quantize_swiglu(buf[:, :F], buf[:, F:], xq=xq, xd=xd))
        nbytes = rows * F * 8 + rows * F * 9 // 8
        out[name] = {"us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    out["note"] = ("per launch: 20 launches captured in one HIP graph, replayed; norm prologues: one "
                   "1024-thread workgroup per row for up to 8 rows, latency-bound; swiglu_q8: eight lanes "
                   "per 32-block, no row reduction")
    return out


def bench_moe(args, dev):
    """MUL_MAT_ID decode (64 experts, 16 tokens, top-8).  Gate and up share
    the routing and each token's row, so they are one stacked expert tensor
    [E][2 * 1408][2048] (one routed call); down [E][2048][1408] takes one row
    per (token, slot).  Bytes count every distinct selected expert's weights
    once, plus the activations and outputs."""
    import torch

    import block_quantized_matmul_q8_amd as q
    import workloads as wl

    cfg = wl.MOE
    ids = torch.from_numpy(wl.expert_ids(0, cfg.T, cfg.E, cfg.top_k)).to(dev)
    copies = moe_weight_copies(dev)
    mats = []
    for i, (M, K, S) in enumerate(((2 * cfg.ffn, cfg.hidden, 1), (cfg.hidden, cfg.ffn, cfg.top_k))):
        x = wl.activation_device(3, 0, i, cfg.T * S, K, dev)
        gw = wl.norm_weight_device(3, 0, i, K, dev)
        xq, xd, _ = q.q8_quantize_rmsnorm(x, gw, 1e-5)
        y = torch.empty((cfg.T, cfg.top_k, M), dtype=torch.float32, device=dev)
        ws = torch.empty(q.mul_mat_id_q4q8_workspace(cfg.E, cfg.T, cfg.top_k), dtype=torch.uint8, device=dev)
        mats.append((xq.view(cfg.T, S, K), xd.view(cfg.T, S, K // 32), y, ws, M, K, S))
    step = [0]

    def fn():
        qsd = copies[step[0] % len(copies)]
        step[0] += 1
        for (qs, d), (xq, xd, y, ws, M, K, S) in zip(qsd, mats):
            q.mul_mat_id_q4q8(qs, d, xq, xd, ids, y=y, ws=ws)
    ms, _ = time_direct(fn, max(8, args.steps // 2), 4)
    distinct = len(set(ids.cpu().numpy().ravel().tolist()))
    nbytes = 0
    for xq, xd, y, ws, M, K, S in mats:
        nbytes += distinct * q4_bytes(M, K) + cfg.T * S * K * 9 // 8 + cfg.T * cfg.top_k * M * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the weighted expert-plane sum of the down projection's planes
    y_down = mats[1][2]
    w = torch.from_numpy(wl.expert_weights(0, cfg.T, cfg.top_k)).to(dev)
    out = torch.empty((cfg.T, cfg.hidden), dtype=torch.float32, device=dev)
    ms_sum = per_launch_graph_ms(lambda: q.moe_expert_sum_f32(y_down, w, out=out))
    sum_bytes = cfg.T * cfg.top_k * (cfg.hidden + 1) * 4 + cfg.T * cfg.hidden * 4
    return {"GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "ms_per_step": round(ms, 4),
            "distinct_experts": distinct, "bytes": nbytes,
            "launches": "2 routed calls (stacked gate/up, down), each one streaming launch whose workgroups route the pairs in LDS before streaming (a small routing)",
            "weight_copies": len(copies),
            "expert_sum": {"us": round(ms_sum * 1e3, 2), "GB/s": round(sum_bytes / (ms_sum * 1e-3) / 1e9, 1),
                           "bytes": sum_bytes,
                           "what": "weighted in-order sum of the down projection's 8 expert planes, "
                                   "[16][8][2048] -> [16][2048], one launch"}}


def cpu_baseline(model, seconds=10.0):
    """The oracle (plain C, output rows split over threads) on this host over
    the same decode step: oracle prologue per activation row, then every
    matrix; repeated until `seconds` have passed (at least once)."""
    import numpy as np

    import oracle

    # every CPU this process may run on, up to the 16 that one GPU's jobs are
    # allotted on the GPU machines
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    nthreads = max(1, min(avail, 16))
    host = []
    for l in range(model.n_layers):
        acts = {s: (x.cpu().numpy(), g.cpu().numpy()) for s, (x, g) in model.acts[l].items()}
        mats = [(m["slot"], m["qs"].cpu().numpy(), m["d"].cpu().numpy().view(np.uint16)) for m in model.mats[l]]
        host.append((acts, mats))
    reps = 0
    t0 = time.perf_counter()
    while True:
        for acts, mats in host:
            q8 = {s: oracle.q8_quantize_rmsnorm(x, g, 1e-5)[:2] for s, (x, g) in acts.items()}
            for slot, qs, d in mats:
                xq, xd = q8[slot]
                oracle.mul_mat(qs, d, xq, xd, nthreads=nthreads, want_y64=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = model.step_bytes * reps / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{reps} full decode step(s) of the Llama-3.2-1B-shaped workload (16 layers, B=1), "
                      f"{el:.1f} s, {nthreads} threads (output rows split over threads)",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "cpus_available": avail,
            "build": "gcc -O2 -ffp-contract=off -fno-fast-math, plain C, no intrinsics"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-extras", action="store_true", help="only the headline step and its roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--gemm-only", type=int, default=0, metavar="N",
                    help="launch N grouped prefill GEMMs (T=2048, Llama-3-8B layer) and exit")
    ap.add_argument("--q8-0-only", type=int, default=0, metavar="N",
                    help="launch N grouped Q8_0 decode launches (B=1) and N grouped Q8_0 prefill launches, and exit")
    ap.add_argument("--moe-only", type=int, default=0, metavar="N",
                    help="launch N routed MoE steps and exit")
    ap.add_argument("--moe-widths", action="store_true",
                    help="routed call time per pass width in the 1536 and 2048 bands, and exit")
    ap.add_argument("--kernel-only", type=int, default=0, metavar="N",
                    help="launch N steps and N streaming passes (after a calibration copy) and exit")
    ap.add_argument("--decode-8b-only", nargs=2, type=int, default=None, metavar=("B", "N"),
                    help="N grouped Llama-3-8B-shaped decode steps at batch B (for rocprofv3 runs)")
    ap.add_argument("--trace-calls", nargs="+", metavar="ARG",
                    help="DIR KERNEL ROLE [ROLE ...]: per-role durations of one kernel's dispatches in launch order")
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG",
                    help="KERNEL_SUBSTRING DIR [DIR ...]: per-dispatch counter medians of rocprofv3 --pmc runs "
                         "(no GPU needed)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace csv run (no GPU needed)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [REQ_DIR]: summarise rocprofv3 --pmc runs of --kernel-only "
                         "(no GPU needed)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.trace_calls:
        trace_calls(args.trace_calls[0], args.trace_calls[1], args.trace_calls[2:])
        return
    if args.counter_summary:
        counter_summary(args.counter_summary[0], args.counter_summary[1:])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library runs the product on one GPU and does not shard it across GPUs "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_matmul_q8_amd as q
    from block_quantized_matmul_q8_amd.build import LIB_PATH, build

    if not os.path.exists(LIB_PATH):
        build()
    q.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.kernel_only:
        kernel_only(args.kernel_only, dev)
        return
    if args.gemm_only:
        gemm_only(args.gemm_only, dev)
        return
    if args.moe_only:
        moe_only(args.moe_only, dev)
        return
    if args.moe_widths:
        moe_widths(dev)
        return
    if args.q8_0_only:
        q8_0_only(args.q8_0_only, dev)
        return
    if args.decode_8b_only:
        decode_8b_only(args.decode_8b_only[0], args.decode_8b_only[1], dev)
        return
    report = {}
    model = bench_decode_1b(args, dev, report)
    print(f"[bench] decode step done: {report['value']} GB/s", file=sys.stderr, flush=True)
    if not args.skip_extras:
        report["decode_8b"] = bench_decode_8b(args, dev)
        print("[bench] 8B decode done", file=sys.stderr, flush=True)
        report["prefill"] = bench_prefill(args, dev)
        p = report["prefill"]["T=2048"]
        report["roofline_gemm"] = {
            "bound": "mfma", "dtype": "i8", "achieved": p["TOPS"], "peak": I8_PEAK_TOPS, "unit": "TOPS",
            "frac": round(p["TOPS"] / I8_PEAK_TOPS, 4), "kernel": p["kernel"],
            "launch": "Llama-3-8B-shaped prefill layer, T = 2048: one grouped tiled launch over the 7 products "
                      "on Q8 planes",
            "ops_per_launch": 2 * 2048 * sum(m.M * m.K for m in __import__("workloads").LLAMA_3_8B),
            "avg_launch_ms": p["ms_per_layer"],
            "timing": "back-to-back launches between two HIP events on the launch stream",
            "profile": "profiles/gemm_prefill_llama8b_t2048.txt",
            "T=512": {"achieved": report["prefill"]["T=512"]["TOPS"],
                      "frac": report["prefill"]["T=512"]["frac_i8_peak"]}}
        print("[bench] prefill done", file=sys.stderr, flush=True)
        report["moe"] = bench_moe(args, dev)
        print("[bench] moe done", file=sys.stderr, flush=True)
        report["prologues"] = bench_prologues(args, dev)
        print("[bench] prologues done", file=sys.stderr, flush=True)
        report["q8_0"] = bench_q8_0(args, dev)
        print("[bench] q8_0 done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        report["cpu_baseline"] = cpu_baseline(model, args.cpu_seconds)
    else:
        report["cpu_baseline"] = None

    line = {
        "metric": report.pop("metric"),
        "value": report.pop("value"),
        "unit": report.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": report.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded, device-drawn N(0,0.02) weights, N(0,1) activations, N(1,0.1) norm weights)",
        "config": {"workload": "llama-3.2-1b-shaped decode, B=1, 16 layers x 7 Q4 matrices; RMSNorm*g->Q8 "
                               "prologue pass over the 64 activation rows + one streaming launch, captured in a "
                               "HIP graph and replayed back to back (mean replay time)",
                   "hidden": 2048, "ffn": 8192, "kv_rows": 512, "layers": 16, "B": 1},
        "roofline": report.pop("roofline"),
        "roofline_gemm": report.pop("roofline_gemm", None),
        "cpu_baseline": report.pop("cpu_baseline"),
    }
    line.update(report)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
