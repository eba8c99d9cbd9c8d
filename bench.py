#!/usr/bin/env python3
"""Benchmark of the W4A16 linear path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = one decode token through the four W4A16 linear layers of a
Llama-3.1-8B-shaped block (fused QKV 4096x6144, O 4096x4096, gate+up
4096x28672, down 14336x4096; asymmetric uint4 with packed zero points,
group 128, bf16 activations, M = 1).  Inputs are seeded synthetic tensors of
those shapes (no checkpoint), resident in HBM before timing starts.  Each
step reads a different copy of the weights from a pool larger than the
256 MB Infinity Cache, so the weights stream from HBM as they do when
consecutive layers differ.  The steps are captured in HIP graphs of one
step per weight copy and replayed, so the host's launch overhead is spread
over many steps and the kernels run back to back, as in a decode loop.

Printed: one JSON line with decode GB/s (algorithmic bytes / time), the
roofline of the decode kernel (per-launch durations from HIP events around
graphs of back-to-back launches of each layer), the prefill TFLOP/s at
M = 1920 on the Llama-3.1-8B prefill layers, and the CPU oracle timed on a
bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "decode HBM GB/s (% of peak) at M=1; prefill TFLOP/s (% MFMA peak) at M=1920"

DECODE_LAYERS = ((4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096))  # (K, N)
PREFILL_LAYERS = ((4096, 6144), (4096, 28672), (14336, 4096))
GROUP = 128


def decode_bytes(M, N, K, g, asym=True, bias=False):
    """Algorithmic bytes of one call: weights, scales, packed zero points, x, y (+bias)."""
    b = N * K // 2 + 2 * N * (K // g) + 2 * M * K + 2 * M * N
    if asym:
        b += (N // 8) * (K // g) * 4
    if bias:
        b += 2 * N
    return b


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "gemv_one_kernel_llama8b_decode_M1_traffic.txt")
DECODE_SOURCES = ("w4a16_gemv.hip", "w4a16_device.hpp", "w4a16_internal.h")


def decode_kernel_name(layer, M=1):
    """The decode kernel the planner picks for a layer (K, N) at M tokens."""
    import int4_weight_only_linear_amd as L
    K, N = layer
    p = L.w4a16_plan(M, N, K, GROUP, L.W4A16_BF16, True, L.PATH_GEMV)
    name = "gemv_one_kernel" if p["kernel"] == 1 else "gemv_small_kernel"
    return f"{name}<bf16, group {GROUP}, asym>"


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by a copy of known size), or None when the decode
    kernel's sources have changed since those counters were taken."""
    import hashlib
    try:
        fields = dict(l.split(": ", 1) for l in open(TRAFFIC_PROFILE).read().splitlines() if ": " in l)
        h = hashlib.sha256()
        csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int4_weight_only_linear_amd", "csrc")
        for f in DECODE_SOURCES:
            h.update(open(os.path.join(csrc, f), "rb").read())
        if fields.get("kernel_source_sha256", "").strip() != h.hexdigest():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def build_layer(K, N, M, seed, device):
    import torch
    from synth import make_case
    import int4_weight_only_linear_amd as L
    c = make_case(M, N, K, GROUP, 1, False, False, seed=seed)
    wq = torch.from_numpy(L.w4a16_pack_weights(c.q)).to(device)
    zp = torch.from_numpy(L.w4a16_pack_zeros(c.zp)).to(device)
    s = torch.from_numpy(c.s_bits.view(np.int16)).to(device).view(torch.bfloat16)
    x = torch.from_numpy(c.x_bits.view(np.int16)).to(device).view(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    return dict(K=K, N=N, M=M, wq=wq, zp=zp, s=s, x=x, y=y, case=c)


class Launcher:
    """Pre-marshalled C calls (pointers resolved once) for capture and timing."""

    def __init__(self, layer, wq, zp, s):
        import torch
        import int4_weight_only_linear_amd as L
        from int4_weight_only_linear_amd import _binding as B
        self.B = B
        # the call holds raw device pointers: keep their tensors alive with it
        # (graph capture empties torch's allocator cache, so a tensor freed
        # here would be unmapped by the time the graph replays)
        self.keep = (layer["x"], layer["y"], wq, zp, s)
        self.args = (layer["x"].data_ptr(), wq.data_ptr(), s.data_ptr(), zp.data_ptr(), None,
                     layer["y"].data_ptr(), layer["M"], layer["N"], layer["K"], GROUP, L.W4A16_BF16)
        need = L.w4a16_workspace_size(layer["M"], layer["N"], layer["K"], GROUP, L.W4A16_BF16, True)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=layer["x"].device) if need else None

    def __call__(self, stream_ptr):
        ws = None if self.ws is None else self.ws.data_ptr()
        nbytes = 0 if self.ws is None else self.ws.numel()
        self.B._check(self.B.lib.w4a16_linear(*self.args, ws, nbytes, stream_ptr))


def capture(launch_lists, stream):
    """One graph replaying the given launch lists back to back."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        sp = torch.cuda.current_stream().cuda_stream
        for launches in launch_lists:
            for fn in launches:
                fn(sp)
    torch.cuda.synchronize()
    return g


def time_steps(step_lists, steps, warmup, stream):
    """Time exactly `steps` steps; step i runs step_lists[i % len(step_lists)].

    The steps are captured in graphs of len(step_lists) consecutive steps
    (plus one graph for the remainder), so the host's launch cost is spread
    over many steps and the GPU runs them back to back.
    """
    import torch
    C = len(step_lists)
    full = capture(step_lists, stream)
    rem = capture(step_lists[: steps % C], stream) if steps % C else None
    for _ in range(max(1, -(-warmup // C))):  # at least `warmup` steps
        full.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps // C):
        full.replay()
    if rem is not None:
        rem.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def per_launch_durations(step_lists, reps, stream, passes=5, replays=4):
    """Mean duration of each launch position, from HIP events on the launch
    stream around `replays` back-to-back replays of a graph holding `passes`
    rounds of that position's launches (one per weight copy), so the graph
    and event overheads are spread over hundreds of launches and the kernels
    run back to back as they do inside a step.  (median, p10, p90) over
    `reps` graph replays, each the mean launch of its replay."""
    import torch
    out = []
    for j in range(len(step_lists[0])):
        g = capture([[fns[j]] for _ in range(passes) for fns in step_lists], stream)
        g.replay()
        torch.cuda.synchronize()
        n = passes * len(step_lists) * replays
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / n)
        out.append((float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))))
    return out


def host_cores() -> int:
    """The host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def graph_launch_ms(fns, stream, passes=5, replays=4, reps=5):
    """Mean duration of one launch from `fns` (one launch each, e.g. one per
    weight copy), from HIP events on the launch stream around `replays`
    replays of a graph of `passes` rounds over them; median over `reps`."""
    import torch
    g = capture([[f] for _ in range(passes) for f in fns], stream)
    g.replay()
    torch.cuda.synchronize()
    n = passes * len(fns) * replays
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(replays):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / n)
    return float(np.median(ts))


PAD_STRIDES = (256, 4096)  # bytes added after each 16-row tile (row-stride padding)


def decode_ceilings(layers, pool, stream):
    """What this device sustains on the decode layers' weight bytes, from
    the ceiling kernels (libw4a16_ceilings), rotating through the same weight
    copies: a plain streaming read of each layer's packed weights, and the
    decode kernel's own weight loads alone in its grid (same workgroups,
    waves and 1 KiB blocks), also on copies whose 16-row tiles are padded
    (row-stride padding).  Times are per launch."""
    import torch
    import int4_weight_only_linear_amd as L
    from int4_weight_only_linear_amd import ceilings as C
    sink = torch.zeros(16, dtype=torch.int32, device=pool[0][0][0].device)
    rows = []
    for i, l in enumerate(layers):
        K, N = l["K"], l["N"]
        tiles = N // 16
        plan = L.w4a16_plan(1, N, K, GROUP, L.W4A16_BF16, True, L.PATH_GEMV)
        waves = plan["waves"]
        kpw = 1 << max(0, (-(-(K // 128) // waves) - 1).bit_length())  # a power of two covering the run
        wqs = [pool[c][i][0] for c in range(len(pool))]
        wbytes = wqs[0].numel() * 4
        t_stream = graph_launch_ms([lambda sp, w=w: C.stream_read(w, sink, sp) for w in wqs], stream)
        t_loads = graph_launch_ms([lambda sp, w=w: C.decode_loads(w, tiles, K, 8 * K, kpw, waves, sink, sp)
                                   for w in wqs], stream)
        row = dict(K=K, N=N, weight_bytes=wbytes, waves=waves, kpw=kpw,
                   stream_read_us=round(t_stream * 1e3, 3), stream_read_GBs=round(wbytes / t_stream / 1e6, 1),
                   loads_only_us=round(t_loads * 1e3, 3), loads_only_GBs=round(wbytes / t_loads / 1e6, 1))
        for pad in PAD_STRIDES:
            stride = 8 * K + pad
            padded = []
            for w in wqs:
                buf = torch.zeros(tiles * stride, dtype=torch.uint8, device=w.device)
                buf.view(tiles, stride)[:, :8 * K].copy_(w.view(torch.uint8).view(tiles, 8 * K))
                padded.append(buf)
            t_pad = graph_launch_ms([lambda sp, w=w: C.decode_loads(w, tiles, K, stride, kpw, waves, sink, sp)
                                     for w in padded], stream)
            row[f"loads_only_pad{pad}_us"] = round(t_pad * 1e3, 3)
            del padded
            torch.cuda.empty_cache()
        rows.append(row)
    return rows


def mfma_ceiling(stream, cu_count, iters=20000):
    """The sustained bf16 matrix-core rate: independent 32x32x16 MFMA chains
    on hashed operands, one and two waves per SIMD (libw4a16_ceilings)."""
    import torch
    from int4_weight_only_linear_amd import ceilings as C
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    out = {}
    for wps in (1, 2):
        blocks = cu_count * wps
        ms = graph_launch_ms([lambda sp, s=s: C.mfma_loop(blocks, iters, s, sink, sp) for s in range(2)],
                             stream, passes=2, replays=2, reps=3)
        out[f"waves_per_simd_{wps}"] = round(blocks * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12, 1)
    return dict(unit="TFLOP/s", kernel="v_mfma_f32_32x32x16_bf16 chains, hashed operands",
                **out, best=max(out.values()))


def cpu_baseline(layers_host, min_s=10.0):
    """The oracle (untuned) on this host's cores: whole M=1 decode steps over
    the layers, repeated until at least `min_s` seconds of oracle work.  Its
    BLAS runs on every core this process may use (numpy's own threading; the
    unpacking and dequantisation are numpy element-wise, one thread)."""
    import contextlib
    import oracle as O
    cores = host_cores()
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=cores)
    except ImportError:  # pragma: no cover
        ctx = contextlib.nullcontext()
    packed = [(K, N, c, O.pack_weights(c.q), O.pack_zeros(c.zp)) for (K, N, c) in layers_host]
    total_bytes, t_total, steps = 0, 0.0, 0
    with ctx:
        while t_total < min_s:
            for (K, N, c, wq, zpk) in packed:
                t0 = time.perf_counter()
                O.linear_ref(c.x_bits, wq, c.s_bits, zpk, None, c.M, N, K, GROUP, 1)
                t_total += time.perf_counter() - t0
                total_bytes += decode_bytes(c.M, N, K, GROUP)
            steps += 1
    layers = ", ".join(f"{K}x{N}" for (K, N, _c) in layers_host)
    return dict(value=total_bytes / t_total / 1e9, unit="GB/s", cores=cores, kind="oracle",
                seconds=round(t_total, 3),
                sample=(f"oracle linear_ref (unpack + exact fp32 dequant + fp64 GEMV) over {steps} M=1 "
                        f"decode step(s), layers {layers} (K x N), BLAS on {cores} threads; packing not "
                        f"timed"))


def _layer_tensors(case, device):
    """Pack a synth case with the library and upload it."""
    import torch
    import int4_weight_only_linear_amd as L
    act = torch.float16 if case.dtype == 0 else torch.bfloat16
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(act)
    wq = torch.from_numpy(L.w4a16_pack_weights(case.q)).to(device)
    zp = None if case.zp is None else torch.from_numpy(L.w4a16_pack_zeros(case.zp)).to(device)
    bias = None if case.bias_bits is None else up(case.bias_bits)
    return wq, zp, up(case.s_bits), up(case.x_bits), bias


def time_point(x, pool, bias, y, M, N, K, g, dt, path, reps, stream):
    """Mean per-launch time (ms) of w4a16_linear_path over a graph of one
    launch per weight copy in `pool`, replayed `reps` times."""
    import torch
    import int4_weight_only_linear_amd as L
    from int4_weight_only_linear_amd import _binding as B
    need = L.w4a16_workspace_size(M, N, K, g, dt, pool[0][1] is not None, path)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=x.device) if need else None
    wsp, wsn = (None, 0) if ws is None else (ws.data_ptr(), ws.numel())

    def launch(wq, zp, s):
        def fn(sp):
            B._check(B.lib.w4a16_linear_path(
                x.data_ptr(), wq.data_ptr(), s.data_ptr(), None if zp is None else zp.data_ptr(),
                None if bias is None else bias.data_ptr(), y.data_ptr(), M, N, K, g, dt,
                wsp, wsn, sp, path))
        return fn
    fns = [[launch(*w)] for w in pool]
    fns[0][0](torch.cuda.current_stream().cuda_stream)  # first call outside capture
    torch.cuda.synchronize()
    graph = capture(fns, stream)
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(pool))


def dense_comparator(players, stream, steps):
    """The dequantised prefill copy on the same layers: w4a16_dequant once,
    then w4a16_linear_dense per call (dense product on the matrix cores).
    Times the dense call alone, like the W4A16 GEMM, plus the one-off
    dequantisation, and states the memory the copy costs."""
    import torch
    import int4_weight_only_linear_amd as L
    from int4_weight_only_linear_amd import _binding as B
    rows = []
    for l in players:
        K, N, M = l["K"], l["N"], l["M"]
        w = L.w4a16_dequant(l["wq"], l["s"], l["zp"], group_size=GROUP)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.w4a16_dequant(l["wq"], l["s"], l["zp"], group_size=GROUP, out=w)
        e1.record()
        torch.cuda.synchronize()
        deq_us = e0.elapsed_time(e1) * 1e3
        need = L.w4a16_dense_workspace_size(M, N, K, L.W4A16_BF16, False)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=w.device)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=w.device)

        def fn(sp, x=l["x"], w=w, y=y, ws=ws, M=M, N=N, K=K):
            B._check(B.lib.w4a16_linear_dense(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), M, N, K,
                                              L.W4A16_BF16, ws.data_ptr(), ws.numel(), sp))
        fn(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ms = time_steps([[fn]] * 4, max(8, steps), 4, stream)
        rows.append(dict(K=K, N=N, us=round(ms * 1e3, 2),
                         tflops=round(2 * M * N * K / (ms * 1e-3) / 1e12, 1),
                         dequant_once_us=round(deq_us, 1), copy_bytes=N * K * 2))
        del w, ws, y
    return dict(what="w4a16_dequant once (kept resident, 4x the packed bytes), then "
                     "w4a16_linear_dense (the prefill GEMM's dense instances: bf16 MFMA, fp32 "
                     "accumulation, weight fragments loaded instead of dequantised) per call",
                per_layer=rows)


def vendor_dense(x, w, steps, stream, copies_bytes=1 << 30):
    """torch's bf16 matmul (the vendor BLAS on this image) of x [M, K] with a
    dequantised copy w [N, K] (transposed once to [K, N]), per call, graphs
    rotating >= copies_bytes of copies: the dense comparator of the prefill
    GEMM.  Returns microseconds per call."""
    import torch
    wt = w.t().contiguous()
    pool = [wt] + [wt.clone() for _ in range(max(1, math.ceil(copies_bytes / (wt.numel() * 2))) - 1)]
    y = torch.empty((x.shape[0], w.shape[0]), dtype=x.dtype, device=x.device)
    with torch.cuda.stream(stream):
        for ww in pool[:2]:  # its first calls set up the library (not allowed under graph capture)
            torch.matmul(x, ww, out=y)
    torch.cuda.synchronize()
    ms = graph_launch_ms([lambda sp, ww=ww: torch.matmul(x, ww, out=y) for ww in pool], stream,
                         passes=3, replays=2, reps=max(3, steps // 10))
    del pool, wt, y
    torch.cuda.empty_cache()
    return ms * 1e3


def run_vendor(path_prefix):
    """The W4A16 prefill GEMM against torch's bf16 matmul (the vendor BLAS)
    on the dequantised copy of the same weights, on the Llama prefill layers
    at M = 128, 256 and 1920; both timed per call over graphs rotating
    >= 1 GiB of weight copies.  Writes <prefix>.md and .json."""
    import torch
    import int4_weight_only_linear_amd as L
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream()
    rows = []
    for (K, N) in PREFILL_LAYERS:
        l = build_layer(K, N, 1920, ("vendor", K, N), dev)
        wbytes = l["wq"].numel() * 4 + l["s"].numel() * 2 + l["zp"].numel() * 4
        pool = [(l["wq"], l["zp"], l["s"])] + [(l["wq"].clone(), l["zp"].clone(), l["s"].clone())
                                               for _ in range(max(2, math.ceil((1 << 30) / wbytes)) - 1)]
        w = L.w4a16_dequant(l["wq"], l["s"], l["zp"], group_size=GROUP)
        for M in (128, 256, 1920):
            x = l["x"][:M].contiguous()
            y = torch.empty((M, N), dtype=x.dtype, device=dev)
            t_w4 = time_point(x, pool, None, y, M, N, K, GROUP, L.W4A16_BF16, L.PATH_GEMM, 20, side) * 1e3
            t_v = vendor_dense(x, w, 30, side)
            tf = lambda t: 2 * M * N * K / (t * 1e-6) / 1e12
            p = L.w4a16_plan(M, N, K, GROUP, L.W4A16_BF16, True, L.PATH_GEMM)
            rows.append(dict(K=K, N=N, M=M, w4a16_us=round(t_w4, 1), w4a16_tflops=round(tf(t_w4), 1),
                             vendor_us=round(t_v, 1), vendor_tflops=round(tf(t_v), 1),
                             speedup=round(t_v / t_w4, 2),
                             plan=f"{p['tile_tokens']}x{p['tile_features']}, {p['splits']} K range(s)"
                                  + (", two-pass" if p["two_pass"] else "") + (", tail launch" if p["tail_tiles"] else "")))
            print(f"[vendor] {K}x{N} M={M}: {rows[-1]}", file=sys.stderr, flush=True)
        del pool, w, l
        torch.cuda.empty_cache()
    with open(path_prefix + ".json", "w") as f:
        json.dump(dict(rows=rows, torch=torch.__version__), f)
    with open(path_prefix + ".md", "w") as f:
        f.write("# W4A16 prefill GEMM against the vendor BLAS on a dequantised copy (Llama-3.1-8B-shaped layers, bf16)\n\n")
        f.write(f"Command: python bench.py --vendor {os.path.basename(path_prefix)}\n\n")
        f.write("Both per call, from HIP events around graphs rotating >= 1 GiB of weight copies: the W4A16 GEMM on the\n"
                "packed weights (asym uint4, g128), and torch.matmul (torch " + torch.__version__ + ", bf16, the image's\n"
                "vendor BLAS) on the same weights dequantised once to bf16 and transposed to [K, N] (4x the packed bytes).\n\n")
        f.write("| K | N | M | W4A16 plan | W4A16 us | TFLOP/s | vendor dense us | TFLOP/s | W4A16 speedup |\n")
        f.write("|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {r['K']} | {r['N']} | {r['M']} | {r['plan']} | {r['w4a16_us']} | {r['w4a16_tflops']} | "
                    f"{r['vendor_us']} | {r['vendor_tflops']} | {r['speedup']} |\n")
    print(json.dumps(dict(vendor=path_prefix + ".md", points=len(rows))), flush=True)


MOE_LAYERS = (("gate_up", 1536, 2048, False), ("down", 2048, 768, True))  # (name, N, K, x per slot)
MOE_EXPERTS, MOE_TOPK = 128, 8


def moe_measure(stream, reps=20):
    """Expert-indexed decode on Qwen3-30B-A3B-shaped experts (128 experts,
    top-8, hidden 2048, expert intermediate 768; gate and up fused), bf16,
    asymmetric uint4, group 128, synthetic routing (distinct random experts
    per token, random router weights).  GB/s counts each distinct expert's
    weights, scales and zero points once per launch, plus x and y.  Timed over
    a graph of launches rotating through >= 1 GiB of stack copies."""
    import torch
    import int4_weight_only_linear_amd as L
    from int4_weight_only_linear_amd import _binding as B
    from synth import make_case, stream_seed
    dev = torch.device("cuda:0")
    E, topk, g = MOE_EXPERTS, MOE_TOPK, GROUP
    rows = []
    for name, N, K, xps in MOE_LAYERS:
        G = K // g
        c = make_case(1, N, K, g, 1, False, False, seed=("bench-moe", name))
        wq1 = torch.from_numpy(L.w4a16_pack_weights(c.q)).to(dev)
        zp1 = torch.from_numpy(L.w4a16_pack_zeros(c.zp)).to(dev)
        s1 = torch.from_numpy(c.s_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        # E experts: the one packed expert perturbed per expert (distinct bytes)
        wq = wq1.unsqueeze(0).repeat(E, 1, 1) ^ torch.arange(E, device=dev, dtype=torch.int32).view(E, 1, 1)
        zp = zp1.unsqueeze(0).repeat(E, 1, 1)
        s = s1.unsqueeze(0).repeat(E, 1, 1).contiguous()
        per_expert = N * K // 2 + N * G * 2 + (N // 8) * G * 4
        copies = max(2, min(16, -(-(1 << 30) // (E * per_expert))))
        stacks = [(wq, zp, s)] + [(wq.clone(), zp.clone(), s.clone()) for _ in range(copies - 1)]
        for M in (1, 4):
            rng = np.random.default_rng(stream_seed("bench-moe-ids", name, M))
            ids_h = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
            ids = torch.from_numpy(ids_h).to(dev)
            w = torch.from_numpy(rng.random((M, topk)).astype(np.float32)).to(dev)
            xr = M * topk if xps else M
            x = torch.from_numpy(make_case(xr, N, K, g, 1, False, False, seed=("bench-moe-x", name, M))
                                 .x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty((M * topk, N), dtype=torch.bfloat16, device=dev)

            def launch(st):
                def fn(sp, st=st):
                    B._check(B.lib.w4a16_moe_linear(x.data_ptr(), st[0].data_ptr(), st[2].data_ptr(),
                                                    st[1].data_ptr(), None, ids.data_ptr(), w.data_ptr(),
                                                    y.data_ptr(), M, topk, E, N, K, g, L.W4A16_BF16,
                                                    int(xps), sp))
                return fn
            fns = [[launch(st)] for st in stacks]
            fns[0][0](torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            ms = time_steps(fns * 4, reps * len(fns), len(fns), stream)
            nbytes = len(set(ids_h.ravel().tolist())) * per_expert + xr * K * 2 + M * topk * N * 2
            gbs = nbytes / (ms * 1e-3) / 1e9
            rows.append(dict(layer=name, N=N, K=K, M=M, us=round(ms * 1e3, 2), GBs=round(gbs, 1),
                             frac=round(gbs / HBM_PEAK_GBS, 4)))
        del stacks, wq, zp, s
        torch.cuda.empty_cache()
    return dict(workload=f"Qwen3-30B-A3B-shaped expert layers: {E} experts, top-{topk}, "
                         "gate_up 2048 -> 1536 (x per token), down 768 -> 2048 (x per slot); "
                         "asym uint4 g128 bf16; synthetic routing",
                per_layer=rows)


def run_report(path_prefix):
    """Every point of the decode, prefill and dispatch-sweep workloads on both
    paths: per-launch time, GB/s and % of HBM peak, TFLOP/s and % of the
    dense MFMA peak, roofline fraction, and the dispatch crossover M* per
    (shape, group, quantisation, dtype).  Beside each point, the CPU oracle
    on this host's cores: unpack + exact dequantisation (once per weight) and
    its fp64 product at that M, with the GPU's speedup over the two.  Writes
    <prefix>.md and <prefix>.json."""
    import contextlib
    import torch
    import int4_weight_only_linear_amd as L
    import oracle as O
    from synth import make_case
    from synth.configs import CONFIGS
    cores = host_cores()
    try:
        from threadpoolctl import threadpool_limits
        pool_ctx = threadpool_limits(limits=cores)
    except ImportError:  # pragma: no cover
        pool_ctx = contextlib.nullcontext()
    pool_ctx.__enter__()
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream()
    rows = []
    t_start = time.time()
    for name in ("llama8b_decode", "qwen3_4b_decode", "llama8b_prefill", "sweep"):
        cfg = CONFIGS[name]
        mmax = max(cfg.Ms)
        for layer in cfg.layers:
            K, N = layer.K, layer.N
            for g in cfg.groups:
                for sym in cfg.symmetric:
                    for dt in cfg.dtypes:
                        for bias in cfg.bias:
                            c = make_case(mmax, N, K, g, dt, sym, bias, seed=("report", name, K, N, g, sym, dt))
                            wq, zp, s, x_all, b = _layer_tensors(c, dev)
                            wbytes = wq.numel() * 4 + s.numel() * 2 + (0 if zp is None else zp.numel() * 4)
                            copies = max(2, min(64, math.ceil((1 << 30) / wbytes)))
                            pool = [(wq, zp, s)] + [(wq.clone(), None if zp is None else zp.clone(), s.clone())
                                                    for _ in range(copies - 1)]
                            # decode layers: a plain streaming read of the same packed weight
                            # copies, the rate a kernel that only reads them reaches
                            t_read = None
                            if name.endswith("_decode"):
                                from int4_weight_only_linear_amd import ceilings as C
                                sink = torch.zeros(16, dtype=torch.int32, device=dev)
                                t_read = graph_launch_ms([lambda sp, w=w: C.stream_read(w, sink, sp)
                                                          for (w, _, _) in pool], side)
                            for M in cfg.Ms:
                                x = x_all[:M].contiguous()
                                y = torch.empty((M, N), dtype=x.dtype, device=dev)
                                for path in (L.PATH_GEMV, L.PATH_GEMM):
                                    if path == L.PATH_GEMV and M > L.GEMV_MAX_M:
                                        continue
                                    reps = 20 if M >= 128 else 50
                                    ms = time_point(x, pool, b, y, M, N, K, g, dt, path, reps, side)
                                    nbytes = decode_bytes(M, N, K, g, asym=not sym, bias=bias)
                                    flops = 2 * M * N * K
                                    gbs = nbytes / (ms * 1e-3) / 1e9
                                    tfl = flops / (ms * 1e-3) / 1e12
                                    frac = max(gbs / HBM_PEAK_GBS, tfl / MFMA_BF16_PEAK_TFLOPS)
                                    rows.append(dict(config=name, K=K, N=N, M=M, group=g,
                                                     quant="uint4b8" if sym else "uint4+zp",
                                                     dtype="fp16" if dt == 0 else "bf16", bias=bias,
                                                     path="gemv" if path == L.PATH_GEMV else "gemm",
                                                     auto=int(L.w4a16_select_path(M, N, K, g, dt, not sym)) == path,
                                                     us=round(ms * 1e3, 3), GBs=round(gbs, 1),
                                                     hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                                                     TFLOPs=round(tfl, 1),
                                                     mfma_frac=round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                                                     roofline_frac=round(frac, 4)))
                                    if t_read is not None:
                                        rows[-1]["read_us"] = round(t_read * 1e3, 3)
                                        rows[-1]["of_read"] = round(t_read / ms, 3)
                            # the oracle on the same case: unpack + exact dequant once,
                            # then its fp64 product for each M
                            wq_o = O.pack_weights(c.q)
                            zp_o = None if sym else O.pack_zeros(c.zp)
                            t0 = time.perf_counter()
                            w64 = O.dequant_f32(wq_o, c.s_bits, zp_o, N, K, g, dt).astype(np.float64)
                            t_deq = time.perf_counter() - t0
                            b64 = None if c.bias_bits is None else O.act_bits_to_f64(c.bias_bits, dt)
                            t_gemm = {}
                            for M in cfg.Ms:
                                x64 = O.act_bits_to_f64(c.x_bits[:M], dt)
                                t0 = time.perf_counter()
                                y64 = x64 @ w64.T
                                if b64 is not None:
                                    y64 = y64 + b64[None, :]
                                t_gemm[M] = time.perf_counter() - t0
                            del w64
                            for r in rows:
                                if (r["config"], r["K"], r["N"], r["group"], r["quant"], r["dtype"], r["bias"]) == \
                                        (name, K, N, g, "uint4b8" if sym else "uint4+zp", "fp16" if dt == 0 else "bf16",
                                         bias) and "oracle_ms" not in r:
                                    r["oracle_dequant_ms"] = round(t_deq * 1e3, 1)
                                    r["oracle_gemm_ms"] = round(t_gemm[r["M"]] * 1e3, 2)
                                    r["oracle_ms"] = round((t_deq + t_gemm[r["M"]]) * 1e3, 1)
                                    r["speedup_vs_oracle"] = round(r["oracle_ms"] / (r["us"] * 1e-3))
                            print(f"[report] {name} K={K} N={N} g={g} {'sym' if sym else 'asym'} "
                                  f"{'fp16' if dt == 0 else 'bf16'} bias={bias}: {len(cfg.Ms)} M values "
                                  f"({time.time() - t_start:.0f}s)", file=sys.stderr, flush=True)
                            del pool, wq, zp, s, x_all, b
                            torch.cuda.empty_cache()
    # dispatch crossover: the largest M at which the decode kernel is faster
    cross = {}
    for r in rows:
        if r["config"] != "sweep":
            continue
        key = (r["K"], r["N"], r["group"], r["quant"], r["dtype"])
        cross.setdefault(key, {}).setdefault(r["M"], {})[r["path"]] = r["us"]
    mstar = []
    for key, byM in sorted(cross.items()):
        best = 0
        for M in sorted(byM):
            t = byM[M]
            if "gemv" in t and t["gemv"] <= t["gemm"]:
                best = M
        mstar.append(dict(K=key[0], N=key[1], group=key[2], quant=key[3], dtype=key[4], Mstar=best))
    with open(path_prefix + ".json", "w") as f:
        json.dump(dict(rows=rows, mstar=mstar), f)
    with open(path_prefix + ".md", "w") as f:
        f.write("# W4A16 linear on MI355X: every decode, prefill and crossover-sweep point on both kernels\n\n")
        f.write(f"Command: python bench.py --report {os.path.basename(path_prefix)}\n\n")
        f.write("Each point: mean time per launch over a HIP graph of back-to-back launches that rotate\n"
                "through >= 1 GiB of weight copies (weights stream from HBM).  GB/s = algorithmic bytes\n"
                "(weights, scales, zp, x, y, bias) / time; TFLOP/s = 2*M*N*K / time; peaks 8 TB/s and\n"
                "2.5 PFLOP/s.  auto (*) marks the kernel W4A16_PATH_AUTO picks.  Oracle: the CPU oracle\n"
                f"on this host ({cores} cores, BLAS on all of them): unpack + exact dequantisation of the\n"
                "layer (deq, once per weight) + its fp64 product at this M (gemm); x = GPU speedup over\n"
                "deq + gemm.  read us: a plain streaming read of the same packed weight copies (decode\n"
                "layers; the rate a kernel that only reads them reaches); of read = read us / us.\n\n")
        f.write("| config | K | N | M | g | quant | dtype | bias | path | auto | us | GB/s | %HBM | TFLOP/s | "
                "%MFMA | read us | of read | oracle deq ms | oracle gemm ms | x |\n")
        f.write("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {r['config']} | {r['K']} | {r['N']} | {r['M']} | {r['group']} | {r['quant']} | "
                    f"{r['dtype']} | {'y' if r['bias'] else 'n'} | {r['path']} | {'*' if r['auto'] else ''} | "
                    f"{r['us']} | {r['GBs']} | {100 * r['hbm_frac']:.1f} | {r['TFLOPs']} | "
                    f"{100 * r['mfma_frac']:.1f} | {r.get('read_us', '')} | {r.get('of_read', '')} | "
                    f"{r.get('oracle_dequant_ms', '')} | "
                    f"{r.get('oracle_gemm_ms', '')} | {r.get('speedup_vs_oracle', '')} |\n")
        f.write("\n| K | N | g | quant | dtype | M* (largest M where the decode kernel is faster) |\n")
        f.write("|---|---|---|---|---|---|\n")
        for m in mstar:
            f.write(f"| {m['K']} | {m['N']} | {m['group']} | {m['quant']} | {m['dtype']} | {m['Mstar']} |\n")
    print(json.dumps(dict(report=path_prefix + ".md", points=len(rows), mstar=mstar)), flush=True)


# ---- rocprofv3 summaries (profiles/) ------------------------------------------

# $R: the repository; $OUT: any directory for the profiler's CSV output
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/{kind}_trace -o run -- "
             "python3 $R/bench.py --profile {kind} --steps {steps}",
    "bench-trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/bench_trace -o run -- "
                   "python3 $R/bench.py",
    "pmc": "rocprofv3 --pmc {counters} --output-format csv -d $OUT/{kind}_pmc{tag} -o run -- "
           "python3 $R/bench.py --profile {kind} --steps {steps}",
    "traffic": "rocprofv3 --pmc {counter} --output-format csv -d $OUT/{kind}_{counter} -o run -- "
               "python3 $R/bench.py --profile {kind} --steps {steps} --calibration-copy-mb 256",
}


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def profile_layers(kind):
    """(K, N, M, expected Grid_Size_X of the layer's main kernel, work) per
    layer of a --profile run; work = algorithmic bytes (decode) or flops.
    Prefill layers also carry their GEMM tile (mb, cb) and, for a plan with
    a tail launch, the tail kernel's grid and tile."""
    import int4_weight_only_linear_amd as L
    shapes, M = (DECODE_LAYERS, 1) if kind == "decode" else (PREFILL_LAYERS, 1920)
    out = []
    for (K, N) in shapes:
        p = L.w4a16_plan(M, N, K, GROUP, L.W4A16_BF16, True)
        threads = 64 * p["waves"]
        units = p["tiles"] * (p["splits"] if kind == "prefill" else 1)
        work = decode_bytes(M, N, K, GROUP) if kind == "decode" else 2 * M * N * K
        l = dict(K=K, N=N, M=M, grid=units * threads, plan=p, work=work, tile=None, tail_grid=0, tail_tile=None)
        if kind == "prefill":
            l["tile"] = (p["tile_tokens"] // 32, p["tile_features"] // 128)
            if p["tail_tiles"]:
                # the first launch covers the tiles before the tail's (two tail tiles per tile)
                l["grid"] = (p["tiles"] - p["tail_tiles"] // 2) * threads
                l["tail_grid"] = p["tail_tiles"] * threads
                l["tail_tile"] = (p["tail_tile_tokens"] // 32, p["tail_tile_features"] // 128)
        out.append(l)
    return out


def _gemm_tile(name):
    """(mb, cb) of a demangled gemm_kernel name, else None."""
    import re
    m = re.search(r"gemm_kernel<\d+, \d+, \w+, (\d+), (\d+), \w+>", name)
    return (int(m.group(1)), int(m.group(2))) if m else None


def _layer_calls(l, disp):
    """The calls of layer l among dispatch records (dicts with grid, tile,
    start, end): one record per dispatch of its kernel, or, for a plan with a
    tail launch, its first launch together with the next tail launch."""
    def match(d, grid, tile):
        return d["grid"] == grid and (tile is None or d["tile"] == tile)
    main = sorted((d for d in disp if match(d, l["grid"], l["tile"])), key=lambda d: d["start"])
    if not l["tail_grid"]:
        return [[d] for d in main]
    tails = sorted((d for d in disp if match(d, l["tail_grid"], l["tail_tile"])), key=lambda d: d["start"])
    calls = []
    for d in main:
        t = next((t for t in tails if t["start"] >= d["end"]), None)
        if t is not None:
            tails.remove(t)
            calls.append([d, t])
    return calls


def _kernel_short(name):
    """'gemm_kernel<1, 128, true, 8, 2, false>' out of a demangled kernel name."""
    import re
    m = re.search(r"(\w+_kernel<[^>]*>)", name)
    return m.group(1) if m else name.split("(")[0]


def _median(v):
    return float(np.median(np.asarray(v, dtype=np.float64))) if len(v) else float("nan")


def summarize_trace(kind, d, steps, of_bench=False):
    """Per layer of a --profile run (or, of_bench, of the bench line's own
    run: its decode graphs rotating the weight copies): launches, mean and
    median kernel time (End - Start), and GB/s (decode) or TFLOP/s
    (prefill) against the peak."""
    rows = [r for r in _csv_rows(os.path.join(d, "run_kernel_trace.csv")) if "w4a16" in r["Kernel_Name"]]
    if of_bench:
        # the decode layers' kernels only: the prefill GEMM runs some of the
        # same grid sizes, the expert-indexed decode instance (last template
        # argument 1) its own
        rows = [r for r in rows if _kernel_short(r["Kernel_Name"]).startswith("gemv_")
                and not _kernel_short(r["Kernel_Name"]).endswith(", 1>")]
    layers = profile_layers(kind)
    unit = "GB/s" if kind == "decode" else "TFLOP/s"
    peak = HBM_PEAK_GBS if kind == "decode" else MFMA_BF16_PEAK_TFLOPS
    cmd = PROFILE_CMDS["bench-trace"] if of_bench else PROFILE_CMDS["trace"].format(kind=kind, steps=steps)
    what = ("every dispatch of the layer's kernel in the bench run: warmup, timed graphs and the per-launch "
            "timing graphs" if of_bench else
            "the first launch of each layer, outside the timed loop, included")
    lines = [f"Command (from /tmp, TMPDIR=/tmp, repository at $R, CSV output under $OUT):",
             "  " + cmd, "",
             f"Per layer (End - Start of each dispatch of the layer's kernel; a call with a tail launch: its two "
             f"kernels' End - Start added; {what}):",
             f"  layer (K,N)      M     kernel grid   launches  mean_ns    median_ns   {unit}(mean)  frac of {peak:g}"]
    disp = [dict(grid=int(r["Grid_Size_X"]), tile=_gemm_tile(_kernel_short(r["Kernel_Name"])),
                 start=int(r["Start_Timestamp"]), end=int(r["End_Timestamp"]), name=_kernel_short(r["Kernel_Name"]))
            for r in rows if "splitk_reduce" not in r["Kernel_Name"]]
    means = []
    for l in layers:
        calls = _layer_calls(l, disp)
        # a call with a tail launch: its two kernels' durations added
        ts = [sum(d["end"] - d["start"] for d in c) for c in calls]
        names = {d["name"] for c in calls for d in c}
        mean = float(np.mean(ts)) if ts else float("nan")
        rate = l["work"] / mean if kind == "decode" else l["work"] / mean / 1e3
        means.append(mean)
        lines.append(f"  ({l['K']:5d},{l['N']:5d})  {l['M']:5d}  {l['grid']:10d}   {len(ts):8d}  {mean:9.0f}  "
                     f"{_median(ts):9.0f}   {rate:10.1f}  {rate / peak:.4f}   {' / '.join(sorted(names))}")
        if l["tail_grid"] and calls:
            first = [c[0]["end"] - c[0]["start"] for c in calls]
            tail = [c[1]["end"] - c[1]["start"] for c in calls]
            lines.append(f"      of which the first launch (grid {l['grid']}) mean {np.mean(first):.0f} ns, the tail "
                         f"launch (grid {l['tail_grid']}) mean {np.mean(tail):.0f} ns; the layer's first call "
                         f"{first[0]} + {tail[0]} ns")
    if kind == "decode":
        mb = float(np.mean([l["work"] for l in layers]))
        mm = float(np.mean(means))
        lines.append(f"  mean over the layers: {mm:.0f} ns per launch, {mb:.0f} bytes per launch -> "
                     f"{mb / mm:.1f} GB/s = {mb / mm / HBM_PEAK_GBS:.4f} of {HBM_PEAK_GBS:g}")
    return "\n".join(lines)


PMC_SETS = {
    "A": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
          "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT"],
    "B": ["SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
          "SQ_WAVES", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"],
    "C": ["TCC_HIT_sum", "TCC_MISS_sum", "MeanOccupancyPerActiveCU", "OccupancyPercent"],  # (the first two and the last are reported)
}
XCDS, SIMDS = 8, 1024


def summarize_pmc(kind, dirs, steps):
    """Per layer, medians over its dispatches: kernel time, the clock
    (GRBM_GUI_ACTIVE per XCD over the kernel time), MFMA utilisation
    (SQ_VALU_MFMA_BUSY_CYCLES over GUI-active cycles of all 1024 SIMDs), the
    bf16 matrix flops the MFMA counters saw, and instructions per MFMA."""
    layers = profile_layers(kind)
    per = {}
    for tag, d in dirs.items():
        for r in _csv_rows(os.path.join(d, "run_counter_collection.csv")):
            if "w4a16" not in r["Kernel_Name"]:
                continue
            e = per.setdefault((tag, r["Dispatch_Id"]), dict(
                grid=int(r["Grid_Size"]), tile=_gemm_tile(_kernel_short(r["Kernel_Name"])),
                start=int(r["Start_Timestamp"]), end=int(r["End_Timestamp"]),
                ns=int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])

    def calls_of(tag, l):
        # a call with a tail launch: both kernels' times and counters added
        out = []
        for c in _layer_calls(l, [e for (t, _), e in per.items() if t == tag]):
            m = dict(c[0])
            for e in c[1:]:
                for k, v in e.items():
                    if k not in ("grid", "tile", "start", "end"):
                        m[k] = m.get(k, 0.0) + v
            out.append(m)
        return out
    lines = ["Commands (from /tmp, TMPDIR=/tmp, repository at $R, CSV output under $OUT), one counter set per run:"]
    for tag in dirs:
        lines.append("  " + PROFILE_CMDS["pmc"].format(kind=kind, steps=steps, tag=tag,
                                                         counters=" ".join(PMC_SETS[tag])))
    lines += ["", "Per layer (median over the layer's dispatches; counters summed over the device):"]
    for l in layers:
        a, b, c = calls_of("A", l), calls_of("B", l), calls_of("C", l)
        tail = (f", the last {l['plan']['tail_tiles'] // 2} as {l['plan']['tail_tiles']} "
                f"{l['plan']['tail_tile_tokens']}x{l['plan']['tail_tile_features']} tiles in a tail launch "
                f"(counters and times of the two kernels added)" if l["tail_grid"] else "")
        lines.append(f"  layer (K,N) = ({l['K']},{l['N']}), M = {l['M']}, plan {l['plan']['tile_tokens']}x"
                     f"{l['plan']['tile_features']} tiles{tail}, {l['plan']['splits']} K range(s), {len(a)} calls")
        if a:
            ns = _median([e["ns"] for e in a])
            clk = _median([e["GRBM_GUI_ACTIVE"] / XCDS / e["ns"] for e in a])
            util = _median([e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) for e in a])
            tf = _median([e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / e["ns"] / 1e3 for e in a])
            valu = _median([e["SQ_INSTS_VALU"] / e["SQ_INSTS_MFMA"] for e in a])
            lds = _median([e["SQ_INSTS_LDS"] / e["SQ_INSTS_MFMA"] for e in a])
            conf = _median([e["SQ_LDS_BANK_CONFLICT"] for e in a])
            busy = _median([e["SQ_VALU_MFMA_BUSY_CYCLES"] / e["SQ_INSTS_MFMA"] for e in a])
            lines.append(f"    kernel {ns / 1e3:.1f} us, clock {clk:.2f} GHz, MFMA busy {util:.3f} of GUI-active "
                         f"SIMD cycles ({busy:.0f} busy cycles per MFMA), {tf:.0f} TFLOP/s from "
                         f"SQ_INSTS_VALU_MFMA_MOPS_BF16*512 ({tf / MFMA_BF16_PEAK_TFLOPS:.3f} of "
                         f"{MFMA_BF16_PEAK_TFLOPS:g}; algorithmic {l['work'] / ns / 1e3:.0f}), "
                         f"VALU instructions per MFMA {valu:.2f} (MFMAs included), LDS instructions per MFMA "
                         f"{lds:.2f}, LDS bank conflicts {conf:.0f}")
        if b:
            co = _median([e["SQ_VALU_MFMA_COEXEC_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) for e in b])
            extra = ""
            if "SQ_WAIT_ANY" in b[0]:
                wc = [e["SQ_WAVE_CYCLES"] for e in b]
                extra = (f"; of the waves' cycles: waiting on a dependency or counter "
                         f"{_median([e['SQ_WAIT_ANY'] / e['SQ_WAVE_CYCLES'] for e in b]):.3f}, waiting to issue "
                         f"{_median([e['SQ_WAIT_INST_ANY'] / e['SQ_WAVE_CYCLES'] for e in b]):.3f}, issuing "
                         f"{_median([e['SQ_ACTIVE_INST_ANY'] / e['SQ_WAVE_CYCLES'] for e in b]):.3f}")
            lines.append(f"    VALU/MFMA co-execution {co:.3f} of GUI-active SIMD cycles; waves "
                         f"{_median([e['SQ_WAVES'] for e in b]):.0f}{extra}")
        if c:
            hit = _median([e["TCC_HIT_sum"] / max(1.0, e["TCC_HIT_sum"] + e["TCC_MISS_sum"]) for e in c])
            pct = _median([e["OccupancyPercent"] for e in c])
            lines.append(f"    L2 hit rate {hit:.3f} (TCC_HIT_sum / (HIT + MISS)); occupancy {pct:.1f} % of the "
                         f"maximum (OccupancyPercent: waves resident over the 32 wave slots of each CU, averaged "
                         f"over the kernel)")
    return "\n".join(lines)


def summarize_traffic(kind, fetch_dir, write_dir, steps, copy_mb=256):
    """HBM bytes per launch of each layer's kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), scaled by what the same counters read for
    the calibration copy (reads and writes copy_mb MiB once)."""
    layers = profile_layers(kind)
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _csv_rows(os.path.join(d, "run_counter_collection.csv"))
        cal = [float(r["Counter_Value"]) for r in rows
               if "bitwise_not" in r["Kernel_Name"] or "BitwiseNot" in r["Kernel_Name"]]
        scale = (copy_mb * 1024) / _median(cal)
        out[counter] = dict(scale=scale, cal=_median(cal), rows=rows)
    lines = ["Commands (from /tmp, TMPDIR=/tmp, repository at $R, CSV output under $OUT), one counter per run:"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append("  " + PROFILE_CMDS["traffic"].format(kind=kind, steps=steps, counter=counter))
    lines += ["", f"Calibration (torch bitwise_not: one elementwise kernel reading and writing {copy_mb} MiB):"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"  {counter} per dispatch: {out[counter]['cal']:.1f} KiB for {copy_mb * 1024} KiB -> "
                     f"scale {out[counter]['scale']:.4f}")
    lines += ["", "Per layer (median KiB per dispatch as counted; bytes after scaling):",
              "  layer (K,N)      FETCH_KiB   WRITE_KiB   traffic_bytes   algorithmic_bytes   ratio"]
    tot_t = tot_a = 0.0
    for l in layers:
        kib = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            v = [float(r["Counter_Value"]) for r in out[counter]["rows"]
                 if "w4a16" in r["Kernel_Name"] and int(r["Grid_Size"]) == l["grid"]]
            kib[counter] = _median(v)
        t = (kib["FETCH_SIZE"] * out["FETCH_SIZE"]["scale"] + kib["WRITE_SIZE"] * out["WRITE_SIZE"]["scale"]) * 1024
        alg = decode_bytes(l["M"], l["N"], l["K"], GROUP)
        tot_t += t
        tot_a += alg
        lines.append(f"  ({l['K']:5d},{l['N']:5d})  {kib['FETCH_SIZE']:10.1f}  {kib['WRITE_SIZE']:10.1f}  "
                     f"{t:14.0f}  {alg:18d}  {t / alg:.4f}")
    n = len(layers)
    lines.append(f"  mean traffic per launch: {tot_t / n:.0f} bytes; algorithmic {tot_a / n:.0f}; "
                 f"ratio {tot_t / tot_a:.4f}")
    return "\n".join(lines), int(round(tot_t / n))


# ---- performance regression check with a control --------------------------------

QWEN_DECODE_LAYERS = ((2560, 6144), (4096, 2560), (2560, 19456), (9728, 2560))  # (K, N), fp16 sym


def perf_points(dev, stream):
    """Per-launch times (us) of the decode layers at M=1 (Llama bf16 asym, Qwen
    fp16 sym; graphs rotating >= 1 GiB of weight copies) and the prefill layers
    at M=1920, plus two controls timed in the same run: a streaming read of
    1 GiB (GB/s) and the sustained MFMA loop (TFLOP/s)."""
    import torch
    import int4_weight_only_linear_amd as L
    from int4_weight_only_linear_amd import ceilings as C
    from synth import make_case
    sink = torch.zeros(16, dtype=torch.int32, device=dev)
    bufs = [torch.empty(1 << 28, dtype=torch.uint8, device=dev) for _ in range(4)]
    t = graph_launch_ms([lambda sp, b=b: C.stream_read(b, sink, sp) for b in bufs], stream, passes=2)
    control = dict(stream_read_GBs=round((1 << 28) / (t * 1e-3) / 1e9, 1),
                   mfma_TFLOPs=mfma_ceiling(stream, torch.cuda.get_device_properties(dev).multi_processor_count)["best"])
    del bufs
    points = {}
    for fam, shapes, dt, sym in (("llama8b_decode", DECODE_LAYERS, 1, False),
                                 ("qwen3_4b_decode", QWEN_DECODE_LAYERS, 0, True)):
        for (K, N) in shapes:
            c = make_case(1, N, K, GROUP, dt, sym, False, seed=("perf", fam, K, N))
            wq, zp, s, x, b = _layer_tensors(c, dev)
            wbytes = wq.numel() * 4 + s.numel() * 2 + (0 if zp is None else zp.numel() * 4)
            copies = max(2, min(64, math.ceil((1 << 30) / wbytes)))
            pool = [(wq, zp, s)] + [(wq.clone(), None if zp is None else zp.clone(), s.clone())
                                    for _ in range(copies - 1)]
            y = torch.empty((1, N), dtype=x.dtype, device=dev)
            ms = min(time_point(x, pool, b, y, 1, N, K, GROUP, dt, L.PATH_AUTO, 50, stream) for _ in range(2))
            points[f"{fam} {K}x{N} M=1"] = round(ms * 1e3, 3)
            del pool, wq, zp, s
            torch.cuda.empty_cache()
    for (K, N) in PREFILL_LAYERS:
        l = build_layer(K, N, 1920, ("bench-prefill", K, N), dev)
        fn = Launcher(l, l["wq"], l["zp"], l["s"])
        fn(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        graph_launch_ms([fn, fn], stream, passes=5, replays=4, reps=2)  # steady clocks
        ms = graph_launch_ms([fn, fn], stream, passes=3, replays=2, reps=3)
        points[f"llama8b_prefill {K}x{N} M=1920"] = round(ms * 1e3, 2)
        del l, fn
        torch.cuda.empty_cache()
    return dict(control=control, points_us=points)


def perf_compare(base, now, band=1.25):
    """Each point's time relative to the baseline, divided by how much faster
    the control runs now than then (stream read for decode points, MFMA loop
    for prefill points); a point regresses when that ratio exceeds `band`."""
    out = []
    for name, t0 in base["points_us"].items():
        t1 = now["points_us"][name]
        key, unit = ("mfma_TFLOPs", "mfma") if "prefill" in name else ("stream_read_GBs", "stream")
        speed = now["control"][key] / base["control"][key]
        ratio = t1 / t0 * speed
        out.append(dict(point=name, base_us=t0, now_us=t1, control=unit, control_speedup=round(speed, 3),
                        normalized_ratio=round(ratio, 3), regressed=ratio > band))
    return out


# Megatron-style tensor-parallel shards of the Llama-3.1-8B layers over P GPUs:
# qkv and gate_up split by output feature (column-parallel: N/P), o and down
# by input feature (row-parallel: K/P; their partial outputs would be summed
# across the GPUs).  (name, K, N, split)
SHARD_LAYERS = (("qkv", 4096, 6144, "N"), ("o", 4096, 4096, "K"), ("gate_up", 4096, 28672, "N"),
                ("down", 14336, 4096, "K"))
SHARD_PREFILL = ("qkv", "gate_up", "down")


def shard_shape(K, N, split, P):
    return (K, N // P) if split == "N" else (K // P, N)


def run_shards(path_prefix):
    """One GPU's share of each Llama-3.1-8B layer under P-way tensor
    parallelism (P = 1, 2, 4, 8), at its real shape: the decode step (M = 1)
    and the prefill layers (M = 1920), bf16 asym g128, on the path the
    dispatcher picks, graphs rotating >= 1 GiB of weight copies.  The
    collectives between the GPUs are not part of it.  Writes <prefix>.md and
    <prefix>.json."""
    import torch
    import int4_weight_only_linear_amd as L
    from synth import make_case
    dev = torch.device("cuda:0")
    side = torch.cuda.Stream()
    g, dt = GROUP, L.W4A16_BF16
    rows = []
    for P in (1, 2, 4, 8):
        for (name, K0, N0, split) in SHARD_LAYERS:
            K, N = shard_shape(K0, N0, split, P)
            Ms = (1, 1920) if name in SHARD_PREFILL else (1,)
            c = make_case(max(Ms), N, K, g, dt, False, False, seed=("shard", name, P))
            wq, zp, sc, x_all, b = _layer_tensors(c, dev)
            wbytes = wq.numel() * 4 + sc.numel() * 2 + zp.numel() * 4
            copies = max(2, min(64, math.ceil((1 << 30) / wbytes)))
            pool = [(wq, zp, sc)] + [(wq.clone(), zp.clone(), sc.clone()) for _ in range(copies - 1)]
            for M in Ms:
                x = x_all[:M].contiguous()
                y = torch.empty((M, N), dtype=x.dtype, device=dev)
                ms = time_point(x, pool, b, y, M, N, K, g, dt, L.PATH_AUTO, 20 if M > 16 else 50, side)
                plan = L.w4a16_plan(M, N, K, g, dt, True)
                nbytes = decode_bytes(M, N, K, g)
                rows.append(dict(P=P, layer=name, split=split, K=K, N=N, M=M, us=round(ms * 1e3, 3),
                                 GBs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                                 TFLOPs=round(2 * M * N * K / (ms * 1e-3) / 1e12, 1),
                                 kernel=("gemv_one" if plan["kernel"] == 1 else "gemv_small")
                                 if M <= 16 and int(L.w4a16_select_path(M, N, K, g, dt, True)) == L.PATH_GEMV
                                 else "gemm", waves=plan["waves"], splits=plan["splits"]))
                print(f"[shards] P={P} {name} K={K} N={N} M={M}: {ms * 1e3:.2f} us", file=sys.stderr, flush=True)
            del pool
            torch.cuda.empty_cache()
    lines = ["# One GPU's share of the Llama-3.1-8B layers under P-way tensor parallelism", "",
             f"Command: python bench.py --shards {os.path.basename(path_prefix)}", "",
             "qkv and gate_up split by output feature (N/P), o and down by input feature (K/P); bf16 activations,",
             "asymmetric uint4, group 128; the path the dispatcher picks; each point the mean launch over graphs",
             "rotating >= 1 GiB of weight copies.  The collectives between the GPUs (an all-gather after the",
             "column-parallel layers where needed, a sum of the row-parallel partial outputs) are not measured.",
             "Scaling = the P = 1 time / (P x this time): 1 when the share takes 1/P of the time.", "",
             "| P | M | layer | K | N | kernel | waves | K ranges | us | GB/s | TFLOP/s |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['P']} | {r['M']} | {r['layer']} | {r['K']} | {r['N']} | {r['kernel']} | {r['waves']} | "
                     f"{r['splits']} | {r['us']} | {r['GBs']} | {r['TFLOPs']} |")
    lines += ["", "| P | decode step (4 layers, M = 1) us | scaling | prefill (3 layers, M = 1920) us | scaling |",
              "|---|---|---|---|---|"]
    tot = {}
    for P in (1, 2, 4, 8):
        d = sum(r["us"] for r in rows if r["P"] == P and r["M"] == 1)
        f = sum(r["us"] for r in rows if r["P"] == P and r["M"] == 1920)
        tot[P] = (d, f)
    for P, (d, f) in tot.items():
        lines.append(f"| {P} | {d:.2f} | {tot[1][0] / (P * d):.3f} | {f:.1f} | {tot[1][1] / (P * f):.3f} |")
    with open(path_prefix + ".md", "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(path_prefix + ".json", "w") as fh:
        json.dump(dict(rows=rows, totals={str(P): dict(decode_us=d, prefill_us=f) for P, (d, f) in tot.items()}), fh,
                  indent=1)
    print(json.dumps(dict(shards=path_prefix + ".md", totals=tot)), flush=True)


def run_profile(kind, steps, dev):
    """Eager launches for a profiler: each layer `steps` times in turn.  Decode
    launches rotate through the bench's >= 1 GiB of weight copies, so that
    every launch streams its weights from HBM as in the bench line (on one
    copy the layer's weights would stay in the 256 MB last-level cache)."""
    import torch
    shapes, M = (DECODE_LAYERS, 1) if kind == "decode" else (PREFILL_LAYERS, 1920)
    layers = [build_layer(K, N, M, ("bench-" + kind, K, N), dev) for (K, N) in shapes]
    copies = 1
    if kind == "decode":
        set_bytes = sum(l["wq"].numel() * 4 + l["s"].numel() * 2 + l["zp"].numel() * 4 for l in layers)
        copies = max(2, math.ceil((1 << 30) / set_bytes))
    pool = [[(l["wq"], l["zp"], l["s"]) for l in layers]]
    for _ in range(copies - 1):
        pool.append([(wq.clone(), zp.clone(), s.clone()) for (wq, zp, s) in pool[0]])
    fns = [[Launcher(l, *pool[c][i]) for c in range(copies)] for i, l in enumerate(layers)]
    sp = torch.cuda.current_stream().cuda_stream
    for per_copy in fns:
        per_copy[0](sp)
    torch.cuda.synchronize()
    for per_copy in fns:
        for i in range(steps):
            per_copy[i % copies](sp)
        torch.cuda.synchronize()
    print(json.dumps(dict(profile=kind, M=M, layers=[f"{K}x{N}" for (K, N) in shapes], launches_per_layer=steps,
                          weight_copies=copies)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies", type=int, default=0, help="weight copies in the rotation pool (0: >= 1 GiB)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-moe", action="store_true", help="skip the expert-indexed decode measurement")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dequantised-copy (dense) comparator of the prefill layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MB (for scaling PMC byte counters)")
    ap.add_argument("--profile", choices=("decode", "prefill"), default="",
                    help="instead of the bench line: --steps eager launches of each decode layer (M=1, "
                         "rotating the bench's >= 1 GiB of weight copies) or prefill layer (M=1920, one "
                         "copy), for rocprofv3 kernel traces and counters (one dispatch per launch, "
                         "kernels named per layer by their grid)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="print a profiles/ summary from rocprofv3 csv output (no GPU needed): "
                         "'trace KIND DIR' (a --profile run), 'trace decode DIR bench' (a trace of the "
                         "bench line's own run), 'pmc KIND DIR_A [DIR_B|- [DIR_C]]' or "
                         "'traffic KIND FETCH_DIR WRITE_DIR'")
    ap.add_argument("--perf-record", default="", metavar="FILE",
                    help="measure the performance-regression points and their controls, write FILE (json)")
    ap.add_argument("--perf-check", default="", metavar="FILE",
                    help="measure the same points and compare with FILE, normalised by the controls; "
                         "exit 1 on a regression beyond 25%%")
    ap.add_argument("--shards", default="", metavar="PREFIX",
                    help="instead of the bench line: time one GPU's share of each Llama-3.1-8B layer under "
                         "P = 1, 2, 4, 8-way tensor parallelism (decode M=1, prefill M=1920), write "
                         "<PREFIX>.md and .json")
    ap.add_argument("--vendor", default="", metavar="PREFIX",
                    help="instead of the bench line: the prefill GEMM against torch's bf16 matmul (vendor BLAS) "
                         "on a dequantised copy, Llama prefill layers at M = 128, 256, 1920; write <PREFIX>.md "
                         "and .json")
    ap.add_argument("--report", default="",
                    help="instead of the bench line: time every point of the decode, prefill and "
                         "dispatch-sweep workloads on both paths, write <REPORT>.md and .json")
    args = ap.parse_args()

    if args.summarize:
        what, kind, dirs = args.summarize[0], args.summarize[1], args.summarize[2:]
        if what == "trace":
            print(summarize_trace(kind, dirs[0], args.steps, of_bench=len(dirs) > 1 and dirs[1] == "bench"))
        elif what == "pmc":
            print(summarize_pmc(kind, {t: d for t, d in zip("ABC", dirs) if d != "-"}, args.steps))
        elif what == "traffic":
            import hashlib
            text, per_launch = summarize_traffic(kind, dirs[0], dirs[1], args.steps)
            h = hashlib.sha256()
            csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int4_weight_only_linear_amd", "csrc")
            for f in DECODE_SOURCES:
                with open(os.path.join(csrc, f), "rb") as fh:
                    h.update(fh.read())
            print(text)
            print("\nmachine-readable (read by bench.py; valid only while the hash of the decode kernel "
                  "sources matches):")
            print(f"traffic_bytes_per_launch: {per_launch}")
            print(f"kernel_source_sha256: {h.hexdigest()}")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libw4a16 has no multi-GPU path (row- and "
              "column-parallel sharding of the layer is a design, not code). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import int4_weight_only_linear_amd as L  # noqa: F401  (loads libw4a16; raises if missing)
    if args.report:
        run_report(args.report)
        return
    if args.shards:
        run_shards(args.shards)
        return
    if args.vendor:
        run_vendor(args.vendor)
        return
    if args.calibration_copy_mb:
        # a plain copy of known size: reads and writes exactly n bytes, so the
        # HBM byte counters of this dispatch give their scale on this device
        n = args.calibration_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)  # one elementwise kernel: n bytes in, n out
        torch.cuda.synchronize()
        del src, dst

    if args.profile:
        run_profile(args.profile, args.steps, dev)
        return
    if args.perf_record or args.perf_check:
        side = torch.cuda.Stream()
        now = perf_points(dev, side)
        now["device"] = torch.cuda.get_device_properties(dev).gcnArchName
        if args.perf_record:
            with open(args.perf_record, "w") as f:
                json.dump(now, f, indent=1)
            print(json.dumps(now), flush=True)
            return
        with open(args.perf_check) as f:
            base = json.load(f)
        res = perf_compare(base, now)
        print(json.dumps(dict(control_now=now["control"], control_base=base["control"], points=res)), flush=True)
        sys.exit(1 if any(r["regressed"] for r in res) else 0)

    # ---- decode: four layers at M = 1, weight copies rotated through HBM ----
    layers = [build_layer(K, N, 1, ("bench-decode", K, N), dev) for (K, N) in DECODE_LAYERS]
    set_bytes = sum(l["wq"].numel() * 4 + l["s"].numel() * 2 + l["zp"].numel() * 4 for l in layers)
    copies = args.copies or max(2, math.ceil((1 << 30) / set_bytes))
    pool = [[(l["wq"], l["zp"], l["s"]) for l in layers]]
    for _ in range(copies - 1):
        pool.append([(wq.clone(), zp.clone(), s.clone()) for (wq, zp, s) in pool[0]])
    launch_lists = [[Launcher(l, *pool[c][i]) for i, l in enumerate(layers)] for c in range(copies)]
    side = torch.cuda.Stream()
    for fns in launch_lists[:1]:            # first calls: device query, outside capture
        for fn in fns:
            fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # graphs of five passes over the weight copies (50 steps), so graph
    # launches are rare between the timed steps
    ms_step = time_steps(launch_lists * 5, args.steps, args.warmup, side)
    step_bytes = sum(decode_bytes(1, l["N"], l["K"], GROUP) for l in layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # per-launch kernel durations of each layer
    durs3 = per_launch_durations(launch_lists, max(5, args.steps // copies), side)
    durs = [d[0] for d in durs3]
    per_layer = []
    for l, (d, d10, d90) in zip(layers, durs3):
        b = decode_bytes(1, l["N"], l["K"], GROUP)
        per_layer.append(dict(K=l["K"], N=l["N"], bytes=b, us=round(d * 1e3, 3),
                              p10_us=round(d10 * 1e3, 3), p90_us=round(d90 * 1e3, 3),
                              GBs=round(b / (d * 1e-3) / 1e9, 1),
                              frac=round(b / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)))
    mean_bytes = step_bytes / len(layers)
    mean_ms = float(np.mean(durs))
    achieved = mean_bytes / (mean_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    ceil_rows = decode_ceilings(layers, pool, side)
    floor_ms = sum(r["stream_read_us"] for r in ceil_rows) * 1e-3
    loads_ms = sum(r["loads_only_us"] for r in ceil_rows) * 1e-3
    measured_ceiling = dict(
        what="ceiling kernels on the same weight copies, per launch (graphs rotating >= 1 GiB)",
        stream_read_GBs=round(step_bytes / (floor_ms * 1e-3) / 1e9, 1),
        decode_loads_only_GBs=round(step_bytes / (loads_ms * 1e-3) / 1e9, 1),
        frac_of_stream_read=round(achieved / (step_bytes / (floor_ms * 1e-3) / 1e9), 4),
        frac_of_decode_loads_only=round(achieved / (step_bytes / (loads_ms * 1e-3) / 1e9), 4),
        note="GB/s = the step's algorithmic bytes over the summed per-layer times of reading only "
             "the packed weights (stream: grid-stride read; loads only: the decode kernel's grid and "
             "1 KiB blocks, nothing computed); padN: 16-row tiles N bytes apart beyond the packed tile",
        per_layer=ceil_rows)
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    traffic_unit="bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
                    kernel=decode_kernel_name(DECODE_LAYERS[0]),
                    mean_launch_us=round(mean_ms * 1e3, 3), bytes_per_launch=int(mean_bytes),
                    per_layer=per_layer, measured_ceiling=measured_ceiling)

    # ---- prefill: M = 1920 on the three prefill layers ----
    prefill = None
    if not args.no_prefill:
        players = [build_layer(K, N, 1920, ("bench-prefill", K, N), dev) for (K, N) in PREFILL_LAYERS]
        plaunch = [[Launcher(l, l["wq"], l["zp"], l["s"]) for l in players]]
        for fn in plaunch[0]:
            fn(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        # five passes per graph, so graph launches do not separate the passes
        pms = time_steps(plaunch * 5, args.prefill_steps, max(5, args.prefill_steps // 4), side)
        pdurs = [d[0] for d in per_launch_durations(plaunch * 4, max(3, args.prefill_steps // 4), side, passes=1,
                                                    replays=2)]
        flops = sum(2 * 1920 * N * K for (K, N) in PREFILL_LAYERS)
        tflops = flops / (pms * 1e-3) / 1e12
        prefill = dict(workload="Llama-3.1-8B-shaped prefill, M=1920, layers (K,N) "
                                + ", ".join(f"({K},{N})" for K, N in PREFILL_LAYERS)
                                + ", asym uint4 g128, bf16",
                       ms_per_pass=round(pms, 4), tflops=round(tflops, 1),
                       frac_of_peak=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                       peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                       per_layer=[dict(K=K, N=N, us=round(d * 1e3, 2),
                                       tflops=round(2 * 1920 * N * K / (d * 1e-3) / 1e12, 1))
                                  for (K, N), d in zip(PREFILL_LAYERS, pdurs)])
        mc = mfma_ceiling(side, torch.cuda.get_device_properties(dev).multi_processor_count)
        prefill["measured_ceiling"] = dict(mc, frac_of_measured=round(tflops / mc["best"], 4))
        if not args.no_dense:
            prefill["dequantised_copy"] = dense_comparator(players, side, args.prefill_steps)
            vrows = []
            for l in players:
                w = L.w4a16_dequant(l["wq"], l["s"], l["zp"], group_size=GROUP)
                t = vendor_dense(l["x"], w, args.prefill_steps, side)
                vrows.append(dict(K=l["K"], N=l["N"], us=round(t, 2),
                                  tflops=round(2 * l["M"] * l["N"] * l["K"] / (t * 1e-6) / 1e12, 1)))
                del w
            prefill["vendor_dense"] = dict(what="torch.matmul (bf16, the vendor BLAS) on the dequantised copy, "
                                                "transposed to [K, N], graphs rotating >= 1 GiB of copies",
                                           per_layer=vrows)
        del players, plaunch

    moe = None
    if not args.no_moe:
        moe = moe_measure(side)

    cpu = None
    if not args.no_cpu_baseline:
        host_layers = [(l["K"], l["N"], l["case"]) for l in layers]
        cpu = cpu_baseline(host_layers)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3.1-8B-shaped decode step, M=1: W4A16 layers (K,N) "
                        + ", ".join(f"({K},{N})" for K, N in DECODE_LAYERS)
                        + "; asymmetric uint4, packed int32 zero points, group 128, bf16",
            "global_batch": 1,
            "weight_copies": copies,
            "weight_pool_bytes": int(set_bytes * copies),
            "bytes_per_step": int(step_bytes),
            "graph_replay": True,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "moe_decode": moe,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
