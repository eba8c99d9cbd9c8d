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
                               "gemv_small_kernel_llama8b_decode_M1_traffic.txt")
DECODE_SOURCES = ("w4a16_gemv.hip", "w4a16_device.hpp", "w4a16_internal.h")


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
    run back to back as they do inside a step.  Median over `reps`."""
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
        out.append(float(np.median(ts)))
    return out


def cpu_baseline(layers_host, min_s=10.0):
    """The oracle (untuned) on this host, 1 thread: whole M=1 decode steps over
    the layers, repeated until at least `min_s` seconds of oracle work."""
    import contextlib
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
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
    return dict(value=total_bytes / t_total / 1e9, unit="GB/s", cores=1, kind="oracle",
                seconds=round(t_total, 3),
                sample=(f"oracle linear_ref (unpack + exact fp32 dequant + fp64 GEMV) over {steps} M=1 "
                        f"decode step(s), layers {layers} (K x N), single thread; packing not timed"))


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
    (shape, group, quantisation, dtype).  Writes <prefix>.md and <prefix>.json."""
    import torch
    import int4_weight_only_linear_amd as L
    from synth import make_case
    from synth.configs import CONFIGS
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
        f.write(f"Command: python bench.py --report {path_prefix}\n\n")
        f.write("Each point: mean time per launch over a HIP graph of back-to-back launches that rotate\n"
                "through >= 1 GiB of weight copies (weights stream from HBM).  GB/s = algorithmic bytes\n"
                "(weights, scales, zp, x, y, bias) / time; TFLOP/s = 2*M*N*K / time; peaks 8 TB/s and\n"
                "2.5 PFLOP/s.  auto (*) marks the kernel W4A16_PATH_AUTO picks.\n\n")
        f.write("| config | K | N | M | g | quant | dtype | bias | path | auto | us | GB/s | %HBM | TFLOP/s | %MFMA |\n")
        f.write("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {r['config']} | {r['K']} | {r['N']} | {r['M']} | {r['group']} | {r['quant']} | "
                    f"{r['dtype']} | {'y' if r['bias'] else 'n'} | {r['path']} | {'*' if r['auto'] else ''} | "
                    f"{r['us']} | {r['GBs']} | {100 * r['hbm_frac']:.1f} | {r['TFLOPs']} | "
                    f"{100 * r['mfma_frac']:.1f} |\n")
        f.write("\n| K | N | g | quant | dtype | M* (largest M where the decode kernel is faster) |\n")
        f.write("|---|---|---|---|---|---|\n")
        for m in mstar:
            f.write(f"| {m['K']} | {m['N']} | {m['group']} | {m['quant']} | {m['dtype']} | {m['Mstar']} |\n")
    print(json.dumps(dict(report=path_prefix + ".md", points=len(rows), mstar=mstar)), flush=True)


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
    ap.add_argument("--report", default="",
                    help="instead of the bench line: time every point of the decode, prefill and "
                         "dispatch-sweep workloads on both paths, write <REPORT>.md and .json")
    args = ap.parse_args()

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
    durs = per_launch_durations(launch_lists, max(5, args.steps // copies), side)
    per_layer = []
    for l, d in zip(layers, durs):
        b = decode_bytes(1, l["N"], l["K"], GROUP)
        per_layer.append(dict(K=l["K"], N=l["N"], bytes=b, us=round(d * 1e3, 3),
                              GBs=round(b / (d * 1e-3) / 1e9, 1),
                              frac=round(b / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)))
    mean_bytes = step_bytes / len(layers)
    mean_ms = float(np.mean(durs))
    achieved = mean_bytes / (mean_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    traffic_unit="bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
                    kernel="gemv_small_kernel<bf16, group 128, asym>",
                    mean_launch_us=round(mean_ms * 1e3, 3), bytes_per_launch=int(mean_bytes),
                    per_layer=per_layer)

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
        pdurs = per_launch_durations(plaunch * 4, max(3, args.prefill_steps // 4), side, passes=1, replays=2)
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
        if not args.no_dense:
            prefill["dequantised_copy"] = dense_comparator(players, side, args.prefill_steps)
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
