#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

Headline: fwd+bwd TFLOP/s of the seven LLaMA-7B-shaped linears (q, k, v, o
[4096x4096], gate, up [11008x4096], down [4096x11008]) at M = 2048 tokens,
rank 64, s = 0.25.  One step = forward (Y, T) and backward (dX, dA, dB) of
all seven on one batch; the NF4 base is quantized once at load, outside the
step, because the base is frozen.  Algorithmic flops per linear:
4MKN + 6Mr(K+N); dequantization and recomputation are not counted.

Second figure: decode (M = 1) effective HBM GB/s on the 65B shapes, with a
pool of weight copies over 1 GB per shape so the 256 MB last-level cache
cannot serve them.

Prints one JSON line (the last line of stdout).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s at M=2048; decode (M=1) effective HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
FAMILIES = {0: "k_fwd_gemm", 1: "k_dx_gemm", 2: "k_fwd_decode", 3: "k_quantize", 4: "rank"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_fine_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, src_hash):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def linear_flops(M, N, K, r):
    """Algorithmic flops of one linear's forward + backward: 4MKN + 6Mr(K+N)
    (base products of Y and dX, and the rank-r products T, LoRA-up, G, dA, dB,
    the LoRA term of dX); dequantization and recomputation are not counted."""
    return 4 * M * K * N + 6 * M * r * (K + N)


def bf16_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


def percentiles(xs):
    """p10, median and p90 of a list of per-step times (ms)."""
    import numpy as np
    return [float(v) for v in np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])]


def run_training(q, torch, steps, warmup, dev, key="llama7b", M=None):
    """One step = fwd + bwd of the workload's seven linears.  The 33B workload
    runs the backward as under gradient checkpointing: T is not kept, the
    backward recomputes it (and dequantizes W again, as every backward does)."""
    import numpy as np

    import workloads
    cfg = workloads.WORKLOADS[key]
    M, r, s = (cfg.M[0] if M is None else M), cfg.r, cfg.s
    recompute = key == "llama33b_recompute"
    layers = []
    t0 = time.time()
    for lin, inp in workloads.workload_inputs(key, M=M):
        w = q.qlora_nf4_quantize(torch.from_numpy(inp.W).to(dev))
        L = dict(lin=lin, w=w, X=bf16_dev(inp.X, dev), A=bf16_dev(inp.A, dev),
                 B=bf16_dev(inp.B, dev), dY=bf16_dev(inp.dY, dev))
        L["Y"] = torch.empty((M, lin.N), dtype=torch.bfloat16, device=dev)
        L["T"] = torch.empty((M, r), dtype=torch.float32, device=dev)
        L["dX"] = torch.empty((M, lin.K), dtype=torch.bfloat16, device=dev)
        L["dA"] = torch.empty((lin.K, r), dtype=torch.bfloat16, device=dev)
        L["dB"] = torch.empty((r, lin.N), dtype=torch.bfloat16, device=dev)
        L["wsf"] = torch.empty(q.lib().qlora_linear_fwd_workspace_bytes(M, lin.N, lin.K, r),
                               dtype=torch.uint8, device=dev)
        L["wsb"] = torch.empty(q.lib().qlora_linear_bwd_workspace_bytes(M, lin.N, lin.K, r),
                               dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()
    log(f"setup (draw + upload + quantize {len(layers)} linears): {time.time() - t0:.1f}s")

    def step():
        for L in layers:
            q.qlora_linear_fwd(L["X"], L["w"], L["A"], L["B"], s, Y=L["Y"], T=L["T"],
                               workspace=L["wsf"])
            q.qlora_linear_bwd(L["dY"], L["X"], L["w"], L["A"], L["B"], s,
                               T=None if recompute else L["T"],
                               dX=L["dX"], dA=L["dA"], dB=L["dB"], workspace=L["wsb"])

    for _ in range(warmup):
        step()
    step()   # the eager reference for the graph check (also when warmup is 0)
    torch.cuda.synchronize()
    outs = ("Y", "T", "dX", "dA", "dB")
    eager = [[L[k].clone() for k in outs] for L in layers]

    # The timed steps replay one step captured as a HIP graph (the library
    # allocates nothing and records no memsets, so a step captures whole);
    # the replay must reproduce the eager outputs bit for bit.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    for L, ref in zip(layers, eager):
        for k, t in zip(outs, ref):
            if not torch.equal(L[k], t):
                raise RuntimeError(f"graph replay differs from the eager step ({L['lin'].name}.{k})")
    # an event after every replay gives the per-step spread (median, p10, p90)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    del graph

    # Kernel durations: the same steps run eagerly with the per-family event
    # timer on (the events sit on the launch stream around each kernel family)
    q.qlora_profile_reset()
    q.qlora_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t0) * 1e3 / steps
    q.qlora_profile_enable(False)
    fam = {FAMILIES[f]: q.qlora_profile_read(f) for f in FAMILIES}

    flops_step = sum(linear_flops(M, L["lin"].N, L["lin"].K, r) for L in layers)
    fwd_flops = sum(2 * M * L["lin"].K * L["lin"].N + 2 * M * r * L["lin"].N for L in layers)
    dx_flops = sum(2 * M * L["lin"].K * L["lin"].N + 2 * M * r * L["lin"].K for L in layers)
    return dict(layers=layers, M=M, r=r, s=s, ms_step=ms_step, ms_step_eager=ms_step_eager,
                step_ms_pct=percentiles(per_step),
                flops_step=flops_step,
                fam=fam, fwd_flops=fwd_flops, dx_flops=dx_flops, cfg=cfg)


def run_stack(q, torch, dev, steps=2, warmup=1):
    """The 65B-shaped stack with the whole NF4 base resident: 80 layers x 7
    linears (hidden 8192, FFN 22016), every weight drawn and quantized on the
    device, r = 64 adapters on every linear.  A training step runs the
    linears in a chain, per layer h = o(v(k(q(x)))), a = gate(h) + up(h),
    x' = down(a), with every linear output scaled by 1/(0.02 sqrt(K)) (a
    torch op outside the library) to keep values O(1); the backward runs the
    chain in reverse.  Also one decode token (M = 1, forward only) through
    the whole chain, so the 33 GB of codes stream from HBM once per token."""
    import workloads
    cfg = workloads.WORKLOADS["stack_65b"]
    M, r, s = cfg.M[0], cfg.r, cfg.s
    t0 = time.time()
    lins = []
    for idx, lin in enumerate(cfg.linears):
        W = workloads.device_weight(torch, dev, lin.N, lin.K, seed=4000 + idx)
        w = q.qlora_nf4_quantize(W)
        del W
        A, B = workloads.device_adapters(torch, dev, lin.N, lin.K, r, seed=5000 + idx)
        lins.append(dict(lin=lin, w=w, A=A, B=B))
    torch.cuda.synchronize()
    nf4_bytes = sum(L["w"].codes.numel() + L["w"].absmax_q.numel() + 4 * L["w"].absmax_scale.numel()
                    for L in lins)
    log(f"setup (draw + quantize {len(lins)} linears on the device): {time.time() - t0:.1f}s, "
        f"NF4 resident {nf4_bytes / 1e9:.2f} GB, device memory in use "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB")
    scale = {K: 1.0 / (0.02 * K ** 0.5) for K in (8192, 22016)}
    ws_f = torch.empty(max(q.lib().qlora_linear_fwd_workspace_bytes(M, L["lin"].N, L["lin"].K, r)
                           for L in lins[:7]), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(q.lib().qlora_linear_bwd_workspace_bytes(M, L["lin"].N, L["lin"].K, r)
                           for L in lins[:7]), dtype=torch.uint8, device=dev)
    for L in lins:
        L["dA"] = torch.empty_like(L["A"])
        L["dB"] = torch.empty_like(L["B"])
    x0 = workloads.device_activations(torch, dev, M, 8192, seed=4900)
    dx_top = workloads.device_activations(torch, dev, M, 8192, seed=4901)

    def lin_fwd(L, x):
        y, T = q.qlora_linear_fwd(x, L["w"], L["A"], L["B"], s, workspace=ws_f)
        y.mul_(scale[L["lin"].K])
        L["X"], L["T"] = x, T
        return y

    def lin_bwd(L, dy):
        dy = dy * scale[L["lin"].K]
        dX, _, _ = q.qlora_linear_bwd(dy, L["X"], L["w"], L["A"], L["B"], s, T=L["T"],
                                      dA=L["dA"], dB=L["dB"], workspace=ws_b)
        return dX

    def step():
        x = x0
        for l in range(0, len(lins), 7):
            Lq, Lk, Lv, Lo, Lg, Lu, Ld = lins[l:l + 7]
            h = lin_fwd(Lo, lin_fwd(Lv, lin_fwd(Lk, lin_fwd(Lq, x))))
            a = lin_fwd(Lg, h) + lin_fwd(Lu, h)
            x = lin_fwd(Ld, a)
        dx = dx_top
        for l in range(len(lins) - 7, -1, -7):
            Lq, Lk, Lv, Lo, Lg, Lu, Ld = lins[l:l + 7]
            da = lin_bwd(Ld, dx)
            dh = lin_bwd(Lg, da) + lin_bwd(Lu, da)
            dx = lin_bwd(Lq, lin_bwd(Lk, lin_bwd(Lv, lin_bwd(Lo, dh))))
        for L in lins:   # saved inputs are freed after the backward
            L.pop("X", None)
            L.pop("T", None)
        return dx

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    flops = sum(linear_flops(M, L["lin"].N, L["lin"].K, r) for L in lins)

    # decode: one token through the chain, forward only
    x1 = workloads.device_activations(torch, dev, 1, 8192, seed=4902)
    ws_d = torch.empty(max(q.lib().qlora_linear_fwd_workspace_bytes(1, L["lin"].N, L["lin"].K, r)
                           for L in lins[:7]), dtype=torch.uint8, device=dev)

    def token():
        x = x1
        for l in range(0, len(lins), 7):
            Lq, Lk, Lv, Lo, Lg, Lu, Ld = lins[l:l + 7]
            f = lambda L, v: q.qlora_linear_fwd(v, L["w"], L["A"], L["B"], s, workspace=ws_d)[0] \
                .mul_(scale[L["lin"].K])
            h = f(Lo, f(Lv, f(Lk, f(Lq, x))))
            x = f(Ld, f(Lg, h) + f(Lu, h))
        return x

    ref = token()
    torch.cuda.synchronize()
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        token()
    torch.cuda.synchronize()
    ms_token_eager = (time.perf_counter() - t0) * 1e3 / reps
    # device time: the token captured as one graph and replayed (the eager
    # time above includes the host path of 560 calls from Python)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = token()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("decode token: graph replay differs from the eager pass")
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    ms_token = (time.perf_counter() - t0) * 1e3 / reps
    del graph
    alg = sum(L["w"].codes.numel() + L["w"].absmax_q.numel() + 4 * L["w"].absmax_scale.numel()
              + 2 * (L["lin"].K + L["lin"].N + L["lin"].K * r + r * L["lin"].N) for L in lins)
    return dict(ms_step=ms_step, tflops=flops / (ms_step * 1e-3) / 1e12, flops_step=flops,
                nf4_gb=nf4_bytes / 1e9, peak_mem_gb=peak / 1e9, ms_token=ms_token,
                ms_token_eager=ms_token_eager, token_gbs=alg / (ms_token * 1e-3) / 1e9)


def run_decode(q, torch, dev, reps=20, pool_bytes=1.1e9):
    """Decode GB/s on the 65B shapes, rotating over >1 GB of weight copies.

    The rate is device time per call: one pass over the pool is captured as
    a graph (the calls allocate nothing and record no memsets) and replayed;
    the eager per-call time, host launch path included, is reported too."""
    import workloads
    cfg = workloads.WORKLOADS["decode_65b"]
    r, s = cfg.r, cfg.s
    g = torch.Generator(device=dev)
    g.manual_seed(2000)
    out = {}
    for M in cfg.M:
        tot_bytes, tot_ms, kern_bytes, kern_ms = 0.0, 0.0, 0.0, 0.0
        per_shape = {}
        for lin in cfg.linears:
            N, K = lin.N, lin.K
            nf4_bytes = N * K // 2 + N * K // 64 + 4 * ((N * K // 64 + 255) // 256)
            copies = max(2, int(pool_bytes // nf4_bytes) + 1)
            pool = []
            for _ in range(copies):
                W = torch.randn((N, K), generator=g, device=dev) * 0.02
                W = torch.where(torch.rand((N, K), generator=g, device=dev) < 0.001, W * 10, W)
                pool.append(q.qlora_nf4_quantize(W))
                del W
            X = (torch.randn((M, K), generator=g, device=dev)).to(torch.bfloat16)
            A = (torch.randn((K, r), generator=g, device=dev) / r).to(torch.bfloat16)
            B = (torch.randn((r, N), generator=g, device=dev) * 0.01).to(torch.bfloat16)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            T = torch.empty((M, r), dtype=torch.float32, device=dev)
            ws = torch.empty(q.lib().qlora_linear_fwd_workspace_bytes(M, N, K, r),
                             dtype=torch.uint8, device=dev)
            for w in pool[:2]:
                q.qlora_linear_fwd(X, w, A, B, s, Y=Y, T=T, workspace=ws)
            torch.cuda.synchronize()
            # eager per-call rate (includes the Python launch path)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for w in pool:
                q.qlora_linear_fwd(X, w, A, B, s, Y=Y, T=T, workspace=ws)
            ev1.record()
            torch.cuda.synchronize()
            ms_eager = ev0.elapsed_time(ev1) / len(pool)
            # device rate: one pass over the pool captured as a graph and
            # replayed, so host launch overhead is not on the clock
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for w in pool:
                    q.qlora_linear_fwd(X, w, A, B, s, Y=Y, T=T, workspace=ws)
            graph.replay()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(reps):
                graph.replay()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1)
            calls = reps * len(pool)
            # the last call of every replay used pool[-1]: recompute it eagerly
            Y_graph = Y.clone()
            q.qlora_linear_fwd(X, pool[-1], A, B, s, Y=Y, T=T, workspace=ws)
            torch.cuda.synchronize()
            if not torch.equal(Y_graph, Y):
                raise RuntimeError(f"decode {N}x{K} M={M}: graph replay differs from eager call")
            del graph
            # decode-kernel time alone: a second pass with the launch profiler on
            q.qlora_profile_reset()
            q.qlora_profile_enable(True)
            for _ in range(max(1, reps // 4)):
                for w in pool:
                    q.qlora_linear_fwd(X, w, A, B, s, Y=Y, T=T, workspace=ws)
            torch.cuda.synchronize()
            q.qlora_profile_enable(False)
            kms, kn = q.qlora_profile_read(2)
            alg = nf4_bytes + 2 * (M * K + M * N + K * r + r * N)
            per_shape[f"{N}x{K}"] = dict(us_per_call=1e3 * ms / calls,
                                         gbs_call=alg * calls / (ms * 1e-3) / 1e9,
                                         us_per_call_eager=1e3 * ms_eager,
                                         us_decode_kernel=1e3 * kms / max(1, kn),
                                         gbs_decode_kernel=alg * kn / (kms * 1e-3) / 1e9,
                                         copies=copies)
            tot_bytes += alg * calls
            tot_ms += ms
            kern_bytes += alg * kn
            kern_ms += kms
            del pool
            torch.cuda.empty_cache()
        out[f"M={M}"] = dict(gbs_call=tot_bytes / (tot_ms * 1e-3) / 1e9,
                             gbs_decode_kernel=kern_bytes / (kern_ms * 1e-3) / 1e9,
                             shapes=per_shape)
        log(f"decode M={M}: {out[f'M={M}']['gbs_call']:.0f} GB/s per call, "
            f"{out[f'M={M}']['gbs_decode_kernel']:.0f} GB/s decode kernel")
    return out


def run_cpu_baseline(train, repeats=3):
    """The oracle (dequantize + forward + backward, float64 products) on a
    bounded sample of the same workload: all seven linears at full M (one
    training step), `repeats` times, on this host's cores."""
    import numpy as np

    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    cfg = workloads.WORKLOADS["llama7b"]
    flops, secs = 0, 0.0
    ctx = threadpool_limits(cores) if threadpool_limits else None
    try:
        for idx in range(len(cfg.linears)):
            (lin, inp), = list(workloads.workload_inputs("llama7b", linears=[idx]))
            codes, e, d, _ = oracle.quantize(inp.W)       # load-time, untimed
            for _ in range(repeats):
                t0 = time.perf_counter()
                What = oracle.dequantize(codes, e, d, lin.N, lin.K)
                oracle.linear_fwd(inp.X, What, inp.A, inp.B, cfg.s)
                oracle.linear_bwd(inp.dY, inp.X, What, inp.A, inp.B, cfg.s)
                secs += time.perf_counter() - t0
                flops += oracle.linear_flops(cfg.M[0], lin.N, lin.K, cfg.r)
        threads = cores
        if threadpool_info:
            nums = [p.get("num_threads", 0) for p in threadpool_info()
                    if p.get("user_api") == "blas"]
            threads = max(nums) if nums else cores
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return dict(value=flops / secs / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                seconds=secs,
                sample=f"{repeats} steps: all seven linears, M=2048, r=64: oracle dequantize + "
                       "fwd + bwd (float64 products); load-time quantization untimed")


def _rocprof_csvs(root, suffix):
    out = []
    for d, _, files in os.walk(root):
        out += [os.path.join(d, f) for f in files if f.endswith(suffix)]
    return sorted(out)


def summarize_rocprof(root, copy_mib, top=16, by_grid=False):
    """Text summary of a rocprofv3 output folder (csv format): the kernel
    statistics table, and per-dispatch counter means per kernel (per kernel
    and grid size with by_grid, which tells shapes of one kernel apart).
    With a calibration copy of `copy_mib` MiB in the run, the
    FETCH_SIZE/WRITE_SIZE scale factors (bytes moved / counter bytes) are
    printed too."""
    import csv
    lines = []
    for path in _rocprof_csvs(root, "kernel_stats.csv"):
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        lines.append(f"{'kernel':70s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} "
                     f"{'max_us':>9s} {'total_%':>7s}")
        for r in rows[:top]:
            lines.append(f"{r['Name'][:70]:70s} {int(r['Calls']):6d} "
                         f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                         f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
    traffic = {}
    for path in _rocprof_csvs(root, "counter_collection.csv"):
        agg = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if by_grid:   # (the calibration copy keeps its name's "neg" in front)
                tag = "neg_kernel " if "neg_kernel" in name else ""
                name = f"{(tag + name.split('(')[0])[:52]} grid={r['Grid_Size']}"
            key = (name, r["Counter_Name"])
            agg.setdefault(key, []).append(float(r["Counter_Value"]))
        lines.append(f"{'kernel':70s} {'counter':>12s} {'dispatches':>10s} {'mean_per_dispatch':>18s}")
        for (k, c), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            mean = sum(v) / len(v)
            traffic.setdefault(k, {})[c] = (mean, len(v))
            lines.append(f"{k[:70]:70s} {c:>12s} {len(v):10d} {mean:18.1f}")
        if copy_mib:
            exp_kib = copy_mib * 1024.0
            for k, cs in traffic.items():
                if "neg" in k:
                    for c, (mean, n) in cs.items():
                        if c in ("FETCH_SIZE", "WRITE_SIZE"):
                            lines.append(f"calibration copy ({k[:40]}): {c} {mean:.0f} KiB for "
                                         f"{exp_kib:.0f} KiB moved -> scale {exp_kib / mean:.4f}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the extra step at one GPU's share of 8-way data parallelism "
                         "(256 of the 2048 tokens)")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode leg (65B shapes, M in {1, 4, 16}) and print its "
                         "numbers (for profiling it on its own)")
    ap.add_argument("--decode-reps", type=int, default=20,
                    help="graph replays per shape in the decode leg")
    ap.add_argument("--workload", default="llama7b",
                    choices=("llama7b", "llama33b_recompute", "stack_65b"),
                    help="llama7b: the headline (LLaMA-7B linears, M=2048); "
                         "llama33b_recompute: the 33B layer at M=4096 with recompute backward; "
                         "stack_65b: the 65B stack of 560 linears resident on the GPU (training "
                         "step and one decode token)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain elementwise copy (torch.neg) of this many MiB before "
                         "the step, as the yardstick for rocprofv3 FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print a text summary of a rocprofv3 csv output folder and exit")
    ap.add_argument("--by-grid", action="store_true",
                    help="with --summarize-rocprof: counter means per kernel and grid size")
    args = ap.parse_args()
    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof, args.copy_calibration_mib,
                                by_grid=args.by_grid))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_fine_amd as q
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    q.lib()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 18          # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.decode_only:
        dec = run_decode(q, torch, dev, reps=args.decode_reps)
        print(json.dumps({"metric": "QLoRA decode (M=1) effective HBM GB/s, 65B shapes",
                          "value": dec["M=1"]["gbs_call"], "unit": "GB/s", "n_gpus": 1,
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "decode": dec}), flush=True)
        return
    if args.workload == "stack_65b":
        st = run_stack(q, torch, dev)
        log(f"65B stack step: {st['ms_step']:.1f} ms, {st['tflops']:.1f} TFLOP/s; one decode token "
            f"through all 560 linears: {st['ms_token']:.2f} ms by graph replay, {st['token_gbs']:.0f} GB/s "
            f"({st['ms_token_eager']:.2f} ms eager from Python)")
        print(json.dumps({
            "metric": "QLoRA fwd+bwd TFLOP/s, 65B-shaped stack resident on one GPU",
            "value": st["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": 2, "warmup": 1,
            "ms_per_step": st["ms_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "80 layers x 7 linears (hidden 8192, FFN 22016), NF4 base "
                                   "quantized on the device, r=64 LoRA on every linear, chained "
                                   "fwd + reverse bwd, M=2048 tokens",
                       "tokens": 2048, "rank": 64, "lora_scale": 0.25},
            "nf4_resident_gb": st["nf4_gb"], "peak_device_memory_gb": st["peak_mem_gb"],
            "decode_token_ms": st["ms_token"], "decode_token_gbs": st["token_gbs"],
            "decode_token_ms_eager": st["ms_token_eager"],
        }), flush=True)
        return

    tr = run_training(q, torch, args.steps, args.warmup, dev, key=args.workload)
    value = tr["flops_step"] / (tr["ms_step"] * 1e-3) / 1e12
    log(f"train step: {tr['ms_step']:.3f} ms ({tr['ms_step_eager']:.3f} ms eager with the kernel "
        f"timer on), {value:.1f} TFLOP/s; kernels: {tr['fam']}")

    fwd_ms, fwd_n = tr["fam"]["k_fwd_gemm"]
    dx_ms, dx_n = tr["fam"]["k_dx_gemm"]
    if fwd_ms >= dx_ms:
        kern, kms, kn, kflops = "k_fwd_gemm", fwd_ms, fwd_n, tr["fwd_flops"]
    else:
        kern, kms, kn, kflops = "k_dx_gemm", dx_ms, dx_n, tr["dx_flops"]
    steps_timed = args.steps
    achieved = kflops * steps_timed / (kms * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    traffic = stored_traffic(kern, src_hash)
    roofline = dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=achieved / PEAK_BF16_TFLOPS, traffic=traffic, kernel=kern,
                    avg_launch_us=1e3 * kms / max(1, kn),
                    flops_per_launch=kflops / len(tr["layers"]), src_hash=src_hash)

    kernels = {}
    for name, (ms, n) in tr["fam"].items():
        if n:
            kernels[name] = dict(ms_per_step=ms / steps_timed, launches_per_step=n / steps_timed,
                                 avg_launch_us=1e3 * ms / n)

    decode = None
    if not args.no_decode:
        decode = run_decode(q, torch, dev, reps=args.decode_reps)

    shard = None
    if args.workload == "llama7b" and not args.no_shard:
        # extra data point: the same step at the per-GPU share of 8-way data
        # parallelism over the 2048-token batch (not the headline value)
        sh = run_training(q, torch, args.steps, args.warmup, dev, key="llama7b", M=256)
        shard = dict(tokens=256, data_parallel=8, ms_per_step=sh["ms_step"],
                     tflops=sh["flops_step"] / (sh["ms_step"] * 1e-3) / 1e12,
                     note="one GPU's share of 8-way data parallelism over the 2048-token "
                          "batch; the dA/dB all-reduce is not part of it")
        shard["kernels_ms_per_step"] = {k: ms / args.steps for k, (ms, n) in sh["fam"].items() if n}
        log(f"dp8 shard (M=256): {sh['ms_step']:.3f} ms per step, {shard['tflops']:.1f} TFLOP/s; "
            f"kernels (ms per step, eager): {shard['kernels_ms_per_step']}")
        del sh

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(tr)
        log(f"cpu baseline: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")

    cfg = tr["cfg"]
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": tr["ms_step"],
        "ms_per_step_eager_timed_kernels": tr["ms_step_eager"],
        "step_ms_p10_p50_p90": tr["step_ms_pct"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("LLaMA-7B-shaped QLoRA linears q,k,v,o [4096x4096], gate,up "
                         "[11008x4096], down [4096x11008]; NF4 base (block 64, DQ 256); "
                         "fwd + bwd (dX, dA, dB)") if args.workload == "llama7b" else
                        ("33B-shaped QLoRA linears q,k,v,o [6656x6656], gate,up "
                         "[17920x6656], down [6656x17920]; NF4 base; fwd + recompute bwd"),
            "global_batch": cfg.M[0], "seq_len": 512 if args.workload == "llama7b" else 2048,
            "batch": 4 if args.workload == "llama7b" else 2, "tokens": cfg.M[0],
            "rank": cfg.r, "lora_scale": cfg.s, "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode_m1_gbs": None if decode is None else decode["M=1"]["gbs_call"],
        "dp8_shard": shard,
        "decode": decode,
        "kernels": kernels,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
