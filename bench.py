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
FAMILIES = {0: "k_fwd_gemm", 1: "k_dx_gemm", 2: "k_fwd_decode", 3: "k_quantize", 4: "rank",
            5: "k_adamw"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources that define each kernel whose HBM traffic the bench reports: a
# stored counter reading is used only while these files are unchanged.
KERNEL_SOURCES = {
    "k_fwd_gemm": ("gemm_fwd.hip", "device_common.hpp", "kernels.hpp"),
    "k_dx_gemm": ("gemm_dx.hip", "device_common.hpp", "kernels.hpp"),
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_fine_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def write_traffic(fetch_dir, write_dir, copy_mib, source_note, path=None):
    """profiles/traffic.json from two rocprofv3 counter runs of the same
    command (FETCH_SIZE, then WRITE_SIZE), each with a calibration copy of
    copy_mib MiB (`--copy-calibration-mib`): per kernel, the mean counter
    reading per dispatch in KiB, scaled by bytes moved / counter reading of
    the copy, and the hash of the kernel's sources."""
    import csv
    means, scale = {}, {}
    for counter, root in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        agg = {}
        for csv_path in _rocprof_csvs(root, "counter_collection.csv"):
            for r in csv.DictReader(open(csv_path)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = ("neg" if "neg_kernel" in name else
                       next((k for k in KERNEL_SOURCES if f"{k}<0>" in name), None))
                if key:
                    agg.setdefault(key, []).append(float(r["Counter_Value"]))
        if "neg" not in agg:
            raise SystemExit(f"{root}: no calibration copy in the {counter} run")
        scale[counter] = copy_mib * 1024.0 / (sum(agg["neg"]) / len(agg["neg"]))
        for k, v in agg.items():
            if k != "neg":
                means.setdefault(k, {})[counter] = (sum(v) / len(v), len(v))
    out = {}
    for k, m in sorted(means.items()):
        fk, wk = m["FETCH_SIZE"][0], m["WRITE_SIZE"][0]
        fb, wb = fk * 1024 * scale["FETCH_SIZE"], wk * 1024 * scale["WRITE_SIZE"]
        out[k] = dict(bytes_per_launch=fb + wb, fetch_bytes_per_launch=fb,
                      write_bytes_per_launch=wb, fetch_kib_raw=round(fk, 1),
                      write_kib_raw=round(wk, 1), fetch_scale=round(scale["FETCH_SIZE"], 4),
                      write_scale=round(scale["WRITE_SIZE"], 4),
                      dispatches=m["FETCH_SIZE"][1], src_hash=kernel_source_hash(k),
                      launches="mean over the dispatches of the profiled run",
                      source=source_note)
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


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


def q4_format(form):
    """(codebook, double_quant) of a 4-bit weight form "int4-fp32", "fp4-dq", ...,
    or None for the NF4 entry points ("nf4") and the bf16 weight ("lora16")."""
    if form in ("nf4", "lora16"):
        return None
    cb, const = form.split("-")
    return cb, const == "dq"


def run_training(q, torch, steps, warmup, dev, key="llama7b", M=None, form="nf4"):
    """One step = fwd + bwd of the workload's seven linears.  The 33B workload
    runs the backward as under gradient checkpointing: T is not kept, the
    backward recomputes it (and dequantizes W again, as every backward does).
    form "lora16" runs the same step with bf16 base weights on the same
    kernels (the 16-bit LoRA comparator) instead of NF4 ones; "int4-fp32",
    "fp4-dq" (codebook - block constants) run it on the 4-bit codebook
    variants through the same kernels."""
    import numpy as np

    import workloads
    cfg = workloads.WORKLOADS[key]
    M, r, s = (cfg.M[0] if M is None else M), cfg.r, cfg.s
    recompute = key == "llama33b_recompute"
    dense = form == "lora16"
    q4 = q4_format(form)
    ws_fwd = (q.lib().qlora_lora16_fwd_workspace_bytes if dense
              else q.lib().qlora_linear_fwd_workspace_bytes)
    ws_bwd = (q.lib().qlora_lora16_bwd_workspace_bytes if dense
              else q.lib().qlora_linear_bwd_workspace_bytes)
    layers = []
    t0 = time.time()
    for lin, inp in workloads.workload_inputs(key, M=M):
        Wg = torch.from_numpy(inp.W).to(dev)
        if dense:
            w = Wg.to(torch.bfloat16)
        elif q4 is not None:
            w = q.qlora_q4_quantize(Wg, q4[0], q4[1])
        else:
            w = q.qlora_nf4_quantize(Wg)
        del Wg
        L = dict(lin=lin, w=w, X=bf16_dev(inp.X, dev), A=bf16_dev(inp.A, dev),
                 B=bf16_dev(inp.B, dev), dY=bf16_dev(inp.dY, dev))
        L["Y"] = torch.empty((M, lin.N), dtype=torch.bfloat16, device=dev)
        L["T"] = torch.empty((M, r), dtype=torch.float32, device=dev)
        L["dX"] = torch.empty((M, lin.K), dtype=torch.bfloat16, device=dev)
        L["dA"] = torch.empty((lin.K, r), dtype=torch.bfloat16, device=dev)
        L["dB"] = torch.empty((r, lin.N), dtype=torch.bfloat16, device=dev)
        L["wsf"] = torch.empty(ws_fwd(M, lin.N, lin.K, r), dtype=torch.uint8, device=dev)
        L["wsb"] = torch.empty(ws_bwd(M, lin.N, lin.K, r), dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()
    log(f"setup (draw + upload + {'convert' if dense else 'quantize'} {len(layers)} linears): "
        f"{time.time() - t0:.1f}s")
    fwd = (q.qlora_lora16_fwd if dense else q.qlora_q4_linear_fwd if q4 is not None
           else q.qlora_linear_fwd)
    bwd = (q.qlora_lora16_bwd if dense else q.qlora_q4_linear_bwd if q4 is not None
           else q.qlora_linear_bwd)

    def step():
        for L in layers:
            fwd(L["X"], L["w"], L["A"], L["B"], s, Y=L["Y"], T=L["T"], workspace=L["wsf"])
            bwd(L["dY"], L["X"], L["w"], L["A"], L["B"], s, T=None if recompute else L["T"],
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


def run_training_torch16(torch, steps, warmup, dev, M=None):
    """Context for the 16-bit LoRA comparator: the same LLaMA-7B layer step as
    plain bf16 torch matmuls (the vendor GEMM library), the way a framework's
    autograd runs a LoRA linear over a bf16 base weight:
      fwd  T = X A, Y = X W^T + s T B
      bwd  G = dY B^T, dX = dY W + s G A^T, dA = s X^T G, dB = s T^T dY
    (T and G in bf16, as autograd keeps them).  Timed by graph replay when the
    library's calls capture and replay to the eager result, else eagerly."""
    import torch.nn.functional as F

    import workloads
    cfg = workloads.WORKLOADS["llama7b"]
    M, r, s = (cfg.M[0] if M is None else M), cfg.r, cfg.s
    layers = []
    for lin, inp in workloads.workload_inputs("llama7b", M=M):
        layers.append(dict(lin=lin, W=torch.from_numpy(inp.W).to(dev).to(torch.bfloat16),
                           X=bf16_dev(inp.X, dev), A=bf16_dev(inp.A, dev),
                           B=bf16_dev(inp.B, dev), dY=bf16_dev(inp.dY, dev)))
    torch.cuda.synchronize()

    def step():
        outs = []
        for L in layers:
            X, W, A, B, dY = L["X"], L["W"], L["A"], L["B"], L["dY"]
            T = torch.matmul(X, A)
            Y = torch.addmm(F.linear(X, W), T, B, alpha=s)
            G = F.linear(dY, B)
            dX = torch.addmm(torch.matmul(dY, W), G, A.t(), alpha=s)
            dA = torch.matmul(X.t(), G).mul_(s)
            dB = torch.matmul(T.t(), dY).mul_(s)
            outs.append((Y, dX, dA, dB))
        return outs

    for _ in range(warmup):
        step()
    ref = step()
    torch.cuda.synchronize()
    mode = "graph replay"
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            got = step()
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            for a, b in zip(ref, got):
                for x, y in zip(a, b):
                    if not torch.equal(x, y):
                        raise RuntimeError("replay differs from the eager step")
        run = graph.replay
    except Exception as e:   # the eager step is the comparator then
        log(f"torch 16-bit LoRA step: no graph ({e}); timing it eagerly")
        mode, graph, run = "eager", None, step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    ms = evs[0].elapsed_time(evs[-1]) / steps
    del graph
    flops = sum(linear_flops(M, L["lin"].N, L["lin"].K, r) for L in layers)
    return dict(ms_per_step=ms, tflops=flops / (ms * 1e-3) / 1e12, timing=mode,
                step_ms_p10_p50_p90=percentiles(per_step), tokens=M,
                what="bf16 torch matmuls (F.linear / addmm / matmul), T and G in bf16")


def run_training_fused(q, torch, steps, warmup, dev, M=None):
    """The LLaMA-7B layer's seven linears as a transformer layer runs them:
    q, k, v read one input and run as one fused block (S = 3, 4096 rows
    each), o alone, gate and up as one block (S = 2, 11008 rows each), down
    alone.  The weights, adapters and output gradients are the per-linear
    workload's; the blocks take q's and gate's input.  Same flops as the
    per-linear step (the input gradient of a block is the sum of its
    projections')."""
    import numpy as np

    import workloads
    cfg = workloads.WORKLOADS["llama7b"]
    M, r, s = (cfg.M[0] if M is None else M), cfg.r, cfg.s
    ins = list(workloads.workload_inputs("llama7b", M=M))
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    units = []
    for g in groups:
        lins = [ins[i][0] for i in g]
        W = np.concatenate([ins[i][1].W for i in g], axis=0)
        A = np.concatenate([ins[i][1].A for i in g], axis=1)
        B = np.concatenate([ins[i][1].B for i in g], axis=1)
        dY = np.concatenate([ins[i][1].dY for i in g], axis=1)
        S = len(g)
        u = dict(S=S, lins=lins, w=q.qlora_nf4_quantize(torch.from_numpy(W).to(dev)),
                 X=bf16_dev(ins[g[0]][1].X, dev), A=bf16_dev(np.ascontiguousarray(A), dev),
                 B=bf16_dev(np.ascontiguousarray(B), dev), dY=bf16_dev(np.ascontiguousarray(dY), dev))
        N, K = W.shape
        u["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        u["T"] = torch.empty((M, S * r), dtype=torch.float32, device=dev)
        u["dX"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        u["dA"] = torch.empty((K, S * r), dtype=torch.bfloat16, device=dev)
        u["dB"] = torch.empty((r, N), dtype=torch.bfloat16, device=dev)
        if S > 1:
            u["wsf"] = torch.empty(q.lib().qlora_block_fwd_workspace_bytes(M, S, N // S, K, r),
                                   dtype=torch.uint8, device=dev)
            u["wsb"] = torch.empty(q.lib().qlora_block_bwd_workspace_bytes(M, S, N // S, K, r),
                                   dtype=torch.uint8, device=dev)
        else:
            u["wsf"] = torch.empty(q.lib().qlora_linear_fwd_workspace_bytes(M, N, K, r),
                                   dtype=torch.uint8, device=dev)
            u["wsb"] = torch.empty(q.lib().qlora_linear_bwd_workspace_bytes(M, N, K, r),
                                   dtype=torch.uint8, device=dev)
        units.append(u)
    del ins
    torch.cuda.synchronize()

    def step():
        for u in units:
            if u["S"] > 1:
                q.qlora_block_fwd(u["X"], u["w"], u["S"], u["A"], u["B"], s, Y=u["Y"], T=u["T"],
                                  workspace=u["wsf"])
                q.qlora_block_bwd(u["dY"], u["X"], u["w"], u["S"], u["A"], u["B"], s, T=u["T"],
                                  dX=u["dX"], dA=u["dA"], dB=u["dB"], workspace=u["wsb"])
            else:
                q.qlora_linear_fwd(u["X"], u["w"], u["A"], u["B"], s, Y=u["Y"], T=u["T"],
                                   workspace=u["wsf"])
                q.qlora_linear_bwd(u["dY"], u["X"], u["w"], u["A"], u["B"], s, T=u["T"],
                                   dX=u["dX"], dA=u["dA"], dB=u["dB"], workspace=u["wsb"])

    for _ in range(warmup):
        step()
    step()
    torch.cuda.synchronize()
    outs = ("Y", "T", "dX", "dA", "dB")
    eager = [[u[k].clone() for k in outs] for u in units]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    for u, ref in zip(units, eager):
        for k, t in zip(outs, ref):
            if not torch.equal(u[k], t):
                raise RuntimeError(f"fused step: graph replay differs from the eager step ({k})")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    ms = evs[0].elapsed_time(evs[-1]) / steps
    del graph
    flops = sum(linear_flops(M, l.N, l.K, r) for u in units for l in u["lins"])
    return dict(ms_per_step=ms, tflops=flops / (ms * 1e-3) / 1e12,
                step_ms_p10_p50_p90=percentiles(per_step), tokens=M,
                blocks="q/k/v fused (S=3), o, gate/up fused (S=2), down")


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


def run_decode(q, torch, dev, reps=20, pool_bytes=1.1e9, form="nf4", Ms=None, shapes=None):
    """Decode GB/s on the 65B shapes, rotating over >1 GB of weight copies.

    The rate is device time per call: one pass over the pool is captured as
    a graph (the calls allocate nothing and record no memsets) and replayed;
    the eager per-call time, host launch path included, is reported too.
    form: "nf4", or a 4-bit codebook variant ("int4-fp32", "fp4-dq", ...)
    whose weight bytes (codes and block constants) are counted as such.
    Ms and shapes ("NxK" strings) restrict the sweep, e.g. to tell one
    shape's counters apart from another's with the same kernel and grid."""
    import workloads
    cfg = workloads.WORKLOADS["decode_65b"]
    r, s = cfg.r, cfg.s
    q4 = q4_format(form)
    fwd_call = q.qlora_q4_linear_fwd if q4 is not None else q.qlora_linear_fwd
    g = torch.Generator(device=dev)
    g.manual_seed(2000)
    out = {}
    for M in (cfg.M if Ms is None else Ms):
        tot_bytes, tot_ms, kern_bytes, kern_ms = 0.0, 0.0, 0.0, 0.0
        per_shape = {}
        for lin in cfg.linears:
            N, K = lin.N, lin.K
            if shapes is not None and f"{N}x{K}" not in shapes:
                continue
            if q4 is not None and not q4[1]:   # one fp32 constant per block
                nf4_bytes = N * K // 2 + 4 * (N * K // 64)
            else:
                nf4_bytes = N * K // 2 + N * K // 64 + 4 * ((N * K // 64 + 255) // 256)
            copies = max(2, int(pool_bytes // nf4_bytes) + 1)
            pool = []
            for _ in range(copies):
                W = torch.randn((N, K), generator=g, device=dev) * 0.02
                W = torch.where(torch.rand((N, K), generator=g, device=dev) < 0.001, W * 10, W)
                pool.append(q.qlora_q4_quantize(W, q4[0], q4[1]) if q4 is not None
                            else q.qlora_nf4_quantize(W))
                del W
            X = (torch.randn((M, K), generator=g, device=dev)).to(torch.bfloat16)
            A = (torch.randn((K, r), generator=g, device=dev) / r).to(torch.bfloat16)
            B = (torch.randn((r, N), generator=g, device=dev) * 0.01).to(torch.bfloat16)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            T = torch.empty((M, r), dtype=torch.float32, device=dev)
            ws = torch.empty(q.lib().qlora_linear_fwd_workspace_bytes(M, N, K, r),
                             dtype=torch.uint8, device=dev)
            for w in pool[:2]:
                fwd_call(X, w, A, B, s, Y=Y, T=T, workspace=ws)
            torch.cuda.synchronize()
            # eager per-call rate (includes the Python launch path)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for w in pool:
                fwd_call(X, w, A, B, s, Y=Y, T=T, workspace=ws)
            ev1.record()
            torch.cuda.synchronize()
            ms_eager = ev0.elapsed_time(ev1) / len(pool)
            # device rate: one pass over the pool captured as a graph and
            # replayed, so host launch overhead is not on the clock
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for w in pool:
                    fwd_call(X, w, A, B, s, Y=Y, T=T, workspace=ws)
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
            fwd_call(X, pool[-1], A, B, s, Y=Y, T=T, workspace=ws)
            torch.cuda.synchronize()
            if not torch.equal(Y_graph, Y):
                raise RuntimeError(f"decode {N}x{K} M={M}: graph replay differs from eager call")
            del graph
            # decode-kernel time alone: a second pass with the launch profiler on
            q.qlora_profile_reset()
            q.qlora_profile_enable(True)
            for _ in range(max(1, reps // 4)):
                for w in pool:
                    fwd_call(X, w, A, B, s, Y=Y, T=T, workspace=ws)
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
        if not per_shape:
            continue
        out[f"M={M}"] = dict(gbs_call=tot_bytes / (tot_ms * 1e-3) / 1e9,
                             gbs_decode_kernel=kern_bytes / (kern_ms * 1e-3) / 1e9,
                             shapes=per_shape)
        log(f"decode {form} M={M}: {out[f'M={M}']['gbs_call']:.0f} GB/s per call, "
            f"{out[f'M={M}']['gbs_decode_kernel']:.0f} GB/s decode kernel")
    return out


def run_adamw(q, torch, dev, reps=20, M=2048):
    """The adapters' AdamW step over the LLaMA-7B layer's seven adapters (A
    and B of q, k, v, o, gate, up, down at r = 64: one flat buffer), with the
    fp32 moments resident in HBM and paged out to pinned host memory; and the
    page-out / page-in times.  22 bytes move per parameter (bf16 p read and
    written, bf16 g read, fp32 m and v read and written)."""
    import workloads
    cfg = workloads.WORKLOADS["llama7b"]
    n = sum(l.K * cfg.r + cfg.r * l.N for l in cfg.linears)
    P = (torch.randn(n, device=dev) * 0.02).to(torch.bfloat16)
    G = (torch.randn(n, device=dev) * 1e-3).to(torch.bfloat16)
    st = q.PagedState(n)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(k0):
        st.step(P, G, k0)   # warm
        torch.cuda.synchronize()
        ev[0].record()
        for k in range(reps):
            st.step(P, G, k0 + 1 + k)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    ms_dev = timed(1)
    t0 = time.perf_counter()
    st.page_out()
    ms_out = (time.perf_counter() - t0) * 1e3
    ms_host = timed(100)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st.page_in()
    torch.cuda.synchronize()
    ms_in = (time.perf_counter() - t0) * 1e3
    st.close()
    bytes_step = 22 * n
    return dict(params=n, bytes_per_step=bytes_step,
                resident_us=1e3 * ms_dev, resident_gbs=bytes_step / (ms_dev * 1e-3) / 1e9,
                paged_out_us=1e3 * ms_host,
                paged_out_link_gbs=16 * n / (ms_host * 1e-3) / 1e9,
                page_out_ms=ms_out, page_in_ms=ms_in, state_mb=8 * n / 1e6,
                note="moments paged out: the kernel reads and writes them in pinned host memory "
                     "(16 of the 22 bytes per parameter cross the host link)")


def run_peaks(q, torch, dev):
    """Rates this GPU reaches on a plain 4 GiB streaming read and on a loop of
    independent bf16 32x32x16 MFMAs (the library's probe kernels), best of
    a few launch sizes, each timed with HIP events over 5 launches."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_gbs = 0.0
    for wg in (1024, 2048, 4096, 8192):
        q.qlora_probe_hbm_read(buf, wg, sink)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(5):
            q.qlora_probe_hbm_read(buf, wg, sink)
        ev1.record()
        torch.cuda.synchronize()
        best_gbs = max(best_gbs, 5 * nbytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9)
    del buf
    best_tf = 0.0
    for wg in (1024, 2048):
        q.qlora_probe_mfma_bf16(100, wg, sink)
        torch.cuda.synchronize()
        ev0.record()
        flops = sum(q.qlora_probe_mfma_bf16(4000, wg, sink) for _ in range(3))
        ev1.record()
        torch.cuda.synchronize()
        best_tf = max(best_tf, flops / (ev0.elapsed_time(ev1) * 1e-3) / 1e12)
    torch.cuda.empty_cache()
    return dict(hbm_read_gbs=best_gbs, mfma_bf16_tflops=best_tf,
                note="4 GiB non-temporal 16-byte streaming read; independent "
                     "v_mfma_f32_32x32x16_bf16 on register operands; best of several grid sizes")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(train, repeats=2):
    """The oracle (plain NumPy: dequantize, then float64 products) timed on a
    bounded sample of each workload on this host's cores.  The value is the
    headline workload's: all seven LLaMA-7B linears at M = 2048 (one
    training step, `repeats` times; load-time quantization untimed).  Also
    timed: the 1024 x 1024 parity linear in full (quantize, dequantize, fwd,
    bwd), one M = 1 forward of the 8192 x 8192 decode shape and one linear
    (q, 6656 x 6656, M = 4096) of the 33B layer with the recompute backward;
    for the last two the codes are drawn at random (the time does not depend
    on their values) instead of quantized."""
    import numpy as np

    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(cores) if threadpool_limits else None
    extra = {}
    try:
        cfg = workloads.WORKLOADS["llama7b"]
        flops, secs = 0, 0.0
        for idx in range(len(cfg.linears)):
            (lin, inp), = list(workloads.workload_inputs("llama7b", linears=[idx]))
            codes, e, d, _ = oracle.quantize(inp.W)       # load-time, untimed
            for _ in range(repeats):
                t0 = time.perf_counter()
                What = oracle.dequantize(codes, e, d, lin.N, lin.K)
                oracle.linear_fwd(inp.X, What, inp.A, inp.B, cfg.s)
                oracle.linear_bwd(inp.dY, inp.X, What, inp.A, inp.B, cfg.s)
                secs += time.perf_counter() - t0
                flops += linear_flops(cfg.M[0], lin.N, lin.K, cfg.r)
        # the parity linear, everything timed
        c0 = workloads.WORKLOADS["parity_1k"]
        (lin, inp), = list(workloads.workload_inputs("parity_1k"))
        t0 = time.perf_counter()
        codes, e, d, _ = oracle.quantize(inp.W)
        What = oracle.dequantize(codes, e, d, lin.N, lin.K)
        oracle.linear_fwd(inp.X, What, inp.A, inp.B, c0.s)
        oracle.linear_bwd(inp.dY, inp.X, What, inp.A, inp.B, c0.s)
        dt = time.perf_counter() - t0
        extra["parity_1k"] = dict(seconds=dt, sample="quantize + dequantize + fwd + bwd, "
                                  "1024x1024, M=16, r=16")
        rng = np.random.default_rng(99)

        def random_weight(N, K):
            codes = rng.integers(0, 256, N * K // 2, dtype=np.uint8)
            e = rng.integers(0, 256, N * K // 64, dtype=np.uint8)
            d = (rng.random((N * K // 64 + 255) // 256, dtype=np.float32) * 1e-3).astype(np.float32)
            return codes, e, d

        # one decode call (M = 1) on the 8192 x 8192 shape: bytes per second
        N = K = 8192
        r = 64
        codes, e, d = random_weight(N, K)
        X = workloads.to_bf16_bits(rng.standard_normal((1, K), dtype=np.float32))
        A = workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) / r)
        B = workloads.to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * 0.01)
        t0 = time.perf_counter()
        What = oracle.dequantize(codes, e, d, N, K)
        oracle.linear_fwd(X, What, A, B, 0.25)
        dt = time.perf_counter() - t0
        alg = N * K // 2 + N * K // 64 + 4 * (N * K // 64 // 256) + 2 * (K + N + K * r + r * N)
        extra["decode_65b_m1"] = dict(seconds=dt, value=alg / dt / 1e9, unit="GB/s",
                                      sample="one M=1 forward of 8192x8192, r=64: oracle "
                                             "dequantize + fwd")
        # one linear of the 33B layer, recompute backward
        cfg3 = workloads.WORKLOADS["llama33b_recompute"]
        N = K = 6656
        M = cfg3.M[0]
        codes, e, d = random_weight(N, K)
        X = workloads.to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        dY = workloads.to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
        A = workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) / r)
        B = workloads.to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * 0.01)
        t0 = time.perf_counter()
        What = oracle.dequantize(codes, e, d, N, K)
        oracle.linear_fwd(X, What, A, B, cfg3.s)
        What = oracle.dequantize(codes, e, d, N, K)   # the backward dequantizes again
        oracle.linear_bwd(dY, X, What, A, B, cfg3.s)
        dt = time.perf_counter() - t0
        extra["llama33b_recompute_q"] = dict(
            seconds=dt, value=linear_flops(M, N, K, r) / dt / 1e12, unit="TFLOP/s",
            sample="one linear (6656x6656, M=4096, r=64): dequantize + fwd + dequantize + bwd")
        threads = cores
        if threadpool_info:
            nums = [p.get("num_threads", 0) for p in threadpool_info()
                    if p.get("user_api") == "blas"]
            threads = max(nums) if nums else cores
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return dict(value=flops / secs / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                seconds=secs, cpu_model=cpu_model(),
                sample=f"{repeats} steps: all seven LLaMA-7B linears, M=2048, r=64: oracle "
                       "dequantize + fwd + bwd (float64 products); load-time quantization untimed",
                other_workloads=extra)


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
    if by_grid:
        # durations per kernel and grid size (tells the shapes of one kernel apart)
        for path in _rocprof_csvs(root, "kernel_trace.csv"):
            agg = {}
            for r in csv.DictReader(open(path)):
                grid = r.get("Grid_Size") or "x".join(
                    r.get(f"Grid_Size_{a}", "?") for a in ("X", "Y", "Z"))
                key = f"{r['Kernel_Name'].split('(')[0][:52]} grid={grid}"
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                agg.setdefault(key, []).append(dur)
            lines.append(f"{'kernel (per grid size)':70s} {'calls':>6s} {'avg_us':>9s} "
                         f"{'median_us':>9s} {'min_us':>9s} {'max_us':>9s}")
            for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:3 * top]:
                v = sorted(v)
                lines.append(f"{k[:70]:70s} {len(v):6d} {sum(v) / len(v):9.2f} "
                             f"{v[len(v) // 2]:9.2f} {v[0]:9.2f} {v[-1]:9.2f}")
    traffic = {}
    for path in _rocprof_csvs(root, "counter_collection.csv"):
        agg = {}
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if by_grid:   # (the calibration copy keeps its name's "neg" in front)
                tag = "neg_kernel " if "neg_kernel" in name else ""
                grid = r.get("Grid_Size") or "x".join(
                    r.get(f"Grid_Size_{a}", "?") for a in ("X", "Y", "Z"))
                name = f"{(tag + name.split('(')[0])[:52]} grid={grid}"
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


def _int_list(text):
    """"1,16" -> [1, 16]: token counts of the decode path (1 <= M <= 16)."""
    vals = [int(v) for v in text.split(",") if v.strip()]
    if not vals or any(not 1 <= v <= 16 for v in vals):
        raise argparse.ArgumentTypeError(f"token counts between 1 and 16 expected, got {text!r}")
    return vals


def _shape_list(text):
    """"8192x8192,22016x8192" -> the same names, checked against the decode sweep's shapes."""
    import workloads
    known = tuple(f"{lin.N}x{lin.K}" for lin in workloads.WORKLOADS["decode_65b"].linears)
    vals = [v.strip() for v in text.split(",") if v.strip()]
    if not vals or any(v not in known for v in vals):
        raise argparse.ArgumentTypeError(f"shapes among {', '.join(known)} expected, got {text!r}")
    return vals


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak probes (4 GiB streaming read, bf16 MFMA loop)")
    ap.add_argument("--no-adamw", action="store_true",
                    help="skip the adapters' AdamW step (resident and paged-out moments)")
    ap.add_argument("--no-lora16", action="store_true",
                    help="skip the 16-bit LoRA comparator steps (bf16 base weight)")
    ap.add_argument("--no-codebooks", action="store_true",
                    help="skip the INT4 / FP4 / fp32-constant variants (step and M=1 decode)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the extra step with q/k/v and gate/up run as fused blocks")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the extra step at one GPU's share of 8-way data parallelism "
                         "(256 of the 2048 tokens)")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode leg (65B shapes, M in {1, 4, 16}) and print its "
                         "numbers (for profiling it on its own)")
    ap.add_argument("--decode-reps", type=int, default=20,
                    help="graph replays per shape in the decode leg")
    ap.add_argument("--decode-m", type=_int_list, default=None, metavar="M[,M...]",
                    help="with --decode-only: only these token counts (of 1, 4, 16)")
    ap.add_argument("--decode-shapes", type=_shape_list, default=None, metavar="NxK[,NxK...]",
                    help="with --decode-only: only these weight shapes (of 8192x8192, "
                         "22016x8192, 8192x22016)")
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
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 run (each with --copy-calibration-mib) and exit")
    args = ap.parse_args()
    if (args.decode_m or args.decode_shapes) and not args.decode_only:
        ap.error("--decode-m and --decode-shapes go with --decode-only")
    if args.write_traffic:
        if not args.copy_calibration_mib:
            raise SystemExit("--write-traffic needs --copy-calibration-mib (the size the runs used)")
        out = write_traffic(*args.write_traffic, args.copy_calibration_mib,
                            "profiles/train_step_traffic.md")
        print(json.dumps(out, indent=1))
        return
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
        dec = run_decode(q, torch, dev, reps=args.decode_reps, Ms=args.decode_m,
                         shapes=args.decode_shapes)
        first = "M=1" if "M=1" in dec else next(iter(dec))
        print(json.dumps({"metric": f"QLoRA decode ({first}) effective HBM GB/s, 65B shapes",
                          "value": dec[first]["gbs_call"], "unit": "GB/s", "n_gpus": 1,
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
    src_hash = kernel_source_hash(kern)
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

    fused = None
    if args.workload == "llama7b" and not args.no_fused:
        fused = run_training_fused(q, torch, args.steps, args.warmup, dev)
        log(f"fused-block step (q/k/v and gate/up as blocks): {fused['ms_per_step']:.3f} ms, "
            f"{fused['tflops']:.1f} TFLOP/s")

    lora16 = torch16 = None
    if args.workload == "llama7b" and not args.no_lora16:
        l16 = run_training(q, torch, args.steps, args.warmup, dev, key="llama7b", form="lora16")
        lora16 = dict(ms_per_step=l16["ms_step"],
                      tflops=l16["flops_step"] / (l16["ms_step"] * 1e-3) / 1e12,
                      step_ms_p10_p50_p90=l16["step_ms_pct"],
                      kernels={k: dict(ms_per_step=ms / args.steps,
                                       avg_launch_us=1e3 * ms / n)
                               for k, (ms, n) in l16["fam"].items() if n},
                      nf4_over_lora16_time=tr["ms_step"] / l16["ms_step"],
                      what="the same step with bf16 base weights on the same kernels "
                           "(weight tile loaded instead of dequantized)")
        log(f"16-bit LoRA step (same kernels, bf16 W): {l16['ms_step']:.3f} ms, "
            f"{lora16['tflops']:.1f} TFLOP/s; NF4/bf16 time {lora16['nf4_over_lora16_time']:.3f}; "
            f"kernels {lora16['kernels']}")
        del l16
        torch16 = run_training_torch16(torch, args.steps, args.warmup, dev)
        log(f"16-bit LoRA step as torch bf16 matmuls: {torch16['ms_per_step']:.3f} ms "
            f"({torch16['timing']}), {torch16['tflops']:.1f} TFLOP/s")

    variants = None
    if args.workload == "llama7b" and not args.no_codebooks:
        # the codebook / constant variants through the same kernels: the
        # training step and the M = 1 decode (weight bytes counted per format)
        variants = {}
        for form in ("int4-fp32", "fp4-dq"):
            v = run_training(q, torch, args.steps, args.warmup, dev, key="llama7b", form=form)
            vd = dict(ms_per_step=v["ms_step"],
                      tflops=v["flops_step"] / (v["ms_step"] * 1e-3) / 1e12,
                      time_over_nf4=v["ms_step"] / tr["ms_step"])
            del v
            if not args.no_decode:
                dm = run_decode(q, torch, dev, reps=args.decode_reps, form=form, Ms=[1])["M=1"]
                vd["decode_m1"] = dict(gbs_call=dm["gbs_call"],
                                       gbs_decode_kernel=dm["gbs_decode_kernel"],
                                       us_per_call={k: x["us_per_call"]
                                                    for k, x in dm["shapes"].items()})
            variants[form] = vd
            log(f"{form}: step {vd['ms_per_step']:.3f} ms ({vd['tflops']:.1f} TFLOP/s, "
                f"{vd['time_over_nf4']:.3f} of the NF4 time)"
                + (f"; decode M=1 {vd['decode_m1']['gbs_call']:.0f} GB/s per call"
                   if "decode_m1" in vd else ""))

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

    opt = None
    if args.workload == "llama7b" and not args.no_adamw:
        opt = run_adamw(q, torch, dev)
        log(f"adamw over {opt['params'] / 1e6:.2f} M adapter parameters: resident "
            f"{opt['resident_us']:.1f} us ({opt['resident_gbs']:.0f} GB/s), paged out "
            f"{opt['paged_out_us']:.1f} us ({opt['paged_out_link_gbs']:.1f} GB/s over the link); "
            f"page-out {opt['page_out_ms']:.2f} ms, page-in {opt['page_in_ms']:.2f} ms")

    peaks = None
    if not args.no_peaks:
        peaks = run_peaks(q, torch, dev)
        log(f"measured peaks: {peaks['hbm_read_gbs']:.0f} GB/s streaming read, "
            f"{peaks['mfma_bf16_tflops']:.0f} TFLOP/s bf16 MFMA")
        roofline["measured_peak"] = peaks["mfma_bf16_tflops"]
        roofline["frac_of_measured_peak"] = roofline["achieved"] / peaks["mfma_bf16_tflops"]
        if decode is not None:
            for mk, dv in decode.items():
                dv["frac_hbm_vendor"] = dv["gbs_call"] / PEAK_HBM_GBS
                dv["frac_hbm_measured"] = dv["gbs_call"] / peaks["hbm_read_gbs"]
        if opt is not None:
            opt["frac_hbm_vendor"] = opt["resident_gbs"] / PEAK_HBM_GBS
            opt["frac_hbm_measured"] = opt["resident_gbs"] / peaks["hbm_read_gbs"]

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
        "measured_peaks": peaks,
        "decode_m1_gbs": None if decode is None else decode["M=1"]["gbs_call"],
        "fused_block_step": fused,
        "lora16_step": lora16,
        "adamw": opt,
        "torch_lora16_step": torch16,
        "codebook_variants": variants,
        "dp8_shard": shard,
        "decode": decode,
        "kernels": kernels,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
