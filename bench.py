#!/usr/bin/env python3
"""MoE-layer decode throughput on one MI355X.

Workload (default): one full-width q4 MoE layer -- d_model 2816, 128 routed
experts (all resident in HBM), top-8, expert FFN 704, shared expert FFN 2816,
MLX-style affine 4-bit weights (group 64) and an 8-bit router -- decoding
10,000 seeded tokens x ~ N(0,1) one token per step.  A step is the whole hot
path for one token: router + top-8 + softmax, shared expert, the 8 routed
experts' gate/up/down, combine, fp16 output.

Prints one JSON line: tokens/s over the timed steps (inputs already resident
in HBM, steps replayed from HIP graphs), the dominant kernel's roofline
(algorithmic bytes per launch / its average duration from hipExtLaunchKernel
start/stop events), and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer decode tokens/s + achieved HBM GB/s (% of peak), 1×MI355X"


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def _event(h):
    e = ctypes.c_void_p()
    assert h.hipEventCreate(ctypes.byref(e)) == 0
    return e


def qmat_bytes(n, k, bits=4):
    return n * k * bits // 8 + 2 * n * (k // 64) * 2


def stage_b_bytes(d, f, fs, k, T=1):
    """Algorithmic bytes of one routed-gate/up + shared-down launch (T tokens,
    every token's experts distinct): weights + x in, h_s in, h_r and y_s out."""
    w = k * T * 2 * qmat_bytes(f, d) + qmat_bytes(d, fs)
    return w + T * d * 2 + T * fs * 4 + T * k * f * 4 + T * d * 4


def layer_bytes(d, f, fs, E, k):
    """Bytes one decode token must move: the 8-bit router, the shared expert,
    k routed experts (q4 codes + fp16 scale/bias), plus x in and y out."""
    router = qmat_bytes(E, d, 8)
    shared = 2 * qmat_bytes(fs, d) + qmat_bytes(d, fs)
    routed = k * (2 * qmat_bytes(f, d) + qmat_bytes(d, f))
    return router + shared + routed + 2 * d + 2 * d


def _traffic_for(kernel_name, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    from bit_routed_expert_tf_amd import profiling
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[kernel_name]
    except (KeyError, ValueError):
        return None
    if (rec.get("source_sha256") != profiling.source_sha256(rec.get("kernel", ""))
            or rec.get("workload") != workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(nbytes=256 << 20, reps=3):
    """Plain device-to-device copies of a known size, for scaling the memory
    counters (rocprofv3 FETCH_SIZE / WRITE_SIZE) of the same run."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def run_decode(args):
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen

    wl = gen.WORKLOADS[1]
    d, E, k, f, fs = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared
    n_tok = wl.n_tokens
    lib = _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    router = gen.router(wl.seed, 0, d, E)
    shared_blob = gen.shared_blob(wl.seed, 0, d, fs)
    pool = gen.expert_pool(wl.seed, 0, d, f, E)
    X = gen.tokens(wl.seed, n_tok, d)
    D = api.DeviceLayer.from_arrays(router, shared_blob, pool, d, f, fs, k, device=dev)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    Y = torch.empty((n_tok, d), dtype=torch.int16, device=dev)
    IDS = torch.empty((n_tok, k), dtype=torch.int32, device=dev)
    W = torch.empty((n_tok, k), dtype=torch.float32, device=dev)
    ws = api.workspace(api.tf_moe_workspace_bytes(D, 1), dev)
    setup_s = time.time() - t0

    stream = torch.cuda.Stream(device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    Lp = ctypes.byref(D.struct)
    xp, yp, ip, wp = Xd.data_ptr(), Y.data_ptr(), IDS.data_ptr(), W.data_ptr()
    wsp, wsn = ctypes.c_void_p(ws.data_ptr()), ws.numel()

    def step(i):
        rc = lib.tf_moe_layer_fwd(Lp, ctypes.c_void_p(xp + 2 * d * i), 1, None,
                                  ctypes.c_void_p(yp + 2 * d * i), None,
                                  ctypes.c_void_p(ip + 4 * k * i), ctypes.c_void_p(wp + 4 * k * i),
                                  None, 0, sh, sh, wsp, wsn)
        if rc:
            raise RuntimeError(lib.tf_last_error().decode())

    with torch.cuda.stream(stream):
        for i in range(8):
            step(i)
    torch.cuda.synchronize()

    chunk = args.graph_chunk
    n_graphs = (n_tok + chunk - 1) // chunk
    graphs = []
    for j in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(j * chunk, min(n_tok, (j + 1) * chunk)):
                step(i)
        graphs.append(g)
    torch.cuda.synchronize()

    def run_steps(nsteps):
        done, j = 0, 0
        with torch.cuda.stream(stream):
            while done < nsteps:
                graphs[j % n_graphs].replay()
                done += min(chunk, n_tok - (j % n_graphs) * chunk)
                j += 1
        return done

    run_steps(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    steps = run_steps(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1)
    tok_s = steps / (ms / 1e3)

    # Per-kernel durations: eager steps whose kernels are launched through
    # hipExtLaunchKernel with start/stop events on the compute stream.
    h = _hip()
    kern = {}
    names = {_lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "router_shared_gateup",
             _lib.TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN: "routed_gateup_shared_down",
             _lib.TF_KERNEL_DOWN_COMBINE: "down_combine"}
    nprof = args.prof_steps
    for kid, name in names.items():
        evs = [(_event(h), _event(h)) for _ in range(nprof)]
        with torch.cuda.stream(stream):
            for i in range(nprof):
                _lib.check(lib.tf_profile_kernel(kid, evs[i][0], evs[i][1]))
                step((i * 37) % n_tok)
        torch.cuda.synchronize()
        durs = []
        for a, b in evs:
            v = ctypes.c_float()
            h.hipEventElapsedTime(ctypes.byref(v), a, b)
            durs.append(v.value * 1e3)
            h.hipEventDestroy(a)
            h.hipEventDestroy(b)
        durs.sort()
        kern[name] = {"avg_us": sum(durs) / len(durs), "median_us": durs[len(durs) // 2],
                      "min_us": durs[0], "launches": len(durs)}

    bytes_b = stage_b_bytes(d, f, fs, k)
    dur_b = kern["routed_gateup_shared_down"]["avg_us"] * 1e-6
    achieved = bytes_b / dur_b / 1e9
    lb = layer_bytes(d, f, fs, E, k)
    traffic = _traffic_for("routed_gateup_shared_down", wl.name)

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms / steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded; random-init q4 weights of the stated shapes)",
        "config": {"workload": wl.name, "d_model": d, "n_experts": E, "top_k": k, "d_ff": f,
                   "d_ff_shared": fs, "tokens": n_tok, "tokens_per_step": 1,
                   "weights": "affine q4 group 64 (fp16 scale/bias), 8-bit router",
                   "io": "fp16 x/y, fp32 accumulate, fp64 router sums",
                   "experts_resident": "all 128 in HBM", "graph_chunk": chunk},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "routed_gateup_shared_down",
                     "algorithmic_bytes_per_launch": bytes_b,
                     "avg_duration_us": round(dur_b * 1e6, 3)},
        "layer": {"bytes_per_token": lb, "GBps": round(lb * tok_s / 1e9, 1),
                  "frac_of_hbm_peak": round(lb * tok_s / 1e9 / HBM_PEAK_GBPS, 4),
                  "wall_s": round(wall, 4), "setup_s": round(setup_s, 1)},
        "kernels": {n: {kk: round(v, 3) if isinstance(v, float) else v for kk, v in r.items()}
                    for n, r in kern.items()},
        "device": torch.cuda.get_device_name(dev),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, router, shared_blob, pool, X, wl)
    return out


def cpu_baseline(args, router, shared_blob, pool, X, wl):
    """The fp64 oracle, as it stands, on the host cores over a bounded sample
    of the same tokens."""
    import oracle
    L = {"router": router, "shared_blob": shared_blob, "pool": pool, "d_model": wl.d_model,
         "d_ff": wl.d_ff, "d_ff_shared": wl.d_ff_shared, "top_k": wl.top_k}
    oracle.moe_token(L, X[0])             # load / first-touch
    n, t0 = 0, time.perf_counter()
    while n < 8 or (time.perf_counter() - t0 < args.cpu_seconds and n < wl.n_tokens):
        oracle.moe_token(L, X[n])
        n += 1
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    # the same oracle on one core, over a shorter sample
    oracle.set_num_threads(1)
    n1, t1 = 0, time.perf_counter()
    while n1 < 2 or (time.perf_counter() - t1 < args.cpu_seconds / 4 and n1 < wl.n_tokens):
        oracle.moe_token(L, X[n1])
        n1 += 1
    dt1 = time.perf_counter() - t1
    oracle.set_num_threads(cores)
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} of the {wl.n_tokens} workload tokens, one at a time "
                      f"({dt:.1f} s, C fp64 oracle, OpenMP over rows)",
            "one_core": {"value": round(n1 / dt1, 3), "unit": "tokens/s", "cores": 1,
                         "sample": f"first {n1} tokens ({dt1:.1f} s)"}}


def _profile(lib, h, kernels, step, nprof, stream):
    """Average durations of the named kernels (hipExtLaunchKernel start/stop
    events on the compute stream) over nprof eager calls of step(i)."""
    import torch

    from bit_routed_expert_tf_amd import _lib
    out = {}
    for kid, name in kernels.items():
        evs = [(_event(h), _event(h)) for _ in range(nprof)]
        with torch.cuda.stream(stream):
            for i in range(nprof):
                _lib.check(lib.tf_profile_kernel(kid, evs[i][0], evs[i][1]))
                step(i)
        torch.cuda.synchronize()
        durs = []
        for a, b in evs:
            v = ctypes.c_float()
            h.hipEventElapsedTime(ctypes.byref(v), a, b)
            durs.append(v.value * 1e3)
            h.hipEventDestroy(a)
            h.hipEventDestroy(b)
        durs.sort()
        out[name] = {"avg_us": round(sum(durs) / len(durs), 3),
                     "median_us": round(durs[len(durs) // 2], 3), "min_us": round(durs[0], 3),
                     "launches": len(durs)}
    return out


def _graphs(step, n, chunk, stream):
    """HIP graphs of `chunk` consecutive steps each, covering steps 0..n-1."""
    import torch
    graphs = []
    for j in range(0, n, chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(j, min(n, j + chunk)):
                step(i)
        graphs.append((g, min(n, j + chunk) - j))
    torch.cuda.synchronize()
    return graphs


def _replay(graphs, nsteps, stream):
    import torch
    done, j = 0, 0
    with torch.cuda.stream(stream):
        while done < nsteps:
            g, c = graphs[j % len(graphs)]
            g.replay()
            done += c
            j += 1
    return done


def _timed(graphs, nsteps, warmup, stream):
    import torch
    _replay(graphs, warmup, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    steps = _replay(graphs, nsteps, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return steps, e0.elapsed_time(e1)


def run_prefill(args):
    """128-token chunks through one full-width layer (natural routing)."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen
    wl = gen.WORKLOADS[3]
    d, E, k, f, fs, C = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared, wl.chunk
    nch = wl.n_tokens // C
    lib = _lib.load()
    dev = torch.device("cuda:0")
    router = gen.router(wl.seed, 0, d, E)
    D = api.DeviceLayer.from_arrays(router, gen.shared_blob(wl.seed, 0, d, fs),
                                    gen.expert_pool(wl.seed, 0, d, f, E), d, f, fs, k, device=dev)
    X = torch.from_numpy(gen.tokens(wl.seed, wl.n_tokens, d).view(np.int16)).to(dev)
    Y = torch.empty((wl.n_tokens, d), dtype=torch.int16, device=dev)
    IDS = torch.empty((wl.n_tokens, k), dtype=torch.int32, device=dev)
    W = torch.empty((wl.n_tokens, k), dtype=torch.float32, device=dev)
    ws = api.workspace(api.tf_prefill_workspace_bytes(D, C), dev)
    stream = torch.cuda.Stream(device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    Lp = ctypes.byref(D.struct)

    def step(i):
        j = i % nch
        _lib.check(lib.tf_moe_prefill_chunk(
            Lp, ctypes.c_void_p(X.data_ptr() + 2 * d * C * j), C,
            ctypes.c_void_p(Y.data_ptr() + 2 * d * C * j), None,
            ctypes.c_void_p(IDS.data_ptr() + 4 * k * C * j),
            ctypes.c_void_p(W.data_ptr() + 4 * k * C * j), sh, ctypes.c_void_p(ws.data_ptr()),
            ws.numel()))

    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    graphs = _graphs(step, nch, nch, stream)
    steps, ms = _timed(graphs, args.steps or nch, nch, stream)
    ids = IDS.cpu().numpy().reshape(nch, C * k)
    distinct = float(np.mean([len(np.unique(r)) for r in ids]))
    qb = lambda n, kk, bits=4: n * kk * bits // 8 + 4 * n * (kk // 64)   # noqa: E731
    blob = 2 * qb(f, d) + qb(d, f)
    chunk_bytes = qb(E, d, 8) + 2 * qb(fs, d) + qb(d, fs) + distinct * blob + 4 * C * d
    kern = _profile(lib, _hip(), {
        _lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "router_topk_group",
        _lib.TF_KERNEL_PREFILL_GATEUP: "gateup_mfma",
        _lib.TF_KERNEL_PREFILL_DOWN: "down_mfma",
        _lib.TF_KERNEL_PREFILL_COMBINE: "combine"}, step, min(args.prof_steps, 64), stream)
    us = ms * 1e3 / steps
    return {"metric": "prefill tokens/s (128-token chunks, one layer)",
            "value": round(C * steps / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": steps, "us_per_chunk": round(us, 2), "higher_is_better": True,
            "data": "synthetic (seeded)", "dtype": "fp32",
            "config": {"workload": wl.name, "chunk": C, "chunks": nch,
                       "distinct_experts_per_chunk": distinct},
            "chunk_bytes": int(chunk_bytes),
            "GBps": round(chunk_bytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(chunk_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "kernels": kern}


def run_stack(args):
    """30 resident layers, batch 1 and 16 independent tokens per step, forced
    uniform routing; every layer of a step consumes the step's x."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen
    wl = gen.WORKLOADS[4]
    d, E, k, f, fs, L = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared, wl.n_layers
    nsteps = args.steps or wl.n_tokens
    warm = wl.extra.get("warmup_steps", 50)
    lib = _lib.load()
    dev = torch.device("cuda:0")
    t0 = time.time()
    stride = gen.blob_bytes(d, f)
    layers = []
    host = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        gen.expert_pool(wl.seed, l, d, f, E, out=host.numpy(), threads=16)
        pool = host.to(dev, non_blocking=False)
        layers.append(api.DeviceLayer.from_arrays(gen.router(wl.seed, l, d, E),
                                                  gen.shared_blob(wl.seed, l, d, fs), pool,
                                                  d, f, fs, k, device=dev))
        print(f"stack: layer {l} resident ({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)
    setup = time.time() - t0
    res = {}
    for B in wl.batches:
        ntok = (nsteps + warm) * B
        X = torch.from_numpy(gen.tokens(wl.seed, ntok, d).view(np.int16)).to(dev)
        ids_f = np.stack([gen.uniform_ids(wl.seed, l, ntok, E, k) for l in range(L)])
        F = torch.from_numpy(ids_f).to(dev)
        Y = torch.empty((L, B, d), dtype=torch.int16, device=dev)
        IDS = torch.empty((L, B, k), dtype=torch.int32, device=dev)
        W = torch.empty((L, B, k), dtype=torch.float32, device=dev)
        ws = api.workspace(api.tf_moe_workspace_bytes(layers[0], B), dev)
        stream = torch.cuda.Stream(device=dev)
        sh = ctypes.c_void_p(stream.cuda_stream)
        Ls = [ctypes.byref(D.struct) for D in layers]

        def step(i, B=B, X=X, F=F, Y=Y, IDS=IDS, W=W, ws=ws, sh=sh, Ls=Ls, ntok=ntok):
            r0 = (i % (ntok // B)) * B
            for l in range(L):
                _lib.check(lib.tf_moe_layer_fwd(
                    Ls[l], ctypes.c_void_p(X.data_ptr() + 2 * d * r0), B,
                    ctypes.c_void_p(F.data_ptr() + 4 * k * (l * ntok + r0)),
                    ctypes.c_void_p(Y.data_ptr() + 2 * d * B * l), None,
                    ctypes.c_void_p(IDS.data_ptr() + 4 * k * B * l),
                    ctypes.c_void_p(W.data_ptr() + 4 * k * B * l), None, 0, sh, sh,
                    ctypes.c_void_p(ws.data_ptr()), ws.numel()))

        with torch.cuda.stream(stream):
            step(0)
        torch.cuda.synchronize()
        graphs = _graphs(step, nsteps + warm, 50, stream)
        steps, ms = _timed(graphs, nsteps, warm, stream)
        # algorithmic bytes: per layer router + shared + distinct experts of the step
        qb = lambda n, kk, bits=4: n * kk * bits // 8 + 4 * n * (kk // 64)   # noqa: E731
        blob = 2 * qb(f, d) + qb(d, f)
        core = qb(E, d, 8) + 2 * qb(fs, d) + qb(d, fs)
        rows = ids_f[:, :(nsteps + warm) * B].reshape(L, nsteps + warm, B * k)
        distinct = float(np.mean([[len(np.unique(r)) for r in lay] for lay in rows]))
        step_bytes = L * (core + distinct * blob + 4 * B * d)
        nexp = B * k if B * k < distinct else distinct
        if B == 1:   # decode kernels A, B, C; B = routed gate/up + shared down
            names = {_lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "router_shared_gateup",
                     _lib.TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN: "routed_gateup_shared_down",
                     _lib.TF_KERNEL_DOWN_COMBINE: "down_combine"}
            gemv = {"routed_gateup_shared_down": nexp * 2 * qb(f, d) + qb(d, fs)}
        else:        # grouped step: router + grouping, gate/up, down, combine
            names = {_lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "router_topk_group",
                     _lib.TF_KERNEL_PREFILL_GATEUP: "gateup_mfma",
                     _lib.TF_KERNEL_PREFILL_DOWN: "down_mfma",
                     _lib.TF_KERNEL_PREFILL_COMBINE: "combine"}
            gemv = {"gateup_mfma": nexp * 2 * qb(f, d) + 2 * qb(fs, d),
                    "down_mfma": nexp * qb(d, f) + qb(d, fs)}
        kern = _profile(lib, _hip(), names, step, min(args.prof_steps, 100), stream)
        us = ms * 1e3 / steps
        gk = {}
        for name, kb in gemv.items():
            dur = kern[name]["avg_us"] * 1e-6
            gk[name] = {"bytes_per_launch": int(kb), "GBps": round(kb / dur / 1e9, 1),
                        "frac": round(kb / dur / 1e9 / HBM_PEAK_GBPS, 4)}
        res[f"batch{B}"] = {
            "tokens_per_s": round(B * steps / (ms / 1e3), 1), "us_per_step": round(us, 2),
            "distinct_experts_per_layer": round(distinct, 2), "step_bytes": int(step_bytes),
            "GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "gemv_kernels": gk, "kernels_per_layer": kern}
        del X, F, Y, IDS, W, ws, graphs
        torch.cuda.synchronize()
    return {"metric": "30-layer resident MoE stack decode tokens/s", "workload": wl.name,
            "setup_s": round(setup, 1), "steps": nsteps, "warmup": warm, "results": res}


def run_slot(args):
    """30 layers, 16-slot LFU cache per layer in HBM, experts in pinned host
    memory, Zipf(1.1) forced routing; misses copied while the shared branch
    runs."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen
    wl = gen.WORKLOADS[2]
    d, E, k, f, fs, L, S = (wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared,
                            wl.n_layers, wl.n_slots)
    ntok = args.steps or wl.n_tokens
    dev = torch.device("cuda:0")
    t0 = time.time()
    stride = gen.blob_bytes(d, f)
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy().reshape(L, E, stride)
    layers = []
    for l in range(L):
        gen.expert_pool(wl.seed, l, d, f, E, out=hv[l], threads=16)
        layers.append(api.DeviceLayer.from_arrays(gen.router(wl.seed, l, d, E),
                                                  gen.shared_blob(wl.seed, l, d, fs),
                                                  torch.empty((S, stride), dtype=torch.uint8,
                                                              device=dev), d, f, fs, k, device=dev))
        print(f"slot: layer {l} generated ({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)
    setup = time.time() - t0
    X = torch.from_numpy(gen.tokens(wl.seed, ntok, d).view(np.int16)).to(dev)
    F = torch.from_numpy(np.stack([gen.zipf_ids(wl.seed, l, ntok, E, k) for l in range(L)])).to(dev)
    Y = torch.empty((L, ntok, d), dtype=torch.float16, device=dev)
    ws = api.workspace(api.tf_moe_workspace_bytes(layers[0], 1), dev)
    copy = torch.cuda.Stream(device=dev)
    # same-run pinned H2D peak: one large copy
    big = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(4):
        big.copy_(host[:256 << 20], non_blocking=True)
    torch.cuda.synchronize()
    peak = 4 * (256 << 20) / (time.perf_counter() - c0) / 1e9
    del big

    Fh = F.cpu().numpy()
    prng = np.random.default_rng([wl.seed, 9200])
    # predicted ids of (layer, token): exact, or with half of them replaced
    pred = {"exact": Fh, "noisy": Fh.copy()}
    for l in range(L):
        for t in range(ntok):
            j = prng.choice(k, size=k // 2, replace=False)
            pred["noisy"][l, t, j] = prng.integers(0, E, size=j.size)

    def one(n_slots, policy, prefetch=None, engine="kernel"):
        """One pass of the token stream through the stack with this cache;
        with `prefetch`, the next layer's predicted experts are copied ahead."""
        slot_pool = torch.empty(L * n_slots * stride, dtype=torch.uint8, device=dev)
        cache = api.SlotCache(L, E, n_slots, k, stride, slot_pool, host, trace_cap=ntok,
                              policy=policy)
        cache.set_copy_engine(engine)
        if prefetch:
            pf_buf = torch.empty(L * k * stride, dtype=torch.uint8, device=dev)
            cache.set_prefetch(pf_buf, k)
            P = pred[prefetch]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        if prefetch:
            cache.prefetch(0, P[0, 0], copy)
        for t in range(ntok):
            for l in range(L):
                api.tf_moe_layer_fwd(layers[l], X[t:t + 1], forced_ids=F[l, t:t + 1],
                                     y=Y[l, t:t + 1], cache=cache, layer_idx=l, ws=ws,
                                     copy_stream=copy)
                nl, nt = (l + 1, t) if l + 1 < L else (0, t + 1)
                if prefetch and nt < ntok:
                    cache.prefetch(nl, P[nl, nt], copy)
            if t % 256 == 255:
                print(f"slot: {policy} {n_slots} slots {prefetch or ''}, token {t + 1}",
                      file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        hits = sum(int(cache.trace(l, ntok * k)[0].sum()) for l in range(L))
        filled = cache.bytes_filled()
        pf_bytes, used, wasted = cache.prefetch_stats() if prefetch else (0, 0, 0)
        cache.close()
        del slot_pool
        r = {"slots": n_slots, "policy": policy, "engine": engine, "value": round(ntok / wall, 2),
             "hit_rate": round(hits / (L * ntok * k), 4), "h2d_bytes": filled + pf_bytes,
             "h2d_GBps": round((filled + pf_bytes) / wall / 1e9, 2), "wall_s": round(wall, 2)}
        if prefetch:
            r.update({"prefetch": prefetch, "prefetch_h2d_bytes": pf_bytes,
                      "prefetch_used": used, "prefetch_unused": wasted,
                      "fill_h2d_bytes": filled})
        return r

    base = one(S, "lfu")
    out = {"metric": "slot-cache stack decode tokens/s (30 layers, 16 slots, PCIe misses)",
           "workload": wl.name, "tokens": ntok, "value": base["value"], "unit": "tokens/s",
           "hit_rate": base["hit_rate"], "h2d_bytes": base["h2d_bytes"],
           "h2d_GBps": base["h2d_GBps"], "pinned_h2d_peak_GBps": round(peak, 2),
           "setup_s": round(setup, 1), "wall_s": base["wall_s"]}
    if args.prefetch:     # speculative fill of the next layer's predicted experts
        out["prefetch"] = [one(S, "lfu", "exact"), one(S, "lfu", "noisy"),
                           one(S, "lfu", None, "dma"), one(S, "lfu", "exact", "dma")]
    if args.slot_sweep:   # slot counts x policies (the LFU reading and the LRU gloss)
        out["sweep"] = [one(n, pol) for n in (8, 16, 32) for pol in ("lfu", "lru")
                        if not (n == S and pol == "lfu")] + [dict(base)]
    return out


def run_sample(args):
    """Next-token sampling over 262,144-id logits at the default knobs
    (temperature 0.2, top-k 64, top-p 0.95), batch 1 and 16."""
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen
    lib = _lib.load()
    dev = torch.device("cuda:0")
    V, K, TEMP, TOP_P = gen.VOCAB, 64, 0.2, 0.95
    stream = torch.cuda.Stream(device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    out = {"metric": "sampled tokens/s (262,144-id logits, top-k 64, top-p 0.95, T 0.2)",
           "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
           "data": "synthetic (seeded)", "dtype": "fp32 keys, fp64 softmax",
           "config": {"workload": "sample-v262144-k64", "vocab": V, "top_k": K,
                      "temperature": TEMP, "top_p": TOP_P}, "batches": {}}
    for T in (1, 16):
        nrow = 64   # distinct logit rows cycled through
        l, u = gen.sample_inputs(11, nrow * T, V, "lm")
        L = torch.from_numpy(l).to(dev)
        U = torch.from_numpy(u).to(dev)
        ids = torch.empty(nrow * T, dtype=torch.int32, device=dev)
        ws = api.workspace(api.tf_sample_workspace_bytes(V, T, K), dev)

        def step(i):
            j = i % nrow
            _lib.check(lib.tf_sample(ctypes.c_void_p(L.data_ptr() + 4 * V * T * j), V, T, TEMP, K,
                                     TOP_P, ctypes.c_void_p(U.data_ptr() + 8 * T * j),
                                     ctypes.c_void_p(ids.data_ptr() + 4 * T * j),
                                     ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh))

        with torch.cuda.stream(stream):
            step(0)
        torch.cuda.synchronize()
        n = args.steps or 2000
        graphs = _graphs(step, nrow, nrow, stream)
        steps, ms = _timed(graphs, n, min(args.warmup, n), stream)
        kern = _profile(lib, _hip(), {_lib.TF_KERNEL_SAMPLE_PART: "k_sample_part",
                                      _lib.TF_KERNEL_SAMPLE_FINAL: "k_sample_final"}, step,
                        min(args.prof_steps, 200), stream)
        us = ms * 1e3 / steps
        kus = kern["k_sample_part"]["avg_us"]
        nbytes = 4 * V * T   # the logits, read once by the slice kernel
        out["batches"][str(T)] = {
            "us_per_call": round(us, 3), "tokens_per_s": round(T * steps / (ms / 1e3), 1),
            "kernels": kern,
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (kus * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(nbytes / (kus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}}
    out["value"] = out["batches"]["16"]["tokens_per_s"]
    return out


def run_attn(args):
    """Decode attention of one token (16 query heads, 8 key/value heads, head
    dim 256): a full layer at its 4,096th token and a 1,024-slot
    sliding-window ring past its first wrap."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen
    lib = _lib.load()
    dev = torch.device("cuda:0")
    H, G, D = 16, 8, 256
    stream = torch.cuda.Stream(device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    out = {"metric": "decode attention us per token (16 q heads, 8 kv heads, head dim 256)",
           "unit": "us", "n_gpus": 1, "higher_is_better": False, "data": "synthetic (seeded)",
           "dtype": "fp16 KV, fp32 scores and sums", "config": {"workload": "attn-decode-h16-g8-d256"},
           "layers": {}}
    for name, S, pos, ring in (("full-4096", 4096, 4095, 0), ("sliding-1024", 1024, 5000, 1)):
        nq = 64   # distinct queries cycled through
        q, k, v = gen.attn_inputs(21, nq, H, G, D)
        kc = torch.from_numpy(np.random.default_rng(5).standard_normal((G, S, D)).astype(np.float16)
                              .view(np.int16)).to(dev)
        vc = torch.from_numpy(np.random.default_rng(6).standard_normal((G, S, D)).astype(np.float16)
                              .view(np.int16)).to(dev)
        Q = torch.from_numpy(q.view(np.int16)).to(dev)
        Kn = torch.from_numpy(k.view(np.int16)).to(dev)
        Vn = torch.from_numpy(v.view(np.int16)).to(dev)
        O = torch.empty((nq, H, D), dtype=torch.float32, device=dev)
        ws = api.workspace(api.tf_attn_workspace_bytes(H, D, S), dev)

        def step(i):
            j = i % nq
            _lib.check(lib.tf_attn_decode(
                ctypes.c_void_p(Q[j].data_ptr()), ctypes.c_void_p(Kn[j].data_ptr()),
                ctypes.c_void_p(Vn[j].data_ptr()), ctypes.c_void_p(kc.data_ptr()),
                ctypes.c_void_p(vc.data_ptr()), H, G, D, S, pos, ring, 1.0 / D ** 0.5,
                ctypes.c_void_p(O[j].data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(), sh))

        with torch.cuda.stream(stream):
            step(0)
        torch.cuda.synchronize()
        graphs = _graphs(step, nq, nq, stream)
        steps, ms = _timed(graphs, args.steps or 4000, min(args.warmup, 1000), stream)
        kern = _profile(lib, _hip(), {_lib.TF_KERNEL_ATTN_CHUNK: "k_attn_chunk",
                                      _lib.TF_KERNEL_ATTN_COMBINE: "k_attn_combine"}, step,
                        min(args.prof_steps, 200), stream)
        seen = min(pos + 1, S)
        nbytes = 2 * G * seen * D * 2   # keys and values the token sees, read once
        kus = kern["k_attn_chunk"]["avg_us"]
        out["layers"][name] = {
            "us_per_call": round(ms * 1e3 / steps, 3), "kv_bytes": nbytes, "kernels": kern,
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (kus * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(nbytes / (kus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}}
    L = out["layers"]
    out["value"] = round(25 * L["sliding-1024"]["us_per_call"] + 5 * L["full-4096"]["us_per_call"], 2)
    out["per_token_30_layers"] = "25 sliding-window layers + 5 full layers"
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--graph-chunk", type=int, default=250)
    ap.add_argument("--prof-steps", type=int, default=300)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run plain 256 MiB device copies (memory-counter calibration)")
    ap.add_argument("--prefetch", action="store_true",
                    help="slot-cache workload: also run with the next layer's experts "
                         "prefetched (exact predictions, and half of them wrong)")
    ap.add_argument("--slot-sweep", action="store_true",
                    help="slot-cache workload: also run 8, 16 and 32 slots under LFU and LRU")
    ap.add_argument("--workload", choices=["decode", "prefill", "stack", "slot-cache", "sample",
                                           "attn"],
                    default="decode",
                    help="decode (default, the headline line); the others measure the "
                         "prefill chunk, the 30-layer resident stack, the slot-cache stack "
                         "next-token sampling and decode attention")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path is built and measured on a single "
              "MI355X (the multi-GPU design is expert sharding, not implemented here).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
    if args.workload == "decode":
        out = run_decode(args)
    else:
        if "--steps" not in sys.argv:
            args.steps = 0   # the workload's own count
        out = {"prefill": run_prefill, "stack": run_stack, "slot-cache": run_slot,
               "sample": run_sample, "attn": run_attn}[args.workload](args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
