#!/usr/bin/env python3
"""MoE-layer decode throughput on one MI355X.

Default workload (resident-stack-30L-e128k8-uniform): 30 MoE layers of the
full-width shape -- d_model 2816, 128 routed experts per layer, all resident
in HBM (12.85 GB of q4 experts), top-8, expert FFN 704, shared expert FFN
2816, MLX-style affine 4-bit weights (group 64) and an 8-bit router --
decoding one token per step with uniform random (forced) routing; every layer
of a step consumes that step's token.  A step is the whole hot path for one
token through all 30 layers: router + top-8 + softmax, shared expert, the 8
routed experts' gate/up/down and the combine, per layer.

Prints one JSON line.  ``value`` is tokens/s over exactly --steps steps,
replayed from HIP graphs after exactly --warmup warm-up steps, each step on a
token (and routing) of its own, inputs already resident in HBM.  The
roofline is that of the dominant kernel (the routed gate/up + shared down
launch): its algorithmic bytes divided by its average duration from
start/stop events attached to the launch (hipEventDisableSystemFence, so the
events do not flush the caches), taken on steps after the timed ones.
Batch 16 on the same stack and the single-layer decode workload
(decode-layer-d2816-e128k8) are reported under their own keys, and the fp64
CPU oracle is timed on a bounded sample of the headline workload.
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
NO_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def _event(h):
    e = ctypes.c_void_p()
    assert h.hipEventCreateWithFlags(ctypes.byref(e), NO_SYSTEM_FENCE) == 0
    return e


def qmat_bytes(n, k, bits=4):
    """Codes plus one fp16 scale and one fp16 bias per group of 64."""
    return n * k * bits // 8 + 4 * n * (k // 64)


def stage_b_bytes(d, f, fs, k):
    """Algorithmic bytes of one single-token routed-gate/up + shared-down
    launch: the k experts' gate/up and the shared down weights, x and h_s in,
    h_r and y_s out."""
    w = k * 2 * qmat_bytes(f, d) + qmat_bytes(d, fs)
    return w + d * 2 + fs * 4 + k * f * 4 + d * 4


def layer_bytes(d, f, fs, E, k):
    """Bytes one decode token must move through one layer: the 8-bit router,
    the shared expert, k routed experts, plus x in and y out."""
    router = qmat_bytes(E, d, 8)
    shared = 2 * qmat_bytes(fs, d) + qmat_bytes(d, fs)
    routed = k * (2 * qmat_bytes(f, d) + qmat_bytes(d, f))
    return router + shared + routed + 2 * d + 2 * d


def _traffic_for(name, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources and this workload; else None."""
    import profiling
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[name]
    except (KeyError, ValueError):
        return None
    if (rec.get("source_sha256") != profiling.source_sha256(rec.get("kernel", ""))
            or rec.get("workload") != workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def calibration(nbytes=256 << 20, reps=3):
    """Kernels of known traffic for scaling the memory counters (rocprofv3
    FETCH_SIZE / WRITE_SIZE) of the same run: a read-only stream of nbytes
    with the GEMVs' 16-byte-per-lane whole-line loads (the library's
    k_stream_read), and a write-only fill of nbytes."""
    import torch

    from bit_routed_expert_tf_amd import _lib
    lib = _lib.load()
    a = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(reps):
        _lib.check(lib.tf_profile_stream_read(ctypes.c_void_p(a.data_ptr()), nbytes, s))
        a.fill_(2)
    torch.cuda.synchronize()
    del a


def same_size_stream(lib, nbytes, dev, n_buf=24, reps=10):
    """What one launch of a plain read-only stream (the library's
    k_stream_read: 16 bytes per lane, loads only) of `nbytes` reaches on this
    GPU: graph-replayed back to back, every launch over a buffer of its own.
    Context for a kernel's roofline fraction at the same launch size."""
    import torch

    from bit_routed_expert_tf_amd import _lib
    n = nbytes // 16 * 16
    bufs = [torch.ones(n // 4, dtype=torch.int32, device=dev) for _ in range(n_buf)]
    stream = torch.cuda.Stream(device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for b in bufs:
            _lib.check(lib.tf_profile_stream_read(ctypes.c_void_p(b.data_ptr()), n, sh))
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (n_buf * reps)
    del g, bufs
    return {"bytes": n, "us_per_launch": round(us, 3), "GBps": round(n / us / 1e3, 1),
            "frac_of_peak": round(n / us / 1e3 / HBM_PEAK_GBPS, 4),
            "kernel": "k_stream_read: read-only, 16 B per lane, graph-replayed, "
                      f"{n_buf} buffers of its size in turn"}


def _profile(lib, h, kernels, step, steps, stream):
    """Average durations of the named kernels over eager calls step(i) for i
    in `steps`: start/stop events attached to the launch (fence-free)."""
    import torch

    from bit_routed_expert_tf_amd import _lib
    out = {}
    for kid, name in kernels.items():
        evs = [(_event(h), _event(h)) for _ in steps]
        with torch.cuda.stream(stream):
            for (a, b), i in zip(evs, steps):
                _lib.check(lib.tf_profile_kernel(kid, a, b))
                step(i)
        torch.cuda.synchronize()
        _lib.check(lib.tf_profile_kernel(0, None, None))   # disarm
        durs = []
        for a, b in evs:
            v = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(v), a, b) == 0:
                durs.append(v.value * 1e3)
            h.hipEventDestroy(a)
            h.hipEventDestroy(b)
        if not durs:
            raise RuntimeError(f"kernel {name} did not run in the profiled steps")
        durs.sort()
        out[name] = {"avg_us": round(sum(durs) / len(durs), 3),
                     "median_us": round(durs[len(durs) // 2], 3), "min_us": round(durs[0], 3),
                     "launches": len(durs)}
    return out


def _graphs(step, first, n, chunk, stream, sides=()):
    """HIP graphs of at most `chunk` consecutive steps each, covering steps
    first .. first + n - 1 in order.  With side streams, every graph forks
    them from `stream` at its start and joins them back at its end (the step
    function picks each step's stream)."""
    import torch
    graphs = []
    for j in range(first, first + n, chunk):
        g = torch.cuda.CUDAGraph()
        m = min(first + n, j + chunk) - j
        with torch.cuda.graph(g, stream=stream):
            if sides:
                fork = torch.cuda.Event()
                fork.record(stream)
                for s in sides:
                    s.wait_event(fork)
            for i in range(j, j + m):
                step(i)
            for s in sides:
                join = torch.cuda.Event()
                join.record(s)
                stream.wait_event(join)
        graphs.append((g, m))
    torch.cuda.synchronize()
    return graphs


def _replay_all(graphs, stream):
    import torch
    with torch.cuda.stream(stream):
        for g, _ in graphs:
            g.replay()
    return sum(m for _, m in graphs)


def _timed(step, warmup, steps, chunk, stream, sides=()):
    """Warm-up steps 0 .. warmup-1, then steps warmup .. warmup+steps-1 timed
    with events on the stream; every step exactly once.  Returns (steps, ms)."""
    import torch
    wg = _graphs(step, 0, warmup, chunk, stream, sides) if warmup else []
    tg = _graphs(step, warmup, steps, chunk, stream, sides)
    _replay_all(wg, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    n = _replay_all(tg, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    del wg, tg
    return n, e0.elapsed_time(e1)


def _stack_layers(wl, dev, keep_host=False):
    """30 layers of the stack workload resident on the device; with
    keep_host, also their host copies (for the oracle)."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import api
    from synth import gen
    d, E, k, f, fs = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared
    stride = gen.blob_bytes(d, f)
    t0 = time.time()
    layers, host_layers = [], []
    buf = torch.empty((E, stride), dtype=torch.uint8, pin_memory=True)
    for l in range(wl.n_layers):
        gen.expert_pool(wl.seed, l, d, f, E, out=buf.numpy(), threads=16)
        router, sb = gen.router(wl.seed, l, d, E), gen.shared_blob(wl.seed, l, d, fs)
        layers.append(api.DeviceLayer.from_arrays(router, sb, buf.to(dev), d, f, fs, k, device=dev))
        if keep_host:
            host_layers.append({"router": router, "shared_blob": sb, "pool": np.array(buf.numpy()),
                                "d_model": d, "d_ff": f, "d_ff_shared": fs, "top_k": k})
        if l % 10 == 9:
            print(f"stack: {l + 1} layers resident ({time.time() - t0:.0f} s)", file=sys.stderr,
                  flush=True)
    return layers, host_layers, time.time() - t0


def run_stack_batch(args, wl, layers, B, lib, dev, roofline):
    """Batch-B decode steps through the resident stack: exactly args.warmup
    warm-up steps, then exactly args.steps timed ones, each step on B tokens
    of its own; then kernel durations on further steps."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen
    d, E, k, f, fs, L = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared, wl.n_layers
    nprof = min(args.prof_steps, 200 if B == 1 else 60)
    nstep = args.warmup + args.steps + nprof
    ntok = nstep * B
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
    xp, fp, yp, ip, wp = X.data_ptr(), F.data_ptr(), Y.data_ptr(), IDS.data_ptr(), W.data_ptr()
    wsp, wsn = ctypes.c_void_p(ws.data_ptr()), ws.numel()

    def step(i):
        r0 = i * B
        for l in range(L):
            rc = lib.tf_moe_layer_fwd(
                Ls[l], ctypes.c_void_p(xp + 2 * d * r0), B,
                ctypes.c_void_p(fp + 4 * k * (l * ntok + r0)), ctypes.c_void_p(yp + 2 * d * B * l),
                None, ctypes.c_void_p(ip + 4 * k * B * l), ctypes.c_void_p(wp + 4 * k * B * l),
                None, 0, sh, sh, wsp, wsn)
            if rc:
                raise RuntimeError(lib.tf_last_error().decode())

    steps, ms = _timed(step, args.warmup, args.steps, args.graph_chunk, stream)
    after = range(args.warmup + args.steps, nstep)
    blob = 2 * qmat_bytes(f, d) + qmat_bytes(d, f)
    core = qmat_bytes(E, d, 8) + 2 * qmat_bytes(fs, d) + qmat_bytes(d, fs)
    used = ids_f[:, args.warmup * B:(args.warmup + args.steps) * B].reshape(L, args.steps, B * k)
    distinct = float(np.mean([[len(np.unique(r)) for r in lay] for lay in used]))
    step_bytes = L * (core + distinct * blob + 4 * B * d)
    if B == 1:
        names = {_lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "k_stage_a",
                 _lib.TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN: "k_stage_b",
                 _lib.TF_KERNEL_DOWN_COMBINE: "k_stage_c1"}
        gemv = {"k_stage_b": stage_b_bytes(d, f, fs, k)}
    else:
        names = {_lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "k_router_rows",
                 _lib.TF_KERNEL_PREFILL_GATEUP: "k_gu",
                 _lib.TF_KERNEL_PREFILL_DOWN: "k_dn",
                 _lib.TF_KERNEL_PREFILL_COMBINE: "k_pf_combine"}
        gemv = {"k_gu": distinct * 2 * qmat_bytes(f, d) + 2 * qmat_bytes(fs, d),
                "k_dn": distinct * qmat_bytes(d, f) + qmat_bytes(d, fs)}
    kern = _profile(lib, _hip(), names, step, after, stream)
    us = ms * 1e3 / steps
    rf = {}
    for name, kb in gemv.items():
        dur = kern[name]["avg_us"] * 1e-6
        rf[name] = {"bound": "hbm", "achieved": round(kb / dur / 1e9, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(kb / dur / 1e9 / HBM_PEAK_GBPS, 4),
                    "traffic": _traffic_for(f"{name}_batch{B}", wl.name),
                    "algorithmic_bytes_per_launch": int(kb),
                    "avg_duration_us": kern[name]["avg_us"]}
    del X, F, Y, IDS, W, ws
    torch.cuda.synchronize()
    return {"tokens_per_s": round(B * steps / (ms / 1e3), 1), "steps": steps, "warmup": args.warmup,
            "ms_per_step": round(ms / steps, 5), "us_per_layer": round(us / L, 3),
            "distinct_experts_per_layer": round(distinct, 2), "step_bytes": int(step_bytes),
            "GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "roofline": rf[roofline], "gemv_kernels": rf, "kernels_per_layer": kern,
            "kernel_timing": f"launch-attached fence-free events, {len(after)} eager steps after "
                             f"the timed ones"}


def run_stack(args):
    """The headline: 30 resident layers, batch 1 (and batch 16 under its own
    key), forced uniform routing."""
    import torch

    from bit_routed_expert_tf_amd import _lib
    from synth import gen
    wl = gen.WORKLOADS[4]
    lib = _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers, host_layers, setup = _stack_layers(wl, dev, keep_host=not args.no_cpu_baseline)
    b1 = run_stack_batch(args, wl, layers, 1, lib, dev, "k_stage_b")
    print(f"stack batch 1: {b1['tokens_per_s']} tokens/s", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": b1["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": b1["steps"], "warmup": args.warmup, "ms_per_step": b1["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (seeded; random-init q4 weights of the stated shapes)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "tokens_per_step": 1,
                   "d_model": wl.d_model, "n_experts": wl.n_experts, "top_k": wl.top_k,
                   "d_ff": wl.d_ff, "d_ff_shared": wl.d_ff_shared,
                   "routing": "uniform random forced ids, a fresh token per step",
                   "weights": "affine q4 group 64 (fp16 scale/bias), 8-bit router",
                   "io": "fp16 x/y, fp32 accumulate, fp64 router sums",
                   "experts_resident": "all 30 x 128 in HBM", "graph_chunk": args.graph_chunk},
        "roofline": dict(b1["roofline"], kernel="k_stage_b (routed gate/up + shared down)",
                         timing=b1["kernel_timing"]),
        "stack": {k: b1[k] for k in ("us_per_layer", "step_bytes", "GBps", "frac_of_hbm_peak",
                                     "distinct_experts_per_layer")},
        "kernels_per_layer": b1["kernels_per_layer"],
        "device": torch.cuda.get_device_name(dev), "setup_s": round(setup, 1),
    }
    if not args.headline_only:
        # context: a plain stream of the dominant kernel's bytes in one launch
        st = same_size_stream(lib, out["roofline"]["algorithmic_bytes_per_launch"], dev)
        st["kernel_over_stream"] = round(out["roofline"]["achieved"] / st["GBps"], 4)
        out["roofline"]["same_size_stream"] = st
        out["batch16"] = run_stack_batch(args, wl, layers, 16, lib, dev, "k_gu")
        print(f"stack batch 16: {out['batch16']['tokens_per_s']} tokens/s", file=sys.stderr,
              flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_stack(args, wl, host_layers)
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.headline_only:
        out["decode_layer"] = run_decode(args)
    return out


def run_decode(args):
    """The single-layer decode workload (decode-layer-d2816-e128k8): one
    layer, all 128 experts resident, natural routing, one token per step."""
    import numpy as np
    import torch

    from bit_routed_expert_tf_amd import _lib, api
    from synth import gen

    wl = gen.WORKLOADS[1]
    d, E, k, f, fs = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared
    lib = _lib.load()
    dev = torch.device("cuda:0")
    D = api.DeviceLayer.from_arrays(gen.router(wl.seed, 0, d, E), gen.shared_blob(wl.seed, 0, d, fs),
                                    gen.expert_pool(wl.seed, 0, d, f, E, threads=16), d, f, fs, k,
                                    device=dev)
    Xd = torch.from_numpy(gen.tokens(wl.seed, wl.n_tokens, d).view(np.int16)).to(dev)
    Y = torch.empty((wl.n_tokens, d), dtype=torch.int16, device=dev)
    IDS = torch.empty((wl.n_tokens, k), dtype=torch.int32, device=dev)
    W = torch.empty((wl.n_tokens, k), dtype=torch.float32, device=dev)
    ws = api.workspace(api.tf_moe_workspace_bytes(D, 1), dev)
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

    nprof = min(args.prof_steps, 200)
    steps_t = max(1, min(args.steps, wl.n_tokens - args.warmup - nprof))
    steps, ms = _timed(step, args.warmup, steps_t, args.graph_chunk, stream)
    after = range(args.warmup + steps, args.warmup + steps + nprof)
    kern = _profile(lib, _hip(), {_lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "k_stage_a",
                                  _lib.TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN: "k_stage_b",
                                  _lib.TF_KERNEL_DOWN_COMBINE: "k_stage_c1"}, step, after, stream)
    tok_s = steps / (ms / 1e3)
    bb = stage_b_bytes(d, f, fs, k)
    dur = kern["k_stage_b"]["avg_us"] * 1e-6
    lb = layer_bytes(d, f, fs, E, k)
    return {"workload": wl.name, "tokens_per_s": round(tok_s, 1), "steps": steps,
            "warmup": args.warmup, "us_per_token": round(ms * 1e3 / steps, 3),
            "roofline": {"bound": "hbm", "achieved": round(bb / dur / 1e9, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(bb / dur / 1e9 / HBM_PEAK_GBPS, 4),
                         "traffic": _traffic_for("k_stage_b_decode_layer", wl.name),
                         "kernel": "k_stage_b", "algorithmic_bytes_per_launch": bb,
                         "avg_duration_us": kern["k_stage_b"]["avg_us"]},
            "layer": {"bytes_per_token": lb, "GBps": round(lb * tok_s / 1e9, 1),
                      "frac_of_hbm_peak": round(lb * tok_s / 1e9 / HBM_PEAK_GBPS, 4),
                      "note": "one layer's 441.6 MB working set partly fits the 256 MB "
                              "Infinity Cache, so these GB/s are not all DRAM bytes"},
            "kernels": kern}


def cpu_baseline_stack(args, wl, host_layers):
    """The fp64 oracle, as it stands, on the host cores: whole steps of the
    headline workload (one token through all 30 layers, the same forced ids)
    over a bounded sample, timed on all cores and on one."""
    import numpy as np

    import oracle
    from synth import gen
    L, d, E, k = wl.n_layers, wl.d_model, wl.n_experts, wl.top_k
    nmax = 200
    X = gen.tokens(wl.seed, nmax, d)
    F = np.stack([gen.uniform_ids(wl.seed, l, nmax, E, k) for l in range(L)])

    def run(seconds, least):
        n, t0 = 0, time.perf_counter()
        while n < least or (time.perf_counter() - t0 < seconds and n < nmax):
            for l in range(L):
                oracle.moe_token(host_layers[l], X[n], F[l, n])
            n += 1
        return n, time.perf_counter() - t0

    oracle.moe_token(host_layers[0], X[0], F[0, 0])    # load / first touch
    n, dt = run(args.cpu_seconds, 2)
    cores = oracle.num_threads()
    oracle.set_num_threads(1)
    n1, dt1 = run(args.cpu_seconds / 4, 1)
    oracle.set_num_threads(cores)
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {n} steps of the workload (one token through all {L} layers "
                      f"each, {dt:.1f} s; C fp64 oracle, OpenMP over rows)",
            "one_core": {"value": round(n1 / dt1, 4), "unit": "tokens/s", "cores": 1,
                         "sample": f"the first {n1} steps ({dt1:.1f} s)"}}


def run_prefill(args):
    """128-token chunks through one full-width layer (natural routing).  The
    chunks of a layer are independent, so the line keeps two in flight:
    consecutive chunks alternate between two streams, each with a workspace of
    its own.  One chunk at a time on one stream is timed as well."""
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
    wss = [api.workspace(api.tf_prefill_workspace_bytes(D, C), dev) for _ in range(2)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    stream = streams[0]
    Lp = ctypes.byref(D.struct)
    # chunk j always runs on stream j % 2 (64 chunks: its rows of Y, IDS and W
    # are written by one stream only)
    assert nch % 2 == 0

    def launch(i, q):
        j = i % nch
        _lib.check(lib.tf_moe_prefill_chunk(
            Lp, ctypes.c_void_p(X.data_ptr() + 2 * d * C * j), C,
            ctypes.c_void_p(Y.data_ptr() + 2 * d * C * j), None,
            ctypes.c_void_p(IDS.data_ptr() + 4 * k * C * j),
            ctypes.c_void_p(W.data_ptr() + 4 * k * C * j),
            ctypes.c_void_p(streams[q].cuda_stream), ctypes.c_void_p(wss[q].data_ptr()),
            wss[q].numel()))

    def step(i):    # one chunk at a time
        launch(i, 0)

    def step2(i):   # two chunks in flight
        launch(i, i % 2)

    steps1, ms1 = _timed(step, args.warmup, args.steps, args.graph_chunk, stream)
    steps, ms = _timed(step2, args.warmup, args.steps, args.graph_chunk, stream, streams[1:])
    ids = IDS.cpu().numpy().reshape(nch, C * k)
    distinct = float(np.mean([len(np.unique(r)) for r in ids]))
    qb = lambda n, kk, bits=4: n * kk * bits // 8 + 4 * n * (kk // 64)   # noqa: E731
    blob = 2 * qb(f, d) + qb(d, f)
    chunk_bytes = qb(E, d, 8) + 2 * qb(fs, d) + qb(d, fs) + distinct * blob + 4 * C * d
    kern = _profile(lib, _hip(), {
        _lib.TF_KERNEL_ROUTER_SHARED_GATEUP: "k_router_mm",
        _lib.TF_KERNEL_ROUTER_TOPK: "k_router_topk",
        _lib.TF_KERNEL_PREFILL_GATEUP: "k_mq_gateup",
        _lib.TF_KERNEL_PREFILL_DOWN: "k_mq_down",
        _lib.TF_KERNEL_PREFILL_COMBINE: "k_pf_combine"}, step, range(min(args.prof_steps, 64)), stream)
    us, us1 = ms * 1e3 / steps, ms1 * 1e3 / steps1
    return {"metric": "prefill tokens/s (128-token chunks, one layer)",
            "value": round(C * steps / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": steps, "us_per_chunk": round(us, 2), "higher_is_better": True,
            "one_chunk_at_a_time": {"tokens_per_s": round(C * steps1 / (ms1 / 1e3), 1),
                                    "us_per_chunk": round(us1, 2)},
            "data": "synthetic (seeded)", "dtype": "fp32",
            "config": {"workload": wl.name, "chunk": C, "chunks": nch,
                       "distinct_experts_per_chunk": distinct,
                       "chunks_in_flight": 2, "schedule": "consecutive chunks alternate between "
                       "two streams, one workspace each; graphs fork and join the streams"},
            "chunk_bytes": int(chunk_bytes),
            "GBps": round(chunk_bytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(chunk_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "kernels": kern}


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

    base = one(S, "lfu", engine=args.slot_engine)
    out = {"metric": "slot-cache stack decode tokens/s (30 layers, 16 slots, PCIe misses)",
           "workload": wl.name, "tokens": ntok, "value": base["value"], "unit": "tokens/s",
           "copy_engine": args.slot_engine,
           "hit_rate": base["hit_rate"], "h2d_bytes": base["h2d_bytes"],
           "h2d_GBps": base["h2d_GBps"], "pinned_h2d_peak_GBps": round(peak, 2),
           "setup_s": round(setup, 1), "wall_s": base["wall_s"]}
    if args.prefetch:     # speculative fill of the next layer's predicted experts
        out["prefetch"] = [one(S, "lfu", "exact"), one(S, "lfu", "noisy"),
                           one(S, "lfu", None, "dma"), one(S, "lfu", "exact", "dma")]
    if args.slot_engines:   # the other copy engines on the same stream
        out["engines"] = [one(S, "lfu", None, e) for e in ("device", "kernel", "dma")
                          if e != args.slot_engine]
    if args.slot_sweep:   # slot counts x policies (the LFU reading and the LRU gloss)
        out["sweep"] = [one(n, pol, None, args.slot_engine) for n in (8, 16, 32) for pol in ("lfu", "lru")
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

        steps, ms = _timed(step, args.warmup, args.steps, args.graph_chunk, stream)
        kern = _profile(lib, _hip(), {_lib.TF_KERNEL_SAMPLE_PART: "k_sample_part",
                                      _lib.TF_KERNEL_SAMPLE_FINAL: "k_sample_final"}, step,
                        range(min(args.prof_steps, 200)), stream)
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

        steps, ms = _timed(step, args.warmup, args.steps, args.graph_chunk, stream)
        kern = _profile(lib, _hip(), {_lib.TF_KERNEL_ATTN_CHUNK: "k_attn_chunk",
                                      _lib.TF_KERNEL_ATTN_COMBINE: "k_attn_combine"}, step,
                        range(min(args.prof_steps, 200)), stream)
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


# steps and warm-up steps of each workload when the flags are not given
DEFAULT_STEPS = {"stack": (1000, 50), "decode": (1000, 50), "prefill": (64, 64),
                 "slot-cache": (2048, 0), "sample": (2000, 200), "attn": (4000, 1000)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's own count; 1000 for the stack)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps before them (default 50 for the stack)")
    ap.add_argument("--graph-chunk", type=int, default=25, help="steps per HIP graph")
    ap.add_argument("--prof-steps", type=int, default=200,
                    help="eager steps whose kernels are timed, after the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="stack workload: batch 1 only (no batch 16, no single-layer decode)")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a 256 MiB read-only reduction and a 256 MiB fill "
                         "(memory-counter calibration)")
    ap.add_argument("--prefetch", action="store_true",
                    help="slot-cache workload: also run with the next layer's experts "
                         "prefetched (exact predictions, and half of them wrong)")
    ap.add_argument("--slot-engine", choices=["device", "kernel", "dma"], default="device",
                    help="copy engine of the slot-cache fills (device: the fill kernel reads "
                         "the miss list on the GPU)")
    ap.add_argument("--slot-engines", action="store_true",
                    help="slot-cache workload: also run the other copy engines")
    ap.add_argument("--slot-sweep", action="store_true",
                    help="slot-cache workload: also run 8, 16 and 32 slots under LFU and LRU")
    ap.add_argument("--workload", choices=list(DEFAULT_STEPS), default="stack",
                    help="stack (default, the headline line: 30 resident layers); decode (one "
                         "layer); prefill (128-token chunks); slot-cache; sample; attn")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path is built and measured on a single "
              "MI355X (the multi-GPU design is expert sharding, not implemented here).",
              file=sys.stderr)
        sys.exit(2)
    ds, dw = DEFAULT_STEPS[args.workload]
    args.steps = ds if args.steps is None else args.steps
    args.warmup = dw if args.warmup is None else args.warmup
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    if args.calibrate:
        calibration()
    if args.workload == "decode":
        out = run_decode(args)
    else:
        out = {"stack": run_stack, "prefill": run_prefill, "slot-cache": run_slot,
               "sample": run_sample, "attn": run_attn}[args.workload](args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
