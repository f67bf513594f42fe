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
import hashlib
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


def _traffic_for(kernel_name, src_path, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[kernel_name]
    except (KeyError, ValueError):
        return None
    sha = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


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
    traffic = _traffic_for("routed_gateup_shared_down",
                           os.path.join(ROOT, "bit_routed_expert_tf_amd", "csrc", "tf_decode.hip"),
                           wl.name)

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
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {n} of the {wl.n_tokens} workload tokens, one at a time "
                      f"({dt:.1f} s, C fp64 oracle, OpenMP over rows)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--graph-chunk", type=int, default=250)
    ap.add_argument("--prof-steps", type=int, default=300)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this hot path is built and measured on a single "
              "MI355X (the multi-GPU design is expert sharding, not implemented here).",
              file=sys.stderr)
        sys.exit(2)
    out = run_decode(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
