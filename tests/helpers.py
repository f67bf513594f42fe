"""Test helpers: build seeded layers for both sides and compare outputs."""
from __future__ import annotations

import numpy as np

import oracle
from synth import gen


def oracle_layer(seed, layer, d, E, k, f, fs, pool=None):
    if pool is None:
        pool = gen.expert_pool(seed, layer, d, f, E)
    return {"router": gen.router(seed, layer, d, E),
            "shared_blob": gen.shared_blob(seed, layer, d, fs), "pool": pool,
            "d_model": d, "d_ff": f, "d_ff_shared": fs, "top_k": k}


def device_layer(L, device="cuda", act=0):
    from bit_routed_expert_tf_amd.api import DeviceLayer
    return DeviceLayer.from_arrays(L["router"], L["shared_blob"], L["pool"], L["d_model"],
                                   L["d_ff"], L["d_ff_shared"], L["top_k"], act=act,
                                   device=device)


def rel_err_floored(y_gpu, y_ref):
    """max_i |y_gpu_i - y_ref_i| / max(|y_ref_i|, rms(y_ref)) for one token,
    over the finite reference elements (the rms too).

    Elements whose fp16 reference overflows are compared separately by
    ``check_token`` (the floor would be meaningless there)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    fin = np.isfinite(y_ref)
    rms = np.sqrt(np.mean(y_ref[fin] ** 2))
    den = np.maximum(np.abs(y_ref[fin]), rms)
    return float(np.max(np.abs(y_gpu[fin] - y_ref[fin]) / den))


def check_token(y16_gpu, y_ref, tol=2e-3):
    """Compare one token's fp16 output with a reference (the fp64 oracle, or
    another fp16 output of the GPU path).

    Finite references: floored relative error <= tol, the floor being the rms
    of the finite reference elements.  Where fp16(y_ref) overflows the GPU
    must give the same infinity; within tol of the overflow threshold (65520)
    either 65504 or inf is accepted; an infinite reference element (an fp16
    reference that overflowed) must be matched exactly.  Returns the error."""
    g = np.asarray(y16_gpu, dtype=np.float16).astype(np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    thr = 65520.0
    rfin = np.isfinite(r)
    assert np.array_equal(g[~rfin], r[~rfin]), "infinite reference element not matched"
    near = rfin & (np.abs(np.abs(r) - thr) <= tol * thr)
    over = rfin & (np.abs(r) >= thr) & ~near
    assert np.all(np.isinf(g[over]) & (np.sign(g[over]) == np.sign(r[over]))), "overflow mismatch"
    ok_near = np.isinf(g[near]) | (np.abs(g[near]) == 65504.0) | \
        (np.abs(g[near] - r[near]) <= tol * np.abs(r[near]))
    assert np.all(ok_near), "near-threshold mismatch"
    fin = rfin & ~(over | near)
    assert np.all(np.isfinite(g[fin])), "unexpected non-finite output"
    rms = np.sqrt(np.mean(r[rfin] ** 2))
    den = np.maximum(np.abs(r[fin]), rms)
    err = float(np.max(np.abs(g[fin] - r[fin]) / den)) if fin.any() else 0.0
    assert err <= tol, f"floored relative error {err:.3g} > {tol}"
    return err


def check_token32(y32_gpu, y_ref, tol=2e-3):
    err = rel_err_floored(y32_gpu, y_ref)
    assert err <= tol, f"fp32 floored relative error {err:.3g} > {tol}"
    return err


def report(name, **vals):
    """One line of parity figures (shown with pytest -s; the GPU runs keep it)."""
    print(f"PARITY {name}: " + ", ".join(f"{k}={v}" for k, v in vals.items()), flush=True)
