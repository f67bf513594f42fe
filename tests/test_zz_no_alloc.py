"""The allocation-free decode step (tf_moe_layer_fwd_noalloc) against the
workspace one (tf_moe_layer_fwd), through the C ABI: the same kernels on the
same inputs, so ids, router weights and outputs must be bitwise equal.  Two
calls in a row, the second with fewer tokens (the scratch keeps the first
call's contents), then a single-token call; a step too large for the scratch
is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import device_layer, oracle_layer
from synth import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tfa():
    import bit_routed_expert_tf_amd as m
    from bit_routed_expert_tf_amd import api
    m.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return api


def _noalloc(api, D, x, forced=None):
    lib = api.load()
    T, d, k = x.shape[0], D.d_model, D.top_k
    y = torch.empty((T, d), dtype=torch.int16, device="cuda")
    y32 = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None   # noqa: E731
    rc = lib.tf_moe_layer_fwd_noalloc(ctypes.byref(D.struct), p(x), T, p(forced), p(y), p(y32),
                                      p(ids), p(w), api.stream_handle())
    assert rc == 0, lib.tf_last_error()
    return y, y32, ids, w


def _with_ws(api, D, x, forced=None):
    y, ids, w, y32 = api.tf_moe_layer_fwd(D, x, forced_ids=forced, want_y32=True)
    return y.view(torch.int16), y32, ids, w


def _same(a, b):
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u,
                           v.view(torch.int32) if v.dtype == torch.float32 else v)


def test_noalloc_matches_workspace_entry_point(tfa):
    wl = gen.WORKLOADS[1]
    d, E, k, f, fs = wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared
    print("no-alloc decode: full width, T=16 then T=3 then T=1", flush=True)
    D = device_layer(oracle_layer(wl.seed, 0, d, E, k, f, fs))
    X = torch.from_numpy(gen.tokens(wl.seed, 32, d).view(np.int16)).cuda()
    _same(_noalloc(tfa, D, X[:16]), _with_ws(tfa, D, X[:16]))
    _same(_noalloc(tfa, D, X[16:19]), _with_ws(tfa, D, X[16:19]))
    _same(_noalloc(tfa, D, X[20:21]), _with_ws(tfa, D, X[20:21]))
    F = torch.from_numpy(gen.uniform_ids(4, 0, 5, E, k)).cuda()
    _same(_noalloc(tfa, D, X[21:26], F), _with_ws(tfa, D, X[21:26], F))


def test_noalloc_small_layer_and_too_large(tfa):
    wl = gen.WORKLOADS[0]
    print("no-alloc decode: tiny layer T=7 then T=2; a step over the scratch", flush=True)
    L = oracle_layer(wl.seed, 0, wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared)
    D = device_layer(L)
    X = torch.from_numpy(gen.tokens(wl.seed, 9, wl.d_model).view(np.int16)).cuda()
    _same(_noalloc(tfa, D, X[:7]), _with_ws(tfa, D, X[:7]))
    _same(_noalloc(tfa, D, X[7:9]), _with_ws(tfa, D, X[7:9]))
    # a layer whose 16-token step needs more scratch than the library holds:
    # refused with TF_E_NOMEM before any launch (pointers are never read)
    from bit_routed_expert_tf_amd import _lib
    lib = tfa.load()
    r = _lib.tf_qmat(1 << 12, 1 << 13, 1 << 14, 1024, 4096, 8, 64)
    big = _lib.tf_moe_layer(r, 1 << 16, 1 << 20, lib.tf_expert_blob_bytes(4096, 4096), 4096,
                            4096, 4096, 1024, 16, 0)
    assert lib.tf_moe_workspace_bytes(ctypes.byref(big), 16) > (8 << 20)
    rc = lib.tf_moe_layer_fwd_noalloc(ctypes.byref(big), ctypes.c_void_p(1 << 12), 16, None,
                                      ctypes.c_void_p(1 << 12), None, ctypes.c_void_p(1 << 12),
                                      ctypes.c_void_p(1 << 12), None)
    assert rc == _lib.TF_E_NOMEM
    assert b"scratch" in lib.tf_last_error()
    # and the scratch still works after the refusal
    _same(_noalloc(tfa, D, X[:4]), _with_ws(tfa, D, X[:4]))
