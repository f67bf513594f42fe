"""The C ABI library loads and exports every entry point of include/tf.h;
argument checks that return before any HIP call behave as documented.
Runs on the CPU (no GPU call is made)."""
import ctypes
import os
import re

import pytest

import bit_routed_expert_tf_amd as tfa
from bit_routed_expert_tf_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "tf.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(tf_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_header_and_binding_agree():
    assert sorted(_lib.exported_names()) == _header_functions()


def test_library_exports_every_declared_symbol():
    lib = tfa.load()
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_blob_bytes_and_view():
    lib = tfa.load()
    assert lib.tf_expert_blob_bytes(2816, 704) == 3_345_408
    assert lib.tf_expert_blob_bytes(256, 128) == 55_296
    assert lib.tf_expert_blob_bytes(2816, 2816) == 13_381_632
    assert lib.tf_expert_blob_bytes(100, 704) == 0
    g, u, d = _lib.tf_qmat(), _lib.tf_qmat(), _lib.tf_qmat()
    base = 1 << 20
    assert lib.tf_expert_view(ctypes.c_void_p(base), 2816, 704, ctypes.byref(g), ctypes.byref(u),
                              ctypes.byref(d)) == 0
    assert (g.n, g.k, d.n, d.k, g.bits, g.group) == (704, 2816, 2816, 704, 4, 64)
    assert g.scale - g.q == 991_232 and g.bias - g.scale == 61_952
    assert u.q - g.q == 1_115_136 and d.q - u.q == 1_115_136
    assert lib.tf_expert_view(ctypes.c_void_p(base), 2816, 700, ctypes.byref(g), ctypes.byref(u),
                              ctypes.byref(d)) == _lib.TF_E_SHAPE


def _layer(**kw):
    r = _lib.tf_qmat(1 << 12, 1 << 13, 1 << 14, 128, 2816, 8, 64)
    L = _lib.tf_moe_layer(r, 1 << 16, 1 << 20, 3_345_408, 2816, 704, 2816, 128, 8, 0)
    for k, v in kw.items():
        setattr(L, k, v)
    return L


@pytest.mark.parametrize("field,value,status", [
    ("top_k", 0, _lib.TF_E_SHAPE), ("top_k", 17, _lib.TF_E_SHAPE),
    ("n_experts", 4, _lib.TF_E_SHAPE), ("d_model", 2800, _lib.TF_E_SHAPE),
    ("d_ff", 8192, _lib.TF_E_SHAPE), ("blob_stride", 3_345_408 + 16, _lib.TF_E_ALIGN),
    ("pool", (1 << 20) + 64, _lib.TF_E_ALIGN), ("act", 7, _lib.TF_E_ARG),
])
def test_layer_fwd_rejects_bad_layers_before_any_launch(field, value, status):
    lib = tfa.load()
    L = _layer(**{field: value})
    if field == "n_experts":
        L.router.n = value
    if field == "d_model":
        L.router.k = value
    x = ctypes.c_void_p(1 << 24)
    rc = lib.tf_moe_layer_fwd(ctypes.byref(L), x, 1, None, x, None, x, x, None, 0, None, None,
                              ctypes.c_void_p(1 << 28), 1 << 26)
    assert rc == status, lib.tf_last_error()


def test_layer_fwd_argument_errors():
    lib = tfa.load()
    L = _layer()
    x = ctypes.c_void_p(1 << 24)
    ws = ctypes.c_void_p(1 << 28)
    fwd = lambda *a: lib.tf_moe_layer_fwd(ctypes.byref(L), *a)
    assert fwd(x, 0, None, x, None, x, x, None, 0, None, None, ws, 1 << 26) == _lib.TF_OK  # T=0
    assert fwd(x, 17, None, x, None, x, x, None, 0, None, None, ws, 1 << 26) == _lib.TF_E_ARG
    assert fwd(None, 1, None, x, None, x, x, None, 0, None, None, ws, 1 << 26) == _lib.TF_E_ARG
    assert fwd(ctypes.c_void_p((1 << 24) + 2), 1, None, x, None, x, x, None, 0, None, None, ws,
               1 << 26) == _lib.TF_E_ALIGN
    need = lib.tf_moe_workspace_bytes(ctypes.byref(L), 1)
    assert need > 0
    assert fwd(x, 1, None, x, None, x, x, None, 0, None, None, ws, need - 1) == _lib.TF_E_NOMEM
    assert b"workspace" in lib.tf_last_error()


def test_router_and_gemv_argument_errors():
    lib = tfa.load()
    r = _lib.tf_qmat(1 << 12, 1 << 13, 1 << 14, 128, 2816, 4, 64)   # wrong bits
    x = ctypes.c_void_p(1 << 24)
    assert lib.tf_router_topk(ctypes.byref(r), x, 1, 8, None, x, x, None, ctypes.c_void_p(1 << 28),
                              1 << 20, None) == _lib.TF_E_SHAPE
    r.bits = 8
    assert lib.tf_router_topk(ctypes.byref(r), x, 0, 8, None, x, x, None, None, 0, None) == 0
    assert lib.tf_router_topk(ctypes.byref(r), x, 1, 0, None, x, x, None, ctypes.c_void_p(1 << 28),
                              1 << 20, None) == _lib.TF_E_SHAPE
    g = lib.tf_expert_q4_gemv
    assert g(None, 0, 2816, 704, x, None, None, 0, x, 0, x, 0, x, 0, None) == 0          # P=0
    assert g(ctypes.c_void_p(1 << 20), 3_345_408, 2816, 704, x, None, None, 2, x, 3, x, 0,
             ctypes.c_void_p(1 << 28), 1 << 26, None) == _lib.TF_E_ARG                  # T != P
    assert g(ctypes.c_void_p(1 << 20), 3_345_400, 2816, 704, x, None, None, 2, x, 2, x, 0,
             ctypes.c_void_p(1 << 28), 1 << 26, None) == _lib.TF_E_ALIGN


def test_slot_cache_create_argument_errors():
    lib = tfa.load()
    h = ctypes.c_void_p()
    p = ctypes.c_void_p(1 << 20)
    assert lib.tf_slot_cache_create(30, 128, 4, 8, 3_345_408, p, p, 0, ctypes.byref(h)) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_create(30, 128, 16, 8, 3_345_400, p, p, 0, ctypes.byref(h)) == _lib.TF_E_ALIGN
    assert lib.tf_slot_cache_create(0, 128, 16, 8, 3_345_408, p, p, 0, ctypes.byref(h)) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_lookup(None, 0, p, 8, None, None) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_fill(None, 0, None, None, None) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_bytes_filled(None) == -1
    assert lib.tf_slot_cache_set_policy(None, _lib.TF_SLOT_LRU) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_set_prefetch(None, p, 8) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_prefetch(None, 0, p, 8, None, None) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_prefetch_stats(None, None, None, None) == _lib.TF_E_ARG
    assert lib.tf_slot_cache_set_copy_engine(None, _lib.TF_SLOT_COPY_KERNEL) == _lib.TF_E_ARG


def test_group_argument_errors():
    lib = tfa.load()
    p = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 28)
    need = lib.tf_group_workspace_bytes(128, 128, 8)
    assert need >= 256 + 4 * 16 * (128 + 1024)
    g = lib.tf_group_by_expert
    assert g(p, 0, 8, 128, p, p, p, ws, need, None) == 0                              # T=0
    assert g(p, 129, 8, 128, p, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE          # T > 128
    assert g(p, 4, 17, 128, p, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE           # k > 16
    assert g(p, 4, 8, 4, p, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE              # E < k
    assert g(p, 4, 8, 1025, p, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE           # E > 1024
    assert g(None, 4, 8, 128, p, p, p, ws, 1 << 30, None) == _lib.TF_E_ARG
    assert g(p, 4, 8, 128, p, p, p, ctypes.c_void_p((1 << 28) + 4), 1 << 30, None) == _lib.TF_E_ALIGN
    assert g(p, 128, 8, 128, p, p, p, ws, need - 1, None) == _lib.TF_E_NOMEM
    assert b"workspace" in lib.tf_last_error()


def test_sample_argument_errors():
    lib = tfa.load()
    p = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 28)
    f = lib.tf_sample
    need = lib.tf_sample_workspace_bytes(262144, 16, 64)
    assert need == 16 * 64 * 64 * 8 == lib.tf_sample_workspace_bytes(262144, 16, 1)
    assert f(p, 262144, 0, 0.7, 64, 0.95, p, p, ws, need, None) == 0                 # T=0
    assert f(p, 262144, 4097, 0.7, 64, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_ARG
    assert f(p, 262145, 1, 0.7, 64, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE  # V > 2**18
    assert f(p, 262145, 1, 0.7, 8, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE
    assert f(p, 100, 1, 0.7, 65, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE    # k > 64
    assert f(p, 100, 1, 0.7, 0, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE     # k = 0
    assert f(p, 7, 1, 0.7, 8, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_SHAPE       # V < k
    assert f(p, 100, 1, -0.5, 8, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_ARG
    assert f(p, 100, 1, 0.7, 8, 0.0, p, p, ws, 1 << 30, None) == _lib.TF_E_ARG
    assert f(p, 100, 1, 0.7, 8, 1.5, p, p, ws, 1 << 30, None) == _lib.TF_E_ARG
    assert f(p, 100, 1, 0.7, 8, 0.95, None, p, ws, 1 << 30, None) == _lib.TF_E_ARG     # u NULL
    assert f(None, 100, 1, 0.7, 8, 0.95, p, p, ws, 1 << 30, None) == _lib.TF_E_ARG
    assert f(ctypes.c_void_p((1 << 20) + 2), 100, 1, 0.7, 8, 0.95, p, p, ws, 1 << 30,
             None) == _lib.TF_E_ALIGN
    assert f(p, 262144, 16, 0.7, 64, 0.95, p, p, ws, need - 1, None) == _lib.TF_E_NOMEM
    assert b"workspace" in lib.tf_last_error()


def test_attn_argument_errors():
    lib = tfa.load()
    p = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 28)
    f = lib.tf_attn_decode
    need = lib.tf_attn_workspace_bytes(16, 256, 4096)
    assert need >= 16 * 128 * 258 * 4
    assert f(p, p, p, p, p, 16, 8, 96, 4096, 0, 0, 0.0625, p, ws, need, None) == _lib.TF_E_SHAPE   # D
    assert f(p, p, p, p, p, 24, 8, 256, 4096, 0, 0, 0.0625, p, ws, need, None) == _lib.TF_E_SHAPE  # H = 3G
    assert f(p, p, p, p, p, 16, 8, 256, 0, 0, 0, 0.0625, p, ws, need, None) == _lib.TF_E_SHAPE     # S
    assert f(p, p, p, p, p, 16, 8, 256, 4096, 4096, 0, 0.0625, p, ws, need, None) == _lib.TF_E_ARG  # linear full
    assert f(p, p, p, p, p, 16, 8, 256, 4096, -1, 1, 0.0625, p, ws, need, None) == _lib.TF_E_ARG
    assert f(p, p, p, p, p, 16, 8, 256, 4096, 5, 1, 0.0, p, ws, need, None) == _lib.TF_E_ARG       # scale
    assert f(None, p, p, p, p, 16, 8, 256, 4096, 5, 1, 0.0625, p, ws, need, None) == _lib.TF_E_ARG
    assert f(ctypes.c_void_p((1 << 20) + 8), p, p, p, p, 16, 8, 256, 4096, 5, 1, 0.0625, p, ws, need,
             None) == _lib.TF_E_ALIGN
    assert f(p, p, p, p, p, 16, 8, 256, 4096, 5, 1, 0.0625, p, ws, need - 1, None) == _lib.TF_E_NOMEM


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: loading a library that is not there raises, naming the build."""
    import subprocess
    import sys
    code = ("import bit_routed_expert_tf_amd._lib as L\n"
            "try:\n"
            f"    L.load({str(tmp_path / 'libtf.so')!r})\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert "raised:" in r.stdout and "build()" in r.stdout, r.stdout + r.stderr
