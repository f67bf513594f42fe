"""ctypes binding of ``libtf.so`` (include/tf.h).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the HIP stream.  Every step of the layer runs in the
library's HIP kernels; nothing here computes.  If the library is missing,
loading fails with an error -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# TF_LIBRARY may name another build of the same sources (the host-sanitizer
# test's); it must exist like the default one -- there is no fallback.
LIB_PATH = os.environ.get("TF_LIBRARY") or os.path.join(HERE, "libtf.so")

TF_OK, TF_E_ARG, TF_E_SHAPE, TF_E_ALIGN, TF_E_HIP, TF_E_NOMEM, TF_E_STATE = range(7)
STATUS_NAMES = {0: "TF_OK", 1: "TF_E_ARG", 2: "TF_E_SHAPE", 3: "TF_E_ALIGN", 4: "TF_E_HIP",
                5: "TF_E_NOMEM", 6: "TF_E_STATE"}
TF_GELU_ERF, TF_GELU_TANH = 0, 1
TF_FLAG_ID_RANGE, TF_FLAG_ID_REPEAT = 1, 2
TF_KERNEL_ROUTER_SHARED_GATEUP, TF_KERNEL_ROUTED_GATEUP_SHARED_DOWN, TF_KERNEL_DOWN_COMBINE = 1, 2, 4
TF_KERNEL_PREFILL_DOWN, TF_KERNEL_PREFILL_COMBINE = 8, 16
TF_KERNEL_PREFILL_GATEUP, TF_KERNEL_GROUP = 32, 64
TF_KERNEL_SAMPLE_PART, TF_KERNEL_SAMPLE_FINAL = 128, 256
TF_KERNEL_ATTN_CHUNK, TF_KERNEL_ATTN_COMBINE = 512, 1024
TF_KERNEL_ROUTER_TOPK = 2048
TF_SLOT_LFU, TF_SLOT_LRU = 0, 1
TF_SLOT_COPY_DMA, TF_SLOT_COPY_KERNEL, TF_SLOT_COPY_DEVICE = 0, 1, 2

c_void_p, c_int32, c_int64, c_size_t = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class tf_qmat(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("scale", c_void_p), ("bias", c_void_p), ("n", c_int32),
                ("k", c_int32), ("bits", c_int32), ("group", c_int32)]


class tf_moe_layer(ctypes.Structure):
    _fields_ = [("router", tf_qmat), ("shared_blob", c_void_p), ("pool", c_void_p),
                ("blob_stride", c_size_t), ("d_model", c_int32), ("d_ff", c_int32),
                ("d_ff_shared", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("act", c_int32)]


class TFError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


# name -> (restype, argtypes)
_SIGS = {
    "tf_last_error": (ctypes.c_char_p, []),
    "tf_version": (ctypes.c_char_p, []),
    "tf_expert_blob_bytes": (c_size_t, [c_int32, c_int32]),
    "tf_expert_view": (c_int32, [c_void_p, c_int32, c_int32, ctypes.POINTER(tf_qmat),
                                 ctypes.POINTER(tf_qmat), ctypes.POINTER(tf_qmat)]),
    "tf_workspace_zero": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "tf_workspace_flags": (c_int32, [c_void_p, ctypes.POINTER(c_int32), c_void_p]),
    "tf_router_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "tf_router_topk": (c_int32, [ctypes.POINTER(tf_qmat), c_void_p, c_int32, c_int32, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "tf_gemv_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "tf_expert_q4_gemv": (c_int32, [c_void_p, c_size_t, c_int32, c_int32, c_void_p, c_void_p,
                                    c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                                    c_void_p, c_size_t, c_void_p]),
    "tf_moe_workspace_bytes": (c_size_t, [ctypes.POINTER(tf_moe_layer), c_int32]),
    "tf_moe_layer_fwd": (c_int32, [ctypes.POINTER(tf_moe_layer), c_void_p, c_int32, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_void_p, c_void_p, c_size_t]),
    "tf_moe_layer_fwd_noalloc": (c_int32, [ctypes.POINTER(tf_moe_layer), c_void_p, c_int32,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p]),
    "tf_prefill_workspace_bytes": (c_size_t, [ctypes.POINTER(tf_moe_layer), c_int32]),
    "tf_group_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "tf_group_by_expert": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_size_t, c_void_p]),
    "tf_moe_prefill_chunk": (c_int32, [ctypes.POINTER(tf_moe_layer), c_void_p, c_int32,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t]),
    "tf_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "tf_attn_decode": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                 c_int32, c_int32, c_int32, c_int32, c_int32, ctypes.c_float,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
    "tf_sample_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "tf_sample": (c_int32, [c_void_p, c_int32, c_int32, ctypes.c_float, c_int32, ctypes.c_float,
                            c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "tf_profile_kernel": (c_int32, [c_int32, c_void_p, c_void_p]),
    "tf_profile_stream_read": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "tf_slot_cache_create": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_size_t, c_void_p,
                                       c_void_p, c_int64, ctypes.POINTER(c_void_p)]),
    "tf_slot_cache_destroy": (None, [c_void_p]),
    "tf_slot_cache_lookup": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "tf_slot_cache_fill": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p,
                                     ctypes.POINTER(c_int32)]),
    "tf_slot_cache_trace": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int64,
                                      ctypes.POINTER(c_int64)]),
    "tf_slot_cache_reset": (c_int32, [c_void_p]),
    "tf_slot_cache_bytes_filled": (c_int64, [c_void_p]),
    "tf_slot_cache_set_policy": (c_int32, [c_void_p, c_int32]),
    "tf_slot_cache_set_prefetch": (c_int32, [c_void_p, c_void_p, c_int32]),
    "tf_slot_cache_set_copy_engine": (c_int32, [c_void_p, c_int32]),
    "tf_slot_cache_prefetch": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                                         ctypes.POINTER(c_int32)]),
    "tf_slot_cache_prefetch_stats": (c_int32, [c_void_p, ctypes.POINTER(c_int64),
                                               ctypes.POINTER(c_int64), ctypes.POINTER(c_int64)]),
}

_lib = None
_lock = threading.Lock()


def load(path=LIB_PATH):
    """Load libtf.so and declare every exported entry point."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                                   "(the HIP library is required; there is no fallback)")
            lib = ctypes.CDLL(path)
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def exported_names():
    return list(_SIGS)


def check(status):
    if status != TF_OK:
        raise TFError(status, load().tf_last_error().decode(errors="replace"))
    return status
