"""Python binding of the C ABI: the same entry points, taking torch tensors.

Only argument marshalling happens here (pointers, sizes, the current HIP
stream); all work runs in ``libtf.so``.  torch provides device memory and
streams.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import check, load, tf_moe_layer, tf_qmat

__all__ = [
    "DeviceLayer", "workspace", "tf_expert_blob_bytes", "tf_moe_workspace_bytes",
    "tf_moe_layer_fwd", "tf_router_workspace_bytes", "tf_router_topk",
    "tf_gemv_workspace_bytes", "tf_expert_q4_gemv", "tf_prefill_workspace_bytes",
    "tf_moe_prefill_chunk", "tf_group_workspace_bytes", "tf_group_by_expert", "tf_sample_workspace_bytes", "tf_sample",
    "tf_attn_workspace_bytes", "tf_attn_decode",
    "tf_workspace_flags", "tf_workspace_zero", "SlotCache",
    "pinned_host", "stream_handle",
]


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def stream_handle(s=None):
    s = s if s is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace(nbytes, device="cuda"):
    """A zero-filled device workspace (256-byte aligned by the allocator)."""
    n = (int(nbytes) + 255) // 256 * 256
    return torch.zeros(n, dtype=torch.uint8, device=device)


def pinned_host(nbytes):
    """Pinned host memory (hipHostMalloc through torch)."""
    return torch.empty(int(nbytes), dtype=torch.uint8, pin_memory=True)


def _to_dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def tf_expert_blob_bytes(d_model, d_ff):
    return int(load().tf_expert_blob_bytes(d_model, d_ff))


class DeviceLayer:
    """Device-resident router, shared expert and expert pool of one layer,
    plus the ``tf_moe_layer`` view the C ABI takes."""

    def __init__(self, router_q, router_scale, router_bias, shared_blob, pool, d_model, d_ff,
                 d_ff_shared, n_experts, top_k, act=_lib.TF_GELU_ERF, blob_stride=None):
        self.router_q, self.router_scale, self.router_bias = router_q, router_scale, router_bias
        self.shared_blob, self.pool = shared_blob, pool
        self.d_model, self.d_ff, self.d_ff_shared = d_model, d_ff, d_ff_shared
        self.n_experts, self.top_k, self.act = n_experts, top_k, act
        self.blob_stride = blob_stride or (pool.shape[1] if pool is not None and pool.dim() == 2
                                           else tf_expert_blob_bytes(d_model, d_ff))
        self.router = tf_qmat(router_q.data_ptr(), router_scale.data_ptr(),
                              router_bias.data_ptr(), n_experts, d_model, 8, 64)
        self.struct = tf_moe_layer(self.router, shared_blob.data_ptr(),
                                   pool.data_ptr() if pool is not None else 0,
                                   self.blob_stride, d_model, d_ff, d_ff_shared, n_experts,
                                   top_k, act)

    def with_pool(self, pool_ptr, blob_stride=None):
        """Same layer, routed experts read from another pool (e.g. slot pool)."""
        s = tf_moe_layer.from_buffer_copy(self.struct)
        s.pool = pool_ptr
        if blob_stride:
            s.blob_stride = blob_stride
        return s

    @classmethod
    def from_arrays(cls, router, shared_blob, pool, d_model, d_ff, d_ff_shared, top_k,
                    act=_lib.TF_GELU_ERF, device="cuda"):
        """``router``: dict(q, scale, bias) numpy; ``shared_blob``: uint8;
        ``pool``: uint8 [E][stride] numpy or a device tensor."""
        rq = _to_dev(router["q"], device)
        rs = _to_dev(np.asarray(router["scale"], np.float16).view(np.uint16).view(np.int16), device)
        rb = _to_dev(np.asarray(router["bias"], np.float16).view(np.uint16).view(np.int16), device)
        sb = _to_dev(shared_blob, device)
        pl = pool if isinstance(pool, torch.Tensor) else _to_dev(pool, device)
        return cls(rq, rs, rb, sb, pl, d_model, d_ff, d_ff_shared, rq.shape[0], top_k, act)


def _layer_ptr(layer):
    s = layer.struct if isinstance(layer, DeviceLayer) else layer
    return ctypes.byref(s)


def tf_moe_workspace_bytes(layer, T):
    return int(load().tf_moe_workspace_bytes(_layer_ptr(layer), T))


def tf_moe_layer_fwd(layer, x, forced_ids=None, y=None, y32=None, ids=None, weights=None,
                     cache=None, layer_idx=0, ws=None, stream=None, copy_stream=None,
                     want_y32=False):
    """One decode step of ``x.shape[0]`` tokens; returns (y, ids, weights, y32)."""
    T = x.shape[0]
    dev = x.device
    d = layer.d_model if isinstance(layer, DeviceLayer) else layer.d_model
    k = layer.top_k if isinstance(layer, DeviceLayer) else layer.top_k
    if y is None:
        y = torch.empty((T, d), dtype=torch.float16, device=dev)
    if want_y32 and y32 is None:
        y32 = torch.empty((T, d), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(tf_moe_workspace_bytes(layer, T), dev)
    s = stream_handle(stream)
    cs = stream_handle(copy_stream) if copy_stream is not None else s
    check(load().tf_moe_layer_fwd(_layer_ptr(layer), _p(x), T, _p(forced_ids), _p(y), _p(y32),
                                  _p(ids), _p(weights), cache.handle if cache else None,
                                  layer_idx, s, cs, _p(ws), ws.numel()))
    return y, ids, weights, y32


def tf_router_workspace_bytes(n_experts, T):
    return int(load().tf_router_workspace_bytes(n_experts, T))


def tf_router_topk(layer, x, top_k=None, forced_ids=None, ids=None, weights=None, logits=None,
                   ws=None, stream=None):
    T = x.shape[0]
    k = top_k or layer.top_k
    E = layer.n_experts
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(tf_router_workspace_bytes(E, T), x.device)
    r = tf_qmat.from_buffer_copy(layer.router)
    check(load().tf_router_topk(ctypes.byref(r), _p(x), T, k, _p(forced_ids), _p(ids),
                                _p(weights), _p(logits), _p(ws), ws.numel(),
                                stream_handle(stream)))
    return ids, weights, logits


def tf_gemv_workspace_bytes(d_ff, P):
    return int(load().tf_gemv_workspace_bytes(d_ff, P))


def tf_expert_q4_gemv(pool, blob_stride, d_model, d_ff, slot, token, coef, x, y32,
                      act=_lib.TF_GELU_ERF, ws=None, stream=None):
    P = slot.shape[0]
    T = x.shape[0]
    if ws is None:
        ws = workspace(tf_gemv_workspace_bytes(d_ff, P), x.device)
    check(load().tf_expert_q4_gemv(_p(pool), blob_stride, d_model, d_ff, _p(slot), _p(token),
                                   _p(coef), P, _p(x), T, _p(y32), act, _p(ws), ws.numel(),
                                   stream_handle(stream)))
    return y32


def tf_prefill_workspace_bytes(layer, T):
    return int(load().tf_prefill_workspace_bytes(_layer_ptr(layer), T))


def tf_moe_prefill_chunk(layer, x, y=None, y32=None, ids=None, weights=None, ws=None,
                         stream=None, want_y32=False):
    T = x.shape[0]
    d, k = layer.d_model, layer.top_k
    dev = x.device
    if y is None:
        y = torch.empty((T, d), dtype=torch.float16, device=dev)
    if want_y32 and y32 is None:
        y32 = torch.empty((T, d), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(tf_prefill_workspace_bytes(layer, T), dev)
    check(load().tf_moe_prefill_chunk(_layer_ptr(layer), _p(x), T, _p(y), _p(y32), _p(ids),
                                      _p(weights), stream_handle(stream), _p(ws), ws.numel()))
    return y, ids, weights, y32


def tf_group_workspace_bytes(n_experts, T, top_k):
    return int(load().tf_group_workspace_bytes(n_experts, T, top_k))


def tf_group_by_expert(ids, n_experts, counts=None, offsets=None, pairs=None, ws=None,
                       stream=None):
    T, k = ids.shape
    dev = ids.device
    if counts is None:
        counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    if pairs is None:
        pairs = torch.empty(T * k, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(tf_group_workspace_bytes(n_experts, T, k), dev)
    check(load().tf_group_by_expert(_p(ids), T, k, n_experts, _p(counts), _p(offsets), _p(pairs),
                                    _p(ws), ws.numel(), stream_handle(stream)))
    return counts, offsets, pairs


def tf_sample_workspace_bytes(V, T, top_k):
    return int(load().tf_sample_workspace_bytes(V, T, top_k))


def tf_sample(logits, temperature, top_k, top_p, u=None, ids=None, ws=None, stream=None):
    """ids [T] int32 from logits [T][V] fp32 (u [T] fp64, NULL only when
    temperature is 0)."""
    T, V = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty(T, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(tf_sample_workspace_bytes(V, T, top_k), dev)
    check(load().tf_sample(_p(logits), V, T, float(temperature), top_k, float(top_p),
                           _p(u), _p(ids), _p(ws), ws.numel(),
                           stream_handle(stream)))
    return ids


def tf_attn_workspace_bytes(H, D, S):
    return int(load().tf_attn_workspace_bytes(H, D, S))


def tf_attn_decode(q, k_new, v_new, k_cache, v_cache, pos, ring, scale=None, out=None, ws=None,
                   stream=None):
    """q [H][D], k_new/v_new [G][D], caches [G][S][D] (fp16 bit patterns as
    int16 or float16 tensors); returns out [H][D] fp32."""
    H, D = q.shape
    G, S, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / D ** 0.5
    if out is None:
        out = torch.empty((H, D), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(tf_attn_workspace_bytes(H, D, S), q.device)
    check(load().tf_attn_decode(_p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), H, G, D, S,
                                pos, int(bool(ring)), float(scale), _p(out), _p(ws), ws.numel(),
                                stream_handle(stream)))
    return out


def tf_workspace_zero(ws, stream=None):
    check(load().tf_workspace_zero(_p(ws), ws.numel(), stream_handle(stream)))


def tf_workspace_flags(ws, stream=None):
    v = ctypes.c_int32(0)
    check(load().tf_workspace_flags(_p(ws), ctypes.byref(v), stream_handle(stream)))
    return v.value


class SlotCache:
    """Owning wrapper of a ``tf_slot_cache`` handle."""

    def __init__(self, n_layers, n_experts, n_slots, top_k, blob_stride, slot_pool, host_pool,
                 trace_cap=0, policy="lfu"):
        self.slot_pool, self.host_pool = slot_pool, host_pool
        self.n_layers, self.n_experts, self.n_slots, self.top_k = n_layers, n_experts, n_slots, top_k
        self.blob_stride = blob_stride
        h = ctypes.c_void_p()
        check(load().tf_slot_cache_create(n_layers, n_experts, n_slots, top_k, blob_stride,
                                          _p(slot_pool), _p(host_pool), trace_cap,
                                          ctypes.byref(h)))
        self.handle = h
        self.set_policy(policy)

    def set_policy(self, policy):
        """Eviction rule of later lookups: "lfu" (default) or "lru"."""
        code = {"lfu": _lib.TF_SLOT_LFU, "lru": _lib.TF_SLOT_LRU}[policy]
        check(load().tf_slot_cache_set_policy(self.handle, code))

    def close(self):
        if self.handle:
            load().tf_slot_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lookup(self, layer, ids, slots=None, stream=None):
        check(load().tf_slot_cache_lookup(self.handle, layer, _p(ids), ids.numel(), _p(slots),
                                          stream_handle(stream)))

    def fill(self, layer, copy_stream=None, event=None):
        n = ctypes.c_int32(0)
        ev = ctypes.c_void_p(event.cuda_event) if event is not None else None
        check(load().tf_slot_cache_fill(self.handle, layer, stream_handle(copy_stream), ev,
                                        ctypes.byref(n)))
        return n.value

    def trace(self, layer, cap):
        hit = np.zeros(cap, dtype=np.int8)
        slot = np.zeros(cap, dtype=np.int16)
        n = ctypes.c_int64(0)
        check(load().tf_slot_cache_trace(self.handle, layer, ctypes.c_void_p(hit.ctypes.data),
                                         ctypes.c_void_p(slot.ctypes.data), cap, ctypes.byref(n)))
        return hit[:n.value].astype(bool), slot[:n.value]

    def reset(self):
        check(load().tf_slot_cache_reset(self.handle))

    def bytes_filled(self):
        return int(load().tf_slot_cache_bytes_filled(self.handle))


    def set_copy_engine(self, engine):
        """"kernel" (one launch per fill or prefetch reading the mapped host
        pool, the default), "dma" (one hipMemcpyAsync per blob) or "device"
        (the fill kernel reads the miss list on the GPU: no host wait)."""
        code = {"dma": _lib.TF_SLOT_COPY_DMA, "kernel": _lib.TF_SLOT_COPY_KERNEL,
                "device": _lib.TF_SLOT_COPY_DEVICE}[engine]
        check(load().tf_slot_cache_set_copy_engine(self.handle, code))

    def set_prefetch(self, buffers, n_buffers):
        """Speculative fill: ``buffers`` is a device uint8 tensor of
        n_layers * n_buffers * blob_stride bytes (kept alive here); 0 turns it off."""
        if n_buffers and buffers.numel() < self.n_layers * n_buffers * self.blob_stride:
            raise ValueError("prefetch buffers too small")
        self.pf_buffers = buffers if n_buffers else None
        check(load().tf_slot_cache_set_prefetch(self.handle, _p(self.pf_buffers), n_buffers))

    def prefetch(self, layer, ids, copy_stream=None):
        """Copy the predicted experts of ``layer`` (host ints) that are not
        resident into free buffers; returns the number of copies issued."""
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
        n = ctypes.c_int32(0)
        check(load().tf_slot_cache_prefetch(self.handle, layer, ctypes.c_void_p(a.ctypes.data),
                                            a.size, stream_handle(copy_stream), ctypes.byref(n)))
        return n.value

    def prefetch_stats(self):
        """(host->device prefetch bytes, buffers used by fills, buffers unused)."""
        v = [ctypes.c_int64(0) for _ in range(3)]
        check(load().tf_slot_cache_prefetch_stats(self.handle, *[ctypes.byref(x) for x in v]))
        return tuple(int(x.value) for x in v)
