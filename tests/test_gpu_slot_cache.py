"""Slot-cache path on the GPU: LFU lookup, miss fill, cached decode.

Bars: the hit/slot sequence of every layer equals the oracle's LFU replay
bitwise; a cached decode step is bitwise identical to the same step with all
experts resident (the kernels read the same bytes from another pool, moved
by the copy kernel or by DMA); sampled tokens match the fp64 oracle within
the floored 2e-3; the bytes copied equal misses x blob stride, split between
fills and prefetches as the predictions allow.  Every layer of a token consumes that token's x, and
routing is forced by per-layer Zipf(1.1) popularity.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import check_token
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


def _stack(api, seed, L, d, E, k, f, fs):
    """Per-layer router/shared on the device, the expert pool pinned on the
    host ([L][E][stride]) and the same pool resident on the device."""
    stride = (gen.blob_bytes(d, f) + 255) // 256 * 256
    host = api.pinned_host(L * E * stride)
    hv = host.numpy().reshape(L, E, stride)
    layers = []
    for l in range(L):
        gen.expert_pool(seed, l, d, f, E, stride=stride, out=hv[l])
        layers.append({"router": gen.router(seed, l, d, E),
                       "shared_blob": gen.shared_blob(seed, l, d, fs), "pool": hv[l],
                       "d_model": d, "d_ff": f, "d_ff_shared": fs, "top_k": k})
    resident = host.cuda().view(L, E, stride)
    dls = [api.DeviceLayer.from_arrays(Ld["router"], Ld["shared_blob"], resident[l], d, f, fs, k)
           for l, Ld in enumerate(layers)]
    return stride, host, layers, dls


def _predicted(ids, l, t, mode, rng, E):
    """Predicted ids of layer l at token t: exact, or with half replaced."""
    p = ids[l][t].copy()
    if mode == "noisy":
        j = rng.choice(p.size, size=p.size // 2, replace=False)
        p[j] = rng.integers(0, E, size=j.size)
    return p


def _run(api, seed, L, d, E, k, f, fs, S, T, check_tokens, policy="lfu", prefetch=None,
         engine="kernel"):
    stride, host, layers, dls = _stack(api, seed, L, d, E, k, f, fs)
    ids = np.stack([gen.zipf_ids(seed, l, T, E, k) for l in range(L)])      # [L][T][k]
    x = gen.tokens(seed, T, d)
    slot_pool = torch.empty(L * S * stride, dtype=torch.uint8, device="cuda")
    cache = api.SlotCache(L, E, S, k, stride, slot_pool, host, trace_cap=T, policy=policy)
    cache.set_copy_engine(engine)
    copy = torch.cuda.Stream()
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    ft = torch.from_numpy(ids).cuda()
    ws = api.workspace(api.tf_moe_workspace_bytes(dls[0], 1))
    ws_r = api.workspace(api.tf_moe_workspace_bytes(dls[0], 1))
    y_c = torch.empty((L, T, d), dtype=torch.float16, device="cuda")
    y_r = torch.empty_like(y_c)
    id_c = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
    w_c = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    id_r, w_r = torch.empty_like(id_c), torch.empty_like(w_c)
    rng = np.random.default_rng([seed, 77])
    if prefetch:
        pf_buf = torch.empty(L * k * stride, dtype=torch.uint8, device="cuda")
        cache.set_prefetch(pf_buf, k)
        cache.prefetch(0, _predicted(ids, 0, 0, prefetch, rng, E), copy)
    for t in range(T):
        for l in range(L):
            api.tf_moe_layer_fwd(dls[l], xt[t:t + 1], forced_ids=ft[l, t:t + 1], y=y_c[l, t:t + 1],
                                 ids=id_c[l, t:t + 1], weights=w_c[l, t:t + 1], cache=cache,
                                 layer_idx=l, ws=ws, copy_stream=copy)
            nl, nt = (l + 1, t) if l + 1 < L else (0, t + 1)
            if prefetch and nt < T:
                cache.prefetch(nl, _predicted(ids, nl, nt, prefetch, rng, E), copy)
            api.tf_moe_layer_fwd(dls[l], xt[t:t + 1], forced_ids=ft[l, t:t + 1], y=y_r[l, t:t + 1],
                                 ids=id_r[l, t:t + 1], weights=w_r[l, t:t + 1], ws=ws_r)
    torch.cuda.synchronize()
    assert api.tf_workspace_flags(ws) == 0 and api.tf_workspace_flags(ws_r) == 0
    assert np.array_equal(id_c.cpu().numpy(), ids)
    assert torch.equal(y_c.view(torch.int16), y_r.view(torch.int16)), "cached != resident"
    assert torch.equal(w_c, w_r)
    misses = 0
    for l in range(L):
        hit, slot = cache.trace(l, T * k)
        h_ref, s_ref, _, _ = oracle.lfu_replay(ids[l], S, E, policy=policy)
        assert np.array_equal(hit.reshape(T, k), h_ref), f"layer {l}: hit sequence"
        assert np.array_equal(slot.reshape(T, k), s_ref), f"layer {l}: slot sequence"
        misses += int((~h_ref).sum())
    pf_bytes, used, wasted = cache.prefetch_stats()
    assert cache.bytes_filled() + used * stride == misses * stride
    assert pf_bytes == (used + wasted) * stride
    if prefetch == "exact":      # every miss was predicted and nothing else fetched
        assert cache.bytes_filled() == 0 and used == misses and wasted == 0
    elif prefetch == "noisy":
        assert 0 < used < misses and wasted > 0
    yc = y_c.cpu().view(torch.int16).numpy().view(np.float16)
    for l in range(L):
        ref = oracle.moe_tokens(layers[l], x[check_tokens], ids[l][check_tokens])
        for i, t in enumerate(check_tokens):
            check_token(yc[l, t], ref["y"][i])
    # reset replays the same sequence from an empty cache
    cache.reset()
    for t in range(min(T, 8)):
        api.tf_moe_layer_fwd(dls[0], xt[t:t + 1], forced_ids=ft[0, t:t + 1], y=y_c[0, t:t + 1],
                             ids=id_c[0, t:t + 1], weights=w_c[0, t:t + 1], cache=cache,
                             layer_idx=0, ws=ws, copy_stream=copy)
    torch.cuda.synchronize()
    hit, slot = cache.trace(0, T * k)
    h_ref, s_ref, _, _ = oracle.lfu_replay(ids[0][:min(T, 8)], S, E, policy=policy)
    assert np.array_equal(hit.reshape(-1, k), h_ref) and np.array_equal(slot.reshape(-1, k), s_ref)
    assert torch.equal(y_c[0, :min(T, 8)].view(torch.int16), y_r[0, :min(T, 8)].view(torch.int16))
    cache.close()
    return misses / (L * T * k)


def test_slot_cache_small_stack(tfa):
    print("slot cache: d=256 E=32 k=4 f=128 fs=256 S=8 L=3 T=96", flush=True)
    miss = _run(tfa, 2, L=3, d=256, E=32, k=4, f=128, fs=256, S=8, T=96, check_tokens=[0, 41, 95])
    assert 0.0 < miss < 1.0


def test_slot_cache_ragged_shapes(tfa):
    print("slot cache: d=320 E=12 k=3 f=192 fs=320 S=5 L=2 T=40", flush=True)
    _run(tfa, 5, L=2, d=320, E=12, k=3, f=192, fs=320, S=5, T=40, check_tokens=[0, 39])


@pytest.mark.parametrize("engine", ["dma", "kernel", "device"])
def test_slot_cache_full_width(tfa, engine):
    # the slot-cache workload's shapes (d=2816, 128 experts, top-8, 16 slots)
    # on two layers and 48 tokens, blobs moved by the copy kernel, by DMA or
    # by the kernel that reads the miss list on the GPU
    print(f"slot cache: {engine} d=2816 E=128 k=8 f=704 fs=2816 S=16 L=2 T=48", flush=True)
    miss = _run(tfa, 2, L=2, d=2816, E=128, k=8, f=704, fs=2816, S=16, T=48,
                check_tokens=[0, 47], engine=engine)
    assert 0.2 < miss < 0.9


@pytest.mark.parametrize("S,policy,E", [(8, "lru", 32), (4, "lfu", 32), (4, "lru", 32),
                                         (16, "lru", 32), (32, "lfu", 96), (32, "lru", 96)])
def test_slot_cache_policies_and_sizes(tfa, S, policy, E):
    """The LRU reading and other slot counts, up to the largest (32 slots, the
    sweep's top size, with more experts than slots so that victims are
    chosen): hit/slot sequences equal the oracle's replay of the same rule,
    cached outputs equal resident ones."""
    print(f"slot cache: {policy} S={S} d=256 E={E} k=4 L=2 T=96", flush=True)
    miss = _run(tfa, 5, L=2, d=256, E=E, k=4, f=128, fs=256, S=S, T=96, check_tokens=[0, 95],
                policy=policy)
    assert 0.0 < miss < 1.0


@pytest.mark.parametrize("S,policy,E,L", [(8, "lfu", 32, 3), (32, "lru", 96, 2), (5, "lfu", 12, 2)])
def test_slot_cache_device_engine(tfa, S, policy, E, L):
    """Fills planned on the GPU (no host wait between lookup and copy): the
    same hit/slot sequences, outputs and byte count as the host-driven fills."""
    print(f"slot cache: device engine {policy} S={S} d=256 E={E} k=4 L={L} T=80", flush=True)
    miss = _run(tfa, 8, L=L, d=256, E=E, k=4, f=128, fs=256, S=S, T=80, check_tokens=[0, 79],
                policy=policy, engine="device")
    assert 0.0 < miss < 1.0


def test_slot_cache_engine_state(tfa):
    """The device engine refuses prefetch buffers (and the reverse), and no
    engine change is taken between a lookup and its fill."""
    from bit_routed_expert_tf_amd import _lib
    L, E, S, k, stride = 2, 16, 8, 4, 4096
    host = tfa.pinned_host(L * E * stride)
    host.copy_((torch.arange(host.numel()) % 251).to(torch.uint8))
    pool = torch.zeros(L * S * stride, dtype=torch.uint8, device="cuda")
    buf = torch.zeros(L * k * stride, dtype=torch.uint8, device="cuda")
    cache = tfa.SlotCache(L, E, S, k, stride, pool, host, trace_cap=4)
    cache.set_copy_engine("device")
    with pytest.raises(_lib.TFError, match="host-driven"):
        cache.set_prefetch(buf, k)
    cache.set_copy_engine("kernel")
    cache.set_prefetch(buf, k)
    with pytest.raises(_lib.TFError, match="prefetch"):
        cache.set_copy_engine("device")
    cache.set_prefetch(buf, 0)
    cache.set_copy_engine("device")
    ids = torch.tensor([3, 1, 4, 9], dtype=torch.int32, device="cuda")
    cache.lookup(0, ids)
    with pytest.raises(_lib.TFError, match="not yet filled"):
        cache.set_copy_engine("kernel")
    assert cache.fill(0) == -1          # the count stays on the GPU
    torch.cuda.synchronize()
    assert cache.bytes_filled() == 4 * stride
    cache.lookup(0, ids)                 # all four resident now
    cache.fill(0)
    torch.cuda.synchronize()
    assert cache.bytes_filled() == 4 * stride
    hit, slot = cache.trace(0, 2 * k)
    assert hit.tolist() == [False] * 4 + [True] * 4 and slot.tolist() == [0, 1, 2, 3] * 2
    assert torch.equal(pool[:4 * stride].cpu(),
                       host[torch.cat([torch.arange(e * stride, (e + 1) * stride) for e in (3, 1, 4, 9)])])
    assert _lib.TF_SLOT_COPY_DEVICE == 2
    cache.close()


@pytest.mark.parametrize("mode,engine,policy", [("exact", "kernel", "lfu"), ("noisy", "kernel", "lfu"),
                                                ("noisy", "dma", "lfu"), ("noisy", "kernel", "lru")])
def test_slot_cache_prefetch(tfa, mode, engine, policy):
    """Speculative fill of the next layer's predicted experts: the hit/slot
    sequences still equal the oracle's replay and the outputs the resident
    ones; with exact predictions every miss is served from a buffer (no
    host->device copy at fill time), with half the predictions wrong the
    rest go over the host path and the unused buffers are counted."""
    print(f"slot cache: prefetch {mode} {engine} {policy} d=256 E=32 k=4 S=8 L=3 T=64", flush=True)
    _run(tfa, 6, L=3, d=256, E=32, k=4, f=128, fs=256, S=8, T=64, check_tokens=[0, 63],
         prefetch=mode, engine=engine, policy=policy)


def test_slot_cache_prefetch_full_width(tfa):
    print("slot cache: prefetch exact d=2816 E=128 k=8 S=16 L=2 T=24", flush=True)
    _run(tfa, 3, L=2, d=2816, E=128, k=8, f=704, fs=2816, S=16, T=24, check_tokens=[0, 23],
         prefetch="exact")
