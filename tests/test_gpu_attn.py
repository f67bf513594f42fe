"""Decode attention on the GPU (tf_attn_decode) against the oracle.

The oracle keeps every token's key and value in token order and attends over
the last `window` tokens (sliding-window layer) or all of them (full layer);
the GPU keeps a ring of S slots (token p in slot p % S) or a linear store
(slot p).  Bars: each step's output within the floored 2e-3 of the oracle
(fp32 scores and sums against fp64; the error seen is about 1e-6), and the
new token's key and value stored bitwise in their slot.  Cases: token
sequences that wrap a ring twice, rings and stores whose sizes are not a
multiple of the 32-slot chunk, 1, 2 and 4 query heads per key/value head,
head dims 64, 128 and 256, stores past 2,048 seen tokens (64-slot chunks),
and the full-size layers (16 query heads, 8 key/value heads, head dim 256):
a 4,096-token full layer at its last position and a 1,024-slot ring at
token 5,000.
"""
import numpy as np
import pytest
import torch

import oracle
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


def _check(got, ref, tol=2e-3):
    worst = 0.0
    for h in range(ref.shape[0]):
        floor = max(np.abs(ref[h]).max(), np.sqrt(np.mean(ref[h] ** 2)))
        err = np.abs(got[h] - ref[h]).max() / floor
        assert err <= tol, (h, err)
        worst = max(worst, err)
    return worst


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _sequence(api, seed, ring, S, H, G, D, N, check_every=1):
    q, k, v = gen.attn_inputs(seed, N, H, G, D)
    kc = torch.zeros((G, S, D), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    ws = api.workspace(api.tf_attn_workspace_bytes(H, D, S))
    for pos in range(N):
        out = api.tf_attn_decode(_dev(q[pos]), _dev(k[pos]), _dev(v[pos]), kc, vc, pos, ring, ws=ws)
        if pos % check_every and pos != N - 1:
            continue
        torch.cuda.synchronize()
        ref = oracle.attn_decode(q[pos], k[:pos + 1], v[:pos + 1], window=S if ring else None)
        _check(out.cpu().numpy(), ref)
        slot = pos % S if ring else pos
        assert np.array_equal(kc[:, slot].cpu().numpy(), k[pos].view(np.int16))
        assert np.array_equal(vc[:, slot].cpu().numpy(), v[pos].view(np.int16))


@pytest.mark.parametrize("ring,S,H,G,D,N", [
    (1, 64, 4, 2, 128, 150),    # wraps the ring twice
    (1, 40, 2, 2, 256, 90),     # ring size off the chunk grid, one head per group
    (0, 100, 8, 2, 64, 100),    # linear store filled to the end, four heads per group
    (0, 33, 16, 8, 256, 33),    # full-size heads, one slot past a chunk
])
def test_attn_token_sequences(tfa, ring, S, H, G, D, N):
    print(f"attn: ring={ring} S={S} H={H} G={G} D={D} N={N}", flush=True)
    _sequence(tfa, 1, ring, S, H, G, D, N)


def _prefilled(api, seed, ring, S, pos, H=16, G=8, D=256):
    """Caches holding the tokens before `pos` as a layer would, then one call."""
    n_tok = pos + 1
    q, k, v = gen.attn_inputs(seed, n_tok, H, G, D)
    kc = np.zeros((G, S, D), dtype=np.float16)
    vc = np.zeros_like(kc)
    first = max(0, pos - S + 1) if ring else 0
    for t in range(first, pos):
        slot = t % S if ring else t
        kc[:, slot] = k[t]
        vc[:, slot] = v[t]
    kt, vt = _dev(kc), _dev(vc)
    out = api.tf_attn_decode(_dev(q[pos]), _dev(k[pos]), _dev(v[pos]), kt, vt, pos, ring)
    torch.cuda.synchronize()
    ref = oracle.attn_decode(q[pos], k, v, window=S if ring else None)
    print(f"attn: max floored rel err {_check(out.cpu().numpy(), ref):.2e}", flush=True)


def test_attn_full_layer_at_4096(tfa):
    print("attn: full layer S=4096 pos=4095 H=16 G=8 D=256", flush=True)
    _prefilled(tfa, 2, 0, 4096, 4095)


def test_attn_sliding_layer_wrapped(tfa):
    print("attn: ring S=1024 pos=5000 H=16 G=8 D=256", flush=True)
    _prefilled(tfa, 3, 1, 1024, 5000)


@pytest.mark.parametrize("ring,S,pos,H,G,D", [
    (0, 2200, 2100, 8, 2, 128),    # past 2,048 seen tokens: 64-slot chunks
    (1, 3000, 4000, 4, 4, 64),     # a wrapped ring with 64-slot chunks, one head per group
    (0, 2048, 2047, 4, 1, 256),    # exactly 2,048 seen tokens: 32-slot chunks
])
def test_attn_long_stores(tfa, ring, S, pos, H, G, D):
    print(f"attn: ring={ring} S={S} pos={pos} H={H} G={G} D={D}", flush=True)
    _prefilled(tfa, 8, ring, S, pos, H=H, G=G, D=D)


def test_attn_first_token_and_scale(tfa):
    """pos 0 sees only itself: out = v of that token, whatever the scale."""
    q, k, v = gen.attn_inputs(4, 1, 4, 4, 64)
    kc = torch.zeros((4, 8, 64), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    for scale in (0.125, 3.0):
        out = tfa.tf_attn_decode(_dev(q[0]), _dev(k[0]), _dev(v[0]), kc, vc, 0, 1, scale=scale)
        torch.cuda.synchronize()
        assert np.allclose(out.cpu().numpy(), v[0].astype(np.float64), rtol=0, atol=1e-6)
