"""Chunked prefill on the GPU (tf_moe_prefill_chunk).

Bars: expert ids bitwise equal to the fp64 oracle; layer outputs within the
floored 2e-3 per token (every token of the full-width chunk); the chunk equal
to the same tokens decoded one at a time (ids bitwise, outputs within the
floored 2e-3 of each other); repeated runs bitwise identical.  The chunk's pairs are grouped by expert inside the
library, so sizes span single and multi-pass items, ragged shapes and the
full-width 128-token chunk.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import check_token, check_token32, device_layer, oracle_layer
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


def _prefill(api, D, x16):
    xt = torch.from_numpy(x16.view(np.int16)).cuda()
    y, ids, w, y32 = api.tf_moe_prefill_chunk(D, xt, want_y32=True)
    torch.cuda.synchronize()
    return (y.cpu().view(torch.int16).numpy().view(np.float16), ids.cpu().numpy(), w.cpu().numpy(),
            y32.cpu().numpy())


def _decode_each(api, D, x16):
    ys, ids = [], []
    ws = api.workspace(api.tf_moe_workspace_bytes(D, 1))
    for t in range(x16.shape[0]):
        xt = torch.from_numpy(x16[t:t + 1].view(np.int16)).cuda()
        y, i, _, _ = api.tf_moe_layer_fwd(D, xt, ws=ws)
        ys.append(y)
        ids.append(i)
    torch.cuda.synchronize()
    return (torch.cat(ys).cpu().view(torch.int16).numpy().view(np.float16),
            torch.cat(ids).cpu().numpy())


# 48 and 128: whole 16-token tiles, which the top-k launch walks in the
# router launch's XCD order; 33: a ragged last tile (plain order)
@pytest.mark.parametrize("T", [1, 2, 7, 33, 48, 128])
def test_prefill_tiny_layer_matches_oracle(tfa, T):
    print(f"prefill tiny layer T={T}", flush=True)
    L = oracle_layer(0, 0, 256, 8, 2, 128, 256)
    x = gen.tokens(0, T, 256)
    y, ids, w, y32 = _prefill(tfa, device_layer(L), x)
    ref = oracle.moe_tokens(L, x)
    assert np.array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["p"])) <= 1e-6
    for t in range(T):
        check_token(y[t], ref["y"][t])
        check_token32(y32[t], ref["y"][t])


def test_prefill_ragged_shapes(tfa):
    print("prefill ragged d=320 E=12 k=3 f=192 fs=320 T=50", flush=True)
    L = oracle_layer(5, 0, 320, 12, 3, 192, 320)
    x = gen.tokens(5, 50, 320)
    y, ids, _, y32 = _prefill(tfa, device_layer(L), x)
    ref = oracle.moe_tokens(L, x)
    assert np.array_equal(ids, ref["ids"])
    for t in range(50):
        check_token(y[t], ref["y"][t])


def test_prefill_full_width_chunk(tfa):
    # the prefill workload's shapes: one 128-token chunk through a full layer
    print("prefill full width d=2816 E=128 k=8 f=704 fs=2816 T=128", flush=True)
    wl = gen.WORKLOADS[3]
    L = oracle_layer(wl.seed, 0, wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared)
    D = device_layer(L)
    x = gen.tokens(wl.seed, 128, wl.d_model)
    y, ids, _, y32 = _prefill(tfa, D, x)
    # every token against the fp64 oracle: ids bitwise, outputs within tolerance
    ref = oracle.moe_tokens(L, x)
    assert np.array_equal(ids, ref["ids"])
    worst = max(check_token(y[t], ref["y"][t]) for t in range(128))
    print(f"PARITY prefill chunk 0: worst floored rel err {worst:.3e}", flush=True)
    # the same tokens decoded one at a time: ids bitwise (path invariant)
    yd, idd = _decode_each(tfa, D, x)
    assert np.array_equal(ids, idd)
    for t in range(128):
        check_token(y[t], yd[t].astype(np.float64))
    # repeat: bitwise identical
    y2, ids2, _, _ = _prefill(tfa, D, x)
    assert np.array_equal(ids, ids2) and np.array_equal(y.view(np.int16), y2.view(np.int16))


def test_prefill_two_chunks_in_flight(tfa):
    # the prefill line's schedule: consecutive chunks alternate between two
    # streams with a workspace each, so two chunks run at once; every output
    # must be bitwise the one-at-a-time result
    print("prefill two streams: 6 chunks of 128, full width", flush=True)
    wl = gen.WORKLOADS[3]
    L = oracle_layer(wl.seed, 0, wl.d_model, wl.n_experts, wl.top_k, wl.d_ff, wl.d_ff_shared)
    D = device_layer(L)
    C, n = 128, 6
    x = torch.from_numpy(gen.tokens(wl.seed, C * n, wl.d_model).view(np.int16)).cuda()
    ws = [tfa.workspace(tfa.tf_prefill_workspace_bytes(D, C), x.device) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]

    def run(two):
        y = torch.empty((C * n, wl.d_model), dtype=torch.int16, device=x.device)
        ids = torch.empty((C * n, wl.top_k), dtype=torch.int32, device=x.device)
        w = torch.empty((C * n, wl.top_k), dtype=torch.float32, device=x.device)
        torch.cuda.synchronize()
        for j in range(n):
            q = j % 2 if two else 0
            tfa.tf_moe_prefill_chunk(D, x[C * j:C * (j + 1)], y=y[C * j:C * (j + 1)],
                                     ids=ids[C * j:C * (j + 1)], weights=w[C * j:C * (j + 1)],
                                     ws=ws[q], stream=streams[q])
        torch.cuda.synchronize()
        return y.cpu(), ids.cpu(), w.cpu()

    one, two = run(False), run(True)
    for a, b in zip(one, two):
        assert torch.equal(a, b)
