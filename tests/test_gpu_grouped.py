"""Grouped steps on the GPU: decode of 2-16 tokens (persistent MFMA units of
at most four tokens) and prefill chunks (16-token tiles), under routings that
stress the grouping -- few experts shared by many tokens (items split into
several units), every token on the same experts, identical tokens in a chunk
(every tile full) -- and a sweep of token counts.

Bars: expert ids bitwise; outputs within the floored 2e-3 of the fp64 oracle
(or of the single-token path where the oracle would be the same token again).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import check_token, device_layer, oracle_layer
from synth import gen

pytestmark = pytest.mark.gpu
FULL = gen.WORKLOADS[1]


@pytest.fixture(scope="module")
def tfa():
    import bit_routed_expert_tf_amd as m
    from bit_routed_expert_tf_amd import api
    m.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return api


@pytest.fixture(scope="module")
def full(tfa):
    L = oracle_layer(FULL.seed, 0, FULL.d_model, FULL.n_experts, FULL.top_k, FULL.d_ff,
                     FULL.d_ff_shared)
    return L, device_layer(L), gen.tokens(FULL.seed, 256, FULL.d_model)


def _decode(api, D, x16, forced=None):
    xt = torch.from_numpy(x16.view(np.int16)).cuda()
    ft = None if forced is None else torch.from_numpy(np.ascontiguousarray(forced, np.int32)).cuda()
    y, ids, w, _ = api.tf_moe_layer_fwd(D, xt, forced_ids=ft)
    torch.cuda.synchronize()
    return y.cpu().view(torch.int16).numpy().view(np.float16), ids.cpu().numpy(), w.cpu().numpy()


def _check(L, x, y, ids, w, forced=None):
    ref = oracle.moe_tokens(L, x, forced)
    assert np.array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["p"])) <= 1e-6
    for t in range(x.shape[0]):
        check_token(y[t], ref["y"][t])


def test_decode_few_experts_many_tokens(tfa, full):
    # 16 tokens drawing their 8 experts from 10: about 13 tokens per expert,
    # so every expert has four items and units of one expert follow each other
    print("grouped decode T=16, experts from a pool of 10", flush=True)
    L, D, X = full
    rng = np.random.default_rng(11)
    pool = rng.permutation(FULL.n_experts)[:10]
    forced = np.stack([pool[rng.permutation(10)[:8]] for _ in range(16)]).astype(np.int32)
    x = X[:16]
    y, ids, w = _decode(tfa, D, x, forced)
    _check(L, x, y, ids, w, forced)


def test_decode_every_token_same_experts(tfa, full):
    print("grouped decode T=16, all tokens on experts 3, 17, ..., 127", flush=True)
    L, D, X = full
    forced = np.tile(np.array([3, 17, 40, 41, 77, 100, 126, 127], np.int32), (16, 1))
    x = X[16:32]
    y, ids, w = _decode(tfa, D, x, forced)
    _check(L, x, y, ids, w, forced)


@pytest.mark.parametrize("T", [3, 4, 5, 8, 9, 12, 13])
def test_decode_token_counts(tfa, full, T):
    print(f"grouped decode natural routing T={T}", flush=True)
    L, D, X = full
    x = X[40:40 + T]
    y, ids, w = _decode(tfa, D, x)
    _check(L, x, y, ids, w)


def test_prefill_identical_tokens(tfa, full):
    # every expert of the chunk gets all 128 tokens: eight full 16-token items
    print("prefill T=128, one token repeated", flush=True)
    L, D, X = full
    x = np.repeat(X[60:61], 128, axis=0)
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    y, ids, w, _ = tfa.tf_moe_prefill_chunk(D, xt)
    torch.cuda.synchronize()
    y = y.cpu().view(torch.int16).numpy().view(np.float16)
    ids = ids.cpu().numpy()
    ref = oracle.moe_tokens(L, x[:1])
    assert all(np.array_equal(ids[t], ref["ids"][0]) for t in range(128))
    for t in (0, 1, 63, 127):
        check_token(y[t], ref["y"][0])
    # the same value in every row: each row sums the same terms in the same order
    assert np.array_equal(y.view(np.int16), np.repeat(y[:1], 128, axis=0).view(np.int16))


@pytest.mark.parametrize("T", [17, 100])
def test_prefill_tile_path_sizes(tfa, full, T):
    print(f"prefill tile path T={T}", flush=True)
    L, D, X = full
    x = X[100:100 + T]
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    y, ids, w, _ = tfa.tf_moe_prefill_chunk(D, xt)
    torch.cuda.synchronize()
    y = y.cpu().view(torch.int16).numpy().view(np.float16)
    sample = [0, T // 2, T - 1]
    ref = oracle.moe_tokens(L, x[sample])
    for i, t in enumerate(sample):
        assert np.array_equal(ids.cpu().numpy()[t], ref["ids"][i])
        check_token(y[t], ref["y"][i])
