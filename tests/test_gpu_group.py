"""Grouping of (token, rank) pairs by expert on the GPU (tf_group_by_expert).

Integer work, so the bar is bitwise: counts, offsets and the pair order
(expert, token, rank) equal the oracle's sort.  Cases span one token, token
counts on and off the 32-token mask words, the full 128-token chunk, every
token on the same experts, a single expert, and the largest shapes
(1,024 experts, top-16).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tfa():
    import bit_routed_expert_tf_amd as m
    from bit_routed_expert_tf_amd import api
    m.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return api


def _random_ids(seed, T, k, E):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _check(api, ids, E):
    T, k = ids.shape
    c, o, p = api.tf_group_by_expert(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    rc, ro, rp = oracle.group_by_expert(ids, E)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(p.cpu().numpy(), rp[:, 1] * k + rp[:, 2])


@pytest.mark.parametrize("T,k,E", [(1, 8, 128), (2, 8, 128), (31, 8, 128), (32, 8, 128),
                                   (33, 8, 128), (64, 8, 128), (100, 8, 128), (128, 8, 128),
                                   (50, 3, 12), (128, 16, 1024), (128, 1, 1), (7, 16, 16)])
def test_group_random_ids(tfa, T, k, E):
    print(f"group T={T} k={k} E={E}", flush=True)
    _check(tfa, _random_ids(T * 1000 + k * 10 + E, T, k, E), E)


def test_group_all_tokens_same_experts(tfa):
    print("group T=128 k=8 E=128, every token on experts 120..127", flush=True)
    ids = np.tile(np.arange(127, 119, -1, dtype=np.int32), (128, 1))
    _check(tfa, ids, 128)


def test_group_repeated_calls_reuse_workspace(tfa):
    print("group: two calls on one workspace, larger then smaller", flush=True)
    ws = tfa.workspace(tfa.tf_group_workspace_bytes(128, 128, 8))
    for T in (128, 9):
        ids = _random_ids(77 + T, T, 8, 128)
        c, o, p = tfa.tf_group_by_expert(torch.from_numpy(ids).cuda(), 128, ws=ws)
        torch.cuda.synchronize()
        rc, ro, rp = oracle.group_by_expert(ids, 128)
        assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(o.cpu().numpy(), ro)
        assert np.array_equal(p.cpu().numpy(), rp[:, 1] * 8 + rp[:, 2])
