"""Next-token sampling on the GPU (tf_sample) against the oracle.

The result is an id, so the bar is bitwise: every row's id equals the
oracle's for the same logits, knobs and draw u.  Both sides take the
decisions in the same precisions: keys from the fp32 logits, the softmax,
the nucleus cut and the draw in fp64 with sequential sums in rank order.
Cases: the full 262,144-id vocabulary at the default knobs (temperature
0.2, top-k 64, top-p 0.95), greedy, top-p 1, a small top-k, top-k 1; ragged
vocabularies (one slice, a partial last slice, top_k == V); many equal
logits (ties go to the lower id); logits sorted ascending (the whole top in
the last slice); NaN, -inf and signed zeros; draws at 0 and just below 1;
the largest row count (4,096) in one call.
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


def _check(api, l, u, temperature, top_k, top_p):
    ids = api.tf_sample(torch.from_numpy(l).cuda(), temperature, top_k, top_p,
                        torch.from_numpy(u).cuda())
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    t32, p32 = float(np.float32(temperature)), float(np.float32(top_p))
    want = np.array([oracle.sample(l[r], t32, top_k, p32, float(u[r])) for r in range(len(u))])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"T={temperature} k={top_k} p={top_p}: rows {bad[:8]} "
                           f"got {got[bad[:8]]} want {want[bad[:8]]}")


@pytest.mark.parametrize("temperature,top_k,top_p", [
    (0.2, 64, 0.95), (0.0, 64, 0.95), (1.0, 64, 1.0), (0.7, 8, 0.5), (1.5, 1, 0.9),
    (2.0, 64, 0.999)])
def test_full_vocab(tfa, temperature, top_k, top_p):
    l, u = gen.sample_inputs(1, 16, gen.VOCAB, "lm")
    _check(tfa, l, u, temperature, top_k, top_p)


@pytest.mark.parametrize("V,top_k", [(100, 8), (4096, 64), (4097, 64), (5000, 16),
                                     (64, 64), (1, 1), (8191, 3), (65536, 64)])
def test_ragged_vocab(tfa, V, top_k):
    l, u = gen.sample_inputs(2, 5, V, "lm")
    for temperature, top_p in [(1.0, 0.9), (0.0, 0.95), (4.0, 1.0)]:
        _check(tfa, l, u, temperature, top_k, top_p)


@pytest.mark.parametrize("pattern", ["ties", "sorted", "special"])
def test_patterns(tfa, pattern):
    l, u = gen.sample_inputs(3, 4, 40000, pattern)
    for temperature, top_k, top_p in [(0.0, 64, 0.95), (0.2, 64, 0.95), (1.0, 64, 1.0),
                                      (3.0, 17, 0.8)]:
        _check(tfa, l, u, temperature, top_k, top_p)


def test_draw_edges(tfa):
    l, _ = gen.sample_inputs(4, 6, 20000, "lm")
    u = np.array([0.0, 1.0 - 2.0 ** -53, 0.5, 0.0, 1.0 - 2.0 ** -53, 0.25])
    _check(tfa, l, u, 1.0, 64, 1.0)
    _check(tfa, l, u, 5.0, 64, 0.95)


def test_all_equal_row_is_uniform_over_lowest_ids(tfa):
    l = np.zeros((64, 3000), dtype=np.float32)
    u = (np.arange(64) + 0.5) / 64
    _check(tfa, l, u, 1.0, 16, 1.0)
    ids = tfa.tf_sample(torch.from_numpy(l).cuda(), 1.0, 16, 1.0, torch.from_numpy(u).cuda())
    assert sorted(set(ids.cpu().tolist())) == list(range(16))


def test_many_rows_and_stream(tfa):
    l, u = gen.sample_inputs(5, 300, 9000, "lm")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lt, ut = torch.from_numpy(l).cuda(), torch.from_numpy(u).cuda()
        ids = tfa.tf_sample(lt, 0.8, 40, 0.9, ut, stream=s)
    s.synchronize()
    want = [oracle.sample(l[r], float(np.float32(0.8)), 40, float(np.float32(0.9)), float(u[r]))
            for r in range(300)]
    assert np.array_equal(ids.cpu().numpy(), np.array(want))


def test_workspace_reuse(tfa):
    """One workspace serves calls of different shapes in a row."""
    ws = tfa.workspace(tfa.tf_sample_workspace_bytes(gen.VOCAB, 16, 64))
    for seed, T, V, knobs in [(6, 16, gen.VOCAB, (0.2, 64, 0.95)), (7, 3, 5000, (1.0, 10, 0.9)),
                              (8, 16, gen.VOCAB, (0.9, 64, 0.99)), (9, 7, 70000, (0.0, 5, 0.5))]:
        l, u = gen.sample_inputs(seed, T, V, "lm")
        ids = tfa.tf_sample(torch.from_numpy(l).cuda(), *knobs, torch.from_numpy(u).cuda(), ws=ws)
        torch.cuda.synchronize()
        t32, p32 = float(np.float32(knobs[0])), float(np.float32(knobs[2]))
        want = [oracle.sample(l[r], t32, knobs[1], p32, float(u[r])) for r in range(T)]
        assert np.array_equal(ids.cpu().numpy(), np.array(want)), (seed, T, V)


def test_maximum_rows(tfa):
    """4,096 rows in one call (the largest T), a 100-id vocabulary."""
    l, u = gen.sample_inputs(10, 4096, 100, "lm")
    _check(tfa, l, u, 0.9, 8, 0.9)
