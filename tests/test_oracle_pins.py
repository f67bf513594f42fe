"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Every pin compares the oracle with something it does not compute: exact
integer arithmetic, hand-built groups, textbook values, brute-force sorts,
hand-derived cache sequences, or the pages' own byte counts.  A plausible
mistake (wrong nibble order, dropped bias term, swapped gate/up, tanh GELU,
wrong tie-break, LRU instead of LFU) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _pack4(codes):
    """Pack an integer code matrix [n][k] (0..15) into MLX-style bytes."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _mat(codes, scale, bias, bits=4):
    codes = np.asarray(codes)
    n, k = codes.shape
    q = _pack4(codes) if bits == 4 else codes.astype(np.uint8)
    s = np.broadcast_to(np.float16(scale), (n, k // 64)).astype(np.float16) \
        if np.isscalar(scale) else np.asarray(scale, np.float16)
    b = np.broadcast_to(np.float16(bias), (n, k // 64)).astype(np.float16) \
        if np.isscalar(bias) else np.asarray(bias, np.float16)
    return {"q": q, "scale": s, "bias": b, "n": n, "k": k, "bits": bits}


# ---------------------------------------------------------------- fp16 decode
def test_half_decode_all_65536_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_double(pats)
    want = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------------ P1 dequant
def test_p1_dequant_hand_built_group():
    codes = np.tile(np.arange(16), 4)[None, :]            # q = 0..15 four times
    m = _mat(codes, 0.5, -2.0)
    for j in range(64):
        assert oracle.weight(m, 0, j) == 0.5 * (j % 16) - 2.0
    x = np.ones(64)
    assert oracle.qmatvec(m, x)[0] == sum(0.5 * (j % 16) - 2.0 for j in range(64))


def test_p1_dequant_8bit_group():
    codes = np.arange(64)[None, :] * 4 % 256
    m = _mat(codes, 1.0 / 256.0, 0.0, bits=8)
    for j in range(64):
        assert oracle.weight(m, 0, j) == codes[0, j] / 256.0


def test_p1_group_boundaries_use_own_scale():
    codes = np.full((1, 128), 3)
    m = _mat(codes, np.array([[0.25, 2.0]]), np.array([[1.0, -1.0]]))
    assert oracle.weight(m, 0, 63) == 0.25 * 3 + 1.0
    assert oracle.weight(m, 0, 64) == 2.0 * 3 - 1.0


# --------------------------------------------------------- P2 nibble / layout
def test_p2_one_hot_columns_expose_nibble_order():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(5, 128))
    m = _mat(codes, 1.0, 0.0)
    for j in (0, 1, 2, 3, 62, 63, 64, 65, 127):
        e = np.zeros(128)
        e[j] = 1.0
        assert np.array_equal(oracle.qmatvec(m, e), codes[:, j].astype(np.float64))
        assert np.array_equal(oracle.np_qmatvec(m, e), codes[:, j].astype(np.float64))


# ------------------------------------------------- P3 integer-exact mat-vec
@pytest.mark.parametrize("bias", [0.0, 0.5, -1.25])
def test_p3_integer_exact_gemv(bias):
    rng = np.random.default_rng(11)
    n, k = 9, 256
    codes = rng.integers(0, 16, size=(n, k))
    x = rng.integers(-8, 9, size=k)
    m = _mat(codes, 1.0, bias)
    want = [sum(int(codes[r, j]) * int(x[j]) for j in range(k)) + bias * int(x.sum())
            for r in range(n)]
    assert np.array_equal(oracle.qmatvec(m, x.astype(np.float64)), np.array(want))


def test_p3_router_8bit_exact():
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, size=(4, 192))
    x = rng.integers(-3, 4, size=192)
    m = _mat(codes, 1.0, 0.0, bits=8)
    want = codes.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(oracle.qmatvec(m, x.astype(np.float64)), want.astype(np.float64))


# --------------------------------------------------------------- P4 top-k
def _brute_topk(l, k):
    return sorted(range(len(l)), key=lambda i: (-l[i], i))[:k]


def test_p4_topk_brute_force_random():
    rng = np.random.default_rng(3)
    for _ in range(200):
        l = rng.standard_normal(8)
        assert list(oracle.topk(l, 2)) == _brute_topk(l, 2)
        assert list(oracle.np_topk(l, 2)) == _brute_topk(l, 2)


def test_p4_topk_ties_break_to_lowest_id():
    l = np.array([1.0, 3.0, 3.0, 0.5, 3.0, -1.0, 2.0, 3.0])
    assert list(oracle.topk(l, 2)) == [1, 2]
    assert list(oracle.topk(l, 5)) == [1, 2, 4, 7, 6]
    assert list(oracle.np_topk(l, 5)) == [1, 2, 4, 7, 6]
    assert list(oracle.topk(np.zeros(8), 3)) == [0, 1, 2]


def test_p4_topk_128_choose_8():
    rng = np.random.default_rng(4)
    for _ in range(20):
        l = np.round(rng.standard_normal(128), 1)       # many exact ties
        assert list(oracle.topk(l, 8)) == _brute_topk(list(l), 8)


# -------------------------------------------------------------- P5 softmax
def test_p5_softmax_identities():
    rng = np.random.default_rng(5)
    for _ in range(50):
        l = rng.standard_normal(8) * 5
        p = oracle.softmax(l)
        assert abs(p.sum() - 1.0) <= 1e-12
        direct = np.array([math.exp(v) for v in l])
        direct /= direct.sum()
        assert np.allclose(p, direct, rtol=1e-14, atol=0)
        assert np.array_equal(np.argsort(-p, kind="stable"), np.argsort(-l, kind="stable"))
    assert oracle.softmax(np.array([123.4]))[0] == 1.0
    assert np.all(oracle.softmax(np.full(4, 7.0)) == 0.25)


# ---------------------------------------------------------------- P7 GELU
def test_p7_gelu_is_the_erf_form():
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(1.0) == pytest.approx(0.8413447460685429, abs=1e-16)   # Phi(1)
    assert abs(oracle.gelu(1.0, tanh=True) - 0.8413447460685429) > 1e-4
    for z in np.linspace(-6, 6, 49):
        assert oracle.gelu(z) - oracle.gelu(-z) == pytest.approx(z, abs=1e-14)
    assert oracle.gelu(-10.0) == pytest.approx(0.0, abs=1e-20)
    assert oracle.gelu(10.0) == pytest.approx(10.0, abs=1e-15)
    zs = np.linspace(-4, 4, 33)
    assert np.allclose([oracle.gelu(z) for z in zs], oracle.np_gelu(zs), rtol=1e-15, atol=1e-16)


def test_p7_gelu_tanh_branch():
    """The tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))), pinned
    against things the oracle does not compute: PyTorch's own fp64 tanh-GELU
    (a library routine), the odd identity gelu(z) - gelu(-z) = z (which a
    non-odd inner polynomial, e.g. a z^2 term, breaks), the two limits, and
    the form's known worst deviation from the erf form (about 4.7e-4, near
    |z| = 2.7): between 3e-4 and 5e-4 over [-6, 6]."""
    import torch
    zs = np.linspace(-6, 6, 241)
    got = np.array([oracle.gelu(z, tanh=True) for z in zs])
    ref = torch.nn.functional.gelu(torch.from_numpy(zs), approximate="tanh").numpy()
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-15)
    ref_erf = torch.nn.functional.gelu(torch.from_numpy(zs), approximate="none").numpy()
    assert np.allclose([oracle.gelu(z) for z in zs], ref_erf, rtol=1e-14, atol=1e-15)
    assert oracle.gelu(1.0, tanh=True) == pytest.approx(0.8411919906082768, abs=1e-15)
    for z in zs:
        assert oracle.gelu(z, tanh=True) - oracle.gelu(-z, tanh=True) == pytest.approx(z, abs=1e-13)
    dev = np.abs(got - np.array([oracle.gelu(z) for z in zs]))
    assert 3e-4 < dev.max() < 5e-4
    assert 2.4 < abs(zs[np.argmax(dev)]) < 3.0
    assert oracle.gelu(-12.0, tanh=True) == pytest.approx(0.0, abs=1e-20)
    assert oracle.gelu(12.0, tanh=True) == pytest.approx(12.0, abs=1e-14)
    assert np.allclose(got, oracle.np_gelu(zs, tanh=True), rtol=1e-14, atol=1e-15)


# ----------------------------------------------------- P8 closed-form expert
def test_p8_selection_matrix_expert_closed_form():
    rng = np.random.default_rng(8)
    d, f = 128, 64
    Pg = (rng.random((f, d)) < 0.05).astype(int)
    Pu = (rng.random((f, d)) < 0.05).astype(int)
    Pd = (rng.random((d, f)) < 0.05).astype(int)
    ex = {"gate": _mat(Pg, 1.0, 0.0), "up": _mat(Pu, 1.0, 0.0), "down": _mat(Pd, 1.0, 0.0)}
    x = rng.standard_normal(d)
    h = []
    for i in range(f):
        g = sum(x[j] for j in range(d) if Pg[i, j])
        u = sum(x[j] for j in range(d) if Pu[i, j])
        h.append(0.5 * g * (1.0 + math.erf(g / math.sqrt(2.0))) * u)
    want = np.array([sum(h[i] for i in range(f) if Pd[r, i]) for r in range(d)])
    assert np.allclose(oracle.expert_ffn(ex, x), want, rtol=1e-13, atol=1e-13)
    # swapping gate and up changes the result: the pin sees operand order
    ex2 = {"gate": ex["up"], "up": ex["gate"], "down": ex["down"]}
    assert not np.allclose(oracle.expert_ffn(ex2, x), want, rtol=1e-6, atol=1e-6)


# --------------------------------------------------- layer-level fixtures
def _layer(wl, zero_shared=False, identical=False, top_k=None):
    seed, d, E, f, fs = wl.seed, wl.d_model, wl.n_experts, wl.d_ff, wl.d_ff_shared
    k = top_k or wl.top_k
    pool = gen.expert_pool(seed, 0, d, f, E, threads=1)
    if identical:
        pool[:] = pool[0]
    sh = gen.shared_expert(seed, 0, d, fs)
    if zero_shared:
        for m in sh.values():
            m["scale"][:] = 0
            m["bias"][:] = 0
    return {"router": gen.router(seed, 0, d, E), "shared_blob": gen.expert_blob(sh),
            "pool": pool, "d_model": d, "d_ff": f, "d_ff_shared": fs, "top_k": k}


TINY = gen.WORKLOADS[0]


def test_p6_one_expert_rule_bitwise():
    L = _layer(TINY, zero_shared=True, top_k=1)
    x = gen.tokens(TINY.seed, 3, TINY.d_model)
    for t in range(3):
        out = oracle.moe_token(L, x[t])
        assert out["p"][0] == 1.0
        e = out["ids"][0]
        ye = oracle.expert_from_blob(L["pool"][e], TINY.d_model, TINY.d_ff,
                                     x[t].astype(np.float64))
        assert np.array_equal(out["y"], ye)


def test_p9_identical_experts_combine_is_routing_independent():
    L = _layer(TINY, identical=True)
    x = gen.tokens(TINY.seed, 1, TINY.d_model)[0]
    xd = x.astype(np.float64)
    want = oracle.expert_from_blob(L["shared_blob"], TINY.d_model, TINY.d_ff_shared, xd) \
        + oracle.expert_from_blob(L["pool"][0], TINY.d_model, TINY.d_ff, xd)
    ys = [oracle.moe_token(L, x)["y"]]
    for forced in ([0, 1], [7, 3], [5, 2]):
        ys.append(oracle.moe_token(L, x, forced=np.array(forced))["y"])
    for y in ys:
        assert np.allclose(y, want, rtol=1e-12, atol=1e-9 * np.abs(want).max())


def test_p13_c_oracle_matches_numpy_twin_tiny_layer():
    L = _layer(TINY)
    x = gen.tokens(TINY.seed, 4, TINY.d_model)
    for t in range(4):
        a = oracle.moe_token(L, x[t])
        b = oracle.np_moe_token(L, x[t])
        assert np.array_equal(a["ids"], b["ids"])
        assert np.allclose(a["logits"], b["logits"], rtol=1e-12, atol=1e-12)
        assert np.allclose(a["p"], b["p"], rtol=1e-12, atol=1e-15)
        scale = np.abs(b["y"]).max()
        assert np.max(np.abs(a["y"] - b["y"])) <= 1e-12 * scale


def test_tiny_layer_output_is_finite_and_topk_is_routers():
    L = _layer(TINY)
    x = gen.tokens(TINY.seed, 1, TINY.d_model)[0]
    out = oracle.moe_token(L, x)
    assert np.all(np.isfinite(out["y"]))
    assert list(out["ids"]) == _brute_topk(list(out["logits"]), TINY.top_k)
    assert np.all(np.isfinite(oracle.to_fp16(out["y"])))      # no fp16 overflow at d=256


def test_forced_ids_rejected_when_repeated_or_out_of_range():
    L = _layer(TINY)
    x = gen.tokens(TINY.seed, 1, TINY.d_model)[0]
    with pytest.raises(ValueError):
        oracle.moe_token(L, x, forced=np.array([3, 3]))
    with pytest.raises(ValueError):
        oracle.moe_token(L, x, forced=np.array([0, 8]))


# ------------------------------------------------------------ P10 LFU cache
def test_p10_lfu_hand_derived_sequences():
    cases = json.load(open(os.path.join(GOLD, "lfu_cases.json")))["cases"]
    for c in cases:
        hit, slot, _, _ = oracle.lfu_replay(np.array(c["ids"]), c["n_slots"])
        assert hit.tolist() == c["hit"], c["name"]
        assert slot.tolist() == c["slot"], c["name"]


def test_lfu_invariants_and_uniform_thrash_rate():
    wl = gen.WORKLOADS[4]
    ids = gen.uniform_ids(wl.seed, 0, 2000, 128, 8)
    hit, slot, expert_of, count = oracle.lfu_replay(ids, 16)
    # every hit names the slot the expert already occupied
    where = {}
    for t in range(ids.shape[0]):
        for r in range(8):
            e, s = int(ids[t, r]), int(slot[t, r])
            if hit[t, r]:
                assert where.get(e) == s
            for e2, s2 in list(where.items()):
                if s2 == s and e2 != e:
                    del where[e2]
            where[e] = s
        assert len(set(slot[t].tolist())) == 8          # a token's slots are distinct
    # uniform routing: a 16-of-128 cache hits about 16/128 of the time
    assert abs(hit.mean() - 16 / 128) < 0.02


def test_lfu_zipf_hit_rate_in_stated_band():
    """Zipf(1.1) popularity is stated to give a ~50-70% hit rate."""
    wl = gen.WORKLOADS[2]
    rates = []
    for layer in (0, 17):
        ids = gen.zipf_ids(wl.seed, layer, 1024, 128, 8, s=wl.zipf_s)
        hit, _, _, _ = oracle.lfu_replay(ids, 16)
        rates.append(hit.mean())
    assert all(0.45 < r < 0.75 for r in rates), rates


def test_lru_hand_derived_sequences():
    """The LRU reading (longest-unused slot goes): hand-derived sequences,
    most of them where LFU decides differently."""
    cases = json.load(open(os.path.join(GOLD, "lru_cases.json")))["cases"]
    for c in cases:
        hit, slot, _, _ = oracle.lfu_replay(np.array(c["ids"]), c["n_slots"], policy="lru")
        assert hit.tolist() == c["hit"], c["name"]
        assert slot.tolist() == c["slot"], c["name"]
    lfu = [oracle.lfu_replay(np.array(c["ids"]), c["n_slots"])[:2] for c in cases[:2]]
    assert any(h.tolist() != c["hit"] or s.tolist() != c["slot"] for (h, s), c in zip(lfu, cases[:2]))


def test_lru_uniform_thrash_rate_and_zipf_band():
    """Uniform routing: 16 of 128 slots hit about 16/128 of the time under
    either rule; Zipf(1.1) popularity favours the count-keeping LFU."""
    ids = gen.uniform_ids(gen.WORKLOADS[4].seed, 0, 2000, 128, 8)
    hit, _, _, _ = oracle.lfu_replay(ids, 16, policy="lru")
    assert abs(hit.mean() - 16 / 128) < 0.02
    wl = gen.WORKLOADS[2]
    z = gen.zipf_ids(wl.seed, 0, 1024, 128, 8, s=wl.zipf_s)
    lru = oracle.lfu_replay(z, 16, policy="lru")[0].mean()
    lfu = oracle.lfu_replay(z, 16)[0].mean()
    assert 0.3 < lru < lfu


def test_lfu_rejects_small_cache_and_repeats():
    with pytest.raises(ValueError):
        oracle.lfu_replay(np.array([[0, 1, 2]]), 2)
    with pytest.raises(ValueError):
        oracle.lfu_replay(np.array([[4, 4]]), 4)
    with pytest.raises(ValueError):
        oracle.lfu_replay(np.array([[0, 1]]), 4, policy="fifo")


# ----------------------------------------------------- grouping by expert
def test_group_by_expert_matches_brute_force_scan():
    rng = np.random.default_rng(9)
    ids = np.array([rng.permutation(16)[:4] for _ in range(12)])
    counts, offsets, pairs = oracle.group_by_expert(ids, 16)
    assert counts.sum() == ids.size and offsets[-1] == ids.size
    for e in range(16):
        scan = [(t, r) for t in range(12) for r in range(4) if ids[t, r] == e]
        got = [tuple(p[1:]) for p in pairs[offsets[e]:offsets[e + 1]]]
        assert got == scan and all(p[0] == e for p in pairs[offsets[e]:offsets[e + 1]])


# ------------------------------------------------------ P11 byte accounting
def test_p11_byte_accounting_against_pages():
    const = json.load(open(os.path.join(GOLD, "page_constants.json")))
    E, L = const["experts_per_layer"]["value"], const["layers"]["value"]
    blob = gen.blob_bytes(2816, 704)
    assert blob == 3_345_408
    total = L * E * blob + const["resident_core_GB"]["value"] * 1e9
    assert abs(total / 1e9 - const["installed_text_model_GB"]["value"]) / 14.3 < 0.01
    per_expert_pages = (const["installed_text_model_GB"]["value"]
                        - const["resident_core_GB"]["value"]) * 1e9 / (L * E)
    assert abs(per_expert_pages - blob) / blob < 0.01
    assert gen.blob_bytes(2816, 2816) == 13_381_632
    r = gen.router(1, 0, 2816, 128)
    assert r["q"].nbytes + r["scale"].nbytes + r["bias"].nbytes == 382_976
    assert gen.blob_bytes(256, 128) == 55_296


def test_blob_sections_round_trip():
    ex = gen.expert(0, 0, 3, 256, 128)
    blob = gen.expert_blob(ex)
    off = gen.blob_offsets(256, 128)
    assert blob.size == off["size"]
    assert np.array_equal(blob[off["up.q"]:off["up.q"] + ex["up"]["q"].nbytes],
                          ex["up"]["q"].reshape(-1))
    x = gen.tokens(0, 1, 256)[0].astype(np.float64)
    assert np.array_equal(oracle.expert_from_blob(blob, 256, 128, x), oracle.expert_ffn(ex, x))


# ------------------------------------------------------------ sampling step
def test_sample_hand_worked_cases():
    cases = json.load(open(os.path.join(GOLD, "sample_cases.json")))["cases"]
    for c in cases:
        logits = np.array(c["logits"], dtype=np.float64)
        k = min(c["top_k"], logits.size)
        got = [oracle.sample(logits, c["temperature"], k, c["top_p"], u) for u in c["u"]]
        assert got == c["ids"], c["name"]


def test_sample_greedy_and_degenerate_knobs_are_argmax():
    rng = np.random.default_rng(7)
    for trial in range(50):
        l = rng.standard_normal(1000).astype(np.float32)
        if trial % 5 == 0:                     # a tie at the top
            j = int(np.argmax(l))
            l[rng.integers(0, 1000)] = l[j]
        best = int(np.argmax(l))               # first maximum = lowest id
        u = float(rng.random())
        assert oracle.sample(l, 0.0, 64, 0.95, u) == best
        assert oracle.sample(l, 0.7, 1, 0.95, u) == best
        assert oracle.sample(l, 0.7, 64, 1e-9, u) == best


def test_sample_frequencies_match_the_nucleus():
    """Sweeping u over a uniform grid draws each kept id in proportion to its
    renormalised probability; ids outside the nucleus never appear."""
    rng = np.random.default_rng(3)
    l = rng.standard_normal(300) * 2
    T, K, P = 0.8, 16, 0.9
    order = np.lexsort((np.arange(l.size), -l))[:K]
    w = np.exp((l[order] - l[order[0]]) / T)
    p = w / w.sum()
    keep = int(np.searchsorted(np.cumsum(p), P) + 1)
    q = p[:keep] / p[:keep].sum()
    N = 20000
    ids = [oracle.sample(l, T, K, P, (i + 0.5) / N) for i in range(N)]
    cnt = {int(i): 0 for i in order}
    for i in ids:
        cnt[i] += 1
    for r, i in enumerate(order):
        want = q[r] if r < keep else 0.0
        assert abs(cnt[int(i)] / N - want) <= 1.0 / N + 1e-12, (r, cnt[int(i)], want)


# ------------------------------------------------------------ decode attention
def test_attn_hand_worked_cases():
    cases = json.load(open(os.path.join(GOLD, "attn_cases.json")))["cases"]
    for c in cases:
        out = oracle.attn_decode(c["q"], c["k"], c["v"], window=c["window"], scale=c["scale"])
        assert np.allclose(out, np.array(c["out"]), rtol=0, atol=1e-12), c["name"]


def _attn_inputs(seed, H=4, G=2, D=8, N=12):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((H, D)), rng.standard_normal((N, G, D)),
            rng.standard_normal((N, G, D)))


def test_attn_uniform_scores_give_the_window_mean():
    _, K, V = _attn_inputs(1)
    q = np.zeros((4, 8))
    for window in (None, 1, 5, 12, 40):
        out = oracle.attn_decode(q, K, V, window=window)
        first = 0 if window is None else max(0, 12 - window)
        for h in range(4):
            assert np.allclose(out[h], V[first:, h // 2].mean(axis=0), rtol=0, atol=1e-12)


def test_attn_window_and_order_invariances():
    q, K, V = _attn_inputs(2)
    full = oracle.attn_decode(q, K, V)
    assert np.allclose(oracle.attn_decode(q, K, V, window=12), full, rtol=0, atol=1e-13)
    assert np.allclose(oracle.attn_decode(q, K, V, window=100), full, rtol=0, atol=1e-13)
    w5 = oracle.attn_decode(q, K, V, window=5)
    K2, V2 = K.copy(), V.copy()
    K2[:7] = 50.0                       # tokens outside the window change freely
    V2[:7] = -1e3
    assert np.array_equal(oracle.attn_decode(q, K2, V2, window=5), w5)
    perm = np.random.default_rng(3).permutation(12)
    assert np.allclose(oracle.attn_decode(q, K[perm], V[perm]), full, rtol=0, atol=1e-12)
    assert not np.allclose(w5, full, atol=1e-3)


def test_attn_query_head_grouping():
    q, K, V = _attn_inputs(4)
    q[1] = q[0]                         # heads 0 and 1 read k/v head 0
    q[2] = q[0]                         # head 2 reads k/v head 1
    out = oracle.attn_decode(q, K, V)
    assert np.array_equal(out[0], out[1])
    assert not np.allclose(out[0], out[2], atol=1e-3)
    one = oracle.attn_decode(q[2:3], K[:, 1:2], V[:, 1:2])
    assert np.allclose(out[2], one[0], rtol=0, atol=1e-14)


def test_attn_dominant_score_selects_its_value():
    q, K, V = _attn_inputs(5, H=1, G=1)
    K[7, 0] = q[0] / np.dot(q[0], q[0]) * 60 * np.sqrt(8)   # score 60 against O(1) others
    out = oracle.attn_decode(q, K, V)
    assert np.allclose(out[0], V[7, 0], rtol=0, atol=np.abs(V).max() * 12 * np.exp(-50))
