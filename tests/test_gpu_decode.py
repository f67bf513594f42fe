"""Parity of the HIP decode path with the fp64 oracle (GPU).

Bars: expert ids bitwise; router weights within 1e-6; layer outputs within a
floored relative error of 2e-3 per token (fp32 accumulation, fp16 I/O); the
integer-exact expert bitwise; repeated runs bitwise identical.
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


def _run_layer(api, D, x16, forced=None, act=0):
    xt = torch.from_numpy(x16.view(np.int16)).cuda()
    ft = torch.from_numpy(np.ascontiguousarray(forced, np.int32)).cuda() if forced is not None else None
    y, ids, w, y32 = api.tf_moe_layer_fwd(D, xt, forced_ids=ft, want_y32=True)
    torch.cuda.synchronize()
    return (y.cpu().numpy().view(np.float16), ids.cpu().numpy(), w.cpu().numpy(),
            y32.cpu().numpy())


def _check_layer(L, api, x16, forced=None, tanh=False, act=0):
    D = device_layer(L, act=act)
    y, ids, w, y32 = _run_layer(api, D, x16, forced, act)
    ref = oracle.moe_tokens(L, x16, forced, tanh=tanh)
    assert np.array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["p"])) <= 1e-6
    errs = [check_token(y[t], ref["y"][t]) for t in range(x16.shape[0])]
    for t in range(x16.shape[0]):
        fin = np.abs(ref["y"][t]) < 65504
        if fin.all():
            check_token32(y32[t], ref["y"][t])
    return max(errs)


# ----------------------------------------------------------- bit-exact pin
def _int_expert(rng, d, f):
    # Redraw until gelu(g) == g exactly (g >= 10, in fp32 and fp64) and every
    # fp32 partial sum of the down projection stays an integer below 2^24.
    while True:
        x = rng.integers(1, 4, size=d)
        G = (rng.random((f, d)) < 0.06).astype(np.uint8)
        U = (rng.random((f, d)) < 0.006).astype(np.uint8)
        Dn = rng.integers(0, 16, size=(d, f)).astype(np.uint8)
        g = G.astype(np.int64) @ x
        h = g * (U.astype(np.int64) @ x)
        if g.min() >= 10 and 32 * 1039 * h.max() < 2 ** 24 and h.max() > 0:
            break

    def mat(codes, scale):
        n, k = codes.shape
        return {"q": (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8),
                "scale": np.full((n, k // 64), scale, np.float16),
                "bias": np.zeros((n, k // 64), np.float16), "n": n, "k": k, "bits": 4}
    ex = {"gate": mat(G, 1.0), "up": mat(U, 1.0), "down": mat(Dn, 0.5)}
    return ex, x


def test_integer_expert_is_bitwise_exact(tfa):
    rng = np.random.default_rng(21)
    d, f = 256, 128
    blobs, xs = [], []
    for _ in range(3):
        ex, x = _int_expert(rng, d, f)
        blobs.append(gen.expert_blob(ex))
        xs.append(x)
    pool = torch.from_numpy(np.stack(blobs)).cuda()
    x16 = np.stack(xs).astype(np.float16)
    slot = torch.tensor([0, 1, 2, 2], dtype=torch.int32, device="cuda")
    token = torch.tensor([0, 1, 2, 2], dtype=torch.int32, device="cuda")
    coef = torch.tensor([1.0, 1.0, 1.0, 0.5], dtype=torch.float32, device="cuda")
    y32 = torch.zeros((3, d), dtype=torch.float32, device="cuda")
    tfa.tf_expert_q4_gemv(pool, pool.shape[1], d, f, slot, token, coef,
                          torch.from_numpy(x16.view(np.int16)).cuda(), y32)
    got = y32.cpu().numpy()
    for t in range(3):
        ref = oracle.expert_from_blob(blobs[t], d, f, xs[t].astype(np.float64))
        if t == 2:
            ref = ref + 0.5 * ref
        assert np.array_equal(got[t], ref.astype(np.float32)), t


# ----------------------------------------------------------- tiny layer
TINY = gen.WORKLOADS[0]


@pytest.fixture(scope="module")
def tiny():
    return oracle_layer(TINY.seed, 0, TINY.d_model, TINY.n_experts, TINY.top_k, TINY.d_ff,
                        TINY.d_ff_shared)


def test_tiny_layer_one_token(tfa, tiny):
    x = gen.tokens(TINY.seed, 1, TINY.d_model)
    _check_layer(tiny, tfa, x)


@pytest.mark.parametrize("T", [2, 5, 16])
def test_tiny_layer_batched(tfa, tiny, T):
    x = gen.tokens(TINY.seed, T, TINY.d_model)
    _check_layer(tiny, tfa, x)


def test_tiny_layer_tanh_variant(tfa, tiny):
    x = gen.tokens(TINY.seed, 3, TINY.d_model)
    _check_layer(tiny, tfa, x, tanh=True, act=1)


def test_one_expert_rule_on_gpu(tfa):
    L = oracle_layer(TINY.seed, 0, TINY.d_model, TINY.n_experts, 1, TINY.d_ff, TINY.d_ff_shared)
    sh = gen.shared_expert(TINY.seed, 0, TINY.d_model, TINY.d_ff_shared)
    for m in sh.values():
        m["scale"][:] = 0
        m["bias"][:] = 0
    L["shared_blob"] = gen.expert_blob(sh)
    x = gen.tokens(TINY.seed, 4, TINY.d_model)
    D = device_layer(L)
    y, ids, w, y32 = _run_layer(tfa, D, x)
    assert np.all(w == 1.0)
    for t in range(4):
        ye = oracle.expert_from_blob(L["pool"][ids[t, 0]], TINY.d_model, TINY.d_ff,
                                     x[t].astype(np.float64))
        check_token(y[t], ye)


def test_forced_ids_and_flags(tfa, tiny):
    x = gen.tokens(TINY.seed, 2, TINY.d_model)
    forced = np.array([[3, 1], [0, 7]], dtype=np.int32)
    _check_layer(tiny, tfa, x, forced=forced)
    D = device_layer(tiny)
    ws = tfa.workspace(tfa.tf_moe_workspace_bytes(D, 2))
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    bad = torch.tensor([[2, 2], [0, 9]], dtype=torch.int32, device="cuda")
    tfa.tf_moe_layer_fwd(D, xt, forced_ids=bad, ws=ws)
    fl = tfa.tf_workspace_flags(ws)
    assert fl == 3, fl
    assert tfa.tf_workspace_flags(ws) == 0       # read-and-clear


# ---------------------------------------------------- ragged shapes
RAG = dict(seed=77, d=320, E=12, k=3, f=192, fs=320)


@pytest.mark.parametrize("T", [1, 7, 16])
def test_ragged_shapes(tfa, T):
    L = oracle_layer(RAG["seed"], 0, RAG["d"], RAG["E"], RAG["k"], RAG["f"], RAG["fs"])
    x = gen.tokens(RAG["seed"], T, RAG["d"])
    _check_layer(L, tfa, x)


# ------------------------------------------- one token, wider d_ff
WIDE = dict(seed=78, d=256, E=16, k=4, f=1024, fs=256)


def test_one_token_wide_ff(tfa):
    """A one-token step with d_ff = 1024 (four 16-byte chunks per lane in the
    routed down, where the full-width layer has three): the same parity bar
    as every other shape."""
    L = oracle_layer(WIDE["seed"], 0, WIDE["d"], WIDE["E"], WIDE["k"], WIDE["f"], WIDE["fs"])
    x = gen.tokens(WIDE["seed"], 4, WIDE["d"])
    for t in range(4):
        _check_layer(L, tfa, x[t:t + 1])


def test_t_zero_is_a_no_op(tfa, tiny):
    D = device_layer(tiny)
    x = torch.zeros((0, TINY.d_model), dtype=torch.int16, device="cuda")
    y = torch.full((1, TINY.d_model), 7, dtype=torch.int16, device="cuda")
    ids = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    w = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    ws = tfa.workspace(tfa.tf_moe_workspace_bytes(D, 1))
    from bit_routed_expert_tf_amd import _lib
    import ctypes
    rc = _lib.load().tf_moe_layer_fwd(ctypes.byref(D.struct), ctypes.c_void_p(ws.data_ptr()), 0,
                                      None, ctypes.c_void_p(y.data_ptr()), None,
                                      ctypes.c_void_p(ids.data_ptr()),
                                      ctypes.c_void_p(w.data_ptr()), None, 0, None, None,
                                      ctypes.c_void_p(ws.data_ptr()), ws.numel())
    torch.cuda.synchronize()
    assert rc == 0 and torch.all(y == 7)


# ------------------------------------------------------ full width
FULL = gen.WORKLOADS[1]


@pytest.fixture(scope="module")
def full(tfa):
    L = oracle_layer(FULL.seed, 0, FULL.d_model, FULL.n_experts, FULL.top_k, FULL.d_ff,
                     FULL.d_ff_shared)
    return L, device_layer(L), gen.tokens(FULL.seed, FULL.n_tokens, FULL.d_model)


def test_full_width_decode_sampled_tokens(tfa, full):
    L, D, X = full
    for t in (0, 1, 2, 1234, 4999, 9999):
        y, ids, w, y32 = _run_layer(tfa, D, X[t:t + 1])
        ref = oracle.moe_token(L, X[t])
        assert np.array_equal(ids[0], ref["ids"]), t
        assert np.max(np.abs(w[0] - ref["p"])) <= 1e-6
        check_token(y[0], ref["y"])


def test_full_width_batch16(tfa, full):
    L, D, X = full
    x = X[100:116]
    y, ids, w, y32 = _run_layer(tfa, D, x)
    ref = oracle.moe_tokens(L, x)
    assert np.array_equal(ids, ref["ids"])
    for t in range(16):
        check_token(y[t], ref["y"][t])


def test_full_width_forced_uniform_routing(tfa, full):
    L, D, X = full
    forced = gen.uniform_ids(4, 0, 16, FULL.n_experts, FULL.top_k)
    x = X[200:216]
    y, ids, w, y32 = _run_layer(tfa, D, x, forced)
    ref = oracle.moe_tokens(L, x, forced)
    assert np.array_equal(ids, forced)
    assert np.max(np.abs(w - ref["p"])) <= 1e-6
    for t in range(16):
        check_token(y[t], ref["y"][t])


def test_repeat_runs_are_bitwise_identical(tfa, full):
    L, D, X = full
    a = _run_layer(tfa, D, X[300:316])
    b = _run_layer(tfa, D, X[300:316])
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_workspace_reused_across_token_counts(tfa, full):
    """One workspace for steps of 16, 3, 1, 5, 1 and 16 tokens: the same
    bits as a fresh workspace each time (the counters never share bytes with
    data regions whose place depends on the token count)."""
    L, D, X = full
    ws = tfa.workspace(tfa.tf_moe_workspace_bytes(D, 16))
    xt = torch.from_numpy(X[400:464].view(np.int16)).cuda()
    r0 = 0
    for T in (16, 3, 1, 5, 1, 16):
        x = xt[r0:r0 + T]
        a = tfa.tf_moe_layer_fwd(D, x, ws=ws, want_y32=True)
        b = tfa.tf_moe_layer_fwd(D, x, want_y32=True)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u.view(torch.int16) if u.dtype == torch.float16 else u,
                               v.view(torch.int16) if v.dtype == torch.float16 else v), T
        r0 += T


def test_one_token_counters_return_to_zero(tfa, full):
    """After one-token steps every counter and ticket of a fresh workspace
    (the router's ticket, the down launch's per-tile tickets) is zero again
    and no flag is set."""
    L, D, X = full
    ws = tfa.workspace(tfa.tf_moe_workspace_bytes(D, 1))
    xt = torch.from_numpy(X[500:506].view(np.int16)).cuda()
    for t in range(6):
        y, ids, w, y32 = tfa.tf_moe_layer_fwd(D, xt[t:t + 1], ws=ws, want_y32=True)
        ref = oracle.moe_token(L, X[500 + t])
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy()[0], ref["ids"])
        check_token(y.cpu().numpy().view(np.float16)[0], ref["y"])
    head = ws[:33024].cpu().numpy()       # header (16,640 B) and the down tickets (16,384 B)
    assert not head.any(), np.nonzero(head)[0][:8]
    assert tfa.tf_workspace_flags(ws) == 0


def test_router_topk_logits_fp64(tfa, full):
    L, D, X = full
    x = X[:64]
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    logits = torch.empty((64, FULL.n_experts), dtype=torch.float64, device="cuda")
    ids, w, _ = tfa.tf_router_topk(D, xt, logits=logits)
    torch.cuda.synchronize()
    ref_l = np.stack([oracle.qmatvec(L["router"], x[t].astype(np.float64)) for t in range(64)])
    got = logits.cpu().numpy()
    assert np.max(np.abs(got - ref_l)) <= 1e-12 * np.abs(ref_l).max()
    ref_ids = np.stack([oracle.topk(ref_l[t], FULL.top_k) for t in range(64)])
    assert np.array_equal(ids.cpu().numpy(), ref_ids)


def test_expert_gemv_pairs_grouped_by_token(tfa, full):
    L, D, X = full
    d, f = FULL.d_model, FULL.d_ff
    slots = np.array([5, 9, 9, 127, 0, 64], dtype=np.int32)
    tokens = np.array([0, 0, 1, 1, 1, 2], dtype=np.int32)
    coef = np.array([0.5, 0.25, 1.0, -0.75, 0.125, 2.0], dtype=np.float32)
    x = X[500:503]
    y0 = np.random.default_rng(3).standard_normal((3, d)).astype(np.float32)
    y32 = torch.from_numpy(y0.copy()).cuda()
    tfa.tf_expert_q4_gemv(D.pool, D.blob_stride, d, f, torch.from_numpy(slots).cuda(),
                          torch.from_numpy(tokens).cuda(), torch.from_numpy(coef).cuda(),
                          torch.from_numpy(x.view(np.int16)).cuda(), y32)
    got = y32.cpu().numpy()
    for t in range(3):
        ref = y0[t].astype(np.float64)
        for p in np.nonzero(tokens == t)[0]:
            ref = ref + coef[p] * oracle.expert_from_blob(L["pool"][slots[p]], d, f,
                                                          x[t].astype(np.float64))
        check_token32(got[t], ref)


# ------------------------------------------------------------ top-k ties
@pytest.mark.parametrize("E,k,pattern", [(128, 8, "all"), (128, 8, "pairs"), (128, 8, "blocks"),
                                         (64, 8, "pairs"), (300, 16, "blocks"), (9, 8, "pairs")])
def test_topk_exact_ties(tfa, E, k, pattern):
    """Router rows copied between experts give exactly equal fp64 logits:
    the selection must break them by the lower id, as the oracle does."""
    d = 256
    L = oracle_layer(TINY.seed + E, 0, d, E, k, 64, 64)
    r = L["router"]
    src = {"all": np.zeros(E, int), "pairs": np.arange(E) & ~1,
           "blocks": (np.arange(E) // 5) * 5}[pattern]
    for key in ("q", "scale", "bias"):
        r[key] = np.ascontiguousarray(r[key][src])
    D = device_layer(L)
    x = gen.tokens(TINY.seed, 8, d)
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    logits = torch.empty((8, E), dtype=torch.float64, device="cuda")
    ids, w, _ = tfa.tf_router_topk(D, xt, logits=logits)
    torch.cuda.synchronize()
    ref_l = np.stack([oracle.qmatvec(r, x[t].astype(np.float64)) for t in range(8)])
    ref_ids = np.stack([oracle.topk(ref_l[t], k) for t in range(8)])
    got = ids.cpu().numpy()
    assert np.array_equal(got, ref_ids)
    if pattern == "all":
        assert np.array_equal(got, np.tile(np.arange(k), (8, 1)))
    ref_p = np.stack([oracle.softmax(ref_l[t][ref_ids[t]]) for t in range(8)])
    assert np.max(np.abs(w.cpu().numpy() - ref_p)) <= 1e-6
