"""fp64 CPU oracle for the q4 MoE layer -- TEST INFRASTRUCTURE ONLY.

Two independent implementations of the same definitions:

* the C library ``oracle/moe_oracle.c`` (fp64, OpenMP over rows), driven
  through ctypes by the ``orc_*``-backed functions below; and
* a NumPy fp64 twin (``np_*``) that dequantises whole matrices and uses
  library matmul / erf.  The two agree to ~1e-12 on the tiny workload.

Plus two integer oracles written as plain Python loops:

* ``lfu_replay``: the 16-slot per-layer expert cache.  The pages name the
  policy LFU (shilu.ai README translation, "推理引擎的工作原理"; the
  sh.edu-sjtu.cn article, "三件事", writes LFU but glosses it as
  longest-unused eviction).  Reading taken: in-cache LFU -- a slot's count is
  1 on fill and +1 per hit; the token's own ids are pinned; misses are handled
  in rank order; the victim is the lowest empty slot, else the unpinned slot
  with the smallest (count, last-use token, slot index); every layer starts
  empty.
* ``sample``: the next-token choice after the stack.  The pages give the
  knobs and their defaults (shilu.ai README translation, "向模型输入
  prompt": temperature 0.2, Top-K 64, Top-P 0.95, temperature 0 for greedy
  output); the order of the steps is a reading: the K largest logits (ties
  to the lower id), their softmax at the temperature, the shortest rank
  prefix whose cumulative probability reaches P, then the first kept rank
  whose cumulative probability exceeds u times the kept total, u in [0, 1)
  given by the caller.  Every sum runs sequentially in rank order.
* ``attn_decode``: one decode step of attention for one new token.  The
  pages give the store and the kind of kernel (shilu.ai README translation,
  "状态和范围": fp16 keys and values; a bounded ring for the 25
  sliding-window layers and linear storage for the 5 full-attention layers;
  exact split-K/V decode attention).  Definition: per query head h, with
  key/value head g = h // (H / G), scores s_t = scale * (q_h . k_{g,t}) over
  the tokens t the layer sees (the last `window` tokens up to and including
  the new one, or all of them), p = softmax(s), out_h = sum_t p_t v_{g,t}.
  The oracle keeps every token's key and value in token order and knows
  nothing of a ring; "exact" is read as the full softmax, no approximation.
* ``group_by_expert``: (token, rank) pairs of a prefill chunk sorted by
  (expert, token, rank) -- the grouping that lets one fetched expert serve
  several rows (shilu.ai, "推理引擎的工作原理": prefill in chunks of at
  most 128 tokens).

The layer definition (configs of the study; the pages only say the shared and
routed outputs are combined -- sh.edu-sjtu.cn "三件事", shilu.ai
"推理引擎的工作原理"):

    y = shared(x) + sum_{k in top-k} softmax(l_topk)_k * expert_k(x)
    expert(x) = W_down (gelu(W_gate x) (.) (W_up x)),   l = W_router x

Parity pins (tests/test_oracle_pins.py): dequant of hand-built groups, nibble
order by one-hot columns, integer-exact GEMV, brute-force top-k with ties,
softmax identities, GELU values (Phi(1)), the one-expert rule, closed-form
0/1 experts, identical-expert combine, hand-derived LFU sequences, byte
accounting against the pages' 14.3 GB / 1.35 GB, fp16 decode of all 65536
patterns, C-vs-NumPy agreement, hand-worked sampling rows, and for attention a
hand-worked two-token case, the uniform-score mean, window and order
invariances and the query-head grouping.  No function here is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
# a separately built copy (the sanitizer test's) when ORACLE_LIBRARY names one
_SO_OVERRIDE = os.environ.get("ORACLE_LIBRARY")
_lock = threading.Lock()
_lib = None

__all__ = [
    "build", "lib", "half_to_double", "qmatvec", "weight", "gelu", "topk",
    "softmax", "expert_ffn", "expert_from_blob", "moe_token", "moe_tokens",
    "np_dequant", "np_qmatvec", "np_gelu", "np_topk", "np_softmax",
    "np_expert", "np_moe_token", "lfu_replay", "group_by_expert", "to_fp16",
    "num_threads", "set_num_threads", "sample", "attn_decode",
]


def build(force=False):
    """Compile the C oracle (gcc, -O2 -fopenmp)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC,
                               "-lm", "-o", tmp])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if _SO_OVERRIDE:
                L = ctypes.CDLL(_SO_OVERRIDE)
            else:
                build()
                L = ctypes.CDLL(_SO)
            P = ctypes.c_void_p
            i32, i64 = ctypes.c_int, ctypes.c_int64
            L.orc_half_to_double.restype = ctypes.c_double
            L.orc_half_to_double.argtypes = [ctypes.c_uint16]
            L.orc_halves_to_double.argtypes = [P, i64, P]
            L.orc_weight.restype = ctypes.c_double
            L.orc_weight.argtypes = [P, P, P, i32, i32, i32, i32, i32]
            L.orc_qmatvec.argtypes = [P, P, P, i32, i32, i32, P, P]
            L.orc_gelu.restype = ctypes.c_double
            L.orc_gelu.argtypes = [ctypes.c_double, i32]
            L.orc_topk.argtypes = [P, i32, i32, P]
            L.orc_softmax.argtypes = [P, i32, P]
            L.orc_set_num_threads.argtypes = [i32]
            L.orc_set_num_threads.restype = None
            L.orc_expert_ffn.argtypes = [P] * 9 + [i32, i32, i32, P, P, P]
            L.orc_expert_blob.argtypes = [P, i32, i32, i32, P, P, P]
            L.orc_moe_token.restype = i32
            L.orc_moe_token.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32,
                                        i32, P, P, P, P, P, P]
            L.orc_num_threads.restype = i32
            _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads():
    return lib().orc_num_threads()


def set_num_threads(n):
    """Threads of later C-oracle calls (timing only; results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------
# C-backed oracle
# --------------------------------------------------------------------------
def half_to_double(h):
    h = _c(np.asarray(h).view(np.uint16) if np.asarray(h).dtype == np.float16 else h,
           np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().orc_halves_to_double(_p(h), h.size, _p(out))
    return out


def _mat(m):
    return (_c(m["q"], np.uint8), _c(m["scale"], np.float16).view(np.uint16),
            _c(m["bias"], np.float16).view(np.uint16))


def weight(m, r, j):
    q, s, b = _mat(m)
    return lib().orc_weight(_p(q), _p(s), _p(b), m["n"], m["k"], m["bits"], r, j)


def qmatvec(m, x):
    """y = W x for a canonical quantised matrix, fp64 (x taken as fp64)."""
    q, s, b = _mat(m)
    x = _c(x, np.float64)
    y = np.empty(m["n"], dtype=np.float64)
    lib().orc_qmatvec(_p(q), _p(s), _p(b), m["n"], m["k"], m["bits"], _p(x), _p(y))
    return y


def gelu(z, tanh=False):
    return lib().orc_gelu(float(z), 1 if tanh else 0)


def topk(logits, k):
    l = _c(logits, np.float64)
    ids = np.empty(k, dtype=np.int32)
    lib().orc_topk(_p(l), l.size, k, _p(ids))
    return ids


def softmax(l):
    l = _c(l, np.float64)
    p = np.empty_like(l)
    lib().orc_softmax(_p(l), l.size, _p(p))
    return p


def expert_ffn(ex, x, tanh=False, return_h=False):
    """expert(x) = W_down (gelu(W_gate x) (.) (W_up x)), fp64."""
    g, u, d = _mat(ex["gate"]), _mat(ex["up"]), _mat(ex["down"])
    dm, f = ex["gate"]["k"], ex["gate"]["n"]
    x = _c(x, np.float64)
    y = np.empty(dm, dtype=np.float64)
    h = np.empty(f, dtype=np.float64)
    lib().orc_expert_ffn(*[_p(a) for a in (*g, *u, *d)], dm, f, 1 if tanh else 0,
                         _p(x), _p(y), _p(h))
    return (y, h) if return_h else y


def expert_from_blob(blob, d_model, d_ff, x, tanh=False):
    blob = _c(blob, np.uint8)
    x = _c(x, np.float64)
    y = np.empty(d_model, dtype=np.float64)
    lib().orc_expert_blob(_p(blob), d_model, d_ff, 1 if tanh else 0, _p(x), _p(y), None)
    return y


def moe_token(layer, x16, forced=None, tanh=False):
    """One token through one layer.

    ``layer``: dict with ``router`` (canonical 8-bit matrix), ``shared_blob``
    (uint8), ``pool`` (uint8 ``[E][stride]``), ``d_model``, ``d_ff``,
    ``d_ff_shared``, ``top_k``.  ``x16``: fp16 ``[d_model]``.
    Returns dict(y fp64 [d], ids int32 [k], p fp64 [k], logits fp64 [E]).
    """
    rq, rs, rb = _mat(layer["router"])
    pool = layer["pool"]
    if not (pool.flags.c_contiguous and pool.dtype == np.uint8):
        raise ValueError("pool must be a C-contiguous uint8 [E][stride] array")
    sb = _c(layer["shared_blob"], np.uint8)
    d, E, k = layer["d_model"], pool.shape[0], layer["top_k"]
    x16 = _c(np.asarray(x16, dtype=np.float16), np.float16).view(np.uint16)
    fr = None if forced is None else _c(forced, np.int32)
    y = np.empty(d, dtype=np.float64)
    ids = np.empty(k, dtype=np.int32)
    p = np.empty(k, dtype=np.float64)
    lg = np.empty(E, dtype=np.float64)
    rc = lib().orc_moe_token(_p(rq), _p(rs), _p(rb), _p(sb), _p(pool), pool.shape[1],
                             d, E, k, layer["d_ff"], layer["d_ff_shared"],
                             1 if tanh else 0, _p(x16), _p(fr), _p(y), _p(ids), _p(p),
                             _p(lg))
    if rc:
        raise ValueError("forced ids out of range or repeated")
    return {"y": y, "ids": ids, "p": p, "logits": lg}


def moe_tokens(layer, X16, forced=None, tanh=False):
    """Apply ``moe_token`` to each row of ``X16`` independently (prefill and
    batched decode are the per-token definition applied row by row)."""
    outs = [moe_token(layer, X16[t], None if forced is None else forced[t], tanh)
            for t in range(X16.shape[0])]
    return {key: np.stack([o[key] for o in outs]) for key in outs[0]}


# --------------------------------------------------------------------------
# NumPy fp64 twin (independent of the C code above)
# --------------------------------------------------------------------------
def np_dequant(m):
    """W = scale * q + bias as a dense fp64 matrix [n][k]."""
    n, k, bits = m["n"], m["k"], m["bits"]
    q = np.asarray(m["q"], dtype=np.uint8)
    if bits == 4:
        codes = np.empty((n, k), dtype=np.float64)
        codes[:, 0::2] = q & 15
        codes[:, 1::2] = q >> 4
    else:
        codes = q.astype(np.float64)
    s = np.repeat(np.asarray(m["scale"], np.float16).astype(np.float64), 64, axis=1)
    b = np.repeat(np.asarray(m["bias"], np.float16).astype(np.float64), 64, axis=1)
    return s * codes + b


def np_qmatvec(m, x):
    return np_dequant(m) @ np.asarray(x, dtype=np.float64)


def np_gelu(z, tanh=False):
    z = np.asarray(z, dtype=np.float64)
    if tanh:
        return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def np_topk(logits, k):
    l = np.asarray(logits, dtype=np.float64)
    order = np.lexsort((np.arange(l.size), -l))   # primary: -l, secondary: id
    return order[:k].astype(np.int32)


def np_softmax(l):
    l = np.asarray(l, dtype=np.float64)
    e = np.exp(l - l.max())
    return e / e.sum()


def np_expert(ex, x, tanh=False):
    x = np.asarray(x, dtype=np.float64)
    h = np_gelu(np_qmatvec(ex["gate"], x), tanh) * np_qmatvec(ex["up"], x)
    return np_qmatvec(ex["down"], h)


def _np_blob_expert(blob, d, f):
    def sec(pos, nbytes):
        return blob[pos:pos + nbytes], pos + nbytes
    out, pos = {}, 0
    for name, (n, k) in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f))):
        q, pos = sec(pos, n * k // 2)
        s, pos = sec(pos, n * (k // 64) * 2)
        b, pos = sec(pos, n * (k // 64) * 2)
        out[name] = {"q": q.reshape(n, k // 2), "scale": s.view(np.float16).reshape(n, -1),
                     "bias": b.view(np.float16).reshape(n, -1), "n": n, "k": k, "bits": 4}
    return out


def np_moe_token(layer, x16, forced=None, tanh=False):
    d, f, fs, k = layer["d_model"], layer["d_ff"], layer["d_ff_shared"], layer["top_k"]
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    l = np_qmatvec(layer["router"], x)
    ids = np.asarray(forced, dtype=np.int32) if forced is not None else np_topk(l, k)
    p = np_softmax(l[ids])
    y = np_expert(_np_blob_expert(np.asarray(layer["shared_blob"]), d, fs), x, tanh)
    for a in range(k):
        y = y + p[a] * np_expert(_np_blob_expert(layer["pool"][ids[a]], d, f), x, tanh)
    return {"y": y, "ids": ids, "p": p, "logits": l}


# --------------------------------------------------------------------------
# Integer oracles
# --------------------------------------------------------------------------
def lfu_replay(ids, n_slots, n_experts=None, policy="lfu"):
    """Replay the per-layer slot cache on a stream of token id rows.

    ``ids``: int ``[T][k]`` in rank order.  Returns (hit bool [T][k],
    slot int16 [T][k], final expert_of_slot int [S], final count [S]).
    ``policy``: "lfu" (the pages' word; victim = least (count, last use,
    slot)) or "lru" (the sh.edu-sjtu.cn article's gloss of it, "三件事":
    the longest-unused slot goes; victim = least (last use, slot)).  Both
    pin the token's own hits and fill the lowest empty slot first.
    """
    if policy not in ("lfu", "lru"):
        raise ValueError("policy must be 'lfu' or 'lru'")
    ids = np.asarray(ids)
    T, k = ids.shape
    S = n_slots
    if S < k:
        raise ValueError("n_slots must be >= top_k")
    expert_of = [-1] * S
    count = [0] * S
    last = [0] * S
    slot_of = {}
    hit = np.zeros((T, k), dtype=bool)
    slot = np.zeros((T, k), dtype=np.int16)
    for t in range(T):
        row = [int(e) for e in ids[t]]
        if len(set(row)) != k:
            raise ValueError("ids repeated within a token")
        pinned = set()
        for r, e in enumerate(row):            # hits first: they are pinned
            if e in slot_of:
                s = slot_of[e]
                count[s] += 1
                last[s] = t
                pinned.add(s)
                hit[t, r] = True
                slot[t, r] = s
        for r, e in enumerate(row):            # misses in rank order
            if hit[t, r]:
                continue
            empty = [s for s in range(S) if expert_of[s] == -1]
            if empty:
                v = empty[0]
            else:
                if policy == "lfu":
                    v = min((count[s], last[s], s) for s in range(S) if s not in pinned)[2]
                else:
                    v = min((last[s], s) for s in range(S) if s not in pinned)[1]
                del slot_of[expert_of[v]]
            expert_of[v] = e
            count[v] = 1
            last[v] = t
            slot_of[e] = v
            pinned.add(v)
            slot[t, r] = v
    return hit, slot, np.array(expert_of), np.array(count)


def sample(logits, temperature, top_k, top_p, u):
    """Next-token id from one row of logits (see the module docstring).

    ``logits``: fp32 or fp64 ``[V]`` (NaN ranks last); ``temperature`` 0 gives
    the greedy choice (largest logit, lowest id on ties); ``u`` in [0, 1).
    """
    l = np.asarray(logits, dtype=np.float64).copy()
    l[np.isnan(l)] = -np.inf
    V = l.size
    if not 1 <= top_k <= V:
        raise ValueError("need 1 <= top_k <= V")
    order = np.lexsort((np.arange(V), -l))          # logit desc, id asc
    if temperature == 0:
        return int(order[0])
    sel = order[:top_k]
    w = [float(np.exp((l[i] - l[sel[0]]) / temperature)) for i in sel]
    s = 0.0
    for x in w:
        s += x
    cum, c = [], 0.0
    for x in w:
        c += x / s
        cum.append(c)
    keep = top_k
    for n, c in enumerate(cum):
        if c >= top_p:
            keep = n + 1
            break
    target = u * cum[keep - 1]
    for n in range(keep):
        if cum[n] > target:
            return int(sel[n])
    return int(sel[keep - 1])


def attn_decode(q, k_hist, v_hist, window=None, scale=None):
    """Attention of one new token (see the module docstring).

    ``q``: [H][D] (fp16 values or floats); ``k_hist``, ``v_hist``: [N][G][D],
    the keys and values of tokens 0..N-1 in token order, the new token last;
    ``window``: the number of most recent tokens a sliding-window layer sees
    (None: all N); ``scale``: default 1/sqrt(D).  Returns fp64 [H][D].
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(k_hist, dtype=np.float64)
    Vv = np.asarray(v_hist, dtype=np.float64)
    H, D = q.shape
    N, G, _ = K.shape
    if H % G:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    first = 0 if window is None else max(0, N - window)
    out = np.empty((H, D))
    for h in range(H):
        g = h // (H // G)
        s = scale * (K[first:, g, :] @ q[h])       # one score per seen token
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ Vv[first:, g, :]
    return out


def group_by_expert(ids, n_experts):
    """(token, rank) pairs sorted by (expert, token, rank).

    Returns counts [E], offsets [E+1], and pairs int32 [T*k][3] of
    (expert, token, rank)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    pairs = [(int(ids[t, r]), t, r) for t in range(T) for r in range(k)]
    pairs.sort()
    counts = np.zeros(n_experts, dtype=np.int32)
    for e, _, _ in pairs:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    return counts, offsets, np.array(pairs, dtype=np.int32).reshape(-1, 3)


def to_fp16(y):
    """IEEE round-to-nearest-even to fp16 (|y| >= 65520 becomes +-inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float16)
