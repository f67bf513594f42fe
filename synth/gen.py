"""Seeded synthetic workloads for the q4 MoE layer.

Everything here is random draws and byte layout -- no dequantisation, no dot
products, no routing decisions.  The shapes and value distributions follow the
five workloads of the q4 MoE-layer study (a tiny single layer, a full-width
decode layer, a 30-layer slot-cache stack, a 128-token prefill chunk and an
all-resident 30-layer roofline case); the model they stand in for is the one
the TurboFieldfare write-ups describe (blog.hypho.cn "它省的不是模型大小":
128 routed experts per layer, 8 chosen per token, plus a dense shared expert;
shilu.ai "概览" table: MLX affine 4-bit weights with group 64, 8-bit router).

Random streams
--------------
Each matrix is drawn from ``numpy.random.default_rng([seed, layer, owner,
matrix])`` with ``owner`` = expert id, ``SHARED`` (1000) or ``ROUTER`` (2000)
and ``matrix`` = router 0, gate 1, up 2, down 3; the draw order is q, then
scale, then bias.  Token activations come from ``default_rng([seed, 9000])``
and forced routing from ``default_rng([seed, 9001, layer])``.  Any expert of
any layer can therefore be regenerated on its own.

Canonical quantised matrix ``W[n][k]`` (affine, group 64)
---------------------------------------------------------
* ``q``: uint8 ``[n][k*bits/8]``.  For 4 bits, element ``j`` of a row sits in
  byte ``j // 2``, in the low nibble when ``j`` is even and the high nibble
  when it is odd.  For 8 bits, one byte per element.
* ``scale``, ``bias``: IEEE fp16 ``[n][k/64]``; group ``g`` covers elements
  ``64g .. 64g+63`` of its row.

Expert blob (one routed expert, the unit a slot holds)
------------------------------------------------------
``gate.q | gate.scale | gate.bias | up.q | up.scale | up.bias | down.q |
down.scale | down.bias`` back to back, with gate/up ``[d_ff][d_model]`` and
down ``[d_model][d_ff]``.  At d_model=2816, d_ff=704 that is 3,345,408 bytes.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GROUP = 64
SHARED = 1000
ROUTER = 2000
MAT_ROUTER, MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2, 3
X_STREAM = 9000
IDS_STREAM = 9001

__all__ = [
    "GROUP", "SHARED", "ROUTER", "Workload", "WORKLOADS", "qmat", "expert",
    "shared_expert", "router", "tokens", "expert_blob", "blob_bytes",
    "blob_offsets", "expert_pool", "zipf_ids", "uniform_ids", "shared_blob",
]


@dataclass(frozen=True)
class Workload:
    """Shapes, seed and routing of one synthetic workload."""
    name: str
    seed: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    d_ff_shared: int
    n_layers: int = 1
    n_tokens: int = 1
    routing: str = "natural"          # natural | zipf | uniform
    zipf_s: float = 1.1
    n_slots: int = 0                  # slot-cache size per layer (0 = all resident)
    chunk: int = 0                    # prefill chunk length (0 = decode)
    batches: tuple = (1,)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload("tiny-layer-d256-e8k2", 0, 256, 8, 2, 128, 256),
    1: Workload("decode-layer-d2816-e128k8", 1, 2816, 128, 8, 704, 2816,
                n_tokens=10_000),
    2: Workload("slot-cache-stack-30L-16slot-zipf1.1", 2, 2816, 128, 8, 704, 2816,
                n_layers=30, n_tokens=2048, routing="zipf", n_slots=16),
    3: Workload("prefill-chunk128-d2816-e128k8", 3, 2816, 128, 8, 704, 2816,
                n_tokens=64 * 128, chunk=128),
    4: Workload("resident-stack-30L-e128k8-uniform", 4, 2816, 128, 8, 704, 2816,
                n_layers=30, n_tokens=1000, routing="uniform", batches=(1, 16),
                extra={"warmup_steps": 50}),
}


def _rng(*key):
    return np.random.default_rng([int(k) for k in key])


def qmat(seed, layer, owner, matrix, n, k, bits=4, scale_lo=0.002, scale_hi=0.02,
         bias_lo=-0.1, bias_hi=0.1):
    """Draw one affine-quantised matrix ``W[n][k]`` (canonical layout above).

    4-bit codes are drawn as whole bytes uniform on 0..255, i.e. two
    independent nibbles uniform on 0..15.
    """
    if k % GROUP:
        raise ValueError("k must be a multiple of 64")
    rng = _rng(seed, layer, owner, matrix)
    q = rng.integers(0, 256, size=(n, k * bits // 8), dtype=np.uint8)
    ng = k // GROUP
    scale = rng.uniform(scale_lo, scale_hi, size=(n, ng)).astype(np.float16)
    bias = rng.uniform(bias_lo, bias_hi, size=(n, ng)).astype(np.float16)
    return {"q": q, "scale": scale, "bias": bias, "n": n, "k": k, "bits": bits}


def expert(seed, layer, e, d_model, d_ff):
    """One routed expert: gate/up ``[d_ff][d_model]``, down ``[d_model][d_ff]``."""
    return {
        "gate": qmat(seed, layer, e, MAT_GATE, d_ff, d_model),
        "up": qmat(seed, layer, e, MAT_UP, d_ff, d_model),
        "down": qmat(seed, layer, e, MAT_DOWN, d_model, d_ff),
    }


def shared_expert(seed, layer, d_model, d_ff_shared):
    return expert(seed, layer, SHARED, d_model, d_ff_shared)


def router(seed, layer, d_model, n_experts):
    """8-bit router ``[n_experts][d_model]``.

    Codes uniform on 0..255; the scale range is the experts' range times
    15/255 so that dequantised router weights span what the 4-bit experts
    span; bias as for the experts.
    """
    f = 15.0 / 255.0
    return qmat(seed, layer, ROUTER, MAT_ROUTER, n_experts, d_model, bits=8,
                scale_lo=0.002 * f, scale_hi=0.02 * f)


def tokens(seed, n_tokens, d_model):
    """Activations x ~ N(0,1) rounded to fp16, ``[n_tokens][d_model]``."""
    return _rng(seed, X_STREAM).standard_normal((n_tokens, d_model)).astype(np.float16)


def _section_sizes(n, k, bits=4):
    qb = n * k * bits // 8
    sb = n * (k // GROUP) * 2
    return qb, sb, sb


def blob_offsets(d_model, d_ff):
    """Byte offsets of the nine sections of an expert blob, plus its size."""
    off = {}
    pos = 0
    for name, (n, k) in (("gate", (d_ff, d_model)), ("up", (d_ff, d_model)),
                         ("down", (d_model, d_ff))):
        qb, sb, bb = _section_sizes(n, k)
        off[name + ".q"] = pos
        pos += qb
        off[name + ".scale"] = pos
        pos += sb
        off[name + ".bias"] = pos
        pos += bb
    off["size"] = pos
    return off


def blob_bytes(d_model, d_ff):
    return blob_offsets(d_model, d_ff)["size"]


def expert_blob(ex):
    """Lay one expert's three matrices out as a contiguous uint8 blob."""
    parts = []
    for name in ("gate", "up", "down"):
        m = ex[name]
        parts += [m["q"].reshape(-1), m["scale"].view(np.uint8).reshape(-1),
                  m["bias"].view(np.uint8).reshape(-1)]
    return np.concatenate(parts)


def shared_blob(seed, layer, d_model, d_ff_shared):
    return expert_blob(shared_expert(seed, layer, d_model, d_ff_shared))


def expert_pool(seed, layer, d_model, d_ff, n_experts, stride=None, out=None,
                experts=None, threads=None):
    """Blobs of ``n_experts`` routed experts of one layer, ``[n_experts][stride]``.

    ``out`` may be a preallocated uint8 array (e.g. pinned host memory viewed
    through numpy) of shape ``[n_experts][stride]``.  ``experts`` restricts the
    draw to a subset of ids (other rows are left untouched).
    """
    size = blob_bytes(d_model, d_ff)
    stride = stride or size
    if out is None:
        out = np.zeros((n_experts, stride), dtype=np.uint8)
    ids = range(n_experts) if experts is None else experts

    def one(e):
        out[e, :size] = expert_blob(expert(seed, layer, e, d_model, d_ff))

    threads = threads or min(8, os.cpu_count() or 1)
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, ids))
    else:
        for e in ids:
            one(e)
    return out


def zipf_ids(seed, layer, n_tokens, n_experts, top_k, s=1.1):
    """Forced routing with Zipf(s) expert popularity, ``int32 [n_tokens][top_k]``.

    A seeded permutation maps popularity rank r (1-based) to an expert id.
    Each token then draws ``top_k`` distinct ranks by successive sampling
    without replacement with weights r**-s, realised as Gumbel-top-k (sorting
    log r**-s + Gumbel noise in descending order gives the same distribution
    over ordered draws).  ids are listed in draw order.
    """
    rng = _rng(seed, IDS_STREAM, layer)
    perm = rng.permutation(n_experts)
    logw = -s * np.log(np.arange(1, n_experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(n_tokens, n_experts))
    order = np.argsort(-(logw[None, :] + g), axis=1, kind="stable")[:, :top_k]
    return perm[order].astype(np.int32)


def uniform_ids(seed, layer, n_tokens, n_experts, top_k):
    """Forced routing: ``top_k`` distinct ids uniform per token, in draw order."""
    rng = _rng(seed, IDS_STREAM, layer)
    keys = rng.random((n_tokens, n_experts))
    return np.argsort(keys, axis=1, kind="stable")[:, :top_k].astype(np.int32)


SAMPLE_STREAM = 9100
VOCAB = 262144   # the vocabulary size taken for the sampling step (2**18)


def sample_inputs(seed, n_rows, vocab=VOCAB, pattern="lm"):
    """Logits ``fp32 [n_rows][vocab]`` and draws ``u fp64 [n_rows]`` in [0, 1).

    ``pattern``:
      * ``"lm"``: N(0, 2) per logit plus a head of 32 ids per row lifted by
        Exp(mean 6), so the top 64 hold most of the mass at temperature 1;
      * ``"ties"``: integers 0..7 (many equal logits);
      * ``"sorted"``: the "lm" row sorted ascending (the largest logits last);
      * ``"special"``: the "lm" row with NaN, -inf, +-0 and a row maximum
        repeated at several ids.
    """
    rng = _rng(seed, SAMPLE_STREAM, n_rows, vocab)
    if pattern == "ties":
        l = rng.integers(0, 8, size=(n_rows, vocab)).astype(np.float32)
    else:
        l = rng.normal(0.0, 2.0, size=(n_rows, vocab))
        for r in range(n_rows):
            head = rng.choice(vocab, size=min(32, vocab), replace=False)
            l[r, head] += rng.exponential(6.0, size=head.size)
        l = l.astype(np.float32)
        if pattern == "sorted":
            l.sort(axis=1)
        elif pattern == "special":
            for r in range(n_rows):
                pos = rng.choice(vocab, size=min(24, vocab), replace=False)
                top = l[r].max()
                l[r, pos[:6]] = np.nan
                l[r, pos[6:12]] = -np.inf
                l[r, pos[12:15]] = 0.0
                l[r, pos[15:18]] = -0.0
                l[r, pos[18:]] = top
    u = rng.random(n_rows)
    return l, u


ATTN_STREAM = 9300


def attn_inputs(seed, n_tokens, n_heads, n_kv_heads, head_dim):
    """Per token: q [H][D], k and v [G][D], fp16 draws of N(0, 1) (the scale
    of per-head normalised queries and keys).  Returns three arrays
    [n_tokens][...] of float16."""
    rng = _rng(seed, ATTN_STREAM, n_tokens, n_heads, n_kv_heads, head_dim)
    q = rng.standard_normal((n_tokens, n_heads, head_dim)).astype(np.float16)
    k = rng.standard_normal((n_tokens, n_kv_heads, head_dim)).astype(np.float16)
    v = rng.standard_normal((n_tokens, n_kv_heads, head_dim)).astype(np.float16)
    return q, k, v
