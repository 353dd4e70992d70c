"""Plain float64 CPU oracle of the routed-expert layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or run this module.  The HIP library never calls it,
and it shares no code, table or helper with the HIP path.  It is deliberately
slow and obvious: numpy in float64, one library primitive per step, no
blocking, fusion or reordering beyond what each definition states.

What the layer computes (sources named per function):

1. route    - per token, the k largest router logits and their normalised
              gate weights;
2. permute  - pairs (token, slot) grouped by expert into per-expert route
              lists;
3. expert FFN (SwiGLU) on each route list;
4. combine  - per token, the gate-weighted sum of its k expert outputs;
5. 3-bit grouped weights decoded to values before the products.

Inputs arrive as the exact stored values (bf16 / fp16 bit patterns, float32
logits, uint32 code words) and are widened exactly to float64.

Parity status: every function here is pinned by CPU tests (brute force on
tiny inputs, closed forms, invariants and hand-worked fixtures).  With respect
to the pages themselves all of it is "parity unpinned": the pages print no
layer-level value, worked example or kernel output to compare against.
"""
from __future__ import annotations

import numpy as np

Q3_GROUP = 128
Q3_WORDS = 13
Q3_FIELDS_PER_WORD = 10
Q3_OFFSET = 4


# ----------------------------------------------------------------- decoding

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (the high half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of IEEE binary16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def q3_fields(words: np.ndarray) -> np.ndarray:
    """Unpack the 128 three-bit fields of each group.

    Reading (the pages name a 3.0 bpw expert format but do not describe it):
    a group of 128 consecutive reduction-index weights of one output row is
    stored in 13 little-endian uint32 words; field j of a word occupies bits
    [3j, 3j+3); words 0..11 carry 10 fields each (bits 30-31 unused) and
    word 12 carries the last 8 (bits 24-31 unused).  Field f of the group sits
    in word f // 10 at position f % 10.

    ``words``: uint32 [..., 13]  ->  uint8 [..., 128]
    """
    words = np.asarray(words, dtype=np.uint32)
    f = np.arange(Q3_GROUP)
    w = words[..., f // Q3_FIELDS_PER_WORD]
    shift = (3 * (f % Q3_FIELDS_PER_WORD)).astype(np.uint32)
    return ((w >> shift) & np.uint32(7)).astype(np.uint8)


def q3_pack(fields: np.ndarray) -> np.ndarray:
    """Inverse of :func:`q3_fields` (used by tests to build words by hand)."""
    fields = np.asarray(fields, dtype=np.uint32)
    assert fields.shape[-1] == Q3_GROUP and int(fields.max(initial=0)) < 8
    words = np.zeros(fields.shape[:-1] + (Q3_WORDS,), dtype=np.uint32)
    for f in range(Q3_GROUP):
        words[..., f // Q3_FIELDS_PER_WORD] |= fields[..., f] << np.uint32(3 * (f % Q3_FIELDS_PER_WORD))
    return words


def q3_dequant(words: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Weights of a 3-bit grouped matrix: scale[n, g] * (field - 4).

    ``words`` uint32 [N, K/128, 13], ``scales`` fp16 bits [N, K/128]
    -> float64 [N, K].  Symmetric codes in [-4, 3], one fp16 scale per
    128-wide group of the reduction index.  Exact in float64.
    """
    codes = q3_fields(words).astype(np.float64) - Q3_OFFSET          # [N, G, 128]
    w = codes * f16_to_f64(scales)[..., None]
    return w.reshape(w.shape[0], -1)


def expert_matrices(raw: dict) -> tuple:
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) of one expert in float64.

    ``raw`` holds one expert's stored arrays: bf16 bits under "gate", "up",
    "down", or 3-bit words under the same names plus fp16 scales under
    "<name>_scale".
    """
    mats = []
    for which in ("gate", "up", "down"):
        if which + "_scale" in raw:
            mats.append(q3_dequant(raw[which], raw[which + "_scale"]))
        else:
            mats.append(bf16_to_f64(raw[which]))
    return tuple(mats)


# ------------------------------------------------------------------- route

def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray) -> np.ndarray:
    """Router logits logits[t, e] = x[t] . w_router[e], float64 over the exact
    bf16 values (x [T, H], w_router [E, H]).

    Source: dsv41-flash-offload wiki, opening paragraph -- tokens are routed to
    a few of the layer's routed experts; the router itself is not written on
    the pages.  Reading used: a bias-free linear layer over the hidden state,
    its rows stored [E, H] like the expert matrices.
    """
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_router_bits).T


def route_topk(logits: np.ndarray, k: int):
    """Top-k expert selection and gate weights for every token.

    Source: dsv41-flash-offload wiki, opening paragraph -- each MoE layer has
    384 routed experts and every token is served by a few of them.  The pages
    do not write the gate down; readings used here:

    * selection: the k largest logits of the token, ordered by value
      descending; equal values are ordered by expert index ascending, and
      -0.0 equals +0.0 (IEEE comparison);
    * weights: softmax over the k selected logits,
      w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), which is the softmax over
      all experts renormalised to the selected ones;
    * no routed scaling factor and no shared expert.

    Returns (ids int32 [T,k], w float64 [T,k]).
    """
    l64 = np.asarray(logits, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(l64)):
        raise ValueError("router logits must be finite")
    T, E = l64.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort of the negated values keeps ascending index among equals
    order = np.argsort(-l64, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(l64, order, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


def expert_histogram(ids: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, slot) pairs routed to each expert, one entry per
    expert (experts no token picked count 0).

    Source: dsv41-flash-offload wiki, repository file table, entry for the
    staged cold-expert prefill patch (per-expert route lists and their
    counts).  Pinned by hand-worked cases in tests/golden/metric_worked.txt.
    """
    return np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int32)


# ----------------------------------------------------------------- permute

def permute(ids: np.ndarray, E: int):
    """Group the (token, slot) pairs by expert into per-expert route lists.

    Source: dsv41-flash-offload wiki, repository file table, entry for the
    staged cold-expert prefill patch: routed work is kept as one list per
    expert and only experts with a positive count are run.  Pair p = t*k + j.
    Reading for a unique order: lists are concatenated in expert order and,
    inside a list, pairs keep ascending pair index (hence ascending token,
    since a token selects an expert at most once) -- a stable sort by expert.

    Returns (counts [E], offsets [E+1], sorted_pair [P], pair_to_sorted [P]),
    all int32; sorted_pair[i] is the pair stored at sorted row i and
    pair_to_sorted is its inverse.
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    sorted_pair = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    pair_to_sorted = np.empty_like(sorted_pair)
    pair_to_sorted[sorted_pair] = np.arange(flat.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_pair.astype(np.int32), pair_to_sorted.astype(np.int32))


# ------------------------------------------------------------- expert FFN

def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(xrows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert's SwiGLU FFN on a batch of token rows, in float64.

    The pages say busy experts run as FP16 GEMMs on reconstructed weights
    (wiki opening paragraph; file table, busy-expert GEMM entry) but never
    give the expert's form.  Reading: the SwiGLU expert of DeepSeek-style MoE
    layers -- g = x W_gate^T, u = x W_up^T, a = silu(g) * u, y = a W_down^T,
    with matrices stored [out, in].
    """
    g = xrows @ wg.T
    u = xrows @ wu.T
    a = silu(g) * u
    return a @ wd.T


def grouped_ffn(x: np.ndarray, expert_raw, offsets, sorted_pair, k: int, rows=None) -> np.ndarray:
    """Run every expert's FFN over its route list.

    ``x`` float64 [T,H]; ``expert_raw(e)`` returns expert e's stored arrays.
    Returns Y float64 [P,H] in sorted-row order (row i belongs to pair
    sorted_pair[i]).  With ``rows`` (a set of sorted-row indices) only those
    rows are computed and the others are left as NaN.
    """
    P = len(sorted_pair)
    H = x.shape[1]
    Y = np.full((P, H), np.nan)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        idx = np.arange(lo, hi)
        if rows is not None:
            idx = np.array([i for i in idx if i in rows], dtype=np.int64)
            if idx.size == 0:
                continue
        tokens = np.asarray(sorted_pair)[idx] // k
        wg, wu, wd = expert_matrices(expert_raw(e))
        Y[idx] = expert_ffn(x[tokens], wg, wu, wd)
    return Y


# ----------------------------------------------------------------- combine

def combine(Y: np.ndarray, w: np.ndarray, pair_to_sorted, k: int, tokens=None) -> np.ndarray:
    """out[t] = sum_j w[t,j] * Y[pair_to_sorted[t*k + j]].

    Source: dsv41-flash-offload wiki, repository file table, CPU-tier entry
    (routed work is split per expert and the results are combined back per
    token on the GPU).  Reading: the combine is the gate-weighted sum.
    """
    T = w.shape[0]
    tokens = range(T) if tokens is None else tokens
    out = np.zeros((len(tokens), Y.shape[1]))
    for r, t in enumerate(tokens):
        for j in range(k):
            out[r] += w[t, j] * Y[pair_to_sorted[t * k + j]]
    return out


# ---------------------------------------------------------- whole layer

def moe_layer(logits, x_bits, expert_raw, k: int, tokens=None) -> dict:
    """Route -> permute -> grouped SwiGLU experts -> combine.

    ``tokens`` (optional) restricts the expert and combine work to those
    tokens; routing and the permutation always cover the whole batch.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids, w = route_topk(logits, k)
    counts, offsets, sorted_pair, p2s = permute(ids, E)
    x = bf16_to_f64(x_bits)
    rows = None
    if tokens is not None:
        tokens = list(tokens)
        rows = {int(p2s[t * k + j]) for t in tokens for j in range(k)}
    Y = grouped_ffn(x, expert_raw, offsets, sorted_pair, k, rows=rows)
    out = combine(Y, w, p2s, k, tokens=tokens)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_pair=sorted_pair,
                pair_to_sorted=p2s, Y=Y, out=out, tokens=tokens)


def dense_layer(logits, x_bits, expert_raw, k: int) -> np.ndarray:
    """Brute force: every expert on every token, masked by the routing.

    out[t] = sum_e [e selected by t] * w_e(t) * FFN_e(x_t).  Uses no route
    list, gather or permutation; it cross-checks permute + grouped_ffn +
    combine on small layers.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids, w = route_topk(logits, k)
    gate = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            gate[t, ids[t, j]] = w[t, j]
    x = bf16_to_f64(x_bits)
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        wg, wu, wd = expert_matrices(expert_raw(e))
        out += gate[:, e:e + 1] * expert_ffn(x, wg, wu, wd)
    return out


def rel_max_err(got, ref) -> float:
    """max |got - ref| / rms(ref) over the whole tensor (the parity metric).

    Reading of the pages' relative-error comparison of two implementations
    (dsv41-flash-offload wiki, paragraph on the fidelity of the busy-expert GEMM path) as a bound on the
    largest element error; an all-zero reference falls back to max |err|.
    Pinned by hand-worked cases in tests/golden/metric_worked.txt.
    """
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))
