"""Vectorised fp64 reference of the MoE layer forward (numpy).

Every function takes float64 arrays (already decoded by ``oracle.formats``)
unless it says otherwise, and follows the plain definition of each step with
no blocking, fusion or reordering beyond a library matmul per step.

Steps and where they come from:
  router logits, top-k weights        -- "Fused MoE kernel on Triton: 5 launches
      vs 24" (ai-manual.ru), section "Fused kernel: one operation instead of
      twenty-four", first item of the fused list (top-k routing weights); the
      k is a run-time value (section "Megablocks? It has been obsolete for two
      years", flexibility item).
  dispatch                            -- same section, second item (tokens
      dispatched to their chosen experts).
  expert FFN on engaged experts       -- same section, third item; the FFN form
      (SwiGLU: down(silu(gate x) * up x)) is a reading, the pages never write it.
  weighted aggregation                -- same section, fourth item.
  shared experts                      -- "llama.cpp: fusing shared experts into
      MMVQ" (ai-manual.ru), sections "Shared experts in MoE: what they are and
      why they exist" and "How shared experts differ from routed ones": always
      active, independent of the router; read here as added with weight 1.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, Wr: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h] + b[e]  (b = 0 when absent)."""
    l = x @ Wr.T
    if b is not None:
        l = l + np.asarray(b, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """p[t, e] = exp(l[t, e] - max_e l[t, :]) / sum_e' exp(l[t, e'] - max)."""
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def select_topk(l: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest logits, by descending logit; equal logits
    go to the lower expert index.  Selecting on the logits is the same as
    selecting on the softmax probabilities (softmax is increasing)."""
    order = np.argsort(-l, axis=-1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalize(p: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, ids[t, j]] / sum_j' p[t, ids[t, j']] (selected weights sum to 1)."""
    sel = np.take_along_axis(p, ids, axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


def route(x, Wr, b, k):
    """Router logits, softmax, top-k and renormalisation.  Returns (l, p, ids, w)."""
    l = router_logits(x, Wr, b)
    p = softmax(l)
    ids = select_topk(l, k)
    w = renormalize(p, ids)
    return l, p, ids, w


def near_ties(l: np.ndarray, k: int, tau: float = 1e-4) -> np.ndarray:
    """Tokens whose selection (set or order) a rounding error below ``tau`` could change.

    A token is flagged when two neighbours among its min(k+1, E) largest
    logits are closer than ``tau``.  The GPU computes logits in fp32, so for a
    flagged token either ordering is an acceptable result."""
    s = -np.sort(-l, axis=-1)[:, : min(k + 1, l.shape[1])]
    if s.shape[1] < 2:
        return np.zeros(l.shape[0], dtype=bool)
    return (np.diff(-s, axis=-1) < tau).any(axis=-1)


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """y = Wd (silu(Wg x) * (Wu x)) for each row x of ``x``.

    Wg, Wu: [I, H]; Wd: [H, I]; x: [n, H] -> y: [n, H]."""
    a = silu(x @ Wg.T) * (x @ Wu.T)
    return a @ Wd.T


def moe_forward_tokens(x, ids, w, Wg, Wu, Wd, shared=None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x[t]) + sum_s FFN^s(x[t]).

    The routing (ids, w) is given; ``shared`` is None or (Wsg, Wsu, Wsd) with
    leading dimension S.  Experts are visited one at a time over the tokens
    routed to them."""
    T, H = x.shape
    out = np.zeros((T, H), dtype=np.float64)
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        y = swiglu_ffn(x[t_idx], Wg[e], Wu[e], Wd[e])
        np.add.at(out, t_idx, w[t_idx, j_idx][:, None] * y)
    if shared is not None:
        Wsg, Wsu, Wsd = shared
        for s in range(Wsg.shape[0]):
            out += swiglu_ffn(x, Wsg[s], Wsu[s], Wsd[s])
    return out


def moe_forward(x, Wr, b, Wg, Wu, Wd, k, shared=None) -> dict:
    """Whole layer: route, then experts and aggregation.

    Returns dict(out, logits, p, ids, w)."""
    l, p, ids, w = route(x, Wr, b, k)
    out = moe_forward_tokens(x, ids, w, Wg, Wu, Wd, shared)
    return dict(out=out, logits=l, p=p, ids=ids, w=w)


def dense_gate_matrix(ids: np.ndarray, w: np.ndarray, E: int) -> np.ndarray:
    """G[t, e] = routing weight of expert e for token t (0 when not selected)."""
    T, k = ids.shape
    G = np.zeros((T, E), dtype=np.float64)
    np.add.at(G, (np.repeat(np.arange(T), k), ids.reshape(-1)), w.reshape(-1))
    return G


# ----------------------------------------------------------------------------
# dispatch (integer only)
# ----------------------------------------------------------------------------

def padded_rows(T: int, k: int, E: int, M: int) -> int:
    """Capacity of the expert-sorted order: T*k + E*(M-1) rounded up to a multiple of M."""
    n = T * k + E * (M - 1)
    return (n + M - 1) // M * M


def dispatch(ids: np.ndarray, E: int, M: int) -> dict:
    """Expert-sorted order of the flat assignments f = t*k + j.

    counts[e]      number of f routed to e
    offsets[e]     start of e's segment; segments are padded to multiples of M
    sorted_ids[p]  the r-th smallest f routed to e sits at offsets[e] + r;
                   padding and the tail up to the capacity hold T*k
    tile_expert[i] expert owning rows [i*M, (i+1)*M), -1 past offsets[E]
    inv[f]         position of f in sorted_ids
    active         experts with counts > 0, ascending
    """
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    n = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    padded = (counts + M - 1) // M * M
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    cap = padded_rows(T, k, E, M)
    sorted_ids = np.full(cap, n, dtype=np.int64)
    inv = np.empty(n, dtype=np.int64)
    for e in range(E):
        fs = np.nonzero(flat == e)[0]          # ascending flat ids
        pos = offsets[e] + np.arange(fs.size)
        sorted_ids[pos] = fs
        inv[fs] = pos
    tile_expert = np.full(cap // M, -1, dtype=np.int64)
    for e in range(E):
        tile_expert[offsets[e] // M: offsets[e + 1] // M] = e
    active = np.nonzero(counts > 0)[0]
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids,
                tile_expert=tile_expert, inv=inv, active=active, capacity=cap)


# ----------------------------------------------------------------------------
# budgeted top-c channel-sparse experts
# ----------------------------------------------------------------------------
# "KAIST removed calibration from MoE decoding and sped up blocks up to
# 2.69x over vLLM" (news.hamidun.com), sections "A threshold promises a
# budget but does not keep it" and "Top-k instead of a threshold": inside an
# expert most intermediate channels barely affect a given token; a selector
# scores the channels and only the chosen channels' weights are read, and the
# page argues for keeping, per token, a fixed number of channels with the
# highest scores rather than those above a threshold.  Given that set the
# computation is the expert FFN restricted to those channels (rows of Wg and
# Wu, columns of Wd).  The scorer itself (the "reader" built from the
# weights) is not part of this computation: scores are an input.

def select_channels(scores: np.ndarray, c: int) -> np.ndarray:
    """Indices of the c highest scores, ascending.

    Ranking: a higher score first; equal scores go to the lower index; a NaN
    score ranks below every number (-inf included), NaNs among themselves by
    index.  The rule is stated as explicit sort keys rather than left to how
    a sort happens to place NaN."""
    s = np.asarray(scores, dtype=np.float64)
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s)                     # placeholder for NaN: decided by the first key
    order = np.lexsort((np.arange(s.size), neg, nan))   # keys: NaN last, then -score, then index
    return np.sort(order[:c])


def masked_swiglu(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, chan: np.ndarray) -> np.ndarray:
    """The expert FFN over the channel set ``chan`` only: Wd[:, C] (silu(Wg[C] x) * (Wu[C] x))."""
    a = silu(x @ Wg[chan].T) * (x @ Wu[chan].T)
    return a @ Wd[:, chan].T


def moe_forward_channel_sparse(x, Wr, b, Wg, Wu, Wd, k, scores, c, shared=None, ids=None) -> dict:
    """The layer with budgeted channel sparsity in the routed experts.

    scores [T, E, I]: channel scores of every token for every expert; c: the
    number of channels kept per (token, engaged expert).  Routing and the
    shared experts are as in ``moe_forward`` (shared experts stay dense).
    ``ids`` (optional) replaces the oracle's own expert choice."""
    l, p, ids_o, _ = route(x, Wr, b, k)
    ids = ids_o if ids is None else ids
    w = renormalize(p, ids)
    T, H = x.shape
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            e = ids[t, j]
            chan = select_channels(scores[t, e], c)
            out[t] += w[t, j] * masked_swiglu(x[t:t + 1], Wg[e], Wu[e], Wd[e], chan)[0]
    if shared is not None:
        Wsg, Wsu, Wsd = shared
        for s in range(Wsg.shape[0]):
            out += swiglu_ffn(x, Wsg[s], Wsu[s], Wsd[s])
    return dict(out=out, logits=l, ids=ids_o, w=w, ids_used=ids)
