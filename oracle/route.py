"""Oracle: top-k routing and the counting sort of (token, expert) pairs.

Test infrastructure only (see the package docstring).  The pages never write the routing down; this
library adopts the usual definition: router logits -> softmax -> top-k, weights renormalized over the
k selected experts [DEF].
"""

import numpy as np


def route_ref(logits, k, renormalize=True):
    """Top-k routing.

    logits: float32 [T, E].  Returns (ids int32 [T, k], w float64 [T, k]).
      * ids[t] are the k largest logits of token t in descending order; equal logits are taken in
        increasing expert index (reading: the pages are silent on ties).  Softmax is monotone, so
        choosing on the logits is choosing on the softmax probabilities, without rounding ties.
      * w[t, j] = exp(l_j - l_max) / S, with S the sum of exp(l - l_max) over the k selected experts
        when renormalize is set, else over all E experts (the plain softmax probability).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    l64 = logits.astype(np.float64)
    ex = np.exp(l64 - l64.max(axis=1, keepdims=True))
    sel = np.take_along_axis(ex, ids.astype(np.int64), axis=1)
    denom = sel.sum(axis=1, keepdims=True) if renormalize else ex.sum(axis=1, keepdims=True)
    return ids, sel / denom


def sort_pairs_ref(ids, E):
    """Counting sort of the T*k pairs p = t*k + j by expert.

    Returns (offsets int32 [E+1], sorted_pairs int32 [T*k]): offsets is the exclusive prefix sum of
    the per-expert pair counts, and the pairs of expert e sit in sorted_pairs[offsets[e]:offsets[e+1]]
    in increasing p (a stable sort).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    return offsets, sorted_pairs
