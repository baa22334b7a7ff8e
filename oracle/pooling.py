"""Incremental pooling (oracle side).

"Efficient Iterative Retrieval with Heterogeneous Batching": §3.3
Incremental Pooler splits an n-token input into chunks c_1..c_K and, for
mean and weighted-mean heads, keeps a running weighted sum of the chunk's
final hidden states and a running total of the weights, dividing at the
end; the summary page (agihunt, incremental-pooling paragraph) completes
the truncated statement and adds that CLS and last-token heads keep the
chosen hidden state.

Readings: mean uses weight 1 per token; weighted mean uses the token's
1-based position in its request (ctx_len + j + 1); CLS keeps the row at
position 0 (first chunk); last keeps the row at position n-1 (the final
chunk).

Summary page, incremental-pooling paragraph: a head that is not a streaming
sum can still be served, at a memory cost of n x d per request, by keeping
every final hidden state until the last chunk and applying the head once
there.  Reading: the BUFFER
kind stores each chunk's final hidden states at their positions in the
request (rows ctx_len .. ctx_len + n - 1 of the slot's buffer) and, on the
last chunk, runs one head over all N buffered rows; the head computed here
is the plain mean (1/N) sum of the rows, and the buffer stays readable for
any other head.

The OpRAG page (§ embedding pipeline) normalises pooled vectors to unit L2
length.  Reading: the L2 flag, OR'ed into any kind, returns
e / max(||e||_2, 1e-12) (the common normalise convention; a zero vector
stays zero).  Without it the pooled vector is returned unnormalised.
"""

import numpy as np

POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST, POOL_BUFFER = 0, 1, 2, 3, 4
POOL_L2 = 8


def l2_normalise(e: np.ndarray) -> np.ndarray:
    e64 = np.asarray(e, np.float64)
    return (e64 / max(float(np.sqrt((e64 * e64).sum())), 1e-12)).astype(e.dtype)


def pool_item(pool, item, H):
    """Update ``pool`` (dict of arrays sum [S,d], wsum [S], kept [S,d] and,
    for the BUFFER kind, buf [S, rows, d]) with the final hidden states
    ``H`` [n, d] of one embedding chunk; return the finished embedding when
    ``item.is_last`` else None."""
    e = _pool_base(pool, item, item.pool_kind & ~POOL_L2, H)
    if e is not None and item.pool_kind & POOL_L2:
        e = l2_normalise(e)
    return e


def _pool_base(pool, item, kind, H):
    s = item.pool_slot
    if item.is_first:
        pool["sum"][s] = 0
        pool["wsum"][s] = 0
        pool["kept"][s] = 0
    n = H.shape[0]
    if kind == POOL_BUFFER:
        c = item.ctx_len
        pool["buf"][s, c:c + n] = H
        if item.is_last:
            return pool["buf"][s, :c + n].mean(axis=0, dtype=np.float64).astype(H.dtype)
        return None
    if kind in (POOL_MEAN, POOL_WMEAN):
        if kind == POOL_MEAN:
            w = np.ones(n, dtype=H.dtype)
        else:
            w = (item.ctx_len + np.arange(n) + 1).astype(H.dtype)
        pool["sum"][s] += w @ H
        pool["wsum"][s] += w.sum()
        if item.is_last:
            return pool["sum"][s] / pool["wsum"][s]
        return None
    if kind == POOL_CLS:
        if item.is_first:
            pool["kept"][s] = H[0]
    else:
        pool["kept"][s] = H[n - 1]
    if item.is_last:
        return pool["kept"][s].copy()
    return None
