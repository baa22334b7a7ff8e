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
chunk).  The pooled vector is returned unnormalised.
"""

import numpy as np

POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST = 0, 1, 2, 3


def pool_item(pool, item, H):
    """Update ``pool`` (dict of arrays sum [S,d], wsum [S], kept [S,d]) with
    the final hidden states ``H`` [n, d] of one embedding chunk; return the
    finished embedding when ``item.is_last`` else None."""
    s = item.pool_slot
    if item.is_first:
        pool["sum"][s] = 0
        pool["wsum"][s] = 0
        pool["kept"][s] = 0
    n = H.shape[0]
    if item.pool_kind in (POOL_MEAN, POOL_WMEAN):
        if item.pool_kind == POOL_MEAN:
            w = np.ones(n, dtype=H.dtype)
        else:
            w = (item.ctx_len + np.arange(n) + 1).astype(H.dtype)
        pool["sum"][s] += w @ H
        pool["wsum"][s] += w.sum()
        if item.is_last:
            return pool["sum"][s] / pool["wsum"][s]
        return None
    if item.pool_kind == POOL_CLS:
        if item.is_first:
            pool["kept"][s] = H[0]
    else:
        pool["kept"][s] = H[n - 1]
    if item.is_last:
        return pool["kept"][s].copy()
    return None
