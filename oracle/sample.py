"""Next-token choice from logit rows (oracle side, numpy).

The full text's §3.1 emit stage hands each generation request's last-row
logits to the sampler (§2.2 Generation: one new token per step).  The page
names no sampling rule, so these readings are taken (the same in the HIP
sampler):
 1. Greedy (temperature <= 0 or no random input): the index of the largest
    logit, the lowest index among equal maxima.
 2. Otherwise p_i = exp((l_i - max) / T) / Z in fp64.  The nucleus is the
    smallest set of highest-probability tokens whose mass reaches top_p * Z
    (top_p in (0, 1]); among equal probabilities lower indices enter first.
    With tau the smallest probability in the nucleus, it holds every token
    with p_i > tau and the lowest-index tokens with p_i == tau up to the
    mass.
 3. The draw walks the nucleus in token-index order and returns the first
    token whose running mass exceeds u * (nucleus mass), u in [0, 1) given
    per row; the last nucleus token if rounding leaves none.
"""

import numpy as np


def greedy(logits: np.ndarray) -> np.ndarray:
    """Row-wise argmax, lowest index on ties."""
    return np.argmax(logits, axis=1).astype(np.int32)


def sample_row(l: np.ndarray, temperature: float, top_p: float, u: float) -> int:
    l = np.asarray(l, np.float32)
    if temperature <= 0:
        return int(np.argmax(l))
    m = np.float64(l.max())
    w = np.exp((l.astype(np.float64) - m) / np.float64(np.float32(temperature)))
    Z = w.sum()
    target = np.float64(np.float32(top_p)) * Z
    order = np.lexsort((np.arange(l.size), -w))      # by probability desc, then index
    cum = np.cumsum(w[order])
    k = int(np.searchsorted(cum, target, side="left")) + 1   # smallest prefix with mass >= target
    k = min(k, l.size)
    nucleus = np.zeros(l.size, bool)
    nucleus[order[:k]] = True
    idx = np.nonzero(nucleus)[0]                     # index order
    mass = w[idx].sum()
    run = np.cumsum(w[idx])
    j = int(np.searchsorted(run, np.float64(u) * mass, side="right"))
    return int(idx[min(j, idx.size - 1)])


def sample(logits: np.ndarray, temperature: float, top_p: float, uniforms=None) -> np.ndarray:
    if uniforms is None or temperature <= 0:
        return greedy(logits)
    return np.array([sample_row(logits[i], temperature, top_p, float(uniforms[i]))
                     for i in range(logits.shape[0])], np.int32)
