"""Next-token choice from logit rows (oracle side; numpy float32 and exact
Python integers) — test infrastructure, never called by the product path.

The full text's §3.1 emit stage hands the last-row logits of every
generation request to the sampler, which picks the request's next token
(§2.2 Generation: one new token per decoding step).  The page names no
sampling rule, so the readings below are taken.  Every decision after the
weights is made on integers, so any implementation that follows them picks
the same token:
 1. Greedy (temperature not > 0): the index of the largest logit, the lowest
    index among equal maxima.
 2. Temperature T > 0, s = fp32(log2(e) / T) (division in fp64, one rounding
    to fp32).  d_i = l_i - max (fp32 subtraction) and t_i = d_i * s (fp32
    multiplication), with t_i = 0 where d_i = 0.  Token i weighs
    q_i = floor(2^(30 + t_i)), and 0 when t_i < -30 (so the maximum weighs
    2^30 and q_i / 2^30 is e^((l_i - max) / T) to about 3e-6).  2^t is
    taken as 2^k * P(f), k = floor(t), f = t - k, P the degree-7 Taylor
    polynomial of e^(f ln 2) with coefficients fp32((ln 2)^j / j!), summed
    by Horner steps each rounded to fp32 (multiply, then add: no fused
    multiply-add); q_i = floor(P(f) * 2^(30 + k)).
 3. Nucleus (top-p): P16 = round-half-even(top_p * 65536) clamped to
    [1, 65536], Z = sum of q, target = ceil(Z * P16 / 65536).  The nucleus
    is the smallest set of highest-weight tokens whose weight reaches the
    target, lower indices first among equal weights: with tau the largest
    weight whose upper set {q >= tau} weighs at least the target, every
    token with q > tau and the first ceil((target - mass(q > tau)) / tau)
    tokens with q = tau in index order.
 4. Draw: a caller-supplied 32-bit uniform U per row gives
    x = floor(mass * U / 2^32) for the nucleus mass; walking the nucleus in
    token-index order, the chosen token is the first whose running weight
    exceeds x.  Token i is therefore drawn for a share q_i / mass of the
    2^32 values of U, to within one value of U.
Logits are taken to be finite.
"""

import math

import numpy as np

F32 = np.float32
COEF = [F32(math.log(2.0) ** j / math.factorial(j)) for j in range(8)]   # fp32((ln 2)^j / j!)
LOG2E = 1.4426950408889634


def greedy(logits: np.ndarray) -> np.ndarray:
    """Row-wise argmax, lowest index on ties (reading 1)."""
    return np.argmax(np.asarray(logits, np.float32), axis=1).astype(np.int32)


def weights(l: np.ndarray, temperature: float) -> np.ndarray:
    """Integer weights q_i of one row (reading 2), int64."""
    l = np.asarray(l, np.float32)
    d = (l - l.max()).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        s = F32(LOG2E / float(temperature))                 # inf when T is tiny
        t = np.where(d == 0, F32(0.0), (d * s).astype(np.float32)).astype(np.float32)
    q = np.zeros(l.size, np.int64)
    ok = t >= F32(-30.0)
    tt = t[ok]
    k = np.floor(tt).astype(np.float32)
    f = (tt - k).astype(np.float32)                          # exact
    p = np.full(tt.size, COEF[7], np.float32)
    for j in range(6, -1, -1):
        p = (p * f).astype(np.float32)
        p = (p + COEF[j]).astype(np.float32)
    # P(f) * 2^(30 + k), k in [-30, 0]: an exact scaling, then truncation
    q[ok] = np.floor(p.astype(np.float64) * np.exp2(30.0 + k.astype(np.float64))).astype(np.int64)
    return q


def nucleus(q: np.ndarray, top_p: float):
    """Membership mask and mass of the nucleus (reading 3)."""
    Z = int(q.sum())
    P16 = min(65536, max(1, int(round(float(top_p) * 65536))))
    target = -(-(Z * P16) // 65536)
    desc = np.sort(q)[::-1]
    cum = np.cumsum(desc)
    tau = int(desc[int(np.searchsorted(cum, target, side="left"))])
    base = int(q[q > tau].sum())
    n_tie = -(-(target - base) // tau)
    member = q > tau
    member[np.nonzero(q == tau)[0][:n_tie]] = True
    return member, base + n_tie * tau


def sample_row(l: np.ndarray, temperature: float, top_p: float, U: int) -> int:
    l = np.asarray(l, np.float32)
    if not temperature > 0:
        return int(np.argmax(l))
    q = weights(l, temperature)
    member, mass = nucleus(q, top_p)
    x = (mass * int(U)) >> 32                                # reading 4
    run = np.cumsum(np.where(member, q, 0))
    return int(np.searchsorted(run, x, side="right"))


def sample(logits: np.ndarray, temperature=None, top_p=None, uniforms=None) -> np.ndarray:
    """Per-row temperature / top_p / uniform (uint32) arrays; temperature
    None means greedy for every row, top_p None means 1."""
    logits = np.asarray(logits, np.float32)
    n = logits.shape[0]
    if temperature is None:
        return greedy(logits)
    out = np.zeros(n, np.int32)
    for i in range(n):
        T = float(np.float32(temperature[i]))
        p = 1.0 if top_p is None else float(np.float32(top_p[i]))
        out[i] = sample_row(logits[i], T, p, int(uniforms[i]) if T > 0 else 0)
    return out


def sample_exact_row(l: np.ndarray, temperature: float, top_p: float, U: int, margin: float = None):
    """The textbook definition the readings above approximate, in fp64:
    softmax weights e^((l_i - max) / T), the nucleus as the smallest set of
    most probable tokens (lower index first among equal probabilities)
    whose probability reaches P16 / 65536, and the draw x = (U / 2^32) times
    the nucleus mass, taking the first token in index order whose running
    nucleus mass exceeds x.  Returns (token, decided): decided is False when
    the draw lies within `margin` (relative to the nucleus mass) of a
    boundary between two tokens, or the nucleus edge within `margin` of the
    target or of a near-tie, where the fp32 weights of the readings may
    legitimately pick a neighbour.  The default margin is the readings'
    error bound: each fp32 weight within about 5e-6 of e^((l - max) / T)
    (the Taylor polynomial and the fp32 rounding of t, doubled here), and
    the floor and the zero weights below 2^-30 of the maximum costing at
    most V / 2^30 of the mass each.  Used to check the readings and the GPU
    sampler against the definition, not to replace them."""
    l = np.asarray(l, np.float32).astype(np.float64)
    if margin is None:
        margin = 1e-5 + 2.0 * l.size / 2.0 ** 30
    if not temperature > 0:
        return int(np.argmax(l)), True
    w = np.exp((l - l.max()) / float(np.float32(temperature)))
    Z = float(w.sum())
    P16 = min(65536, max(1, int(round(float(top_p) * 65536))))
    decided = True
    if P16 == 65536:
        member = np.ones(l.size, bool)
    else:
        thr = P16 / 65536.0 * Z
        order = np.lexsort((np.arange(l.size), -w))          # by weight descending, then index
        ws = w[order]
        cum = np.cumsum(ws)
        k = int(np.searchsorted(cum, thr, side="left"))      # nucleus = order[:k + 1]
        k = min(k, l.size - 1)
        if abs(cum[k] - thr) < margin * Z or (k > 0 and abs(cum[k - 1] - thr) < margin * Z):
            decided = False
        if k + 1 < l.size and 0.0 < ws[k] - ws[k + 1] < margin * ws[k]:
            decided = False
        member = np.zeros(l.size, bool)
        member[order[:k + 1]] = True
    run = np.cumsum(np.where(member, w, 0.0))
    M = float(run[-1])
    x = int(U) / 2.0 ** 32 * M
    tok = int(np.searchsorted(run, x, side="right"))
    edges = run[member]
    if np.min(np.abs(edges - x)) < margin * M:
        decided = False
    return min(tok, l.size - 1), decided
