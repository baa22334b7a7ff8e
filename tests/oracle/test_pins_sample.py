"""Pins of the sampling oracle against what does not depend on it: greedy is
the first maximum; the integer weights follow e^((l - max) / T) within the
degree-7 Taylor bound; over an even grid of uniforms the draw frequencies
match the softmax of l / T restricted to the nucleus (textbook temperature
sampling, scipy's softmax); the nucleus is the smallest set of most
probable tokens whose probability reaches top_p (the top-p definition);
ties split by index; hand-worked rows whose weights are exact powers of
two; the degenerate temperatures."""

import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle.sample import greedy, weights, nucleus, sample_row, sample

LOG2E32 = float(np.float32(1.4426950408889634))   # T at which s = fp32(log2 e / T) is exactly 1


def _grid_freq(l, T, p, N=1 << 14):
    """Draw frequencies over the uniforms U_k = floor((k + 1/2) 2^32 / N)."""
    cnt = np.zeros(len(l))
    for k in range(N):
        U = int((k + 0.5) * 2 ** 32 / N)
        cnt[sample_row(np.asarray(l, np.float32), T, p, U)] += 1
    return cnt / N


def test_greedy_first_maximum():
    l = np.array([[1, 3, 3, 2], [5, 5, 5, 5], [-1, -2, -0.5, -0.5], [0, 0, 0, 7]], np.float32)
    assert greedy(l).tolist() == [1, 0, 2, 3]
    for T in (0.0, -1.0, float("nan")):
        assert sample_row(l[0], T, 0.9, 12345) == 1


@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_weights_follow_the_exponential(T):
    rng = np.random.default_rng(int(T * 10))
    l = (rng.standard_normal(4000) * 4).astype(np.float32)
    q = weights(l, T)
    e = np.exp((l.astype(np.float64) - l.max()) / T) * 2.0 ** 30
    assert q[np.argmax(l)] == 2 ** 30
    # Taylor remainder (ln 2)^8 / 8! e^(ln 2) < 2.7e-6, plus fp32 roundings of t
    # (|t| <= 30, 2^-24 relative) and the truncation to an integer
    bound = e * (2.7e-6 + 30 * 2 ** -24 * math.log(2) + 4 * 2 ** -24) + 1
    assert np.all(np.abs(q - e) <= bound)
    t = (l.astype(np.float64) - l.max()) / T * math.log2(math.e)
    assert np.all(q[t < -30.001] == 0) and np.all(q[t > -29.999] >= 1)


def test_hand_worked_powers_of_two():
    # s = 1: weights 2^(30 + d) exactly for integer d
    l = np.array([1, 0, 1, 0, -1], np.float32)
    q = weights(l, LOG2E32)
    assert q.tolist() == [2 ** 30, 2 ** 29, 2 ** 30, 2 ** 29, 2 ** 28]
    # Z = 3.25 * 2^30; top_p 0.5 -> target 1.625 * 2^30 -> tau 2^30, both maxima
    m, mass = nucleus(q, 0.5)
    assert m.tolist() == [True, False, True, False, False] and mass == 2 ** 31
    # top_p 0.7 -> P16 45875, target 2442752000 -> tau 2^29, one tie (index 1) in
    m, mass = nucleus(q, 0.7)
    assert m.tolist() == [True, True, True, False, False] and mass == 2 ** 31 + 2 ** 29
    # draws over that nucleus: x = floor(mass U / 2^32); cumulative 2^30, 1.5 2^30, 2.5 2^30
    assert sample_row(l, LOG2E32, 0.7, 0) == 0
    U_edge = -(-(2 ** 30) * 2 ** 32 // mass)            # smallest U with x >= 2^30
    assert sample_row(l, LOG2E32, 0.7, U_edge - 1) == 0
    assert sample_row(l, LOG2E32, 0.7, U_edge) == 1
    assert sample_row(l, LOG2E32, 0.7, 2 ** 32 - 1) == 2


def test_ties_split_by_index():
    l = np.zeros(4, np.float32)
    # four equal weights 2^30, top_p 1/2: the nucleus is tokens 0 and 1
    assert sample_row(l, 1.0, 0.5, 0) == 0
    assert sample_row(l, 1.0, 0.5, 2 ** 31 - 1) == 0
    assert sample_row(l, 1.0, 0.5, 2 ** 31) == 1
    assert sample_row(l, 1.0, 0.5, 2 ** 32 - 1) == 1
    assert sample_row(l, 1.0, 0.0, 2 ** 32 - 1) == 0       # smallest nucleus: one token


@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_full_nucleus_frequencies_are_the_softmax(T):
    rng = np.random.default_rng(3)
    l = (rng.standard_normal(7) * 1.5).astype(np.float32)
    N = 1 << 14
    f = _grid_freq(l, T, 1.0, N)
    pr = softmax(l.astype(np.float64) / T)
    assert np.all(np.abs(f - pr) <= 1.0 / N + 4e-6 + 3e-6 * pr), (f, pr)


@pytest.mark.parametrize("p", [0.3, 0.62, 0.9, 0.97])
def test_top_p_is_the_smallest_probable_set(p):
    rng = np.random.default_rng(11)
    l = (rng.standard_normal(9) * 1.2).astype(np.float32)
    T = 0.8
    pr = softmax(l.astype(np.float64) / T)
    order = np.argsort(-pr)
    cum = np.cumsum(pr[order])
    assert np.min(np.abs(cum - p)) > 1e-3                  # p away from a boundary
    k = int(np.searchsorted(cum, p)) + 1
    expect = set(order[:k].tolist())
    N = 1 << 13
    f = _grid_freq(l, T, p, N)
    assert set(np.nonzero(f)[0].tolist()) == expect
    ren = np.zeros_like(pr)
    ren[order[:k]] = pr[order[:k]] / pr[order[:k]].sum()
    assert np.all(np.abs(f - ren) <= 1.0 / N + 1e-5)


def test_degenerate_temperatures_and_sizes():
    rng = np.random.default_rng(4)
    l = rng.standard_normal(50).astype(np.float32)
    # vanishing temperature: only the maximum keeps weight
    for T in (1e-30, 1e-45):
        for U in (0, 2 ** 31, 2 ** 32 - 1):
            assert sample_row(l, T, 1.0, U) == int(np.argmax(l))
    # infinite temperature: every token weighs 2^30, the draw is uniform
    q = weights(l, float("inf"))
    assert np.all(q == 2 ** 30)
    f = _grid_freq(l, float("inf"), 1.0, 1 << 12)
    assert np.allclose(f, 1 / 50, atol=1 / 4096)
    # one token
    assert sample_row(np.array([3.0], np.float32), 0.7, 0.1, 2 ** 32 - 1) == 0
    # batch entry point: greedy rows and sampled rows mixed
    L = rng.standard_normal((4, 30)).astype(np.float32)
    out = sample(L, np.array([0, 1, 0, 1e-30], np.float32), np.ones(4, np.float32),
                 np.array([0, 7, 0, 9], np.uint32))
    assert out[0] == np.argmax(L[0]) and out[2] == np.argmax(L[2]) and out[3] == np.argmax(L[3])


def test_reading_matches_exact_definition_away_from_boundaries():
    """The readings (fp32 Taylor weights, integer nucleus and draw) pick the
    token of the textbook definition (fp64 softmax with temperature, top-p
    nucleus, inverse-CDF draw in index order) on every draw that is not
    within the readings' error bound of a boundary; the bound leaves most
    draws decided."""
    from oracle.sample import sample_exact_row
    rng = np.random.default_rng(21)
    decided = agree = total = 0
    for _ in range(500):
        V = int(rng.choice([2, 37, 1000, 5000]))
        l = (rng.standard_normal(V) * rng.choice([1.0, 3.0])).astype(np.float32)
        T = float(rng.choice([0.0, 0.3, 0.7, 1.0, 1.6]))
        p = float(rng.choice([0.05, 0.5, 0.9, 0.99, 1.0]))
        U = int(rng.integers(0, 2 ** 32))
        tok, ok = sample_exact_row(l, T, p, U)
        total += 1
        if ok:
            decided += 1
            agree += tok == sample_row(l, T, p, U if T > 0 else 0)
    assert agree == decided
    assert decided > 0.8 * total, (decided, total)
