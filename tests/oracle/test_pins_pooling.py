"""Pins of the incremental pooler: closed forms of the weight totals,
chunk-invariance of the streaming sum, the kept-state heads, the buffered
head (every row kept at its position, the mean over the whole input at the
end, the same function as the streaming mean) and the L2 flag (unit
length, same direction, constant rows give h / |h|, zero stays zero)."""

import numpy as np
import pytest

import oracle
from synth.workloads import Item, EMBED, POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST, POOL_BUFFER, POOL_L2

RNG = np.random.default_rng(7)


def _run_chunks(kind, H, chunks, dtype=np.float64):
    pool = oracle.new_pool(4, H.shape[1], dtype)
    n = H.shape[0]
    off = 0
    out = None
    for c in chunks:
        it = Item(kind=EMBED, req_id=1, n_tokens=c, ctx_len=off, pool_slot=2,
                  pool_kind=kind, is_first=int(off == 0), is_last=int(off + c == n))
        out = oracle.pool_item(pool, it, H[off:off + c].astype(dtype))
        off += c
    return out, pool


@pytest.mark.parametrize("n", [1, 7, 100, 5791])
def test_weight_totals_closed_form_fp32(n):
    H = np.ones((n, 3), np.float32)
    chunks = [256] * (n // 256) + ([n % 256] if n % 256 else [])
    _, pm = _run_chunks(POOL_MEAN, H, chunks, np.float32)
    _, pw = _run_chunks(POOL_WMEAN, H, chunks, np.float32)
    assert pm["wsum"][2] == n
    # n(n+1)/2 < 2^24 for n < 5792: exact in fp32
    assert pw["wsum"][2] == n * (n + 1) // 2


@pytest.mark.parametrize("kind", [POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST])
def test_constant_rows_give_that_row(kind):
    h = RNG.standard_normal(9)
    H = np.tile(h, (50, 1))
    e, _ = _run_chunks(kind, H, [16, 16, 16, 2])
    np.testing.assert_allclose(e, h, rtol=1e-14)


def test_mean_and_wmean_match_definition_and_are_chunk_invariant():
    H = RNG.standard_normal((300, 5))
    w = np.arange(1, 301, dtype=np.float64)
    for chunks in ([300], [256, 44], [100, 100, 100], [1] * 300):
        em, _ = _run_chunks(POOL_MEAN, H, chunks)
        ew, _ = _run_chunks(POOL_WMEAN, H, chunks)
        np.testing.assert_allclose(em, H.mean(axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ew, (w[:, None] * H).sum(0) / w.sum(), rtol=1e-12, atol=1e-14)


def test_cls_keeps_first_row_and_last_keeps_final_row():
    H = RNG.standard_normal((40, 6))
    ec, pc = _run_chunks(POOL_CLS, H, [16, 16, 8])
    el, _ = _run_chunks(POOL_LAST, H, [16, 16, 8])
    np.testing.assert_array_equal(ec, H[0])
    np.testing.assert_array_equal(el, H[39])


def test_is_first_resets_slot():
    H = RNG.standard_normal((10, 4))
    pool = oracle.new_pool(4, 4, np.float64)
    pool["sum"][2] = 99.0
    pool["wsum"][2] = 5.0
    it = Item(kind=EMBED, req_id=1, n_tokens=10, ctx_len=0, pool_slot=2,
              pool_kind=POOL_MEAN, is_first=1, is_last=1)
    e = oracle.pool_item(pool, it, H)
    np.testing.assert_allclose(e, H.mean(0), rtol=1e-14)


def test_unfinished_chunk_returns_nothing_and_keeps_state():
    H = RNG.standard_normal((8, 4))
    pool = oracle.new_pool(4, 4, np.float64)
    it = Item(kind=EMBED, req_id=1, n_tokens=8, ctx_len=0, pool_slot=0,
              pool_kind=POOL_WMEAN, is_first=1, is_last=0)
    assert oracle.pool_item(pool, it, H) is None
    assert pool["wsum"][0] == 36


def _run_chunks_buf(kind, H, chunks, dtype=np.float64, rows=None):
    pool = oracle.new_pool(4, H.shape[1], dtype, buf_rows=rows or H.shape[0])
    n, off, out = H.shape[0], 0, None
    for c in chunks:
        it = Item(kind=EMBED, req_id=1, n_tokens=c, ctx_len=off, pool_slot=2,
                  pool_kind=kind, is_first=int(off == 0), is_last=int(off + c == n))
        out = oracle.pool_item(pool, it, H[off:off + c].astype(dtype))
        off += c
    return out, pool


def test_buffer_head_keeps_every_row_and_runs_the_mean_at_the_end():
    # Summary page, incremental pooling: every row is kept (n x d) and the head runs once at the end
    H = RNG.standard_normal((300, 5))
    for chunks in ([300], [256, 44], [7] * 42 + [6], [1] * 300):
        e, pool = _run_chunks_buf(POOL_BUFFER, H, chunks, rows=320)
        np.testing.assert_array_equal(pool["buf"][2, :300], H)          # rows at their positions
        assert not pool["buf"][2, 300:].any()
        np.testing.assert_allclose(e, H.mean(axis=0), rtol=1e-12, atol=1e-14)
        em, _ = _run_chunks(POOL_MEAN, H, chunks)                        # same function as the streaming mean
        np.testing.assert_allclose(e, em, rtol=1e-12, atol=1e-14)
    # nothing is emitted before the last chunk
    pool = oracle.new_pool(4, 5, np.float64, buf_rows=300)
    it = Item(kind=EMBED, req_id=1, n_tokens=10, ctx_len=0, pool_slot=2, pool_kind=POOL_BUFFER, is_first=1, is_last=0)
    assert oracle.pool_item(pool, it, H[:10]) is None


@pytest.mark.parametrize("kind", [POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST, POOL_BUFFER])
def test_l2_flag_normalises_the_head_output(kind):
    H = RNG.standard_normal((60, 7)) + 0.5
    e0, _ = _run_chunks_buf(kind, H, [16, 16, 16, 12])
    e1, _ = _run_chunks_buf(kind | POOL_L2, H, [16, 16, 16, 12])
    assert abs(np.linalg.norm(e1) - 1.0) < 1e-12
    np.testing.assert_allclose(e1 * np.linalg.norm(e0), e0, rtol=1e-12, atol=1e-14)   # same direction
    # constant rows: every head gives h / |h|
    h = RNG.standard_normal(7)
    e, _ = _run_chunks_buf(kind | POOL_L2, np.tile(h, (20, 1)), [8, 12])
    np.testing.assert_allclose(e, h / np.linalg.norm(h), rtol=1e-12)
    # a zero vector stays zero
    z, _ = _run_chunks_buf(kind | POOL_L2, np.zeros((5, 7)), [5])
    assert not z.any()
