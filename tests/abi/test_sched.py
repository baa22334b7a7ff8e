"""The C++ intra-batch scheduler (orthrus_sched_*) against the scheduling
oracle, decision for decision: on seeded runs with requests arriving
between steps, every emitted batch (items, token ids, page ids, logit-row
count) and the credit accumulators must be identical; plus the error paths
of the scheduler calls."""

import numpy as np
import pytest

import heterogeneous_embed_decode_amd as hed
from oracle.ibs import IBSOracle, EMBED, PREFILL, DECODE

FIELDS = ("kind", "req_id", "n_tokens", "ctx_len", "page_off", "n_pages", "pool_slot", "pool_kind",
          "is_first", "is_last")


def _oracle_items(items):
    return np.array([[it[f] for f in FIELDS] for it in items], np.int32).reshape(-1, 10)


@pytest.mark.parametrize("seed", range(8))
def test_scheduler_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([32, 64, 256, 1024]))
    C = int(rng.choice([8, 16, 64, 256]))
    ps = int(rng.choice([1, 5, 8, 16]))
    n_pages = int(rng.integers(200, 3000))
    slots = int(rng.integers(1, 9))
    free = rng.permutation(n_pages).astype(np.int32)
    orc = IBSOracle(B, C, ps, free, slots)
    st, s = hed.orthrus_sched_create(B, C, ps, free, slots)
    assert st == hed.OK
    nid = 0
    for step in range(150):
        # arrivals
        for _ in range(int(rng.poisson(1.5))):
            kind = EMBED if rng.random() < 0.5 else PREFILL
            toks = rng.integers(0, 50000, int(rng.integers(1, 3 * C + 5)))
            pk = int(rng.integers(0, 4)) if kind == EMBED else 0
            mn = int(rng.integers(1, 20)) if kind == PREFILL else 0
            orc.submit(nid, kind, toks, pool_kind=pk, max_new=mn)
            assert hed.orthrus_sched_submit(s, nid, kind, toks, pk, mn) == hed.OK
            nid += 1
        ref = orc.next()
        st, got, nl = hed.orthrus_sched_next(s)
        assert st == hed.OK
        if ref is None:
            assert got is None
            continue
        items, toks, pages = ref
        assert np.array_equal(got.items_np, _oracle_items(items)), (seed, step)
        assert np.array_equal(got.tok_np, toks), (seed, step)
        assert np.array_equal(got.pages_np, pages), (seed, step)
        n_logit = sum(1 for it in items if it["kind"] == DECODE or (it["kind"] == PREFILL and it["is_last"]))
        assert nl == n_logit
        sampled = rng.integers(0, 50000, n_logit).astype(np.int32)
        orc.commit(sampled)
        assert hed.orthrus_sched_commit(s, sampled) == hed.OK
        st, stats = hed.orthrus_sched_stats(s)
        assert stats[:7] == [len(orc.emb_q), len(orc.gen_q), len(orc.decoding), len(orc.free_pages),
                             len(orc.free_slots), orc.a_e, orc.a_g]
    hed.orthrus_sched_destroy(s)


def test_scheduler_errors():
    assert hed.orthrus_sched_create(0, 16, 16, [0, 1], 1)[0] == hed.EINVAL
    assert hed.orthrus_sched_create(16, 0, 16, [0, 1], 1)[0] == hed.EINVAL
    st, s = hed.orthrus_sched_create(64, 16, 16, list(range(10)), 1)
    assert st == hed.OK
    assert hed.orthrus_sched_submit(s, 1, DECODE, [1, 2], 0, 0) == hed.EINVAL       # kind
    assert hed.orthrus_sched_submit(s, 1, EMBED, [1, 2], 7, 0) == hed.EINVAL        # pool kind
    assert hed.orthrus_sched_submit(s, 1, EMBED, [1, 2], 16, 0) == hed.EINVAL       # unknown flag
    assert hed.orthrus_sched_submit(s, 1, PREFILL, [1, 2], 0, 0) == hed.EINVAL      # no new tokens
    assert hed.orthrus_sched_submit(s, 1, EMBED, [], 0, 0) == hed.EINVAL            # empty
    assert hed.orthrus_sched_submit(s, 1, EMBED, [1, 2], 0, 0) == hed.OK
    assert hed.orthrus_sched_submit(s, 1, PREFILL, [3], 0, 2) == hed.EINVAL         # id reused
    assert hed.orthrus_sched_commit(s, []) == hed.ESTATE                          # nothing pending
    st, b, nl = hed.orthrus_sched_next(s)
    assert st == hed.OK and b is not None and nl == 0
    assert hed.orthrus_sched_next(s)[0] == hed.ESTATE                                # not committed
    assert hed.orthrus_sched_commit(s, [5]) == hed.EINVAL                         # wrong count
    assert hed.orthrus_sched_commit(s, []) == hed.OK
    st, stats = hed.orthrus_sched_stats(s)
    assert stats[0] == 0 and stats[3] == 10 and stats[4] == 1 and stats[7] == 0
    st, b, nl = hed.orthrus_sched_next(s)
    assert st == hed.OK and b is None
    hed.orthrus_sched_destroy(s)
