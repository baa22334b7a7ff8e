"""Pins of the oracle packer: a hand-worked batch and one case per error code."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.pack import Limits
from synth import model as sm
from synth.workloads import Item, Batch

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "..", "golden", "pack_small.json")))
CFG = sm.TINY


def gold_batch():
    items = [Item(**d) for d in GOLD["items"]]
    return Batch(items, np.array(GOLD["token_ids"], np.int32), np.array(GOLD["page_ids"], np.int32))


def limits(**kw):
    base = dict(n_pages=GOLD["n_pages"], max_tokens=64, max_items=8, max_pool_slots=4)
    base.update(kw)
    return Limits(**base)


def test_hand_worked_batch():
    m = oracle.pack_py(CFG, gold_batch(), limits())
    for k, v in GOLD["expect"].items():
        if isinstance(v, list):
            np.testing.assert_array_equal(np.asarray(m[k]).reshape(np.asarray(v).shape), v, err_msg=k)
        else:
            assert m[k] == v, k


def _mutated(fn):
    b = gold_batch()
    fn(b)
    return b


CASES = [
    ("unsorted kinds", lambda b: b.items.reverse(), oracle.EINVAL, {}),
    ("decode with 2 tokens", lambda b: setattr(b.items[2], "n_tokens", 2), oracle.EINVAL, {}),
    ("empty item", lambda b: setattr(b.items[0], "n_tokens", 0), oracle.EINVAL, {}),
    ("duplicate request", lambda b: setattr(b.items[1], "req_id", 5), oracle.EINVAL, {}),
    ("token out of range", lambda b: b.token_ids.__setitem__(0, 256), oracle.EINVAL, {}),
    ("too few pages", lambda b: setattr(b.items[1], "ctx_len", 15), oracle.ENOPAGES, {}),
    ("page id out of range", lambda b: b.page_ids.__setitem__(5, 8), oracle.ENOPAGES, {}),
    ("pool slot out of range", lambda b: setattr(b.items[0], "pool_slot", 4), oracle.ESTATE, {}),
    ("first chunk not at 0", lambda b: setattr(b.items[0], "ctx_len", 1), oracle.ESTATE, {}),
    ("too many tokens", lambda b: None, oracle.ECAPACITY, {"max_tokens": 5}),
    ("too many items", lambda b: None, oracle.ECAPACITY, {"max_items": 2}),
    ("shared KV slot", lambda b: b.page_ids.__setitem__(2, 4), oracle.EINVAL, {}),
]


@pytest.mark.parametrize("name,fn,code,lim", CASES, ids=[c[0] for c in CASES])
def test_error_codes(name, fn, code, lim):
    with pytest.raises(oracle.PackError) as e:
        oracle.pack_py(CFG, _mutated(fn), limits(**lim))
    assert e.value.code == code
