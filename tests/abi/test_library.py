"""The C-ABI library loads on a CPU-only host, exports every symbol the
header declares, and its host packer matches the oracle's packer bit for
bit (metadata) and code for code (validation)."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import heterogeneous_embed_decode_amd as hed
import oracle
from oracle.pack import Limits
from synth import model as sm
from synth import workloads as wl
from synth.workloads import Item, Batch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "pack_small.json")))


def header_symbols():
    src = open(os.path.join(ROOT, "include", "orthrus.h")).read()
    return sorted(set(re.findall(r"\b(orthrus_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    syms = header_symbols()
    assert {"orthrus_pack", "orthrus_create", "orthrus_step", "orthrus_destroy"} <= set(syms)
    lib = ctypes.CDLL(hed.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert set(hed.EXPORTS) == set(syms)


def cfg_for(dims, n_pages, max_tokens=4096, max_items=256, slots=16):
    return hed.make_cfg(dims.n_layers, dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim,
                        dims.ffn_dim, dims.vocab, dims.lora_rank, dims.page_size, n_pages,
                        max_tokens, max_items, slots, dims.rope_theta, dims.rms_eps, dims.lora_scale)


def both(dims, batch, n_pages, max_tokens=4096, max_items=256, slots=16):
    st, got, msg = hed.orthrus_pack(cfg_for(dims, n_pages, max_tokens, max_items, slots),
                                    hed.BatchArgs(batch.items_array(), batch.token_ids, batch.page_ids))
    try:
        ref = oracle.pack_py(dims, batch, Limits(n_pages, max_tokens, max_items, slots))
        code = oracle.OK
    except oracle.PackError as e:
        ref, code = None, e.code
    return st, got, code, ref


def gold_batch():
    return Batch([Item(**d) for d in GOLD["items"]], np.array(GOLD["token_ids"], np.int32),
                 np.array(GOLD["page_ids"], np.int32))


def test_hand_worked_batch_matches_golden():
    st, got, msg = hed.orthrus_pack(cfg_for(sm.TINY, GOLD["n_pages"]),
                                    hed.BatchArgs(gold_batch().items_array(), GOLD["token_ids"],
                                                  GOLD["page_ids"]))
    assert st == hed.OK, msg
    for k, v in GOLD["expect"].items():
        np.testing.assert_array_equal(np.asarray(got[k]).reshape(np.asarray(v).shape), v, err_msg=k)


def _compare(st, got, code, ref):
    assert st == code
    if code == oracle.OK:
        for k in ("cu_q", "pos", "slot", "row_item", "logit_rows", "pool_segs"):
            np.testing.assert_array_equal(got[k], np.asarray(ref[k]).reshape(np.asarray(got[k]).shape), err_msg=k)
        for k in ("n_embed_rows", "n_prefill_rows", "n_decode_rows", "n_logits", "n_emb"):
            assert got[k] == ref[k], k


@pytest.mark.parametrize("seed", range(40))
def test_random_batches_bit_exact(seed):
    dims = sm.TINY if seed % 2 else sm.MISTRAL_7B
    b, n_pages = wl.random_batch(dims, seed, max_items=15, max_len=70, max_ctx=300)
    _compare(*both(dims, b, n_pages))


def test_workload_batches_bit_exact():
    cfg, batches, n_pages = wl.tiny_workload()
    for b in batches:
        _compare(*both(cfg, b, n_pages))
    cfg2, b2, n2 = wl.one_layer_workload()
    _compare(*both(cfg2, b2, n2, max_tokens=8192))


def _mut(fn):
    b = gold_batch()
    fn(b)
    return b


CASES = [
    ("unsorted kinds", lambda b: b.items.reverse(), {}),
    ("decode with 2 tokens", lambda b: setattr(b.items[2], "n_tokens", 2), {}),
    ("empty item", lambda b: setattr(b.items[0], "n_tokens", 0), {}),
    ("duplicate request", lambda b: setattr(b.items[1], "req_id", 5), {}),
    ("token out of range", lambda b: b.token_ids.__setitem__(0, 256), {}),
    ("too few pages", lambda b: setattr(b.items[1], "ctx_len", 15), {}),
    ("page id out of range", lambda b: b.page_ids.__setitem__(5, 8), {}),
    ("pool slot out of range", lambda b: setattr(b.items[0], "pool_slot", 16), {}),
    ("pool slot reused", lambda b: (setattr(b.items[1], "kind", 0), setattr(b.items[1], "pool_slot", 2),
                                    setattr(b.items[1], "ctx_len", 0)), {}),
    ("first chunk not at 0", lambda b: setattr(b.items[0], "ctx_len", 1), {}),
    ("bad pool kind", lambda b: setattr(b.items[0], "pool_kind", 7), {}),
    ("bad flag", lambda b: setattr(b.items[1], "is_last", 2), {}),
    ("negative ctx", lambda b: setattr(b.items[2], "ctx_len", -1), {}),
    ("page range outside list", lambda b: setattr(b.items[2], "n_pages", 9), {}),
    ("too many tokens", lambda b: None, {"max_tokens": 5}),
    ("too many items", lambda b: None, {"max_items": 2}),
    ("shared KV slot", lambda b: b.page_ids.__setitem__(2, 4), {}),
]


@pytest.mark.parametrize("name,fn,lim", CASES, ids=[c[0] for c in CASES])
def test_error_codes_match_oracle(name, fn, lim):
    st, got, code, ref = both(sm.TINY, _mut(fn), GOLD["n_pages"], **lim)
    assert code != oracle.OK
    assert st == code, (name, st, code)


def test_capacity_of_pack_outputs():
    b = gold_batch()
    ba = hed.BatchArgs(b.items_array(), b.token_ids, b.page_ids)
    small = np.zeros(2, np.int32)
    p = hed.ctypes.POINTER(ctypes.c_int32)
    pk = hed.orthrus_packed(2, 2, *[small.ctypes.data_as(p)] * 6)
    st = hed.LIB.orthrus_pack(ctypes.byref(cfg_for(sm.TINY, 8)), ctypes.byref(ba.struct),
                              ctypes.byref(pk), None, 0)
    assert st == hed.ECAPACITY


def test_gemm_rejects_operands_of_2gib():
    """The GEMM kernels address A, B and a residual C through 32-bit buffer
    offsets; an operand spanning 2 GiB is refused before any device work
    (the pointers are never dereferenced)."""
    big = 1 << 17   # rows: 131072 x 8192 bf16 = 2 GiB
    assert hed.orthrus_gemm_bf16(8, 8192, 8, 8192, 8, 64, big, 64, 8192, hed.EPI_BF16) == hed.EINVAL
    assert hed.orthrus_gemm_bf16(8, 8192, 8, 8192, 8, big, 64, big, 8192, hed.EPI_BF16) == hed.EINVAL
    # residual C: 65536 x 8192 fp32 = 2 GiB (A and B are small)
    assert hed.orthrus_gemm_bf16(8, 64, 8, 64, 8, 8192, 65536, 8192, 64, hed.EPI_RESID) == hed.EINVAL


def test_create_rejects_unknown_dtype_before_device_work():
    """A model dtype other than bf16 (0) or fp32 (1) is refused by the
    argument checks, before any HIP call (the pointers are never used)."""
    from synth import model as sm
    t = sm.TINY
    for dt, want in ((2, hed.EINVAL), (-1, hed.EINVAL)):
        cfg = hed.make_cfg(t.n_layers, t.d_model, t.n_q_heads, t.n_kv_heads, t.head_dim, t.ffn_dim, t.vocab,
                           0, t.page_size, 16, 64, 8, 4, t.rope_theta, t.rms_eps, 1.0, dt)
        layers = [{k: 8 for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_ffn")}] * t.n_layers
        with pytest.raises(hed.OrthrusError) as e:
            hed.orthrus_create(cfg, 8, 8, 8, layers, 8, 8)
        assert e.value.code == want


def test_lora_shrink_rejects_bad_sizes_before_device_work():
    """orthrus_lora_shrink_bf16's argument checks run before any HIP call
    (the dummy pointers are never dereferenced)."""
    p = 256
    assert hed.orthrus_lora_shrink_bf16(p, 32, p, 1, 1, 4, 1.0, p) == hed.EINVAL        # K < 8
    assert hed.orthrus_lora_shrink_bf16(p, 32, p, 1, 1, 40, 1.0, p) == hed.EINVAL       # ldx < K
    assert hed.orthrus_lora_shrink_bf16(p, 36, p, 1, 1, 36, 1.0, p) == hed.EINVAL       # K % 8
    assert hed.orthrus_lora_shrink_bf16(p, 44, p, 1, 1, 40, 1.0, p) == hed.EINVAL       # ldx % 8
    assert hed.orthrus_lora_shrink_bf16(p, 32, p, -1, 1, 32, 1.0, p) == hed.EINVAL      # rows < 0
    assert hed.orthrus_lora_shrink_bf16(p, 32, p, 1, -2, 32, 1.0, p) == hed.EINVAL      # nr < 0
    assert hed.orthrus_lora_shrink_bf16(None, 32, p, 1, 1, 32, 1.0, p) == hed.EINVAL    # NULL X
    assert hed.orthrus_lora_shrink_bf16(p, 32, p, 1, 1, 32, 1.0, None) == hed.EINVAL    # NULL U
    assert hed.orthrus_lora_shrink_bf16(p, 1 << 20, p, 1 << 11, 1, 1024, 1.0, p) == hed.EINVAL  # X spans 4 GiB
    assert hed.orthrus_lora_shrink_bf16(p, 32, p, 1, 1, 32, 1.0, p, p, -1) == hed.EINVAL  # workspace bytes < 0
    assert hed.orthrus_lora_shrink_bf16(None, 32, None, 0, 1, 32, 1.0, None) == hed.OK  # nothing to do
