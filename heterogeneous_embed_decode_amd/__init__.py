"""Python binding of liborthrus.so (argument marshalling only).

Every function below forwards to the C entry point of the same name in
``include/orthrus.h``; all computation runs in the library's HIP kernels.
Device buffers are passed as integer addresses (e.g. ``tensor.data_ptr()``)
and streams as ``hipStream_t`` handles (``torch.cuda.current_stream().cuda_stream``).
Importing this module loads the library and raises if it has not been built.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liborthrus.so")

OK, EINVAL, ENOPAGES, ECAPACITY, ESTATE, ENOMEM, EHIP = range(7)
STATUS_NAMES = ["OK", "EINVAL", "ENOPAGES", "ECAPACITY", "ESTATE", "ENOMEM", "EHIP"]
EMBED, PREFILL, DECODE = 0, 1, 2
POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST = 0, 1, 2, 3
EPI_BF16, EPI_F32, EPI_RESID, EPI_SWIGLU = 0, 1, 2, 3
DTYPE_BF16, DTYPE_F32 = 0, 1

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)


class orthrus_model_cfg(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
        "lora_rank", "page_size", "n_pages", "max_tokens", "max_items", "max_pool_slots")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("lora_scale", ctypes.c_float),
        ("dtype", _i32)]


class orthrus_layer_w(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_ffn",
                                   "lora_a_qkv", "lora_b_qkv", "lora_a_o", "lora_b_o")]


class orthrus_weights(ctypes.Structure):
    _fields_ = [("tok_emb", _vp), ("lm_head", _vp), ("g_final", _vp),
                ("layers", ctypes.POINTER(orthrus_layer_w))]


class orthrus_item(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("kind", "req_id", "n_tokens", "ctx_len", "page_off", "n_pages",
                                    "pool_slot", "pool_kind", "is_first", "is_last")]


class orthrus_batch(ctypes.Structure):
    _fields_ = [("n_items", _i32), ("n_tokens", _i32), ("n_page_ids", _i32),
                ("items", ctypes.POINTER(orthrus_item)), ("token_ids", _i32p), ("page_ids", _i32p)]


class orthrus_pool_state(ctypes.Structure):
    _fields_ = [("sum", _vp), ("wsum", _vp), ("kept", _vp), ("buf", _vp), ("buf_rows", _i32)]


class orthrus_packed(ctypes.Structure):
    _fields_ = [("cap_tokens", _i32), ("cap_items", _i32)] + [
        (n, _i32p) for n in ("cu_q", "pos", "slot", "row_item", "logit_rows", "pool_segs")] + [
        (n, _i32) for n in ("n_embed_rows", "n_prefill_rows", "n_decode_rows", "n_logits", "n_emb",
                            "n_pool_segs")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python heterogeneous_embed_decode_amd/build.py`")
    # One HIP runtime per process.  PyTorch's ROCm build ships its own
    # libamdhip64 (same SONAME, loaded by file name); when it is loaded first
    # the library's dependency resolves to that copy.  Loaded the other way
    # round, the process holds two runtimes and the second to initialise
    # finds no device.  The memory the caller passes comes from PyTorch.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    lib.orthrus_pack.argtypes = [ctypes.POINTER(orthrus_model_cfg), ctypes.POINTER(orthrus_batch),
                                 ctypes.POINTER(orthrus_packed), ctypes.c_char_p, _i32]
    lib.orthrus_pack.restype = ctypes.c_int
    lib.orthrus_create.argtypes = [ctypes.POINTER(orthrus_model_cfg), ctypes.POINTER(orthrus_weights),
                                   _vp, _vp, ctypes.POINTER(_vp)]
    lib.orthrus_create.restype = ctypes.c_int
    lib.orthrus_step.argtypes = [_vp, ctypes.POINTER(orthrus_batch), ctypes.POINTER(orthrus_pool_state),
                                 _vp, _i32, _vp, _i32, _i32p, _i32p, _i32p, _i32p, _vp, _vp]
    lib.orthrus_step.restype = ctypes.c_int
    lib.orthrus_step_noalloc.argtypes = lib.orthrus_step.argtypes
    lib.orthrus_step_noalloc.restype = ctypes.c_int
    lib.orthrus_last_error.argtypes = [_vp]
    lib.orthrus_last_error.restype = ctypes.c_char_p
    lib.orthrus_destroy.argtypes = [_vp]
    lib.orthrus_destroy.restype = None
    lib.orthrus_gemm_bf16.argtypes = [_vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    lib.orthrus_gemm_bf16.restype = ctypes.c_int
    lib.orthrus_lora_shrink_bf16.argtypes = [_vp, _i32, _vp, _i32, _i32, _i32, ctypes.c_float, _vp, _vp,
                                             ctypes.c_int64, _vp]
    lib.orthrus_lora_shrink_bf16.restype = ctypes.c_int
    lib.orthrus_sample.argtypes = [_vp, ctypes.c_int64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.orthrus_sample.restype = ctypes.c_int
    lib.orthrus_fill_hash_bf16.argtypes = [_vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64, _vp]
    lib.orthrus_fill_hash_bf16.restype = ctypes.c_int
    lib.orthrus_set_layer_dump.argtypes = [_vp, _vp, ctypes.c_int64]
    lib.orthrus_set_layer_dump.restype = ctypes.c_int
    lib.orthrus_profile.argtypes = [_vp, _i32]
    lib.orthrus_profile.restype = ctypes.c_int
    lib.orthrus_profile_read.argtypes = [_vp, ctypes.c_char_p, _i32]
    lib.orthrus_profile_read.restype = _i32
    lib.orthrus_sched_create.argtypes = [_i32, _i32, _i32, _i32p, _i32, _i32, ctypes.POINTER(_vp)]
    lib.orthrus_sched_create.restype = ctypes.c_int
    lib.orthrus_sched_submit.argtypes = [_vp, _i32, _i32, _i32p, _i32, _i32, _i32]
    lib.orthrus_sched_submit.restype = ctypes.c_int
    lib.orthrus_sched_next.argtypes = [_vp, ctypes.POINTER(orthrus_batch), _i32p]
    lib.orthrus_sched_next.restype = ctypes.c_int
    lib.orthrus_sched_commit.argtypes = [_vp, _i32p, _i32]
    lib.orthrus_sched_commit.restype = ctypes.c_int
    lib.orthrus_sched_stats.argtypes = [_vp, ctypes.POINTER(ctypes.c_int64)]
    lib.orthrus_sched_stats.restype = ctypes.c_int
    lib.orthrus_sched_destroy.argtypes = [_vp]
    lib.orthrus_sched_destroy.restype = None
    return lib


LIB = _load()
EXPORTS = ("orthrus_pack", "orthrus_create", "orthrus_step", "orthrus_last_error",
           "orthrus_destroy", "orthrus_gemm_bf16", "orthrus_profile", "orthrus_profile_read",
           "orthrus_fill_hash_bf16", "orthrus_sched_create", "orthrus_sched_submit",
           "orthrus_sched_next", "orthrus_sched_commit", "orthrus_sched_stats", "orthrus_sched_destroy",
           "orthrus_sample", "orthrus_set_layer_dump", "orthrus_step_noalloc", "orthrus_lora_shrink_bf16")


class OrthrusError(RuntimeError):
    def __init__(self, code, msg=""):
        super().__init__(f"{STATUS_NAMES[code] if 0 <= code < len(STATUS_NAMES) else code}: {msg}")
        self.code = code


# ---- marshalling helpers ----------------------------------------------------

def make_cfg(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, lora_rank,
             page_size, n_pages, max_tokens, max_items, max_pool_slots, rope_theta, rms_eps,
             lora_scale, dtype=DTYPE_BF16) -> orthrus_model_cfg:
    return orthrus_model_cfg(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab,
                             lora_rank, page_size, n_pages, max_tokens, max_items, max_pool_slots,
                             rope_theta, rms_eps, lora_scale, dtype)


class BatchArgs:
    """An orthrus_batch whose host arrays stay alive with this object.

    items: int32 array [n_items, 10] in orthrus_item field order."""

    def __init__(self, items, token_ids, page_ids):
        self.items_np = np.ascontiguousarray(np.asarray(items, np.int32).reshape(-1, 10))
        self.tok_np = np.ascontiguousarray(np.asarray(token_ids, np.int32).reshape(-1))
        self.pages_np = np.ascontiguousarray(np.asarray(page_ids, np.int32).reshape(-1))
        self.struct = orthrus_batch(
            self.items_np.shape[0], self.tok_np.shape[0], self.pages_np.shape[0],
            self.items_np.ctypes.data_as(ctypes.POINTER(orthrus_item)),
            self.tok_np.ctypes.data_as(_i32p), self.pages_np.ctypes.data_as(_i32p))


def orthrus_pack(cfg: orthrus_model_cfg, batch: BatchArgs):
    """Returns (status, dict of int32 arrays and counts, error message)."""
    T = max(batch.tok_np.shape[0], 1)
    n = max(batch.items_np.shape[0], 1)
    arrs = {"cu_q": np.zeros(n + 1, np.int32), "pos": np.zeros(T, np.int32),
            "slot": np.zeros(T, np.int32), "row_item": np.zeros(T, np.int32),
            "logit_rows": np.zeros(n, np.int32), "pool_segs": np.zeros(n * 8, np.int32)}
    pk = orthrus_packed(T, n, *[arrs[k].ctypes.data_as(_i32p) for k in
                                ("cu_q", "pos", "slot", "row_item", "logit_rows", "pool_segs")])
    err = ctypes.create_string_buffer(256)
    st = LIB.orthrus_pack(ctypes.byref(cfg), ctypes.byref(batch.struct), ctypes.byref(pk), err, 256)
    out = {}
    if st == OK:
        nt, ni = batch.tok_np.shape[0], batch.items_np.shape[0]
        out = {"cu_q": arrs["cu_q"][:ni + 1], "pos": arrs["pos"][:nt], "slot": arrs["slot"][:nt],
               "row_item": arrs["row_item"][:nt], "logit_rows": arrs["logit_rows"][:pk.n_logits],
               "pool_segs": arrs["pool_segs"][:pk.n_pool_segs * 8].reshape(-1, 8),
               "n_embed_rows": pk.n_embed_rows, "n_prefill_rows": pk.n_prefill_rows,
               "n_decode_rows": pk.n_decode_rows, "n_logits": pk.n_logits, "n_emb": pk.n_emb}
    return st, out, err.value.decode()


def orthrus_create(cfg: orthrus_model_cfg, tok_emb, lm_head, g_final, layers, k_pages, v_pages):
    """layers: list of dicts of device addresses keyed like orthrus_layer_w.
    Returns (engine handle, weights struct kept alive by the caller)."""
    arr = (orthrus_layer_w * len(layers))()
    for i, L in enumerate(layers):
        for k, _ in orthrus_layer_w._fields_:
            setattr(arr[i], k, L.get(k) or None)
    w = orthrus_weights(tok_emb, lm_head, g_final, ctypes.cast(arr, ctypes.POINTER(orthrus_layer_w)))
    h = _vp()
    st = LIB.orthrus_create(ctypes.byref(cfg), ctypes.byref(w), k_pages, v_pages, ctypes.byref(h))
    if st != OK:
        raise OrthrusError(st, "orthrus_create failed: " + orthrus_last_error(None))
    return h, (w, arr)


def orthrus_step(eng, batch: BatchArgs, pool_sum, pool_wsum, pool_kept, logits, logits_cap_rows,
                 emb, emb_cap_rows, hidden_out=None, stream=None, logit_req_ids=None, emb_req_ids=None,
                 pool_buf=None, buf_rows=0, noalloc=False):
    """Returns (status, n_logits, n_emb).  logit_req_ids / emb_req_ids:
    optional int32 numpy arrays of at least logits_cap_rows / emb_cap_rows
    entries that receive the req_id of each output row.  pool_buf /
    buf_rows: the BUFFER pooling kind's hidden-state buffer.  noalloc:
    call orthrus_step_noalloc instead (same arguments)."""
    ps = orthrus_pool_state(pool_sum, pool_wsum, pool_kept, pool_buf, buf_rows)
    nl, ne = _i32(0), _i32(0)

    def ids(a, cap):
        if a is None:
            return None
        assert a.dtype == np.int32 and a.flags.c_contiguous and a.size >= cap
        return a.ctypes.data_as(_i32p)

    fn = LIB.orthrus_step_noalloc if noalloc else LIB.orthrus_step
    st = fn(eng, ctypes.byref(batch.struct), ctypes.byref(ps), logits, logits_cap_rows,
            emb, emb_cap_rows, ctypes.byref(nl), ctypes.byref(ne),
            ids(logit_req_ids, logits_cap_rows), ids(emb_req_ids, emb_cap_rows), hidden_out, stream)
    return st, nl.value, ne.value


def orthrus_last_error(eng) -> str:
    return LIB.orthrus_last_error(eng).decode()


def orthrus_destroy(eng) -> None:
    LIB.orthrus_destroy(eng)


def orthrus_gemm_bf16(A, lda, B, ldb, C, ldc, M, N, K, epilogue, b_up_row=0, stream=None) -> int:
    return LIB.orthrus_gemm_bf16(A, lda, B, ldb, C, ldc, M, N, K, epilogue, b_up_row, stream)


def orthrus_lora_shrink_bf16(X, ldx, A, rows, nr, K, scale, U, workspace=None, workspace_bytes=0,
                             stream=None) -> int:
    return LIB.orthrus_lora_shrink_bf16(X, ldx, A, rows, nr, K, scale, U, workspace, workspace_bytes, stream)


def orthrus_set_layer_dump(eng, dst, cap_rows) -> int:
    """dst: device address of fp32 [n_layers][cap_rows][d], or None to stop."""
    return LIB.orthrus_set_layer_dump(eng, dst, cap_rows if dst else 0)


def orthrus_profile(eng, enable: bool) -> int:
    return LIB.orthrus_profile(eng, 1 if enable else 0)


def orthrus_profile_read(eng) -> dict:
    import json
    n = LIB.orthrus_profile_read(eng, None, 0)
    if n < 0:
        raise OrthrusError(EINVAL, "null engine")
    buf = ctypes.create_string_buffer(n + 1)
    LIB.orthrus_profile_read(eng, buf, n + 1)
    return json.loads(buf.value.decode())


def orthrus_sample(logits, ld, n_rows, vocab, tokens, temperature=None, top_p=None, uniforms=None,
                   stream=None) -> int:
    """Device pointers; temperature/top_p/uniforms may be None."""
    return LIB.orthrus_sample(logits, ld, n_rows, vocab, temperature, top_p, uniforms, tokens, stream)


def orthrus_fill_hash_bf16(dst, n, seed, tensor_id, start=0, stream=None) -> int:
    return LIB.orthrus_fill_hash_bf16(dst, n, seed, tensor_id, start, stream)


def orthrus_sched_create(token_budget, chunk, page_size, free_pages, n_pool_slots):
    """Returns (status, handle)."""
    fp = np.ascontiguousarray(np.asarray(free_pages, np.int32).reshape(-1))
    h = _vp()
    st = LIB.orthrus_sched_create(token_budget, chunk, page_size, fp.ctypes.data_as(_i32p), fp.shape[0],
                                  n_pool_slots, ctypes.byref(h))
    return st, h


def orthrus_sched_submit(s, req_id, kind, tokens, pool_kind=0, max_new_tokens=0) -> int:
    t = np.ascontiguousarray(np.asarray(tokens, np.int32).reshape(-1))
    return LIB.orthrus_sched_submit(s, req_id, kind, t.ctypes.data_as(_i32p), t.shape[0], pool_kind,
                                    max_new_tokens)


def orthrus_sched_next(s):
    """Returns (status, BatchArgs copy of the batch or None, n_logits)."""
    b = orthrus_batch()
    nl = _i32(0)
    st = LIB.orthrus_sched_next(s, ctypes.byref(b), ctypes.byref(nl))
    if st != OK or b.n_items == 0:
        return st, None, 0
    items = np.ctypeslib.as_array(ctypes.cast(b.items, _i32p), shape=(b.n_items * 10,)).reshape(-1, 10).copy()
    toks = np.ctypeslib.as_array(b.token_ids, shape=(b.n_tokens,)).copy()
    pages = np.ctypeslib.as_array(b.page_ids, shape=(b.n_page_ids,)).copy() if b.n_page_ids else \
        np.zeros(0, np.int32)
    return st, BatchArgs(items, toks, pages), nl.value


def orthrus_sched_commit(s, sampled) -> int:
    a = np.ascontiguousarray(np.asarray(sampled, np.int32).reshape(-1))
    return LIB.orthrus_sched_commit(s, a.ctypes.data_as(_i32p) if a.size else None, a.shape[0])


def orthrus_sched_stats(s):
    out = (ctypes.c_int64 * 8)()
    st = LIB.orthrus_sched_stats(s, out)
    return st, list(out)


def orthrus_sched_destroy(s) -> None:
    LIB.orthrus_sched_destroy(s)
