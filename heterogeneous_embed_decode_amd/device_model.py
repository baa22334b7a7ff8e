"""Device-memory holder for one engine: weights, KV pools, pooling state.

PyTorch is used only to own device memory and to name the stream; every
step runs through ``orthrus_step`` in liborthrus.so.
"""

import numpy as np
import torch

from . import (BatchArgs, make_cfg, orthrus_create, orthrus_step, orthrus_destroy,
               orthrus_last_error, OrthrusError, OK, DTYPE_BF16, DTYPE_F32)

_LAYER_KEYS = ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_ffn",
               "lora_a_qkv", "lora_b_qkv", "lora_a_o", "lora_b_o")


def _dev_bits(a, device):
    """uint16 bf16 bit patterns (numpy) -> device int16 tensor with the same
    bits; float32 arrays (fp32 models) -> device float32 tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(a.view(np.int16)).to(device)


def _widen_bits(a):
    """bf16 bit patterns -> float32 (exact), for fp32 models given bf16 data."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a
    return (a.astype(np.uint32) << 16).view(np.float32)


class DeviceModel:
    """Weights, KV pools and pooling state on one device plus an engine.

    dims: an object with n_layers, d_model, n_q_heads, n_kv_heads, head_dim,
    ffn_dim, vocab, lora_rank, page_size, rope_theta, rms_eps, lora_scale and
    optionally dtype ("bf16" or "f32").
    weights: {name: uint16 bf16 bits, or float32 for an fp32 model} (globals
    and 'layers.<l>.<name>').
    kv_bits: optional (K, V) uint16 arrays of the full pool shape
    [L, n_pages, Hkv, page_size, hd] to upload as prior KV content.
    """

    def __init__(self, dims, weights, n_pages, max_tokens, max_items, max_pool_slots,
                 device="cuda:0", kv_bits=None, kv_tensors=None, buf_rows=0):
        self.dims = dims
        self.device = torch.device(device)
        torch.cuda.set_device(self.device)
        self.f32 = getattr(dims, "dtype", "bf16") == "f32"
        cast = _widen_bits if self.f32 else (lambda a: a)
        self.w = {k: _dev_bits(cast(v), self.device) for k, v in weights.items()}
        shape = (dims.n_layers, n_pages, dims.n_kv_heads, dims.page_size, dims.head_dim)
        kv_dtype = torch.float32 if self.f32 else torch.int16
        if kv_tensors is not None:
            self.K, self.V = kv_tensors
        elif kv_bits is not None:
            self.K = _dev_bits(cast(kv_bits[0]), self.device).reshape(shape)
            self.V = _dev_bits(cast(kv_bits[1]), self.device).reshape(shape)
        else:
            self.K = torch.zeros(shape, dtype=kv_dtype, device=self.device)
            self.V = torch.zeros(shape, dtype=kv_dtype, device=self.device)
        d = dims.d_model
        self.pool_sum = torch.zeros((max(max_pool_slots, 1), d), dtype=torch.float32, device=self.device)
        self.pool_wsum = torch.zeros(max(max_pool_slots, 1), dtype=torch.float32, device=self.device)
        self.pool_kept = torch.zeros((max(max_pool_slots, 1), d), dtype=torch.float32, device=self.device)
        # hidden-state buffer of the BUFFER pooling kind: [slots][buf_rows][d]
        self.buf_rows = buf_rows
        self.pool_buf = (torch.zeros((max(max_pool_slots, 1), buf_rows, d), dtype=torch.float32, device=self.device)
                         if buf_rows else None)
        self.max_tokens, self.max_items = max_tokens, max_items
        self.cfg = make_cfg(dims.n_layers, d, dims.n_q_heads, dims.n_kv_heads, dims.head_dim,
                            dims.ffn_dim, dims.vocab, dims.lora_rank, dims.page_size, n_pages,
                            max_tokens, max_items, max_pool_slots, dims.rope_theta, dims.rms_eps,
                            dims.lora_scale, DTYPE_F32 if self.f32 else DTYPE_BF16)
        layers = []
        for l in range(dims.n_layers):
            L = {}
            for k in _LAYER_KEYS:
                t = self.w.get(f"layers.{l}.{k}")
                L[k] = t.data_ptr() if (t is not None and t.numel() > 0) else None
            layers.append(L)
        self.eng, self._keep = orthrus_create(self.cfg, self.w["tok_emb"].data_ptr(),
                                              self.w["lm_head"].data_ptr(),
                                              self.w["g_final"].data_ptr(), layers,
                                              self.K.data_ptr(), self.V.data_ptr())
        self.logits = torch.empty((max_items, dims.vocab), dtype=torch.float32, device=self.device)
        self.emb = torch.empty((max_items, d), dtype=torch.float32, device=self.device)
        self.hidden = torch.empty((max_tokens, d), dtype=torch.float32, device=self.device)
        self.logit_req = np.zeros(max_items, np.int32)
        self.emb_req = np.zeros(max_items, np.int32)

    def step_args(self, batch):
        return BatchArgs(batch.items_array(), batch.token_ids, batch.page_ids)

    def step(self, batch, want_hidden=False, stream=None, args=None, noalloc=False):
        """Launch one step; returns (status, n_logits, n_emb).  Outputs live in
        self.logits[:n_logits], self.emb[:n_emb], self.hidden[:T].  noalloc:
        through orthrus_step_noalloc."""
        a = args if args is not None else self.step_args(batch)
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        st, nl, ne = orthrus_step(self.eng, a, self.pool_sum.data_ptr(), self.pool_wsum.data_ptr(),
                                  self.pool_kept.data_ptr(), self.logits.data_ptr(),
                                  self.logits.shape[0], self.emb.data_ptr(), self.emb.shape[0],
                                  self.hidden.data_ptr() if want_hidden else None, stream,
                                  self.logit_req, self.emb_req,
                                  self.pool_buf.data_ptr() if self.pool_buf is not None else None, self.buf_rows,
                                  noalloc=noalloc)
        return st, nl, ne

    def step_checked(self, batch, want_hidden=False):
        st, nl, ne = self.step(batch, want_hidden=want_hidden)
        if st != OK:
            raise OrthrusError(st, orthrus_last_error(self.eng))
        torch.cuda.synchronize(self.device)
        out = {"logits": self.logits[:nl].cpu().numpy(), "emb": self.emb[:ne].cpu().numpy(),
               "logit_req": self.logit_req[:nl].copy(), "emb_req": self.emb_req[:ne].copy()}
        if want_hidden:
            out["hidden"] = self.hidden[:batch.n_tokens].cpu().numpy()
        return out

    def close(self):
        if self.eng:
            orthrus_destroy(self.eng)
            self.eng = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
