"""Benchmark: mixed-batch tokens/s of one heterogeneous-batch step on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--workload W]

Default workload (mix91): the full 32-layer Mistral-7B-shaped decoder in
bf16 (d 4096, 32 q / 8 kv heads of 128, SwiGLU 14336, RoPE theta 1e6, vocab
32768, N(0, 0.02) weights, LoRA rank 16 on q/k/v/o for embedding rows only)
at a 9:1 embedding:generation token mix with a budget of 8192 rows per
step: 819 decode rows with KV contexts uniform in [500, 3500] reserved
first, then embedding requests of U[256, 4096] tokens in chunks of 256
(mean pooling) admitted first come first served; ten consecutive distinct
steps with KV and pooling state carried.  Inputs are seeded and synthetic
and already resident in HBM.  Other workloads: one_layer (one such layer,
8 x 512-token embedding chunks + 64 decode rows), mix55, mix19.

A step is one orthrus_step call (embed gather, every layer, final norm, LM
head on the logit rows, pooling); the timed region is K steps cycling
through the distinct steps, bracketed by device synchronisation, and
`value` is the rows of those steps over the wall time.  Further untimed
passes give per-step times (HIP events around each step) and per-kernel
averages (HIP events around each launch, on the step's stream) for the
roofline figures.  The CPU baseline times the oracle on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

METRIC = "mixed-batch tokens/s per step (embed+decode) @Mistral-7B shape; % MFMA/HBM roofline"


def kernel_work(cfg, batch, meta):
    """Algorithmic work per launch of each kernel: (flops, bytes)."""
    T = batch.n_tokens
    d, F, V = cfg.d_model, cfg.ffn_dim, cfg.vocab
    qd, kvd, qkvd, r = cfg.q_dim, cfg.kv_dim, cfg.qkv_dim, cfg.lora_rank
    TE = meta["n_embed_rows"]
    G = meta["n_logits"]
    hd = cfg.head_dim
    # causal chunk pairs and decode keys (KV read once per kv head)
    pairs = 0
    dec_keys = 0
    for it in batch.items:
        if it.kind == 2:
            dec_keys += it.ctx_len + 1
        else:
            n, c = it.n_tokens, it.ctx_len
            pairs += n * c + n * (n + 1) // 2
    # chunk attention: QK^T and PV over the causal pairs; decode attention:
    # every key of every decode row read once per KV head (K and V, bf16)
    chunk_flops = 4.0 * hd * cfg.n_q_heads * pairs
    chunk_bytes = 2.0 * 2 * kvd * sum(it.ctx_len + it.n_tokens for it in batch.items if it.kind != 2)
    dec_flops = 4.0 * hd * cfg.n_q_heads * dec_keys
    dec_bytes = 2.0 * 2 * kvd * dec_keys
    qkv_work = (2.0 * T * qkvd * d + 2.0 * TE * r * qkvd, 2.0 * (T * d + qkvd * d + T * qkvd))
    return {
        "gemm_qkv": qkv_work,
        # the same projection with RoPE and the KV append in its epilogue:
        # the same flops, plus the step's cos/sin table read once
        "gemm_qkv_rope": (qkv_work[0], qkv_work[1] + 4.0 * T * hd),
        "rope_table": (0.0, 4.0 * T * hd + 4.0 * T),
        "gemm_o": (2.0 * T * d * qd + 2.0 * TE * r * d, 2.0 * (T * qd + d * qd) + 8.0 * T * d),
        "gemm_gate_up": (2.0 * T * 2 * F * d, 2.0 * (T * d + 2 * F * d + T * F)),
        "gemm_down": (2.0 * T * d * F, 2.0 * (T * F + d * F) + 8.0 * T * d),
        "lm_head": (2.0 * G * V * d, 2.0 * (G * d + V * d) + 4.0 * G * V),
        "attn_chunk": (chunk_flops, chunk_bytes),
        "attn_decode": (dec_flops, dec_bytes),
        "attn_ragged": (chunk_flops + dec_flops, chunk_bytes + dec_bytes),
        "lora_shrink_qkv": (2.0 * TE * 3 * r * d, 2.0 * (TE * d + 3 * r * d)),
        "lora_shrink_o": (2.0 * TE * r * qd, 2.0 * (TE * qd + r * qd)),
        "pool": (0.0, pool_bytes(cfg, batch)),
    }


def qkv_rope_fused(cfg, T):
    """Whether the library runs RoPE and the KV append in the QKV
    projection's epilogue for a batch of T rows (head dim 128, an even
    number of q and of KV heads, at least 512 rows)."""
    return cfg.head_dim == 128 and T >= 512 and cfg.n_q_heads % 2 == 0 and cfg.n_kv_heads % 2 == 0


def step_roofline_ms(cfg, batch, meta):
    """Ideal time of one step: every kernel at the larger of its algorithmic
    flops over the bf16 MFMA peak and its algorithmic HBM bytes over the HBM
    peak, summed over the step's launches (per-layer kernels times the
    depth).  Terms: the four projections with their adapter shrinks, chunk
    and decode attention, the two norms and the RoPE/KV append per layer,
    and the LM head, final norm and pooling once."""
    w = kernel_work(cfg, batch, meta)
    L, T, d = cfg.n_layers, batch.n_tokens, cfg.d_model
    P, BW = PEAK_BF16_TFLOPS * 1e12, PEAK_HBM_GBS * 1e9

    def t(fl, by):
        return max(fl / P, by / BW)

    per_layer = ["gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attn_chunk", "attn_decode"]
    if meta["n_embed_rows"] and cfg.lora_rank:
        per_layer += ["lora_shrink_qkv", "lora_shrink_o"]
    terms = {k: L * t(*w[k]) for k in per_layer}
    terms["rmsnorm"] = L * 2 * t(0.0, T * d * (4.0 + 2.0))
    if qkv_rope_fused(cfg, T):
        # RoPE and the KV append run inside the QKV projection, which is
        # matrix-bound; the step builds one cos/sin table
        terms["rope_table"] = t(*w["rope_table"])
    else:
        terms["rope_kv"] = L * t(0.0, 2.0 * T * (cfg.q_dim + cfg.kv_dim) * 2 + 2.0 * T * 2 * cfg.kv_dim)
    # the final norm reads the embedding and logit rows of the residual and
    # writes the logit rows (bf16) and one 1/rms per embedding row
    terms["final_norm"] = t(0.0, (meta["n_embed_rows"] + meta["n_logits"]) * d * 4.0 + meta["n_logits"] * d * 2.0)
    terms["lm_head"] = t(*w["lm_head"])
    terms["pool"] = t(*w["pool"])
    return 1e3 * sum(terms.values()), {k: round(1e3 * v, 4) for k, v in terms.items()}


def host_description():
    """CPU model, logical CPUs and the BLAS numpy calls into."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": blas}


def sub_batch(batch, keep):
    """The items of a batch that `keep` selects, as a batch of their own
    (page lists re-based), for timing one side of the ragged attention."""
    from synth import workloads as wl
    items, toks, pages = [], [], []
    t = 0
    for i, it in enumerate(batch.items):
        if keep(it):
            items.append(wl.Item(**{**it.__dict__, "page_off": len(pages)}))
            pages.extend(batch.item_pages(i).tolist())
            toks.extend(int(x) for x in batch.token_ids[t:t + it.n_tokens])
        t += it.n_tokens
    import numpy as np
    return wl.Batch(items, np.asarray(toks, np.int32), np.asarray(pages, np.int32))


def decode_only(batch):
    from synth import workloads as wl
    return sub_batch(batch, lambda it: it.kind == wl.DECODE)


def chunk_only(batch):
    from synth import workloads as wl
    return sub_batch(batch, lambda it: it.kind != wl.DECODE)


def pool_bytes(cfg, batch):
    """HBM bytes of the pooling kernels per step: streaming heads read the
    chunk's fp32 residual rows once (and one 1/rms per row, not counted);
    the buffered head also writes them to the
    slot's buffer and, on the last chunk, reads the rows buffered by earlier
    chunks; kept heads touch one row; every head reads and writes its
    d-vector state and the emitted row (read again when the L2 flag
    rescales it)."""
    d4 = 4.0 * cfg.d_model
    tot = 0.0
    for it in batch.items:
        if it.kind != 0:
            continue
        k, l2 = it.pool_kind & ~8, it.pool_kind & 8
        n = it.n_tokens
        if k in (0, 1):
            tot += n * d4 + 2 * d4
        elif k == 4:
            tot += 2 * n * d4 + it.ctx_len * d4 * it.is_last
        else:
            tot += 2 * d4
        tot += d4 * it.is_last * (3 if l2 else 1)
    return tot


def kernel_source_digest(names):
    """First 16 hex digits of the SHA-256 of the named csrc files' contents,
    concatenated in the order given (names separated by spaces)."""
    h = hashlib.sha256()
    for name in names.split():
        h.update(open(os.path.join(ROOT, "heterogeneous_embed_decode_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel on this workload, if it was taken on the current kernel
    source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(p):
        return None
    rec = {}
    for line in open(p):
        if ":" in line and not line.startswith(("|", "#", " ", "`")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    src = rec.get("kernel_source_file")
    if not src or rec.get("kernel_source_sha256_16") != kernel_source_digest(src):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


WORKLOAD_TEXT = {
    "one_layer": "one Mistral-7B-shaped layer, LoRA r16 on embedding rows; 8 embedding chunks x 512 tokens "
                 "(last-token pooling) + 64 decode rows, KV contexts U[500,3500], page 16",
    "mix91": "32-layer Mistral-7B shape, 9:1 embed:gen tokens, budget 8192, 819 decode rows (KV U[500,3500]) + "
             "embedding requests U[256,4096] in chunks of 256 (mean), ten distinct steps, LoRA r16",
    "mix55": "32-layer Mistral-7B shape, 5:5 mix, budget 8192, LoRA r64: 4 x 1024-token weighted-mean chunks, "
             "7 x 500-token prefill chunks, 596 decode rows (KV U[500,3500])",
    "mix19": "32-layer Llama-3.1-8B shape, 1:9 requests, budget 8192: 256 decode rows (KV U[500,3500]) + "
             "15 CLS chunks of 512 tokens, LoRA r16",
}


def cpu_baseline_one_layer(cfg, batch, n_pages, bits, n_slots, prior_wsum):
    """The oracle on one full-batch layer of a deep workload (prior KV of the
    batch's pages regenerated on the host), scaled to the full depth."""
    import numpy as np
    import oracle
    from synth.hashfill import splitmix64_fill
    from synth.bf16 import bf16_bits_to_f32
    from synth import workloads as wl
    from threadpoolctl import threadpool_info
    c1 = cfg.with_(n_layers=1)
    keep = {k: v for k, v in bits.items() if not k.startswith("layers.") or k.startswith("layers.0.")}
    W = oracle.widen_weights(keep, np.float32)
    used = sorted(set(int(p) for p in batch.page_ids))
    remap = {p: i for i, p in enumerate(used)}
    blk = cfg.n_kv_heads * cfg.page_size * cfg.head_dim
    shape = (cfg.n_kv_heads, cfg.page_size, cfg.head_dim)
    K = np.stack([bf16_bits_to_f32(splitmix64_fill(wl.KV_SEED, 0, blk, p * blk)).reshape(shape) for p in used])
    V = np.stack([bf16_bits_to_f32(splitmix64_fill(wl.KV_SEED, 1, blk, p * blk)).reshape(shape) for p in used])
    sub = wl.Batch(batch.items, batch.token_ids, np.asarray([remap[int(p)] for p in batch.page_ids], np.int32))
    pool = oracle.new_pool(n_slots, cfg.d_model, np.float32)
    for slot, v in prior_wsum.items():
        pool["wsum"][slot] = v
    t0 = time.perf_counter()
    oracle.step(c1, W, sub, ([K], [V]), pool, np.float32)
    dt1 = time.perf_counter() - t0
    # one layer plus the head; the other layers cost the same as the first
    est = dt1 * cfg.n_layers
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": batch.n_tokens / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": True, "host": host_description(),
            "sample": f"one full-batch layer of the first step ({batch.n_tokens} rows) through the numpy fp32 "
                      f"oracle, {dt1:.2f} s, extrapolated to {cfg.n_layers} layers (extrapolated from 1 measured "
                      f"layer)"}


def cpu_baseline(cfg, batch, n_pages, bits, kv_bits):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    W = oracle.widen_weights(bits, np.float32)
    K, V = oracle.new_kv(cfg, n_pages, np.float32, kv_bits[0], kv_bits[1])
    pool = oracle.new_pool(16, cfg.d_model, np.float32, buf_rows=max((it.ctx_len + it.n_tokens for it in batch.items if it.kind == 0), default=0))
    t0 = time.perf_counter()
    oracle.step(cfg, W, batch, (K, V), pool, np.float32)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": batch.n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": False, "host": host_description(),
            "sample": f"one full step of the same workload ({batch.n_tokens} rows) through the numpy fp32 "
                      f"oracle, {dt:.2f} s"}


def measure_sampler(dev, cfg, meta, stream, run, calls=50, greedy_too=True):
    """Time orthrus_sample on the logit rows of the workload's first step
    (temperature 0.8, top-p 0.9 on every row: the full radix-select path;
    greedy rows stop after the max pass).  HIP events on the step's stream."""
    import numpy as np
    import torch
    import heterogeneous_embed_decode_amd as hed
    nl = int(meta["n_logits"])
    if not nl:
        return None
    g = np.random.default_rng(0)
    temp_d = torch.full((nl,), 0.8, dtype=torch.float32, device="cuda")
    top_d = torch.full((nl,), 0.9, dtype=torch.float32, device="cuda")
    uni_d = torch.from_numpy(g.integers(0, 2 ** 32, nl, dtype=np.uint64).astype(np.uint32).view(np.int32)).cuda()
    tok_d = torch.empty(nl, dtype=torch.int32, device="cuda")
    sptr = stream.cuda_stream
    run(1)

    def smp(k, greedy=False):
        for _ in range(k):
            st_ = hed.orthrus_sample(dev.logits.data_ptr(), cfg.vocab, nl, cfg.vocab, tok_d.data_ptr(),
                                     None if greedy else temp_d.data_ptr(), top_d.data_ptr(), uni_d.data_ptr(), sptr)
            assert st_ == hed.OK

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for mode in (("sampled", "greedy") if greedy_too else ("sampled",)):
        smp(3, mode == "greedy")
        e0.record(stream)
        smp(calls, mode == "greedy")
        e1.record(stream)
        torch.cuda.synchronize()
        res[mode] = e0.elapsed_time(e1) / calls * 1e3
    by = nl * cfg.vocab * 4
    out = {"kernel": "sample_kernel", "rows": nl, "vocab": cfg.vocab, "temperature": 0.8, "top_p": 0.9,
           "us_per_call": round(res["sampled"], 2), "logit_bytes": by,
           "hbm_gbs": round(by / (res["sampled"] * 1e-6) / 1e9, 1),
           "hbm_frac": round(by / (res["sampled"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    if "greedy" in res:
        out["greedy_us_per_call"] = round(res["greedy"], 2)
    print(f"sampler: {nl} rows x {cfg.vocab}: " + ", ".join(f"{k} {v:.1f} us" for k, v in res.items()),
          file=sys.stderr, flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="mix91", choices=["one_layer", "mix91", "mix55", "mix19"],
                    help="mix91 (default): the 32-layer 9:1 workload, ten distinct steps; mix55 (rank 64) and "
                         "mix19 (Llama-3.1-8B shape, 1:9); one_layer: one Mistral-7B-shaped layer, 4160 rows")
    ap.add_argument("--layers", type=int, default=32, help="depth of the mixed workloads")
    ap.add_argument("--pool-kind", default="last", choices=["last", "mean", "wmean", "cls", "buffer", "last+l2",
                                                              "mean+l2", "buffer+l2"],
                    help="pooling head of the one-layer workload's embedding chunks (default: last-token)")
    ap.add_argument("--sampler-only", action="store_true",
                    help="run one step of the workload, then time only the sampler on its logit rows "
                         "(temperature 0.8, top-p 0.9); prints the sampler object")
    ap.add_argument("--decode-only", action="store_true",
                    help="with --counters: run only the decode items of each step (decode attention alone)")
    ap.add_argument("--chunk-only", action="store_true",
                    help="with --counters: run only the embedding and prefill items of each step")
    ap.add_argument("--counters", action="store_true",
                    help="run only --warmup + --steps steps of the workload and exit (for rocprofv3 counter "
                         "passes; no JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB (read) into 1 GiB (write), 5 times; "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the step needs no collective and each replica is "
              "independent, so run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration:
        n = 1 << 28  # float32 elements: 1 GiB
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "launches": 5}), flush=True)
        return
    import heterogeneous_embed_decode_amd as hed
    from heterogeneous_embed_decode_amd.device_model import DeviceModel
    from synth import model as sm
    from synth import workloads as wl

    t_setup = time.time()
    prior_wsum, n_slots = {}, 16
    if args.workload == "one_layer":
        pk_names = {"mean": wl.POOL_MEAN, "wmean": wl.POOL_WMEAN, "cls": wl.POOL_CLS, "last": wl.POOL_LAST,
                    "buffer": wl.POOL_BUFFER}
        base, _, l2 = args.pool_kind.partition("+")
        pool_kind = pk_names[base] | (wl.POOL_L2 if l2 else 0)
        cfg, batch, n_pages = wl.one_layer_workload(pool_kind=pool_kind)
        batches = [batch]
        bits = sm.make_weights(cfg, seed=0)
        kv_bits = wl.synthetic_kv(cfg, n_pages, seed=3)
    else:
        build = {"mix91": wl.nine_to_one_workload, "mix55": wl.five_to_five_workload,
                 "mix19": wl.one_to_nine_workload}[args.workload]
        w = build(n_layers=args.layers)
        cfg, batches, n_pages, n_slots, prior_wsum = w.cfg, w.batches, w.n_pages, w.n_slots, w.prior_wsum
        batch = batches[0]
        bits = sm.make_weights(cfg, seed=0)
        kv_bits = None
    max_t = max(b.n_tokens for b in batches)
    max_i = max(b.n_items for b in batches)
    buf_rows = max((it.ctx_len + it.n_tokens for b in batches for it in b.items
                    if it.kind == wl.EMBED and (it.pool_kind & ~wl.POOL_L2) == wl.POOL_BUFFER), default=0)
    dev = DeviceModel(cfg, bits, n_pages, max_tokens=max_t, max_items=max_i,
                      max_pool_slots=n_slots, kv_bits=kv_bits, buf_rows=buf_rows)
    if kv_bits is None:
        # prior KV and pooling state of the mixed workloads: SplitMix64 values
        # laid down on the device
        st0 = torch.cuda.current_stream().cuda_stream
        assert hed.orthrus_fill_hash_bf16(dev.K.data_ptr(), dev.K.numel(), wl.KV_SEED, 0, 0, st0) == hed.OK
        assert hed.orthrus_fill_hash_bf16(dev.V.data_ptr(), dev.V.numel(), wl.KV_SEED, 1, 0, st0) == hed.OK
        tmp = torch.empty(n_slots * cfg.d_model, dtype=torch.int16, device="cuda")
        for tid, dst in ((wl.POOL_SUM_TID, dev.pool_sum), (wl.POOL_KEPT_TID, dev.pool_kept)):
            assert hed.orthrus_fill_hash_bf16(tmp.data_ptr(), tmp.numel(), wl.KV_SEED, tid, 0, st0) == hed.OK
            dst[:n_slots].copy_((tmp.to(torch.int32) << 16).view(torch.float32).view(n_slots, cfg.d_model))
        for slot, v in prior_wsum.items():
            dev.pool_wsum[slot] = v
        torch.cuda.synchronize()
    metas = []
    for b in batches:
        st, m, _ = hed.orthrus_pack(dev.cfg, dev.step_args(b))
        assert st == hed.OK
        metas.append(m)
    meta = metas[0]
    bargs = [dev.step_args(b) for b in batches]
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    print(f"setup {time.time() - t_setup:.1f}s workload={args.workload} layers={cfg.n_layers} "
          f"rows={[b.n_tokens for b in batches]} items={batch.n_items}", file=sys.stderr, flush=True)

    rows_done = [0]

    def run(k):
        # cycles through the workload's distinct steps (one for the single-step workloads)
        for i in range(k):
            j = i % len(batches)
            s, _, _ = dev.step(batches[j], stream=sptr, args=bargs[j])
            if s != hed.OK:
                raise hed.OrthrusError(s, hed.orthrus_last_error(dev.eng))
            rows_done[0] += batches[j].n_tokens

    if args.counters:
        if args.decode_only or args.chunk_only:
            batches[:] = [(decode_only if args.decode_only else chunk_only)(b) for b in batches]
            bargs[:] = [dev.step_args(b) for b in batches]
        run(args.warmup + args.steps)
        torch.cuda.synchronize()
        print(f"ran {args.warmup + args.steps} steps", file=sys.stderr, flush=True)
        dev.close()
        return
    if args.sampler_only:
        print(json.dumps({"sampler": measure_sampler(dev, cfg, meta, stream, run, greedy_too=False)}), flush=True)
        dev.close()
        return
    run(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows_done[0] = 0
    t0 = time.perf_counter()
    e0.record(stream)
    run(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)
    ms_per_step = 1e3 * wall / args.steps
    value = rows_done[0] / wall
    print(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step wall, {ev_ms / args.steps:.3f} ms/step events",
          file=sys.stderr, flush=True)

    # per distinct step: HIP events around R repeats of the step on its
    # stream, after one untimed repeat, so the host enqueues ahead of the
    # device (a step timed alone between two events would include the host's
    # launch time while the device idles)
    per_step = []
    reps = max(2, args.steps // len(batches))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in batches]
    for j, b in enumerate(batches):
        for r in range(reps + 1):
            if r == 1:
                ev[j][0].record(stream)
            s_, _, _ = dev.step(b, stream=sptr, args=bargs[j])
            assert s_ == hed.OK
        ev[j][1].record(stream)
    torch.cuda.synchronize()
    for j, b in enumerate(batches):
        ms = ev[j][0].elapsed_time(ev[j][1]) / reps
        roof_ms, _ = step_roofline_ms(cfg, b, metas[j])
        per_step.append({"step": j, "rows": b.n_tokens, "embed_rows": int(metas[j]["n_embed_rows"]),
                         "decode_rows": int(metas[j]["n_decode_rows"]), "ms": round(ms, 3),
                         "tokens_per_s": round(b.n_tokens / (ms * 1e-3), 1), "roofline_ms": round(roof_ms, 3),
                         "roofline_frac": round(roof_ms / ms, 4)})
    t_roof = sum(r["roofline_ms"] for r in per_step)
    t_meas = sum(r["ms"] for r in per_step)
    _, terms0 = step_roofline_ms(cfg, batches[0], metas[0])
    step_roof = {"definition": "sum over the step's launches of max(algorithmic flops / 2.5 PFLOP/s, algorithmic "
                               "HBM bytes / 8 TB/s), over the measured step time (HIP events), summed over the "
                               "distinct steps",
                 "t_roof_ms": round(t_roof, 3), "t_measured_ms": round(t_meas, 3),
                 "frac": round(t_roof / t_meas, 4), "terms_step0_ms": terms0}
    print(f"per step: " + ", ".join(f"{r['ms']:.1f}" for r in per_step) + f" ms; step roofline fraction "
          f"{t_roof / t_meas:.3f}", file=sys.stderr, flush=True)

    # per-kernel durations over an identical pass
    hed.orthrus_profile(dev.eng, True)
    run(args.steps)
    torch.cuda.synchronize()
    prof = hed.orthrus_profile_read(dev.eng)
    hed.orthrus_profile(dev.eng, False)
    # algorithmic work per launch, averaged over the distinct steps that ran
    works = [kernel_work(cfg, b, m) for b, m in zip(batches, metas)]
    work = {k: tuple(sum(w_[k][i] for w_ in works) / len(works) for i in range(2)) for k in works[0]}
    kernels = {}
    for name, rec in prof.items():
        avg = rec["total_ms"] / max(rec["count"], 1)
        ent = {"avg_ms": round(avg, 5), "launches_per_step": rec["count"] // args.steps}
        if name in work:
            fl, by = work[name]
            ent["tflops"] = round(fl / (avg * 1e-3) / 1e12, 2)
            ent["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
        kernels[name] = ent
    dom = max(prof, key=lambda k: prof[k]["total_ms"])
    fl, by = work.get(dom, (0.0, 0.0))
    avg_s = prof[dom]["total_ms"] / prof[dom]["count"] * 1e-3
    if dom.startswith("gemm") or dom == "attn_chunk" or (dom == "lm_head" and fl / max(by, 1) > 312):
        achieved, peak, unit, bound = fl / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = by / avg_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    traffic = traffic_from_profiles(dom, args.workload)
    roof = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "algorithmic_per_launch": fl if bound == "mfma" else by, "avg_ms": round(avg_s * 1e3, 5)}
    # ragged attention runs chunk tiles (matrix-bound) and decode splits
    # (HBM-bound) in one launch: its fraction is the sum of both terms over
    # its time
    if "attn_ragged" in prof:
        r_avg = prof["attn_ragged"]["total_ms"] / prof["attn_ragged"]["count"] * 1e-3
        t_r = work["attn_chunk"][0] / (PEAK_BF16_TFLOPS * 1e12) + work["attn_decode"][1] / (PEAK_HBM_GBS * 1e9)
        roof["attn_ragged_frac"] = round(t_r / r_avg, 4)
    # the two sides of the ragged attention, each timed on the same steps'
    # rows alone: decode rows (HBM-bound: K/V bytes over 8 TB/s) and chunk
    # rows (matrix-bound: causal-pair flops over 2.5 PFLOP/s)
    def attn_alone(subs):
        sargs = [dev.step_args(b) for b in subs]
        for j, b in enumerate(subs):
            s_, _, _ = dev.step(b, stream=sptr, args=sargs[j])
            assert s_ == hed.OK
        torch.cuda.synchronize()
        hed.orthrus_profile(dev.eng, True)
        for _ in range(max(1, args.steps // len(subs))):
            for j, b in enumerate(subs):
                s_, _, _ = dev.step(b, stream=sptr, args=sargs[j])
                assert s_ == hed.OK
        torch.cuda.synchronize()
        sprof = hed.orthrus_profile_read(dev.eng)
        hed.orthrus_profile(dev.eng, False)
        return sprof["attn_ragged"]["total_ms"] / sprof["attn_ragged"]["count"] * 1e-3

    dec_batches = [decode_only(b) for b in batches]
    if any(b.n_items for b in dec_batches):
        d_avg = attn_alone(dec_batches)
        d_bytes = sum(kernel_work(cfg, b, m)["attn_decode"][1] for b, m in zip(batches, metas)) / len(batches)
        roof["attn_decode_hbm_gbs"] = round(d_bytes / d_avg / 1e9, 1)
        roof["attn_decode_hbm_frac"] = round(d_bytes / d_avg / 1e9 / PEAK_HBM_GBS, 4)
        roof["attn_decode_avg_ms"] = round(d_avg * 1e3, 5)
        roof["attn_decode_traffic"] = traffic_from_profiles("attn_ragged_decode", args.workload)
    chk_batches = [chunk_only(b) for b in batches]
    if any(b.n_items for b in chk_batches):
        c_avg = attn_alone(chk_batches)
        c_flops = sum(kernel_work(cfg, b, m)["attn_chunk"][0] for b, m in zip(batches, metas)) / len(batches)
        roof["attn_chunk_tflops"] = round(c_flops / c_avg / 1e12, 1)
        roof["attn_chunk_mfma_frac"] = round(c_flops / c_avg / 1e12 / PEAK_BF16_TFLOPS, 4)
        roof["attn_chunk_avg_ms"] = round(c_avg * 1e3, 5)

    sampler = measure_sampler(dev, cfg, meta, stream, run)
    cpu = None
    if not args.no_cpu_baseline:
        print("timing the CPU oracle on the same step ...", file=sys.stderr, flush=True)
        if args.workload == "one_layer":
            cpu = cpu_baseline(cfg, batch, n_pages, bits, kv_bits)
        else:
            cpu = cpu_baseline_one_layer(cfg, batch, n_pages, bits, n_slots, prior_wsum)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (WORKLOAD_TEXT[args.workload] if args.pool_kind == "last" or args.workload != "one_layer"
                                else WORKLOAD_TEXT[args.workload].replace("last-token pooling",
                                                                          f"{args.pool_kind} pooling")),
                   "rows": batch.n_tokens, "distinct_steps": len(batches), "embed_rows": meta["n_embed_rows"],
                   "decode_rows": meta["n_decode_rows"], "layers": cfg.n_layers, "d_model": cfg.d_model,
                   "ffn_dim": cfg.ffn_dim, "vocab": cfg.vocab, "lora_rank": cfg.lora_rank},
        "roofline": roof,
        "step_roofline": step_roof,
        "per_step": per_step,
        "cpu_baseline": cpu,
        "sampler": sampler,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    dev.close()


if __name__ == "__main__":
    main()
