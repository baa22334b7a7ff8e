"""Benchmark: mixed-batch tokens/s of one heterogeneous-batch step on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one Mistral-7B-shaped decoder layer in bf16 (d 4096, 32 q / 8 kv
heads of 128, SwiGLU 14336, RoPE theta 1e6, vocab 32768, N(0, 0.02)
weights, LoRA rank 16 on q/k/v/o for embedding rows only) over a batch of
8 embedding chunks x 512 tokens (last-token pooling) and 64 decode rows with
KV contexts uniform in [500, 3500], KV pages of 16 tokens: 4160 rows per
step, all inputs seeded and synthetic, already resident in HBM.

A step is one orthrus_step call (embed gather, the layer, final norm, LM
head on the 64 logit rows, pooling).  The timed region is K steps bracketed
by device synchronisation; a second pass of K steps with per-kernel HIP
events gives each kernel's average duration for the roofline figure.  The
CPU baseline times the oracle on the same step on the host cores.
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
    attn_flops = 4.0 * hd * cfg.n_q_heads * (pairs + dec_keys)
    attn_bytes = 2.0 * 2 * kvd * dec_keys
    return {
        "gemm_qkv": (2.0 * T * qkvd * d + 2.0 * TE * r * qkvd, 2.0 * (T * d + qkvd * d + T * qkvd)),
        "gemm_o": (2.0 * T * d * qd + 2.0 * TE * r * d, 2.0 * (T * qd + d * qd) + 8.0 * T * d),
        "gemm_gate_up": (2.0 * T * 2 * F * d, 2.0 * (T * d + 2 * F * d + T * F)),
        "gemm_down": (2.0 * T * d * F, 2.0 * (T * F + d * F) + 8.0 * T * d),
        "lm_head": (2.0 * G * V * d, 2.0 * (G * d + V * d) + 4.0 * G * V),
        "attention": (attn_flops, attn_bytes),
        "lora_shrink_qkv": (2.0 * TE * 3 * r * d, 2.0 * (TE * d + 3 * r * d)),
        "lora_shrink_o": (2.0 * TE * r * qd, 2.0 * (TE * qd + r * qd)),
    }


def kernel_source_digest():
    h = hashlib.sha256()
    p = os.path.join(ROOT, "heterogeneous_embed_decode_amd", "csrc", "kernels_gemm.hip")
    h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_one_layer_traffic.md")
    if not os.path.exists(p):
        return None
    rec = {}
    for line in open(p):
        if ":" in line and not line.startswith(("|", "#", " ", "`")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, batch, n_pages, bits, kv_bits):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    W = oracle.widen_weights(bits, np.float32)
    K, V = oracle.new_kv(cfg, n_pages, np.float32, kv_bits[0], kv_bits[1])
    pool = oracle.new_pool(16, cfg.d_model, np.float32)
    t0 = time.perf_counter()
    oracle.step(cfg, W, batch, (K, V), pool, np.float32)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": batch.n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one full step of the same workload ({batch.n_tokens} rows) through the numpy fp32 "
                      f"oracle, {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    cfg, batch, n_pages = wl.one_layer_workload()
    bits = sm.make_weights(cfg, seed=0)
    kv_bits = wl.synthetic_kv(cfg, n_pages, seed=3)
    dev = DeviceModel(cfg, bits, n_pages, max_tokens=batch.n_tokens, max_items=batch.n_items,
                      max_pool_slots=16, kv_bits=kv_bits)
    st, meta, _ = hed.orthrus_pack(dev.cfg, dev.step_args(batch))
    assert st == hed.OK
    bargs = dev.step_args(batch)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    print(f"setup {time.time() - t_setup:.1f}s rows={batch.n_tokens} items={batch.n_items}",
          file=sys.stderr, flush=True)

    def run(k):
        for _ in range(k):
            s, _, _ = dev.step(batch, stream=sptr, args=bargs)
            if s != hed.OK:
                raise hed.OrthrusError(s, hed.orthrus_last_error(dev.eng))

    run(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    run(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)
    ms_per_step = 1e3 * wall / args.steps
    value = batch.n_tokens * args.steps / wall
    print(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step wall, {ev_ms / args.steps:.3f} ms/step events",
          file=sys.stderr, flush=True)

    # per-kernel durations over an identical pass
    hed.orthrus_profile(dev.eng, True)
    run(args.steps)
    torch.cuda.synchronize()
    prof = hed.orthrus_profile_read(dev.eng)
    hed.orthrus_profile(dev.eng, False)
    work = kernel_work(cfg, batch, meta)
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
    if dom.startswith("gemm") or dom == "lm_head" and fl / max(by, 1) > 312:
        achieved, peak, unit, bound = fl / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = by / avg_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    roof = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_from_profiles(dom),
            "algorithmic_per_launch": fl if bound == "mfma" else by, "avg_ms": round(avg_s * 1e3, 5)}
    # decode attention is the HBM-bound part of the path: report its bandwidth too
    if "attention" in prof:
        a_avg = prof["attention"]["total_ms"] / prof["attention"]["count"] * 1e-3
        roof["attention_hbm_gbs"] = round(work["attention"][1] / a_avg / 1e9, 1)

    cpu = None
    if not args.no_cpu_baseline:
        print("timing the CPU oracle on the same step ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, batch, n_pages, bits, kv_bits)

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
        "config": {"workload": "one Mistral-7B-shaped layer, LoRA r16 on embedding rows; 8 embedding "
                               "chunks x 512 tokens (last-token pooling) + 64 decode rows, KV contexts "
                               "U[500,3500], page 16",
                   "rows": batch.n_tokens, "embed_rows": meta["n_embed_rows"],
                   "decode_rows": meta["n_decode_rows"], "layers": cfg.n_layers, "d_model": cfg.d_model,
                   "ffn_dim": cfg.ffn_dim, "vocab": cfg.vocab, "lora_rank": cfg.lora_rank},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    dev.close()


if __name__ == "__main__":
    main()
