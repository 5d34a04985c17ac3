"""Throughput of the decode step on one MI355X.

Default workload: the 8B-shaped bf16 model, batch 1, a 512-token prompt
prefilled as one ubatch, then 128 greedy decode steps (f16 KV cache, n_ctx
4096).  One timed "step" is that whole job: clear the cache, prefill,
decode 128 tokens with on-device greedy picks.  Weights, prompt and KV cache
live in HBM before timing starts.

Prints one JSON line on stdout: whole-job tokens/s plus prefill / decode
rates, the roofline of the dominant decode kernel (bf16 gate|up matvec)
timed with HIP events inside the library, the prefill GEMM's MFMA
fraction, and the CPU oracle timed on a bounded sample of the same job.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILES = {
    "decode.ffn_gate_up": os.path.join(ROOT, "profiles", "decode_ffn_gate_up_8b_bf16_traffic.txt"),
    "decode.attention": os.path.join(ROOT, "profiles", "decode_attention_8b_16seq_32k_traffic.txt"),
    "prefill.ffn_gate_up": os.path.join(ROOT, "profiles", "prefill_ffn_gate_up_8b_bf16_traffic.txt"),
}
KERNEL_SRC = os.path.join(ROOT, "llama_decode_ubatch_amd", "csrc", "kernels.hip")


def measured_traffic(kernel_class):
    """HBM bytes per launch of the roofline kernel from the committed
    rocprofv3 counter summary, if kernels.hip is unchanged since then."""
    import hashlib
    try:
        lines = dict(l.split(":", 1) for l in open(TRAFFIC_FILES[kernel_class]).read().splitlines() if ":" in l)
        src_hash = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]
        if lines.get("kernels_hip_sha256_16", "").strip() != src_hash:
            return None
        return int(float(lines["hbm_bytes_per_launch"].strip()))
    except Exception:
        return None
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def run_job(ctx, w, prompt, first_tokens=None):
    """One pass of the workload.  Returns (t_prefill_s, t_decode_s, ids)."""
    import numpy as np
    if w.kv_prefill:
        for s in range(w.n_seqs):          # back to the pre-filled state
            ctx.seq_rm(s, w.kv_prefill, -1)
    else:
        ctx.seq_rm(-1, -1, -1)
    ids = []
    t0 = time.perf_counter()
    if w.n_prompt:
        assert ctx.decode(prompt) == 0
        tok = ctx.greedy(-1)            # synchronises
    else:
        tok = first_tokens
    t1 = time.perf_counter()
    ids.append(tok)
    for _ in range(w.n_decode):
        if w.n_seqs == 1:
            assert ctx.decode([tok]) == 0
            tok = ctx.greedy(-1)
        else:
            assert ctx.decode(tok, seq_id=np.arange(w.n_seqs), logits=np.ones(w.n_seqs)) == 0
            tok = ctx.greedy_all()
        ids.append(tok)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1, ids


def fill_kv(torch, ctx, w):
    """Pre-fill every sequence's KV stream with the seeded f16 values,
    generated on the device, before any timing."""
    import numpy as np
    from workloads import device as wdev
    P, L, ne = w.kv_prefill, w.model.n_layer, w.model.n_embd_kv
    t0 = time.perf_counter()
    for s in range(w.n_seqs):
        kv = [[wdev.fill_kv_block(torch, w, s, il, which,
                                  torch.empty((P, ne), dtype=torch.int16, device="cuda:0"))
               for il in range(L)] for which in (0, 1)]
        torch.cuda.synchronize()
        assert ctx.kv_fill(s, P, kv[0], kv[1], "f16") == 0
        del kv
    torch.cuda.empty_cache()
    log(f"KV pre-filled: {w.n_seqs} x {P} positions in {time.perf_counter() - t0:.1f}s")


def cpu_baseline(w, sample_layers=2, n_prefill=32, n_decode=2):
    """The oracle as it stands on a bounded sample of the same job: a
    `sample_layers`-layer model of the same shape (its own seeded weights),
    prefill of n_prefill tokens and n_decode single-token decodes; layer
    time is scaled to the full depth and the output head added once."""
    import dataclasses
    import numpy as np
    from oracle import OracleModel, OracleContext, Batch
    from workloads import gen_tensor, gen_tensor_rows, prompt_tokens
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count()
    shape = dataclasses.replace(w.model, n_layer=sample_layers)
    om = OracleModel(shape, lambda name: gen_tensor(shape, name), dtype=np.float32, cache=True,
                     rows_fn=lambda name, rows: gen_tensor_rows(shape, name, rows))
    ctx = OracleContext(om, w.n_ctx, w.n_batch, w.n_ubatch, w.n_seq_max, w.type_k, w.type_v)
    # generate and upcast every weight before timing
    for il in range(sample_layers):
        for t in ("attn_norm", "attn_q", "attn_k", "attn_v", "attn_output", "ffn_norm",
                  "ffn_gate", "ffn_up", "ffn_down"):
            om.w(f"blk.{il}.{t}.weight")
    om.w("output_norm.weight")
    om.w("output.weight")
    L = w.model.n_layer
    if w.kv_prefill:
        return _cpu_baseline_prefilled(w, om, ctx, shape, sample_layers, n_decode, blas_threads)
    prompt = prompt_tokens(w, 0)[:n_prefill]
    h = np.zeros((1, shape.n_embd), np.float32)
    t0 = time.perf_counter()
    ctx.head(h)
    t_head = time.perf_counter() - t0
    t0 = time.perf_counter()
    assert ctx.decode(Batch(prompt)) == 0
    t_pp = time.perf_counter() - t0
    tok = ctx.greedy(-1)
    t0 = time.perf_counter()
    for _ in range(n_decode):
        assert ctx.decode(Batch([tok])) == 0
        tok = ctx.greedy(-1)
    t_tg = (time.perf_counter() - t0) / n_decode
    pp_full = (t_pp - t_head) * L / sample_layers + t_head
    tg_full = (t_tg - t_head) * L / sample_layers + t_head
    job_s = pp_full * w.n_prompt / n_prefill + tg_full * w.n_decode
    return {
        "value": (w.n_prompt + w.n_decode) / job_s,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "prefill_tok_s": n_prefill / pp_full,
        "decode_tok_s": 1.0 / tg_full,
        "sample": (f"oracle (NumPy float32) on a {sample_layers}-layer model of the same shape: "
                   f"{n_prefill}-token prefill + {n_decode} decodes, layer time x{L}/{sample_layers} "
                   f"plus the output head, job = {w.n_prompt}-token prefill + {w.n_decode} decodes"),
        "host_cpus": os.cpu_count(),
    }


def _cpu_baseline_prefilled(w, om, ctx, shape, sample_layers, n_decode, blas_threads):
    """Pre-filled KV workload: the sample model's layers hold every
    sequence's pre-filled KV; n_decode steps of one token per sequence."""
    import numpy as np
    from oracle import Batch
    from workloads import kv_prefill_block, prompt_tokens
    for s in range(w.n_seqs):
        K = [kv_prefill_block(w, s, il, 0).view(np.float16) for il in range(sample_layers)]
        V = [kv_prefill_block(w, s, il, 1).view(np.float16) for il in range(sample_layers)]
        assert ctx.kv_fill(s, w.kv_prefill, K, V)
    seqs = np.arange(w.n_seqs)
    tok = np.array([prompt_tokens(w, s, 1)[0] for s in seqs])
    t0 = time.perf_counter()
    ctx.head(np.zeros((w.n_seqs, shape.n_embd), np.float32))
    t_head = time.perf_counter() - t0
    t0 = time.perf_counter()
    for _ in range(n_decode):
        assert ctx.decode(Batch(tok, seq_id=seqs, logits=np.ones(w.n_seqs, np.int8))) == 0
        tok = np.array([int(np.argmax(ctx.logits_ith(i))) for i in range(w.n_seqs)])
    t_tg = (time.perf_counter() - t0) / n_decode
    L = w.model.n_layer
    step_full = (t_tg - t_head) * L / sample_layers + t_head
    return {
        "value": w.n_seqs / step_full,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "decode_tok_s": w.n_seqs / step_full,
        "sample": (f"oracle (NumPy float32) on a {sample_layers}-layer model of the same shape with "
                   f"{w.n_seqs} sequences x {w.kv_prefill} pre-filled f16 KV positions: {n_decode} "
                   f"decode steps of {w.n_seqs} tokens, layer time x{L}/{sample_layers} plus the output head"),
        "host_cpus": os.cpu_count(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--kv-type", choices=["f16", "q8_0"], default=None,
                    help="override the workload's KV cache type (q8_0: 34 bytes per 32 values)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy 256 MiB device-to-device (reference dispatch for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from llama_decode_ubatch_amd import Model, Context
    from workloads import WORKLOADS, prompt_tokens
    from workloads import device as wdev

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = WORKLOADS[args.config]
    if args.kv_type:
        import dataclasses
        w = dataclasses.replace(w, type_k=args.kv_type, type_v=args.kv_type)
    shape = w.model
    t0 = time.perf_counter()
    if shape.wtype == "f32":
        from workloads import gen_tensor, tensor_specs
        tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    else:
        tens = wdev.model_tensors(torch, shape, "cuda:0")
        torch.cuda.synchronize()
    model = Model(shape, tens, device=0)
    del tens
    torch.cuda.empty_cache()
    log(f"model {shape.tag}: {model.size() / 2**30:.2f} GiB on device, built in {time.perf_counter() - t0:.1f}s")
    ctx = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, n_seq_max=w.n_seq_max,
                  type_k=w.type_k, type_v=w.type_v, kv_unified=w.kv_unified)
    prompt = prompt_tokens(w, 0) if w.n_prompt else None
    first = None
    if w.kv_prefill:
        fill_kv(torch, ctx, w)
        first = np.array([prompt_tokens(w, s, 1)[0] for s in range(w.n_seqs)], np.int32)
    # the kernel whose roofline is reported: the FFN gate|up matvec when the
    # weights dominate, the attention when the KV cache does
    hot = "decode.attention" if w.kv_prefill else "decode.ffn_gate_up"

    for i in range(args.warmup):
        tp, td, _ = run_job(ctx, w, prompt, first)
        log(f"warmup {i}: prefill {tp * 1e3:.1f} ms, decode {td * 1e3:.1f} ms")

    # HIP events only around the two roofline kernels inside the timed region
    ctx.kernel_timing([hot, "prefill.ffn_gate_up"])
    ctx.kernel_stats()                   # reset
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    tp_sum = td_sum = 0.0
    for i in range(args.steps):
        tp, td, ids = run_job(ctx, w, prompt, first)
        tp_sum += tp
        td_sum += td
        log(f"step {i}: prefill {tp * 1e3:.1f} ms, decode {td * 1e3:.1f} ms")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    stats = ctx.kernel_stats()
    # per-class breakdown from one more (untimed) job with events on every class
    ctx.kernel_timing(None)
    run_job(ctx, w, prompt, first)
    breakdown = ctx.kernel_stats()
    ctx.kernel_timing([])

    n_tok = (w.n_prompt + w.n_decode * w.n_seqs) * args.steps
    value = n_tok / elapsed
    prefill_tps = w.n_prompt * args.steps / tp_sum if w.n_prompt else None
    decode_tps = w.n_decode * w.n_seqs * args.steps / td_sum

    d, F, V = shape.n_embd, shape.n_ff, shape.n_vocab
    wbytes = {"f32": 4, "bf16": 2, "q8_0": 34 / 32}[shape.wtype]
    kernels = {k: {"launches": n, "avg_us": 1e3 * ms / n} for k, (n, ms) in stats.items()}
    per_class = {k: {"launches": n, "avg_us": 1e3 * ms / n} for k, (n, ms) in breakdown.items()}
    log("per-class breakdown of one job (events on every launch):")
    for k, v in sorted(per_class.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["launches"]):
        log(f"  {k:22s} {v['launches']:6d} launches  avg {v['avg_us']:9.2f} us  "
            f"total {v['avg_us'] * v['launches'] / 1e3:9.2f} ms")
    roofline = None
    if hot == "decode.attention" and hot in kernels:
        # every launch reads each sequence's K and V rows (f16) once; the
        # cache grows by one cell per sequence per step
        kvb = {"f16": 2.0, "f32": 4.0, "q8_0": 34 / 32}[w.type_k]
        cells = w.n_seqs * (w.kv_prefill + (w.n_decode + 1) / 2.0)
        alg = 2 * cells * shape.n_embd_kv * kvb + 2 * w.n_seqs * d * 4
        avg_s = kernels[hot]["avg_us"] * 1e-6
        ach = alg / avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(hot) if w.type_k == "f16" else None,
                    "kernel": "decode.attention (attn_mfma_kernel split-K + attn_merge_kernel)",
                    "bytes_per_launch": int(alg)}
    elif "decode.ffn_gate_up" in kernels:
        T = w.n_seqs
        alg = 2 * F * d * wbytes + T * d * 4 + T * F * 4     # weights + input + output
        avg_s = kernels["decode.ffn_gate_up"]["avg_us"] * 1e-6
        ach = alg / avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4),
                    # the committed counter summary covers the bf16 configuration
                    "traffic": measured_traffic(hot) if shape.wtype == "bf16" and w.n_seqs == 1 else None,
                    "kernel": "decode.ffn_gate_up (linear_ldsx_kernel, fused RMSNorm, SwiGLU epilogue)",
                    "bytes_per_launch": int(alg)}
    roofline_prefill = None
    if "prefill.ffn_gate_up" in kernels and w.n_prompt:
        flops = 2.0 * w.n_prompt * 2 * F * d
        avg_s = kernels["prefill.ffn_gate_up"]["avg_us"] * 1e-6
        ach = flops / avg_s / 1e12
        roofline_prefill = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                            "kernel": "prefill.ffn_gate_up (gemm_lds_kernel, SwiGLU epilogue)",
                            "flops_per_launch": flops,
                            "traffic": measured_traffic("prefill.ffn_gate_up")
                            if shape.wtype == "bf16" and w.n_prompt == 512 else None}

    cpu = None
    if not args.no_cpu_baseline and shape.wtype != "f32":
        try:
            cpu = cpu_baseline(w)
            log(f"cpu baseline: {cpu}")
        except Exception as e:  # report, do not fail the GPU measurement
            log(f"cpu baseline failed: {e!r}")

    out = {
        "metric": "decode & prefill tokens/s, 8B-shape bf16, 1 MI355X; % of HBM / MFMA roofline",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.wtype,
        "data": "synthetic (seeded counter-based generator; random weights, uniform token ids)",
        "config": {"workload": w.name, "n_prompt": w.n_prompt, "n_decode": w.n_decode,
                   "n_seqs": w.n_seqs, "n_ctx": w.n_ctx, "n_ubatch": w.n_ubatch,
                   "kv_type": w.type_k, "parallelism": "single-gpu"},
        "prefill_tok_s": None if prefill_tps is None else round(prefill_tps, 1),
        "decode_tok_s": round(decode_tps, 2),
        "roofline": roofline,
        "roofline_prefill": roofline_prefill,
        "cpu_baseline": cpu,
        "kernels_one_job": {k: {"launches": v["launches"], "avg_us": round(v["avg_us"], 2)}
                            for k, v in per_class.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
