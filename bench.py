"""Throughput of the decode step on one MI355X.

Headline workload: the 8B-shaped bf16 model, batch 1, a 512-token prompt
prefilled as one ubatch, then 128 greedy decode steps (f16 KV cache, n_ctx
4096).  One timed "step" is that whole job: clear the cache, prefill,
decode 128 tokens with on-device greedy picks.  Weights, prompt and KV cache
live in HBM before timing starts, and nothing else is recorded while the
steps run.

The same run then measures, outside the timed region:
  * kernel durations from HIP events tied to the kernel dispatches (the
    first kernel of a launch records its start, the last its end, as a
    kernel trace does) on every kernel class over one extra job
    (`kernels_one_job`; the roofline kernels' figures in `roofline`,
    `roofline_prefill` come from it);
  * end-to-end fractions: decode tok/s x algorithmic bytes per token against
    8 TB/s of HBM, prefill FLOPs / prefill time against 2.5 PFLOP/s bf16;
  * compact summaries of the 16-sequence 32K-cell decode (`config4`, same
    bf16 weights) and of the q8_0 model (`config5`);
  * the CPU oracle on a bounded sample of the headline job (`cpu_baseline`).

Prints one JSON line on stdout.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
TRAFFIC_FILES = {
    "decode.ffn_gate_up": os.path.join(ROOT, "profiles", "decode_ffn_gate_up_8b_bf16_traffic.txt"),
    "decode.attention": os.path.join(ROOT, "profiles", "decode_attention_8b_16seq_32k_traffic.txt"),
    "prefill.ffn_gate_up": os.path.join(ROOT, "profiles", "prefill_ffn_gate_up_8b_bf16_traffic.txt"),
}
KERNEL_SRC = os.path.join(ROOT, "llama_decode_ubatch_amd", "csrc", "kernels.hip")
# committed kernel-trace summaries (rocprofv3 --kernel-trace --stats of this
# script) and the roofline kernels' names in them
TRACE_FILES = {
    ("decode.ffn_gate_up", "bf16"): (os.path.join(ROOT, "profiles", "decode_prefill_8b_bf16_kernel_stats.md"),
                                     ("linear_ldsx_kernel<2, 2, 4, true>",)),
    ("prefill.ffn_gate_up", "bf16"): (os.path.join(ROOT, "profiles", "decode_prefill_8b_bf16_kernel_stats.md"),
                                      ("gemm_wide_kernel<2, 1, 2, 4, 4>",)),
    # split pass + combine pass, as the events span both
    ("decode.attention", "bf16"): (os.path.join(ROOT, "profiles", "decode_8b_16seq_32k_kernel_stats.md"),
                                   ("attn_mfma_kernel<128, true, false, 1, true>", "attn_merge_kernel<128>")),
    ("decode.ffn_gate_up", "q8_0"): (os.path.join(ROOT, "profiles", "decode_prefill_8b_q8_0_kernel_stats.md"),
                                     ("linear_ldsx_kernel<3, 2, 4, true>",)),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _src_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def traced_avg_us(kernel_class, wtype):
    """Average dispatch duration of a roofline kernel in the committed
    rocprofv3 kernel trace, if kernels.hip is unchanged since then."""
    try:
        path, names = TRACE_FILES[(kernel_class, wtype)]
        text = open(path).read()
        if f"sha256 prefix {_src_hash()}" not in text:
            return None
        avg = {}
        for line in text.splitlines():
            for name in names:
                if line.startswith(f"| `{name}` |"):
                    avg[name] = float(line.split("|")[3])
        return round(sum(avg.values()), 2) if len(avg) == len(names) else None
    except Exception:
        return None


def measured_traffic(kernel_class):
    """HBM bytes per launch of a roofline kernel from the committed
    rocprofv3 counter summary, if kernels.hip is unchanged since then."""
    try:
        lines = dict(l.split(":", 1) for l in open(TRAFFIC_FILES[kernel_class]).read().splitlines() if ":" in l)
        if lines.get("kernels_hip_sha256_16", "").strip() != _src_hash():
            return None
        return int(float(lines["hbm_bytes_per_launch"].strip()))
    except Exception:
        return None


# ------------------------------------------------------------ algorithmic work
def weight_bytes_per_elem(shape):
    return {"f32": 4.0, "bf16": 2.0, "q8_0": 34.0 / 32.0}[shape.wtype]


def kv_bytes_per_elem(t):
    return {"f32": 4.0, "f16": 2.0, "q8_0": 34.0 / 32.0}[t]


def layer_params(shape):
    d, hd, F = shape.n_embd, shape.head_dim, shape.n_ff
    return d * (shape.n_head + 2 * shape.n_head_kv) * hd + shape.n_head * hd * d + 3 * F * d


def decode_bytes_per_step(w):
    """Bytes one decode step must move: every layer matrix and the output
    matrix once, each sequence's visible K and V cells (the average over the
    workload's steps), the embedding rows gathered and the logits rows
    written."""
    s = w.model
    wb = weight_bytes_per_elem(s)
    weights = (s.n_layer * layer_params(s) + s.n_vocab * s.n_embd) * wb
    cells_avg = (w.kv_prefill or w.n_prompt) + (w.n_decode + 1) / 2.0
    kv = w.n_seqs * cells_avg * 2 * s.n_layer * s.n_embd_kv * kv_bytes_per_elem(w.type_k)
    rows = w.n_seqs * (s.n_embd * wb + s.n_vocab * 4)
    return weights + kv + rows


def prefill_flops(w):
    """Matrix products over T prompt tokens, causal attention (query i sees
    i cells) and the logits of the one output row."""
    s = w.model
    T = w.n_prompt
    lin = 2.0 * s.n_layer * layer_params(s) * T
    attn = 4.0 * s.n_head * s.head_dim * (T * (T + 1) / 2.0) * s.n_layer
    return lin + attn + 2.0 * s.n_vocab * s.n_embd


# ------------------------------------------------------------------- the job
def run_job(ctx, w, prompt, first_tokens=None, chain=True):
    """One pass of the workload.  Returns (t_prefill_s, t_decode_s, ids).
    One sequence: the greedy steps run as one chain (ubd_greedy_chain: each
    pick goes from the argmax kernel straight into the next step's token
    table, the same picks as decode + greedy step by step), or with
    chain=False as ubd_decode + ubd_sample_greedy per step; several
    sequences: one decode of a token per sequence, then the greedy picks,
    per step."""
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
    if w.n_seqs == 1 and chain:
        picks = ctx.greedy_chain(tok, w.n_decode)
        assert picks.size == w.n_decode
        ids.extend(int(t) for t in picks)
    elif w.n_seqs == 1:
        for _ in range(w.n_decode):
            assert ctx.decode([tok]) == 0
            tok = ctx.greedy(-1)
            ids.append(tok)
    else:
        for _ in range(w.n_decode):
            assert ctx.decode(tok, seq_id=np.arange(w.n_seqs), logits=np.ones(w.n_seqs)) == 0
            tok = ctx.greedy_all()
            ids.append(tok)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1, ids


def fill_kv(torch, ctx, w):
    """Pre-fill every sequence's KV stream with the seeded f16 values,
    generated on the device, before any timing."""
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


def build_model(torch, shape):
    from llama_decode_ubatch_amd import Model
    from workloads import device as wdev
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
    return model


def measure(torch, model, w, steps, warmup):
    """Times `steps` whole jobs of workload w with nothing else recorded,
    then runs one job with HIP events on every kernel class (the roofline
    kernels among them)."""
    import numpy as np
    from llama_decode_ubatch_amd import Context
    from workloads import prompt_tokens
    ctx = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, n_seq_max=w.n_seq_max,
                  type_k=w.type_k, type_v=w.type_v, kv_unified=w.kv_unified)
    prompt = prompt_tokens(w, 0) if w.n_prompt else None
    first = None
    if w.kv_prefill:
        fill_kv(torch, ctx, w)
        first = np.array([prompt_tokens(w, s, 1)[0] for s in range(w.n_seqs)], np.int32)
    for i in range(warmup):
        tp, td, _ = run_job(ctx, w, prompt, first)
        log(f"[{w.name}] warmup {i}: prefill {tp * 1e3:.1f} ms, decode {td * 1e3:.1f} ms")

    ctx.kernel_timing([])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    tp_sum = td_sum = 0.0
    for i in range(steps):
        tp, td, _ = run_job(ctx, w, prompt, first)
        tp_sum += tp
        td_sum += td
        log(f"[{w.name}] step {i}: prefill {tp * 1e3:.1f} ms, decode {td * 1e3:.1f} ms")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    # kernel durations outside the timed region: one job with events on
    # every kernel class (the roofline kernels included)
    ctx.kernel_timing(None)
    ctx.kernel_stats()
    run_job(ctx, w, prompt, first)
    per_class = {k: {"launches": n, "avg_us": 1e3 * ms / n} for k, (n, ms) in ctx.kernel_stats().items()}
    ctx.kernel_timing([])
    # one sequence: the same decode steps once more with the host picking each
    # token (ubd_decode + ubd_sample_greedy per step), for comparison
    td_steps, same_ids = None, None
    if w.n_seqs == 1 and w.n_decode:
        _, _, ids_chain = run_job(ctx, w, prompt, first)
        _, td_steps, ids_steps = run_job(ctx, w, prompt, first, chain=False)
        same_ids = ids_chain == ids_steps
        log(f"[{w.name}] decode step by step (host picks): {w.n_decode / td_steps:.1f} tok/s, "
            f"ids equal to the chain's: {same_ids}")
    ctx.free()
    log(f"[{w.name}] per-class breakdown of one job (kernel execution, events on every launch):")
    for k, v in sorted(per_class.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["launches"]):
        log(f"  {k:22s} {v['launches']:6d} launches  avg {v['avg_us']:9.2f} us  "
            f"total {v['avg_us'] * v['launches'] / 1e3:9.2f} ms")

    n_tok = (w.n_prompt + w.n_decode * w.n_seqs) * steps
    r = {
        "value": n_tok / elapsed,
        "ms_per_step": 1e3 * elapsed / steps,
        "prefill_tok_s": w.n_prompt * steps / tp_sum if w.n_prompt else None,
        "decode_tok_s": w.n_decode * w.n_seqs * steps / td_sum,
        "per_class": per_class,
    }
    if td_steps:
        r["decode_step_by_step"] = {"tok_s": round(w.n_decode / td_steps, 2), "ids_equal": same_ids,
                                    "loop": "ubd_decode + ubd_sample_greedy per step, one job after the timed region"}
    # end-to-end fractions of the rooflines
    step_bytes = decode_bytes_per_step(w)
    r["e2e"] = {
        "decode_bytes_per_token": round(step_bytes / w.n_seqs),
        "decode_hbm_frac": round(r["decode_tok_s"] / w.n_seqs * step_bytes / (HBM_PEAK_GBS * 1e9), 4),
    }
    if w.n_prompt:
        fl = prefill_flops(w)
        r["e2e"]["prefill_flops"] = fl
        r["e2e"]["prefill_mfma_frac"] = round(fl * r["prefill_tok_s"] / w.n_prompt / (BF16_PEAK_TFLOPS * 1e12), 4)
    return r


def roofline_of(w, r):
    """The dominant decode kernel against HBM: the gate|up product when the
    weights dominate, the split attention when the KV cache does."""
    shape = w.model
    d, F = shape.n_embd, shape.n_ff
    hot = "decode.attention" if w.kv_prefill else "decode.ffn_gate_up"
    if hot not in r["per_class"]:
        return None
    avg_s = r["per_class"][hot]["avg_us"] * 1e-6
    if hot == "decode.attention":
        # each launch reads every sequence's visible K and V cells once; the
        # cache grows by one cell per sequence per step
        cells = w.n_seqs * (w.kv_prefill + (w.n_decode + 1) / 2.0)
        alg = 2 * cells * shape.n_embd_kv * kv_bytes_per_elem(w.type_k) + 2 * w.n_seqs * d * 4
        kernel = ("decode.attention (attn_mfma_kernel split over cells, K/V loaded non-temporally, + attn_merge_kernel), "
                  "per layer-step")
        traffic = measured_traffic(hot) if w.type_k == "f16" else None
    else:
        T = w.n_seqs
        alg = 2 * F * d * weight_bytes_per_elem(shape) + T * d * 4 + T * F * 4   # weights + input + output
        kernel = "decode.ffn_gate_up (linear_ldsx_kernel, fused RMSNorm, SwiGLU epilogue)"
        traffic = measured_traffic(hot) if shape.wtype == "bf16" and T == 1 else None
    ach = alg / avg_s / 1e9
    out = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
           "bytes_per_launch": int(alg), "avg_us": round(r["per_class"][hot]["avg_us"], 2),
           "timing": "HIP events tied to the kernel dispatches (start of the first kernel to end of the last), "
                     "one job after the timed region with every kernel class timed"}
    tr = traced_avg_us(hot, shape.wtype)
    if tr:
        out["trace_avg_us"] = tr
        out["trace_frac"] = round(alg / (tr * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    return out


def roofline_prefill_of(w, r):
    if "prefill.ffn_gate_up" not in r["per_class"] or not w.n_prompt:
        return None
    shape = w.model
    flops = 2.0 * w.n_prompt * 2 * shape.n_ff * shape.n_embd
    avg_us = r["per_class"]["prefill.ffn_gate_up"]["avg_us"]
    ach = flops / (avg_us * 1e-6) / 1e12
    out = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(ach / BF16_PEAK_TFLOPS, 4),
           "kernel": "prefill.ffn_gate_up (gemm_wide_kernel 256 x 128 tiles, SwiGLU epilogue; the method's FLOPs, the activations' "
                     "hi and lo planes make twice that of matrix-core work)",
           "flops_per_launch": flops, "avg_us": round(avg_us, 2),
           "traffic": measured_traffic("prefill.ffn_gate_up")
           if shape.wtype == "bf16" and w.n_prompt == 512 else None,
           "timing": "HIP events tied to the kernel dispatches (start of the first kernel to end of the last), "
                     "one job after the timed region with every kernel class timed"}
    tr = traced_avg_us("prefill.ffn_gate_up", shape.wtype)
    if tr:
        out["trace_avg_us"] = tr
        out["trace_frac"] = round(flops / (tr * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
    return out


# -------------------------------------------------------------- CPU baseline
def cpu_baseline(w, sample_layers=8, n_decode=None):
    """The oracle as it stands on a bounded sample of the same job: a
    `sample_layers`-layer model of the same shape (its own seeded weights)
    prefills the whole prompt as one ubatch (so the causal attention costs
    what it costs in the full job) and then decodes n_decode tokens (default:
    the job's decode count, so the scans cover the same context lengths);
    layer time is scaled to the full depth and the output head added once
    per output row."""
    import numpy as np
    from oracle import OracleModel, OracleContext, Batch
    from workloads import gen_tensor, gen_tensor_rows, prompt_tokens
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    try:
        import psutil
        physical = psutil.cpu_count(logical=False)
    except Exception:
        physical = None
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
    n_decode = w.n_decode if n_decode is None else n_decode
    prompt = prompt_tokens(w, 0)
    t0 = time.perf_counter()
    ctx.head(np.zeros((1, shape.n_embd), np.float32))
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
    job_s = pp_full + tg_full * w.n_decode
    return {
        "value": round((w.n_prompt + w.n_decode) / job_s, 3),
        "unit": "tokens/s",
        "cores": blas_threads,
        "kind": "oracle",
        "prefill_tok_s": round(w.n_prompt / pp_full, 2),
        "decode_tok_s": round(1.0 / tg_full, 3),
        "sample": (f"oracle (NumPy float32 BLAS) on a {sample_layers}-layer model of the same shape: the whole "
                   f"{w.n_prompt}-token prompt as one ubatch + {n_decode} decodes after it; layer time "
                   f"x{L}/{sample_layers} plus the output head; job = {w.n_prompt}-token prefill + "
                   f"{w.n_decode} decodes"),
        "physical_cores": physical,
        "logical_cpus": os.cpu_count(),
        "cpus_allowed": len(os.sched_getaffinity(0)),
        "sample_seconds": round(t_pp + n_decode * t_tg, 1),
    }


def summary(w, r):
    s = {"workload": w.name, "value": round(r["value"], 2), "unit": "tokens/s",
         "ms_per_step": round(r["ms_per_step"], 3),
         "decode_tok_s": round(r["decode_tok_s"], 2), "e2e": r["e2e"],
         **({"decode_step_by_step": r["decode_step_by_step"]} if "decode_step_by_step" in r else {}),
         "roofline": roofline_of(w, r)}
    if r["prefill_tok_s"] is not None:
        s["prefill_tok_s"] = round(r["prefill_tok_s"], 1)
    s["kernels_one_job"] = {k: {"launches": v["launches"], "avg_us": round(v["avg_us"], 2)}
                            for k, v in r["per_class"].items()}
    return s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--configs", type=int, nargs="+", default=[3, 4, 5],
                    help="workloads to measure; the first is the headline (default 3 4 5)")
    ap.add_argument("--kv-type", choices=["f16", "q8_0"], default=None,
                    help="override the workloads' KV cache type (q8_0: 34 bytes per 32 values)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy 256 MiB device-to-device (reference dispatch for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def workload(c):
        w = WORKLOADS[c]
        return dataclasses.replace(w, type_k=args.kv_type, type_v=args.kv_type) if args.kv_type else w

    results = {}
    model, model_tag = None, None
    for c in args.configs:
        w = workload(c)
        if model_tag != w.model.tag:
            if model is not None:
                model.free()
                torch.cuda.empty_cache()
            model, model_tag = build_model(torch, w.model), w.model.tag
        results[c] = measure(torch, model, w, args.steps, args.warmup)
    model.free()
    torch.cuda.empty_cache()

    head = args.configs[0]
    w, r = workload(head), results[head]
    cpu = None
    if not args.no_cpu_baseline and w.model.wtype != "f32" and not w.kv_prefill:
        try:
            cpu = cpu_baseline(w)
            log(f"cpu baseline: {cpu}")
        except Exception as e:  # report, do not fail the GPU measurement
            log(f"cpu baseline failed: {e!r}")

    out = {
        "metric": "decode & prefill tokens/s, 8B-shape bf16, 1 MI355X; % of HBM / MFMA roofline",
        "value": round(r["value"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.model.wtype,
        "data": "synthetic (seeded counter-based generator; random weights, uniform token ids)",
        "config": {"workload": w.name, "n_prompt": w.n_prompt, "n_decode": w.n_decode,
                   "n_seqs": w.n_seqs, "n_ctx": w.n_ctx, "n_ubatch": w.n_ubatch,
                   "kv_type": w.type_k, "parallelism": "single-gpu",
                   "decode_loop": "greedy chain (ubd_greedy_chain)" if w.n_seqs == 1
                   else "decode + greedy of every sequence per step"},
        "prefill_tok_s": None if r["prefill_tok_s"] is None else round(r["prefill_tok_s"], 1),
        "decode_tok_s": round(r["decode_tok_s"], 2),
        "decode_step_by_step": r.get("decode_step_by_step"),
        "e2e": r["e2e"],
        "roofline": roofline_of(w, r),
        "roofline_prefill": roofline_prefill_of(w, r),
        "cpu_baseline": cpu,
        "kernels_one_job": {k: {"launches": v["launches"], "avg_us": round(v["avg_us"], 2)}
                            for k, v in r["per_class"].items()},
    }
    for c in args.configs[1:]:
        out[f"config{c}"] = summary(workload(c), results[c])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
