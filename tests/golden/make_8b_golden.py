"""Write the oracle's end-to-end results for the 8B-shaped workloads.

Runs only oracle/ (NumPy, float32 with exactly upcast / dequantised
weights) on the seeded synthetic inputs of workloads/ and stores, per
workload, the greedy token sequence and, for every step, the top-64 logits
and the logits at 4096 fixed vocabulary indices.  The GPU tests teacher-force
these tokens and compare.  No value here comes from the GPU path.

    python tests/golden/make_8b_golden.py [--configs 3 5 4]

By default every step of each workload is recorded: the prefill logits and
all 128 (512-token prompt) or 256 (256-token prompt) decode steps, and four
of the sixteen pre-filled sequences over all 64 steps.  Needs about 40 GB of
host memory and a few hours of CPU time.
"""
import argparse
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import OracleModel, OracleContext, Batch  # noqa: E402
from workloads import (WORKLOADS, gen_tensor, gen_tensor_rows, prompt_tokens,  # noqa: E402
                       kv_prefill_block)

OUT_DIR = os.path.dirname(os.path.abspath(__file__))
N_SAMPLE = 4096
TOPK = 64
MULTI_SEQS = (0, 5, 9, 15)


def sample_indices(n_vocab):
    return np.random.default_rng(12345).choice(n_vocab, N_SAMPLE, replace=False).astype(np.int64)


def record(z, idx):
    top = np.argsort(-z, kind="stable")[:TOPK]
    return top.astype(np.int32), z[top].astype(np.float32), z[idx].astype(np.float32), np.float32(np.abs(z).max())


def model_for(w):
    return OracleModel(w.model, lambda n: gen_tensor(w.model, n), dtype=np.float32, cache=True,
                       rows_fn=lambda n, r: gen_tensor_rows(w.model, n, r))


def run_single(cfg, steps, log):
    w = WORKLOADS[cfg]
    om = model_for(w)
    ctx = OracleContext(om, w.n_ctx, w.n_batch, w.n_ubatch, w.n_seq_max, w.type_k, w.type_v)
    idx = sample_indices(w.model.n_vocab)
    prompt = prompt_tokens(w, 0)
    t0 = time.time()
    assert ctx.decode(Batch(prompt)) == 0
    log(f"config {cfg}: prefill {prompt.size} tokens in {time.time() - t0:.0f}s")
    toks, tops, topv, samp, zmax = [], [], [], [], []
    for step in range(steps + 1):
        z = ctx.logits_ith(-1)
        a, b, c, m = record(z, idx)
        tok = int(np.argmax(z))
        toks.append(tok); tops.append(a); topv.append(b); samp.append(c); zmax.append(m)
        if step == steps:
            break
        t0 = time.time()
        assert ctx.decode(Batch([tok])) == 0
        log(f"  step {step}: token {tok} ({time.time() - t0:.1f}s)")
    np.savez_compressed(os.path.join(OUT_DIR, f"oracle_cfg{cfg}.npz"), prompt=prompt, tokens=np.array(toks),
                        top_ids=np.array(tops), top_vals=np.array(topv), sample_idx=idx,
                        sample_vals=np.array(samp), zmax=np.array(zmax))
    om.drop_cache()


def run_multi(cfg, steps, seqs, log):
    """Workload with pre-filled KV: each sequence is independent (own KV
    stream), so the oracle runs one sequence at a time."""
    w = WORKLOADS[cfg]
    om = model_for(w)
    idx = sample_indices(w.model.n_vocab)
    first = np.array([prompt_tokens(w, s, 1)[0] for s in range(w.n_seqs)])
    res = {}
    for s in seqs:
        ctx = OracleContext(om, w.n_ctx, w.n_batch, w.n_ubatch, w.n_seq_max, w.type_k, w.type_v)
        t0 = time.time()
        K = [kv_prefill_block(w, s, il, 0).view(np.float16) for il in range(w.model.n_layer)]
        V = [kv_prefill_block(w, s, il, 1).view(np.float16) for il in range(w.model.n_layer)]
        assert ctx.kv_fill(s, w.kv_prefill, K, V)
        del K, V
        log(f"config {cfg} seq {s}: KV pre-filled in {time.time() - t0:.0f}s")
        tok = int(first[s])
        toks, tops, topv, samp, zmax = [tok], [], [], [], []
        for step in range(steps):
            t0 = time.time()
            assert ctx.decode(Batch([tok], seq_id=[s])) == 0
            z = ctx.logits_ith(-1)
            a, b, c, m = record(z, idx)
            tok = int(np.argmax(z))
            toks.append(tok); tops.append(a); topv.append(b); samp.append(c); zmax.append(m)
            log(f"  seq {s} step {step}: token {tok} ({time.time() - t0:.1f}s)")
        res[s] = (toks, tops, topv, samp, zmax)
        del ctx
    np.savez_compressed(os.path.join(OUT_DIR, f"oracle_cfg{cfg}.npz"), seqs=np.array(seqs), first=first,
                        tokens=np.array([res[s][0] for s in seqs]), top_ids=np.array([res[s][1] for s in seqs]),
                        top_vals=np.array([res[s][2] for s in seqs]), sample_idx=idx,
                        sample_vals=np.array([res[s][3] for s in seqs]), zmax=np.array([res[s][4] for s in seqs]))
    om.drop_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=0, help="decode steps (0: the workload's own count)")
    ap.add_argument("--multi-steps", type=int, default=0, help="steps with pre-filled KV (0: all)")
    ap.add_argument("--configs", type=int, nargs="+", default=[3, 5, 4])
    args = ap.parse_args()

    def log(m):
        print(time.strftime("%H:%M:%S"), m, flush=True)
    for cfg in args.configs:
        w = WORKLOADS[cfg]
        if w.kv_prefill:
            run_multi(cfg, args.multi_steps or w.n_decode, list(MULTI_SEQS), log)
        else:
            run_single(cfg, args.steps or w.n_decode, log)


if __name__ == "__main__":
    main()
