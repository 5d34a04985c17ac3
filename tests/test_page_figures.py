"""Model geometry checked against the figures the architecture page prints
for its tiny model (tests/golden/tiny_model_figures.json).  These pin tensor
shapes, parameter counts, KV / output buffer sizes and the 34-byte q8_0
block, i.e. the sizes the oracle and the library are built on (CPU only)."""
import json
import os

import pytest

from workloads import MODELS, WORKLOADS, tensor_specs
from oracle.planner import context_geometry

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_model_figures.json")))
TINY = MODELS["tiny-f32"]
MIB = 1024 * 1024


def q8_0_bytes(n_values):
    assert n_values % 32 == 0
    return n_values // 32 * G["ex2_q8_0_block_bytes"]


def test_hparams_and_derived():
    assert (TINY.n_embd, TINY.n_layer, TINY.n_head, TINY.n_head_kv, TINY.n_ff, TINY.n_vocab) == (
        G["ex8_n_embd"], G["ex8_n_layer"], G["ex8_n_head"], G["ex8_n_head_kv"], G["ex8_n_ff"], G["ex8_n_vocab"])
    assert TINY.head_dim == G["ex8_n_embd_head_k"]
    assert TINY.n_gqa == G["ex8_n_gqa"]
    assert TINY.n_embd_kv == G["ex8_n_embd_k_gqa"]


def test_param_counts():
    specs = tensor_specs(TINY)
    assert len(specs) == G["ex8_tensor_count"]
    assert round(TINY.n_params() / 1e6, 2) == G["ex8_model_params_M"]
    per_layer = sum(s.shape[0] * (s.shape[1] if len(s.shape) > 1 else 1)
                    for s in specs if s.name.startswith("blk.0."))
    assert per_layer == G["ex13_params_per_layer"]


def test_bytes_and_flops_per_token():
    specs = {s.name: s for s in tensor_specs(TINY)}
    out = specs["output.weight"].shape[0] * specs["output.weight"].shape[1]
    layers = TINY.n_layer * G["ex13_params_per_layer"] + TINY.n_embd
    assert round((out + layers) * 4 / 1e6, 1) == G["ex13_weights_read_per_generated_token_MB"]
    assert round(2 * layers / 1e6, 2) == G["ex13_flops_per_prompt_token_M"]


def test_node_shapes():
    specs = {s.name: s for s in tensor_specs(TINY)}
    for name, ne in G["ex4_shapes_ggml"].items():
        if name in specs:
            # ggml {K, M} is M rows of K values: our [out][in] reversed
            assert list(reversed(specs[name].shape)) == ne, name
    assert [TINY.head_dim, TINY.n_head] == G["ex4_shapes_ggml"]["Qcur_heads"]
    assert [TINY.n_embd_kv, 256] == G["ex4_shapes_ggml"]["cache_k_l0_at_c256"]
    assert [TINY.head_dim, 256, TINY.n_head_kv] == G["ex4_shapes_ggml"]["flash_attn_k_view"]


def test_kv_and_output_buffer_sizes():
    n_ctx, n_stream, cells = context_geometry(G["ex10_kv_cells"], 1, False)
    k_f16 = TINY.n_layer * TINY.n_embd_kv * cells * 2
    assert round(k_f16 / MIB, 2) == G["ex10_k_f16_MiB"] == G["ex10_v_f16_MiB"]
    assert round(TINY.n_layer * q8_0_bytes(TINY.n_embd_kv * cells) / MIB, 2) == G["ex10_k_q8_0_MiB"]
    from oracle.numerics import kv_cache_bytes
    assert kv_cache_bytes(TINY.n_layer, TINY.n_embd_kv, cells, "f16") == k_f16
    assert round(kv_cache_bytes(TINY.n_layer, TINY.n_embd_kv, cells, "q8_0") / MIB, 2) == G["ex10_k_q8_0_MiB"]
    assert round(TINY.n_vocab * 4 / MIB, 2) == G["ex10_output_row_MiB"]
    for ub, mib in G["ex10_logits_full_ubatch_MiB"].items():
        assert round(int(ub) * TINY.n_vocab * 4 / MIB, 2) == mib


def test_q8_0_tensor_bytes():
    rows, cols = 704, 256          # ffn_gate {256, 704}
    b = G["ex2_ffn_gate_bytes"]
    assert rows * cols * 4 == b["f32"] and rows * cols * 2 == b["f16"]
    assert q8_0_bytes(cols) == G["ex2_ffn_gate_row_bytes_q8_0"]
    assert rows * q8_0_bytes(cols) == b["q8_0"]


def test_workload_context_geometry():
    # per-sequence cell counts the five workloads rely on
    expect = {1: 512, 2: 256, 3: 4096, 4: 32768, 5: 4096}
    for cid, cells in expect.items():
        w = WORKLOADS[cid]
        assert context_geometry(w.n_ctx, w.n_seq_max, w.kv_unified)[2] == cells
    assert WORKLOADS[4].kv_prefill + WORKLOADS[4].n_decode == 32768
