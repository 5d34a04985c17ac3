"""Model shapes and the five workloads (sizes only; no arithmetic).

Shapes follow the tiny random Llama-architecture model that the
"llama.cpp Architecture" page (codeloopback.dev) runs throughout (Example 8:
4 layers, 256-wide embeddings, 8 query / 2 KV heads, FFN 704, 151 936-token
vocabulary, untied input/output matrices) and a Llama-3-8B-shaped model of the
same architecture.  Tensor names are the GGUF names that the per-layer tensor
loading step lists on the "llama.cpp AI LLM Engine — how it works" page
(Step 6): token_embd, output_norm, output and, per layer, attn_norm, attn_q,
attn_k, attn_v, attn_output, ffn_norm, ffn_gate, ffn_up, ffn_down.

Matrices are held as ``[rows][cols]`` = ``[out][in]``; this is ggml's
``{K, M}`` shape read as M rows of K values (Example 4 of the architecture
page).
"""
from dataclasses import dataclass, field
from typing import Dict, List, Tuple


@dataclass(frozen=True)
class ModelShape:
    tag: str
    model_id: int          # selects the generator's key space
    n_layer: int
    n_embd: int
    n_head: int
    n_head_kv: int
    n_ff: int
    n_vocab: int
    n_ctx_train: int
    rope_base: float
    rms_eps: float = 1e-5
    wtype: str = "f32"     # "f32" | "bf16" | "q8_0" for every 2-D matrix

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    @property
    def n_gqa(self) -> int:
        return self.n_head // self.n_head_kv

    @property
    def n_embd_kv(self) -> int:
        return self.head_dim * self.n_head_kv

    def n_params(self) -> int:
        return sum(int(_prod(s.shape)) for s in tensor_specs(self))


def _prod(shape):
    p = 1
    for v in shape:
        p *= v
    return p


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]   # [out][in] for matrices, [n] for norm gains
    kind: str                # "matrix" | "gain"
    index: int               # enumeration order, part of the generator key


def tensor_specs(m: ModelShape) -> List[TensorSpec]:
    """All tensors of the model in a fixed enumeration order."""
    d, hd, F, V = m.n_embd, m.head_dim, m.n_ff, m.n_vocab
    specs: List[TensorSpec] = []

    def add(name, shape, kind):
        specs.append(TensorSpec(name, tuple(shape), kind, len(specs)))

    add("token_embd.weight", (V, d), "matrix")
    for il in range(m.n_layer):
        p = f"blk.{il}."
        add(p + "attn_norm.weight", (d,), "gain")
        add(p + "attn_q.weight", (m.n_head * hd, d), "matrix")
        add(p + "attn_k.weight", (m.n_head_kv * hd, d), "matrix")
        add(p + "attn_v.weight", (m.n_head_kv * hd, d), "matrix")
        add(p + "attn_output.weight", (d, m.n_head * hd), "matrix")
        add(p + "ffn_norm.weight", (d,), "gain")
        add(p + "ffn_gate.weight", (F, d), "matrix")
        add(p + "ffn_up.weight", (F, d), "matrix")
        add(p + "ffn_down.weight", (d, F), "matrix")
    add("output_norm.weight", (d,), "gain")
    add("output.weight", (V, d), "matrix")
    return specs


MODELS: Dict[str, ModelShape] = {
    "tiny-f32": ModelShape("tiny-f32", 1, n_layer=4, n_embd=256, n_head=8,
                           n_head_kv=2, n_ff=704, n_vocab=151936,
                           n_ctx_train=4096, rope_base=10000.0, wtype="f32"),
    "8b-bf16": ModelShape("8b-bf16", 2, n_layer=32, n_embd=4096, n_head=32,
                          n_head_kv=8, n_ff=14336, n_vocab=128256,
                          n_ctx_train=131072, rope_base=500000.0,
                          wtype="bf16"),
    "8b-q8_0": ModelShape("8b-q8_0", 3, n_layer=32, n_embd=4096, n_head=32,
                          n_head_kv=8, n_ff=14336, n_vocab=128256,
                          n_ctx_train=131072, rope_base=500000.0,
                          wtype="q8_0"),
}


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    model: ModelShape
    n_ctx: int
    n_batch: int
    n_ubatch: int
    n_seq_max: int
    type_k: str
    type_v: str
    kv_unified: bool
    n_seqs: int          # sequences decoded together
    n_prompt: int        # prompt tokens per sequence (0: no prefill)
    n_decode: int        # decode calls, one new token per sequence each
    kv_prefill: int = 0  # positions pre-filled per sequence from the generator
    description: str = ""


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny-1seq-f32kv", MODELS["tiny-f32"], n_ctx=512,
                n_batch=512, n_ubatch=512, n_seq_max=1, type_k="f32",
                type_v="f32", kv_unified=False, n_seqs=1, n_prompt=32,
                n_decode=16,
                description="tiny model, one sequence, 32-token prompt then "
                            "16 greedy decode steps, f32 KV, n_ctx 512"),
    2: Workload(2, "tiny-8seq-f16kv", MODELS["tiny-f32"], n_ctx=2048,
                n_batch=1024, n_ubatch=128, n_seq_max=8, type_k="f16",
                type_v="f16", kv_unified=False, n_seqs=8, n_prompt=128,
                n_decode=32,
                description="tiny model, 8 sequences x 128-token prompts in "
                            "one 1024-token batch split into 128-token "
                            "ubatches, then 32 decode steps x 8 tokens, f16 KV"),
    3: Workload(3, "8b-bf16-pp512-tg128", MODELS["8b-bf16"], n_ctx=4096,
                n_batch=2048, n_ubatch=512, n_seq_max=1, type_k="f16",
                type_v="f16", kv_unified=False, n_seqs=1, n_prompt=512,
                n_decode=128,
                description="8B-shaped bf16 model, batch 1, 512-token prefill "
                            "then 128 greedy decode steps, f16 KV, n_ctx 4096"),
    4: Workload(4, "8b-bf16-16seq-32k", MODELS["8b-bf16"], n_ctx=16 * 32768,
                n_batch=2048, n_ubatch=512, n_seq_max=16, type_k="f16",
                type_v="f16", kv_unified=False, n_seqs=16, n_prompt=0,
                n_decode=64, kv_prefill=32704,
                description="8B-shaped bf16 model, 16 sequences with KV "
                            "pre-filled to 32704 positions of N(0,1) values, "
                            "64 decode steps x 16 tokens, n_ctx 32768 per "
                            "sequence, f16 KV"),
    5: Workload(5, "8b-q8_0-pp256-tg256", MODELS["8b-q8_0"], n_ctx=4096,
                n_batch=2048, n_ubatch=512, n_seq_max=1, type_k="f16",
                type_v="f16", kv_unified=False, n_seqs=1, n_prompt=256,
                n_decode=256,
                description="8B-shaped model with 32-element int8 blocks + "
                            "f16 scale, batch 1, 256-token prefill then 256 "
                            "greedy decode steps, f16 KV, n_ctx 4096"),
}
