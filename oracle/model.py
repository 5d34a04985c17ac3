"""Plain CPU forward of a Llama-architecture decoder over ubatches with a KV
cache, plus the logits readout and the greedy pick.  Oracle - test
infrastructure only.

The layer follows the per-layer graph outline on the engine page ("llama.cpp
AI LLM Engine - how it works", Step 13b: input norm -> attention with Q, K, V,
RoPE on Q and K, scores Q x K^T, causal mask, softmax, weighted sum with V,
output projection -> residual -> norm -> feed-forward -> residual; after the
last layer keep only the rows that asked for output, final norm, output
matrix) and the node list of one decode step on the "llama.cpp Architecture"
page (Example 4: GET_ROWS, RMS_NORM, MUL, MUL_MAT, ROPE, SET_ROWS,
attention, ADD, SWIGLU).  KV handling follows the engine page's KV-cache
section: the new token's K and V are appended first, then Q attends to every
cached key of its (first) sequence, its own included.

Precision: the arrays are float64 for the tiny model and float32 for the
8B shape (the pages' graph computes every node in f32).
Stored K/V are rounded to type_k / type_v.
"""
from typing import Callable, Dict, Mapping, Optional, Union

import numpy as np

from . import numerics as nm
from .planner import (Batch, KVMemory, Plan, UBatch, plan_batch,
                      rollback_ubatch, context_geometry, RC_OK, RC_ABORTED,
                      RC_COMPUTE, RC_INVALID)


def tensor_to_float(t: dict, dtype) -> np.ndarray:
    """Dequantise / upcast one stored tensor to ``dtype``."""
    if t["type"] == "f32":
        return np.asarray(t["data"]).astype(dtype)
    if t["type"] == "bf16":
        return nm.bf16_bits_to_f32(np.asarray(t["data"])).astype(dtype)
    if t["type"] == "q8_0":
        return nm.q8_0_dequant(np.asarray(t["q"]), np.asarray(t["scale"])).astype(dtype)
    raise ValueError(t["type"])


class OracleModel:
    """Weights of one model.

    ``tensors`` maps GGUF tensor names to stored tensors ({"type": "f32",
    "data"} | {"type": "bf16", "data": uint16 bits} | {"type": "q8_0", "q",
    "scale"}), or is a callable name -> stored tensor for lazy generation.
    ``rows_fn(name, rows)``, if given, returns selected rows of a stored
    matrix (used for the embedding gather so the table is never expanded).
    A mapping without "output.weight" is a tied model (engine page, Step 6:
    the output tensor is optional and then duplicates token_embd); for a
    callable, ``tied`` says so.
    """

    def __init__(self, shape, tensors: Union[Mapping[str, dict], Callable],
                 dtype=np.float64, cache: bool = True,
                 rows_fn: Optional[Callable] = None, tied: Optional[bool] = None):
        self.hp = shape
        self.dtype = dtype
        self._get = tensors if callable(tensors) else tensors.__getitem__
        if tied is None:
            tied = not callable(tensors) and "output.weight" not in tensors
        self.tied = bool(tied)
        self.output_name = "token_embd.weight" if self.tied else "output.weight"
        self._rows = rows_fn
        self._cache_on = cache
        self._cache: Dict[str, np.ndarray] = {}

    def w(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        a = tensor_to_float(self._get(name), self.dtype)
        if self._cache_on:
            self._cache[name] = a
        return a

    def drop_cache(self):
        self._cache.clear()

    def embed(self, tokens: np.ndarray) -> np.ndarray:
        """GET_ROWS(token_embd, tokens) with dequantisation of the rows read
        (engine page, "Tokens to embeddings"; architecture page, Example 4)."""
        name = "token_embd.weight"
        if name in self._cache:
            return self._cache[name][tokens]
        if self._rows is not None:
            return tensor_to_float(self._rows(name, np.asarray(tokens)), self.dtype)
        t = self._get(name)
        if t["type"] == "q8_0":
            sub = {"type": "q8_0", "q": t["q"][tokens], "scale": t["scale"][tokens]}
        else:
            sub = {"type": t["type"], "data": np.asarray(t["data"])[tokens]}
        return tensor_to_float(sub, self.dtype)


class OracleContext:
    """A context: cparams, KV cells and per-layer K/V storage, outputs."""

    def __init__(self, model: OracleModel, n_ctx: int, n_batch: int = 2048,
                 n_ubatch: int = 512, n_seq_max: int = 1, type_k: str = "f16",
                 type_v: str = "f16", kv_unified: bool = False):
        hp = model.hp
        self.model = model
        self.n_seq_max = max(1, n_seq_max)
        self.n_ctx, self.n_stream, self.n_cells = context_geometry(
            n_ctx or hp.n_ctx_train, self.n_seq_max, kv_unified)
        # causal model: n_batch is clamped to n_ctx, n_ubatch to n_batch
        self.n_batch = min(self.n_ctx, n_batch)
        self.n_ubatch = min(self.n_batch, n_ubatch or self.n_batch)
        self.type_k, self.type_v = type_k, type_v
        self.mem = KVMemory(self.n_stream, self.n_cells, kv_unified, self.n_seq_max)
        self._kv: Dict[tuple, tuple] = {}      # (layer, stream) -> (K, V)
        self.logits: Optional[np.ndarray] = None
        self.out_row: Optional[np.ndarray] = None
        self.n_outputs = 0
        self.last_plan: Optional[Plan] = None
        self.last_defrag_src = None    # per stream: new cell j <- old cell src[j]
        self.record = None   # optional dict collecting per-layer residuals

    # ------------------------------------------------------------ storage
    def kv(self, layer: int, stream: int):
        key = (layer, stream)
        if key not in self._kv:
            ne = self.model.hp.n_embd_kv
            self._kv[key] = (
                np.zeros((self.n_cells, ne), nm.kv_storage_dtype(self.type_k)),
                np.zeros((self.n_cells, ne), nm.kv_storage_dtype(self.type_v)))
        return self._kv[key]

    def kv_fill(self, seq: int, n_pos: int, k_layers, v_layers) -> bool:
        """Pre-fill positions 0..n_pos-1 of an empty sequence with given K/V
        rows (stored type values, [n_pos][n_embd_kv] per layer)."""
        cells = self.mem.fill_sequence(seq, n_pos)
        if cells is None:
            return False
        st = self.mem.stream_of(seq)
        for il in range(self.model.hp.n_layer):
            K, V = self.kv(il, st)
            K[cells] = np.asarray(k_layers[il]).astype(K.dtype)
            V[cells] = np.asarray(v_layers[il]).astype(V.dtype)
        return True

    # ------------------------------------------------------------ API
    def seq_pos_max(self, s):
        return self.mem.seq_pos_max(s)

    def seq_pos_min(self, s):
        return self.mem.seq_pos_min(s)

    def seq_rm(self, s, p0, p1):
        return self.mem.seq_rm(s, p0, p1)

    def seq_cp(self, src, dst, p0, p1):
        """Between streams the K/V rows of the whole stream go along."""
        ss, sd = self.mem.stream_of(src), self.mem.stream_of(dst)
        if not self.mem.seq_cp(src, dst, p0, p1):
            return False
        if ss != sd:
            for il in range(self.model.hp.n_layer):
                K, V = self.kv(il, ss)
                self._kv[(il, sd)] = (K.copy(), V.copy())
        return True

    def seq_keep(self, s):
        return self.mem.seq_keep(s)

    def _move_cells(self, src):
        self.last_defrag_src = src
        for st, order in enumerate(src):
            for il in range(self.model.hp.n_layer):
                if (il, st) in self._kv:
                    K, V = self._kv[(il, st)]
                    K[:order.size] = K[order].copy()
                    V[:order.size] = V[order].copy()

    def defrag(self):
        """Compact the cells of every stream and move their K/V rows along;
        returns the number of cells whose index changed."""
        src = self.mem.defrag()
        self._move_cells(src)
        return int(sum(int(np.count_nonzero(o != np.arange(o.size))) for o in src))

    def decode(self, batch: Batch, abort_at: Optional[int] = None,
               fail_at: Optional[int] = None) -> int:
        """One ``llama_decode`` call (engine page, Steps 11-12).  ``abort_at``
        / ``fail_at`` force the abort / compute-failure path at that ubatch
        index (test hooks)."""
        hp = self.model.hp
        plan = plan_batch(batch, self.mem, hp.n_vocab, self.n_seq_max,
                          self.n_batch, self.n_ubatch)
        self.last_plan = plan
        self.logits, self.out_row, self.n_outputs = None, None, 0
        if plan.rc != RC_OK:
            return plan.rc
        logits = np.zeros((plan.n_outputs, hp.n_vocab), self.model.dtype)
        for k, (ub, cells) in enumerate(zip(plan.ubatches, plan.cells)):
            self.mem.apply(ub, cells)          # commit before compute
            if k == abort_at or k == fail_at:
                rollback_ubatch(self.mem, ub)
                return RC_ABORTED if k == abort_at else RC_COMPUTE
            z = self.forward_ubatch(ub, cells)
            rows = plan.out_row[ub.idx[ub.output]]
            logits[rows] = z
        self.logits, self.out_row, self.n_outputs = logits, plan.out_row, plan.n_outputs
        return RC_OK

    def logits_ith(self, i: int) -> Optional[np.ndarray]:
        """Row for batch index i (i >= 0), or the i-th row from the end
        (i < 0); None if that token asked for no output (engine page,
        Step 14)."""
        if self.logits is None:
            return None
        if i < 0:
            r = self.n_outputs + i
            return self.logits[r] if 0 <= r < self.n_outputs else None
        if i >= self.out_row.size or self.out_row[i] < 0:
            return None
        return self.logits[self.out_row[i]]

    def greedy(self, i: int) -> int:
        """Most likely token; the lowest id wins a tie (reading)."""
        z = self.logits_ith(i)
        return -1 if z is None else int(np.argmax(z))

    # ------------------------------------------------------------ forward
    def forward_ubatch(self, ub: UBatch, cells: np.ndarray) -> np.ndarray:
        """Logits [n_output_tokens_of_ubatch, n_vocab] for one committed
        ubatch; the ubatch's K/V go into ``cells`` of every layer."""
        m, hp = self.model, self.model.hp
        x = m.embed(ub.token)
        if self.record is not None:
            self.record.setdefault("x", []).append(x.copy())
        for il in range(hp.n_layer):
            x = self.layer_forward(il, x, ub, cells)
            if self.record is not None:
                self.record["x"].append(x.copy())
        return self.head(x[ub.output])

    def head(self, x_out: np.ndarray) -> np.ndarray:
        """Final norm of the output rows, then the output matrix."""
        m, hp = self.model, self.model.hp
        h = nm.rms_norm(x_out, m.w("output_norm.weight"), hp.rms_eps)
        return h @ m.w(m.output_name).T

    def layer_forward(self, il: int, x: np.ndarray, ub: UBatch,
                      cells: np.ndarray) -> np.ndarray:
        m, hp = self.model, self.model.hp
        T, H, Hk, hd, g = ub.n_tokens, hp.n_head, hp.n_head_kv, hp.head_dim, hp.n_gqa
        p = f"blk.{il}."
        xn = nm.rms_norm(x, m.w(p + "attn_norm.weight"), hp.rms_eps)
        q = (xn @ m.w(p + "attn_q.weight").T).reshape(T, H, hd)
        k = (xn @ m.w(p + "attn_k.weight").T).reshape(T, Hk, hd)
        v = xn @ m.w(p + "attn_v.weight").T
        q = nm.rope_normal(q, ub.pos, hp.rope_base)
        k = nm.rope_normal(k, ub.pos, hp.rope_base).reshape(T, Hk * hd)
        # append every token's K/V before any attention
        streams = np.array([self.mem.stream_of(int(s)) for s in ub.seq])
        for t in range(T):
            K, V = self.kv(il, int(streams[t]))
            K[cells[t]] = nm.round_to_kv_type(k[t], self.type_k)
            V[cells[t]] = nm.round_to_kv_type(v[t], self.type_v)
        attn = np.zeros((T, H, hd), x.dtype)
        scale = 1.0 / np.sqrt(hd)
        cache = {}
        for t in range(T):
            st = int(streams[t])
            if st not in cache:
                nkv = self.mem.n_kv(st)
                K, V = self.kv(il, st)
                cache[st] = (nkv, K[:nkv].astype(x.dtype), V[:nkv].astype(x.dtype))
            nkv, Kf, Vf = cache[st]
            # the cells of the token's first sequence, up to its position
            vis = self.mem.has[st, :nkv, ub.seq[t]] & (self.mem.pos[st, :nkv] <= ub.pos[t])
            for gi in range(Hk):
                hs = slice(gi * g, (gi + 1) * g)
                cs = slice(gi * hd, (gi + 1) * hd)
                attn[t, hs], _ = nm.attention_heads(q[t, hs], Kf[:, cs], Vf[:, cs], vis, scale)
        x = x + attn.reshape(T, H * hd) @ m.w(p + "attn_output.weight").T
        xn = nm.rms_norm(x, m.w(p + "ffn_norm.weight"), hp.rms_eps)
        u = nm.swiglu(xn @ m.w(p + "ffn_gate.weight").T, xn @ m.w(p + "ffn_up.weight").T)
        return x + u @ m.w(p + "ffn_down.weight").T
