"""GGUF files of the synthetic models (input generation only).

Writes the layout the loading pages describe ("llama.cpp AI LLM Engine - how
it works", "GGUF format" reference and Step 4; the loading page's
header-parsing and split-file stages): magic, version, tensor count, key
count, the key/value pairs, the tensor records (name, dimensions, element
type, offset into the data block), then the data block.  The pages give no
numeric codes or alignment; the ones used here are those of the public GGUF
specification, so real files and these share a layout:

  value types  0 u8, 1 i8, 2 u16, 3 i16, 4 u32, 5 i32, 6 f32, 7 bool,
               8 string, 9 array, 10 u64, 11 i64, 12 f64
  tensor types 0 F32, 1 F16, 8 Q8_0 (blocks of one f16 scale + 32 int8
               codes, 34 bytes), 30 BF16
  strings      u64 byte length, then the bytes (no terminator)
  alignment    general.alignment (u32) or 32; the data block starts at the
               first aligned offset after the records, every tensor at an
               aligned offset inside it

Nothing here reads files: the oracle's reader (oracle/gguf.py) and the
library's reader parse them independently.
"""
import struct
from typing import List, Sequence, Tuple

import numpy as np

from .configs import ModelShape, tensor_specs
from .gen import gen_tensor

U8, I8, U16, I16, U32, I32, F32, BOOL, STR, ARR, U64, I64, F64 = range(13)
T_F32, T_F16, T_Q8_0, T_BF16 = 0, 1, 8, 30

_SCALAR = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f",
           BOOL: "<?", U64: "<Q", I64: "<q", F64: "<d"}


def _str(s) -> bytes:
    b = s.encode() if isinstance(s, str) else bytes(s)
    return struct.pack("<Q", len(b)) + b


def _value(vtype: int, v) -> bytes:
    if vtype == STR:
        return _str(v)
    if vtype == ARR:
        etype, items = v
        out = struct.pack("<IQ", etype, len(items))
        return out + b"".join(_value(etype, x) for x in items)
    return struct.pack(_SCALAR[vtype], v)


def write_gguf(path: str, kvs: Sequence[Tuple[str, int, object]],
               tensors: Sequence[Tuple[str, int, Sequence[int], bytes]],
               version: int = 3, alignment: int = 32, magic: bytes = b"GGUF") -> None:
    """kvs: (key, value type, value); an array value is (element type, list).
    tensors: (name, tensor type, dims with dims[0] innermost, raw bytes)."""
    head = magic + struct.pack("<IQQ", version, len(tensors), len(kvs))
    for key, vtype, v in kvs:
        head += _str(key) + struct.pack("<I", vtype) + _value(vtype, v)
    offs, off = [], 0
    for _, _, _, raw in tensors:
        offs.append(off)
        off = (off + len(raw) + alignment - 1) // alignment * alignment
    for (name, ttype, dims, _), o in zip(tensors, offs):
        head += _str(name) + struct.pack("<I", len(dims))
        head += b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", ttype, o)
    pad = (-len(head)) % alignment
    with open(path, "wb") as f:
        f.write(head + b"\0" * pad)
        for (_, _, _, raw), o in zip(tensors, offs):
            f.write(raw)
            f.write(b"\0" * ((-len(raw)) % alignment))


def q8_0_blocks(q: np.ndarray, scale_bits: np.ndarray) -> bytes:
    """Interleave int8 codes [rows][K] and f16 scale bits [rows][K/32] into
    34-byte blocks, row by row."""
    rows, K = q.shape
    blk = np.empty((rows, K // 32, 34), np.uint8)
    blk[:, :, :2] = np.ascontiguousarray(scale_bits, np.uint16).reshape(rows, K // 32, 1).view(np.uint8)
    blk[:, :, 2:] = q.reshape(rows, K // 32, 32).view(np.uint8)
    return blk.tobytes()


def tensor_record(name: str, t: dict) -> Tuple[str, int, List[int], bytes]:
    """A generated tensor ({"type": ...} as gen_tensor returns) as a GGUF
    record: matrices [out][in] get dims (in, out); gains (n,)."""
    if t["type"] == "q8_0":
        q = np.asarray(t["q"])
        return name, T_Q8_0, [q.shape[1], q.shape[0]], q8_0_blocks(q, np.asarray(t["scale"]))
    a = np.asarray(t["data"])
    ttype = {"f32": T_F32, "bf16": T_BF16, "f16": T_F16}[t["type"]]
    if ttype == T_F32:
        a = a.astype(np.float32)
    dims = list(a.shape[::-1])
    return name, ttype, dims, np.ascontiguousarray(a).tobytes()


def model_kvs(m: ModelShape, extra=()) -> List[Tuple[str, int, object]]:
    """Architecture and hyperparameter keys of a llama model (engine page,
    Step 4 key list; architecture page, Example 8 metadata listing)."""
    kv = [
        ("general.architecture", STR, "llama"),
        ("general.name", STR, m.tag),
        ("llama.context_length", U32, m.n_ctx_train),
        ("llama.embedding_length", U32, m.n_embd),
        ("llama.block_count", U32, m.n_layer),
        ("llama.feed_forward_length", U32, m.n_ff),
        ("llama.attention.head_count", U32, m.n_head),
        ("llama.attention.head_count_kv", U32, m.n_head_kv),
        ("llama.rope.freq_base", F32, float(m.rope_base)),
        ("llama.attention.layer_norm_rms_epsilon", F32, float(m.rms_eps)),
        ("general.alignment", U32, 32),
        # keys the loader does not need: skipped by name
        ("tokenizer.ggml.model", STR, "synthetic"),
        ("tokenizer.ggml.scores", ARR, (F32, [0.0, -1.5, 2.25])),
        ("tokenizer.ggml.tokens", ARR, (STR, ["<s>", "</s>", "a"])),
    ]
    return kv + list(extra)


def write_model_gguf(m: ModelShape, path_prefix: str, n_split: int = 1,
                     tensors: dict = None, tied: bool = False) -> List[str]:
    """Write the synthetic model as one GGUF file (``<prefix>.gguf``) or as
    n_split files ``<prefix>-0000k-of-0000n.gguf`` (the loading page's
    split stage: every part is a whole GGUF file; the first holds the model
    keys, every part holds split.no / split.count / split.tensors.count).
    ``tied`` leaves output.weight out (a model whose output matrix is its
    token embedding).  Returns the paths, first part first."""
    recs = []
    for s in tensor_specs(m):
        if tied and s.name == "output.weight":
            continue
        t = tensors[s.name] if tensors is not None else gen_tensor(m, s)
        recs.append(tensor_record(s.name, t))
    if n_split == 1:
        path = f"{path_prefix}.gguf"
        write_gguf(path, model_kvs(m), recs)
        return [path]
    parts = np.array_split(np.arange(len(recs)), n_split)
    paths = []
    for k, idx in enumerate(parts):
        path = f"{path_prefix}-{k + 1:05d}-of-{n_split:05d}.gguf"
        split = [("split.no", U16, k), ("split.count", U16, n_split), ("split.tensors.count", I32, len(recs))]
        write_gguf(path, (model_kvs(m) if k == 0 else []) + split, [recs[i] for i in idx])
        paths.append(path)
    return paths
