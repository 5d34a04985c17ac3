"""GGUF reader (test infrastructure: the CPU oracle).

Follows the file layout the pages describe ("llama.cpp AI LLM Engine - how
it works", "GGUF format" reference: magic "GGUF", format version, tensor
count, key count, then key/value pairs - name, value type, value; arrays
carry element type and count first - then per tensor its name, number of
dimensions (at most four) and sizes, element type and offset from the start
of the data block after the metadata; the version must be the current one,
3, else the file is rejected; a repeated tensor name makes the model
invalid), with the numeric codes and the alignment rule of the public GGUF
specification, which the pages leave out:

  value types  0 u8, 1 i8, 2 u16, 3 i16, 4 u32, 5 i32, 6 f32, 7 bool,
               8 string, 9 array, 10 u64, 11 i64, 12 f64
  tensor types 0 F32 (4 bytes), 1 F16 (2), 30 BF16 (2), 8 Q8_0 (34-byte
               blocks of 32 values: f16 scale, then 32 int8 codes)
  alignment    general.alignment (u32), default 32: the data block starts
               at the first multiple after the records; offsets are
               multiples of it.
A dimension must be a positive size (reading: the pages give sizes only).

``model_info`` restates the architecture page's Example 8 summary: the
parameter count from the tensor shapes, bits per weight = file bits over
parameters, and the file type named after the most common tensor type.
"""
import struct
from collections import Counter
from typing import Dict, List, Tuple

import numpy as np

VERSION = 3
_SCALAR = {0: ("<B", 1), 1: ("<b", 1), 2: ("<H", 2), 3: ("<h", 2), 4: ("<I", 4), 5: ("<i", 4),
           6: ("<f", 4), 7: ("<?", 1), 10: ("<Q", 8), 11: ("<q", 8), 12: ("<d", 8)}
STR, ARR = 8, 9
# tensor type -> (values per block, bytes per block, name)
TYPES = {0: (1, 4, "F32"), 1: (1, 2, "F16"), 30: (1, 2, "BF16"), 8: (32, 34, "Q8_0")}


class GGUFError(ValueError):
    pass


class _Cursor:
    def __init__(self, buf: bytes):
        self.buf, self.at = buf, 0

    def take(self, n: int) -> bytes:
        if n < 0 or self.at + n > len(self.buf):
            raise GGUFError("truncated file")
        b = self.buf[self.at:self.at + n]
        self.at += n
        return b

    def unpack(self, fmt: str, n: int):
        return struct.unpack(fmt, self.take(n))[0]

    def string(self) -> str:
        n = self.unpack("<Q", 8)
        return self.take(n).decode("utf-8", errors="surrogateescape")

    def value(self, vtype: int):
        if vtype in _SCALAR:
            return self.unpack(*_SCALAR[vtype])
        if vtype == STR:
            return self.string()
        if vtype == ARR:
            etype = self.unpack("<I", 4)
            n = self.unpack("<Q", 8)
            if etype not in _SCALAR and etype not in (STR, ARR):
                raise GGUFError(f"unknown array element type {etype}")
            if etype in _SCALAR and n * _SCALAR[etype][1] > len(self.buf) - self.at:
                raise GGUFError("truncated file")
            return etype, [self.value(etype) for _ in range(n)]
        raise GGUFError(f"unknown value type {vtype}")


class GGUF:
    """Parsed header, metadata and tensor records of one file; tensor data
    are read on request."""

    def __init__(self, path: str):
        self.path = path
        with open(path, "rb") as f:
            self.raw = f.read()
        c = _Cursor(self.raw)
        if c.take(4) != b"GGUF":
            raise GGUFError("not a GGUF file")
        self.version = c.unpack("<I", 4)
        if self.version != VERSION:
            raise GGUFError(f"unsupported GGUF version {self.version}")
        n_tensors = c.unpack("<Q", 8)
        n_kv = c.unpack("<Q", 8)
        self.kv: Dict[str, Tuple[int, object]] = {}
        self.keys: List[str] = []
        for _ in range(n_kv):
            key = c.string()
            vtype = c.unpack("<I", 4)
            if key in self.kv:
                raise GGUFError(f"duplicate key {key}")
            self.kv[key] = (vtype, c.value(vtype))
            self.keys.append(key)
        self.alignment = self.get("general.alignment", 32)
        if self.alignment <= 0 or self.alignment & (self.alignment - 1):
            raise GGUFError("alignment must be a power of two")
        self.tensors: List[dict] = []
        names = set()
        for _ in range(n_tensors):
            name = c.string()
            n_dims = c.unpack("<I", 4)
            if not 1 <= n_dims <= 4:
                raise GGUFError(f"tensor {name}: {n_dims} dimensions")
            dims = [c.unpack("<Q", 8) for _ in range(n_dims)]
            if min(dims) < 1 or max(dims) >= 2 ** 63:
                raise GGUFError(f"tensor {name}: bad dimensions")
            ttype = c.unpack("<I", 4)
            offset = c.unpack("<Q", 8)
            if name in names:
                raise GGUFError(f"tensor {name} is duplicated")
            names.add(name)
            if ttype not in TYPES:
                raise GGUFError(f"tensor {name}: unknown type {ttype}")
            per, size, _ = TYPES[ttype]
            n = int(np.prod(dims, dtype=object))
            if dims[0] % per:
                raise GGUFError(f"tensor {name}: rows not a whole number of blocks")
            if offset % self.alignment:
                raise GGUFError(f"tensor {name}: misaligned offset")
            self.tensors.append(dict(name=name, dims=dims, type=ttype, offset=offset,
                                     nbytes=n // per * size))
        self.data_start = (c.at + self.alignment - 1) // self.alignment * self.alignment
        for t in self.tensors:
            if self.data_start + t["offset"] + t["nbytes"] > len(self.raw):
                raise GGUFError(f"tensor {t['name']}: data past the end of the file")
        self.by_name = {t["name"]: t for t in self.tensors}

    def get(self, key: str, default=None):
        return self.kv[key][1] if key in self.kv else default

    def tensor_bytes(self, name: str) -> bytes:
        t = self.by_name[name]
        a = self.data_start + t["offset"]
        return self.raw[a:a + t["nbytes"]]

    def stored(self, name: str) -> dict:
        """The tensor in the oracle's stored form: {"type": "f32", "data"},
        {"type": "bf16", "data": uint16 bits} or {"type": "q8_0", "q",
        "scale"}; F16 becomes f32 (exactly); shapes are [dims[1]][dims[0]]
        for matrices, [dims[0]] for vectors."""
        t = self.by_name[name]
        raw = self.tensor_bytes(name)
        shape = tuple(t["dims"][::-1]) if len(t["dims"]) > 1 else (t["dims"][0],)
        if t["type"] == 0:
            return {"type": "f32", "data": np.frombuffer(raw, "<f4").reshape(shape).copy()}
        if t["type"] == 1:
            return {"type": "f32", "data": np.frombuffer(raw, "<f2").astype(np.float32).reshape(shape)}
        if t["type"] == 30:
            return {"type": "bf16", "data": np.frombuffer(raw, "<u2").reshape(shape).copy()}
        rows = int(np.prod(shape[:-1]))
        blk = np.frombuffer(raw, np.uint8).reshape(rows, shape[-1] // 32, 34)
        scale = blk[:, :, :2].copy().view("<u2").reshape(rows, shape[-1] // 32)
        q = blk[:, :, 2:].copy().view(np.int8).reshape(shape)
        return {"type": "q8_0", "q": q, "scale": scale}


def open_model(paths: List[str]) -> Tuple[GGUF, Dict[str, GGUF]]:
    """The first file and a map tensor name -> file over all parts of a
    split model (loading page, split stage: the parts' tensors go into one
    map; a name seen twice is an error)."""
    files = [GGUF(p) for p in paths]
    where: Dict[str, GGUF] = {}
    for g in files:
        for t in g.tensors:
            if t["name"] in where:
                raise GGUFError(f"tensor {t['name']} is duplicated")
            where[t["name"]] = g
    return files[0], where


def hparams(g: GGUF, where: Dict[str, GGUF]) -> dict:
    """Llama hyperparameters from the architecture-prefixed keys (engine
    page, Step 4); n_vocab from the embedding table's second dimension;
    n_head_kv defaults to n_head, the RoPE base to 10000."""
    arch = g.get("general.architecture")
    if arch != "llama":
        raise GGUFError(f"unsupported architecture {arch!r}")
    need = lambda k: g.get(f"llama.{k}") if g.get(f"llama.{k}") is not None else _missing(k)
    n_head = need("attention.head_count")
    return dict(
        n_layer=need("block_count"), n_embd=need("embedding_length"), n_head=n_head,
        n_head_kv=g.get("llama.attention.head_count_kv", n_head), n_ff=need("feed_forward_length"),
        n_vocab=where["token_embd.weight"].by_name["token_embd.weight"]["dims"][1],
        n_ctx_train=need("context_length"),
        rms_eps=need("attention.layer_norm_rms_epsilon"),
        rope_freq_base=g.get("llama.rope.freq_base", 10000.0))


def _missing(k):
    raise GGUFError(f"missing key llama.{k}")


def model_info(files: List[GGUF]) -> dict:
    """Summary lines of the architecture page's Example 8: parameter count,
    file size, bits per weight, file type."""
    n_params = sum(int(np.prod(t["dims"], dtype=object)) for g in files for t in g.tensors)
    size = sum(len(g.raw) for g in files)
    counts = Counter(t["type"] for g in files for t in g.tensors)
    top = counts.most_common(1)[0][0]
    ftype = ("all " if len(counts) == 1 else "mostly ") + TYPES[top][2]
    return dict(n_params=n_params, file_bytes=size, bpw=size * 8.0 / n_params, file_type=ftype,
                type_counts={TYPES[k][2]: v for k, v in counts.items()})
