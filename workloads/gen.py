"""Counter-based generator for every synthetic input (host side).

Every value is a pure function of (key, element index), so any slice of any
tensor - one layer, a few rows of the output matrix, one sequence's KV block -
can be regenerated on its own, and the device-side twin in
``workloads/synth.hip`` produces bit-identical values.

Definition (published generator, restated):
  * ``mix64`` is the output finaliser of SplitMix64 (G. Steele, D. Lea,
    C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
    the constants are D. Stafford's "Mix13" variant that SplitMix64 uses).
  * The SplitMix64 stream of a 64-bit state ``key`` is
    ``h(i) = mix64(key + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64)``; element ``i``
    of a tensor takes ``h(i)``.
  * Keys are chained: ``derive(a, b, ...) = mix64(... mix64(SEED + (a+1)*G) ...)``.
  * Normal draws use the top 16 bits of ``h(i)`` as an index into a 65536-entry
    table of the normal quantiles ``Phi^-1((j + 0.5) / 65536)``, scaled and
    rounded to the storage type on the host once; a value is then a table
    lookup on either side (exact).  This is a 16-bit discretised normal.
  * Uniform integers use ``(h(i) >> 32) mod n``.

Seed 1 follows the pages' ``--seed 1`` runs (architecture page, Example 4).
"""
import os
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache

import numpy as np

from .configs import ModelShape, Workload, tensor_specs, TensorSpec

SEED = 1
GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

# key domains
_DOM_TENSOR, _DOM_PROMPT, _DOM_KV = 1, 2, 3
# sub-streams of a tensor
SUB_VALUES, SUB_SCALES = 0, 1
# q8_0 scale grid: m * 2^-19 for m in [263, 263 + 786), all exact in f16
Q8_SCALE_M0, Q8_SCALE_NM, Q8_SCALE_EXP = 263, 786, -19
Q8_BLOCK = 32


def _mix64_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (returns a new array)."""
    z = z ^ (z >> np.uint64(30))
    z *= np.uint64(_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(_M2)
    z ^= z >> np.uint64(31)
    return z


def derive(*ids: int) -> int:
    k = SEED
    for v in ids:
        k = _mix64_int(k + GOLDEN * (int(v) + 1))
    return k


def tensor_key(model: ModelShape, index: int, sub: int) -> int:
    return derive(_DOM_TENSOR, model.model_id, index, sub)


def prompt_key(w: Workload, seq: int) -> int:
    return derive(_DOM_PROMPT, w.cfg_id, seq)


def kv_key(w: Workload, seq: int, layer: int, which: int) -> int:
    """which: 0 = K, 1 = V."""
    return derive(_DOM_KV, w.cfg_id, seq, layer, which)


def hashes(key: int, idx: np.ndarray) -> np.ndarray:
    """h(i) for an array of element indices (int64/uint64)."""
    z = idx.astype(np.uint64) + np.uint64(1)
    z *= np.uint64(GOLDEN)
    z += np.uint64(key)
    return mix64(z)


def _hash_range(key: int, start: int, count: int) -> np.ndarray:
    return hashes(key, np.arange(start, start + count, dtype=np.uint64))


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        n = min(16, os.cpu_count() or 1)
        _POOL = ThreadPoolExecutor(max_workers=n)
    return _POOL


def _fill_parallel(out: np.ndarray, fn, chunk=1 << 21):
    """out.flat[s:s+n] = fn(s, n) over chunks, in threads (NumPy releases the
    GIL inside its ufunc loops)."""
    flat = out.reshape(-1)
    n = flat.size
    if n <= chunk:
        flat[:] = fn(0, n)
        return out
    starts = list(range(0, n, chunk))

    def work(s):
        c = min(chunk, n - s)
        flat[s:s + c] = fn(s, c)

    list(_pool().map(work, starts))
    return out


# ---------------------------------------------------------------- tables
@lru_cache(maxsize=None)
def _quantiles() -> np.ndarray:
    from scipy.special import ndtri
    return ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


@lru_cache(maxsize=None)
def normal_table_f32(sigma: float) -> np.ndarray:
    t = (sigma * _quantiles()).astype(np.float32)
    t.setflags(write=False)
    return t


@lru_cache(maxsize=None)
def normal_table_bf16(sigma: float) -> np.ndarray:
    t = _f32_to_bf16_bits(normal_table_f32(sigma))
    t.setflags(write=False)
    return t


@lru_cache(maxsize=None)
def gain_table_f32() -> np.ndarray:
    """Norm gains 1 + 0.02 * N(0, 1)."""
    t = (1.0 + 0.02 * _quantiles()).astype(np.float32)
    t.setflags(write=False)
    return t


@lru_cache(maxsize=None)
def kv_table_f16() -> np.ndarray:
    """N(0, 1) rounded to bf16, then to f16 (bit patterns)."""
    bf = normal_table_bf16(1.0).astype(np.uint32) << np.uint32(16)
    t = bf.view(np.float32).astype(np.float16).view(np.uint16)
    t.setflags(write=False)
    return t


# ---------------------------------------------------------------- draws
def q8_codes_from_hash(h: np.ndarray) -> np.ndarray:
    return (((h >> np.uint64(32)) % np.uint64(255)).astype(np.int16)
            - 127).astype(np.int8)


def q8_scale_bits_from_hash(h: np.ndarray) -> np.ndarray:
    m = ((h >> np.uint64(32)) % np.uint64(Q8_SCALE_NM)).astype(np.float32) \
        + np.float32(Q8_SCALE_M0)
    return (m * np.float32(2.0 ** Q8_SCALE_EXP)).astype(np.float16).view(np.uint16)


def _table_fill(key, table, out):
    def fn(s, c):
        return table[(_hash_range(key, s, c) >> np.uint64(48)).astype(np.intp)]
    return _fill_parallel(out, fn)


def _table_rows(key, table, rows, ncol):
    idx = (np.asarray(rows, dtype=np.uint64)[:, None] * np.uint64(ncol)
           + np.arange(ncol, dtype=np.uint64)[None, :])
    return table[(hashes(key, idx) >> np.uint64(48)).astype(np.intp)]


def _spec(model: ModelShape, name_or_spec) -> TensorSpec:
    if isinstance(name_or_spec, TensorSpec):
        return name_or_spec
    for s in tensor_specs(model):
        if s.name == name_or_spec:
            return s
    raise KeyError(name_or_spec)


def gen_tensor(model: ModelShape, name_or_spec, literal_gains=False) -> dict:
    """Whole tensor.  Returns a dict with "type" and the arrays:
    f32: data float32; bf16: data uint16 bit patterns; q8_0: q int8 [out][in]
    and scale uint16 f16 bit patterns [out][in/32]; gains: data float32."""
    s = _spec(model, name_or_spec)
    if s.kind == "gain":
        table = normal_table_f32(0.02) if literal_gains else gain_table_f32()
        out = np.empty(s.shape, np.float32)
        return {"type": "f32", "data": _table_fill(
            tensor_key(model, s.index, SUB_VALUES), table, out)}
    rows, cols = s.shape
    if model.wtype == "f32":
        out = np.empty(s.shape, np.float32)
        return {"type": "f32", "data": _table_fill(
            tensor_key(model, s.index, SUB_VALUES), normal_table_f32(0.02), out)}
    if model.wtype == "bf16":
        out = np.empty(s.shape, np.uint16)
        return {"type": "bf16", "data": _table_fill(
            tensor_key(model, s.index, SUB_VALUES), normal_table_bf16(0.02), out)}
    if model.wtype == "q8_0":
        kq = tensor_key(model, s.index, SUB_VALUES)
        ks = tensor_key(model, s.index, SUB_SCALES)
        q = np.empty(s.shape, np.int8)
        _fill_parallel(q, lambda st, c: q8_codes_from_hash(_hash_range(kq, st, c)))
        sc = np.empty((rows, cols // Q8_BLOCK), np.uint16)
        _fill_parallel(sc, lambda st, c: q8_scale_bits_from_hash(_hash_range(ks, st, c)))
        return {"type": "q8_0", "q": q, "scale": sc}
    raise ValueError(model.wtype)


def gen_tensor_rows(model: ModelShape, name_or_spec, rows,
                    literal_gains=False) -> dict:
    """Selected rows of a matrix (same values as the whole-tensor draw)."""
    s = _spec(model, name_or_spec)
    if s.kind == "gain":
        return gen_tensor(model, s, literal_gains)
    rows = np.asarray(rows, dtype=np.int64)
    ncol = s.shape[1]
    if model.wtype == "f32":
        return {"type": "f32", "data": _table_rows(
            tensor_key(model, s.index, SUB_VALUES), normal_table_f32(0.02), rows, ncol)}
    if model.wtype == "bf16":
        return {"type": "bf16", "data": _table_rows(
            tensor_key(model, s.index, SUB_VALUES), normal_table_bf16(0.02), rows, ncol)}
    if model.wtype == "q8_0":
        kq = tensor_key(model, s.index, SUB_VALUES)
        ks = tensor_key(model, s.index, SUB_SCALES)
        nb = ncol // Q8_BLOCK
        iq = rows.astype(np.uint64)[:, None] * np.uint64(ncol) + np.arange(ncol, dtype=np.uint64)[None, :]
        isc = rows.astype(np.uint64)[:, None] * np.uint64(nb) + np.arange(nb, dtype=np.uint64)[None, :]
        return {"type": "q8_0", "q": q8_codes_from_hash(hashes(kq, iq)),
                "scale": q8_scale_bits_from_hash(hashes(ks, isc))}
    raise ValueError(model.wtype)


def prompt_tokens(w: Workload, seq: int, n: int = None) -> np.ndarray:
    """Uniform token ids over [0, n_vocab) for one sequence."""
    n = w.n_prompt if n is None else n
    h = _hash_range(prompt_key(w, seq), 0, n)
    return ((h >> np.uint64(32)) % np.uint64(w.model.n_vocab)).astype(np.int32)


def kv_prefill_block(w: Workload, seq: int, layer: int, which: int,
                     p0: int = 0, n: int = None) -> np.ndarray:
    """f16 bit patterns [n][n_head_kv * head_dim] for positions p0..p0+n of one
    sequence; element (p, j) takes index p * n_embd_kv + j."""
    n = w.kv_prefill - p0 if n is None else n
    ne = w.model.n_embd_kv
    out = np.empty((n, ne), np.uint16)
    key = kv_key(w, seq, layer, which)
    table = kv_table_f16()
    base = p0 * ne

    def fn(s, c):
        return table[(_hash_range(key, base + s, c) >> np.uint64(48)).astype(np.intp)]
    return _fill_parallel(out, fn)
