"""Per-element and per-head arithmetic of the Llama layer, written out plainly.

Every routine works in the dtype of its input arrays (float64 for the tiny
model, float32 for the 8B shape) unless it says otherwise.  Oracle - test
infrastructure only.
"""
import numpy as np


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis, then the learned per-channel scale.

    "llama.cpp Architecture" page, Example 4: RMS_NORM rescales the vector to
    a standard size and the following MUL applies the learned weight
    (attn_norm / ffn_norm / output_norm).  Reading: x / sqrt(mean(x^2) + eps)
    with eps inside the root.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_normal(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding, "normal" (rope type 0) layout.

    "llama.cpp Architecture" page, Example 4 (ROPE of Qcur/Kcur by inp_pos) and
    Example 8 (rope type 0 is the normal Llama layout, NEOX differs).
    Reading: each head's adjacent pairs (2i, 2i+1) turn by the angle
    pos * base^(-2i/hd).  Angles and the rotation are evaluated in float64.

    x: [T, n_heads, hd]; pos: [T] integers.
    """
    T, nh, hd = x.shape
    i = np.arange(hd // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / hd)
    ang = pos.astype(np.float64)[:, None] * inv_freq[None, :]       # [T, hd/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x0 = x[..., 0::2].astype(np.float64)
    x1 = x[..., 1::2].astype(np.float64)
    out = np.empty(x.shape, np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out.astype(x.dtype)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SWIGLU(ffn_gate, ffn_up) of Example 4: silu(gate) * up (reading)."""
    return silu(gate) * up


def softmax(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis; -inf entries get 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_heads(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                    visible: np.ndarray, scale: float):
    """Unfused attention of several query heads against one KV head.

    Follows the non-flash node list on the architecture page (Example 11:
    kq = K x Q, SOFT_MAX with the mask, kqv = V x softmax): scores over all
    cells, masked cells at -inf, softmax, weighted sum of V.

    q: [nq, hd]; K, V: [n_cells, hd]; visible: bool [n_cells].
    Returns (out [nq, hd], probabilities [nq, n_cells]).
    """
    s = (q @ K.T) * scale
    s = np.where(visible[None, :], s, -np.inf)
    p = softmax(s)
    return p @ V, p


# ------------------------------------------------------------ storage types
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to float32 (exact: bf16 is the top half of f32)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float32)


Q8_0_BLOCK = 32


def q8_0_dequant(q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """32-element int8 blocks with one 2-byte scale each.

    Architecture page, Example 2: a q8_0 block packs 32 values as 32 int8 plus
    one 2-byte scale that turns the integers back into real numbers (34 bytes).
    Reading: w = f16(scale) * q, no offset, blocks run along a row.
    The product of an 11-bit and a 7-bit significand is exact in float32.

    q: int8 [rows, cols]; scale_bits: uint16 [rows, cols / 32] -> float32.
    """
    rows, cols = q.shape
    assert cols % Q8_0_BLOCK == 0
    s = f16_bits_to_f32(scale_bits)
    return (q.astype(np.float32).reshape(rows, cols // Q8_0_BLOCK, Q8_0_BLOCK)
            * s[:, :, None]).reshape(rows, cols)


def q8_0_quantize(x: np.ndarray):
    """Blocks of 32 consecutive values of each row to (int8 codes, f16 scale).

    The pages fix the block (architecture page, Example 2: 32 one-byte
    integers and a 2-byte scale; Example 10: a q8_0 KV cache stores 34 bytes
    per 32 values) but not how the codes are chosen.  Reading: symmetric,
    the block's largest magnitude maps to 127.  In float32: d = amax / 127,
    codes = x * (1 / d) rounded to nearest with halves away from zero (all
    codes 0 when d = 0); the scale kept is f16(d) (round to nearest even).

    x: float32 [..., n], n a multiple of 32 -> (int8 [..., n], uint16 [..., n / 32]).
    """
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    assert n % Q8_0_BLOCK == 0
    b = x.reshape(x.shape[:-1] + (n // Q8_0_BLOCK, Q8_0_BLOCK))
    amax = np.abs(b).max(axis=-1)
    d = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(d > 0, np.float32(1) / d, np.float32(0)).astype(np.float32)
    v = (b * inv[..., None]).astype(np.float32)
    q = np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))
    codes = q.astype(np.int8).reshape(x.shape)
    return codes, d.astype(np.float16).view(np.uint16)


def round_to_kv_type(x: np.ndarray, kv_type: str) -> np.ndarray:
    """Value as stored in a KV cell of type_k / type_v.

    "llama.cpp Architecture" page, Example 4: SET_ROWS writes the f32 key into
    an F16 cache tensor; "-ctk/-ctv" choose the cache types (engine page,
    KV-cache section; decode-loop page, context parameters: F16, Q8_0, ...).
    f16 uses IEEE round-to-nearest-even (NumPy's cast); q8_0 quantises each
    32-value block of the row (q8_0_quantize) and stores what dequantises
    back, f16(d) * code.
    """
    if kv_type == "f32":
        return x.astype(np.float32)
    if kv_type == "f16":
        return x.astype(np.float16)
    if kv_type == "q8_0":
        x = np.asarray(x, np.float32)
        codes, sc = q8_0_quantize(x.reshape(-1, x.shape[-1]))
        return q8_0_dequant(codes, sc).reshape(x.shape)
    raise ValueError(kv_type)


def kv_storage_dtype(kv_type: str):
    return {"f32": np.float32, "f16": np.float16, "q8_0": np.float32}[kv_type]


def kv_cache_bytes(n_layer: int, n_embd_kv: int, n_cells: int, kv_type: str) -> int:
    """Bytes of one of the K or V caches: n_layer x n_cells rows of n_embd_kv
    values (architecture page, Example 10: 2 bytes per value for f16, 34
    bytes per 32 values for q8_0)."""
    per_row = {"f32": 4 * n_embd_kv, "f16": 2 * n_embd_kv, "q8_0": 34 * n_embd_kv // Q8_0_BLOCK}[kv_type]
    return n_layer * n_cells * per_row
