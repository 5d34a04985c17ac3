"""ctypes binding of libubd (include/ubd.h): argument marshalling only.

Every step of the decode path runs inside libubd's HIP kernels; this module
builds the C structs, hands PyTorch's device allocator and current stream to
the library, and converts results to NumPy.  If libubd.so is missing it
raises instead of falling back to anything else.
"""
import ctypes as C
import os
import types
import weakref

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libubd.so")

UBD_TYPE_F32, UBD_TYPE_F16, UBD_TYPE_BF16, UBD_TYPE_Q8_0 = 0, 1, 2, 3
UBD_OK, UBD_NO_KV_SLOT, UBD_ABORTED = 0, 1, 2
UBD_INVALID, UBD_ALLOC_FAILED, UBD_COMPUTE_FAILED = -1, -2, -3
UBD_MAX_SEQ = 256
UBD_GREEDY_STATIC_MAX_ROWS = 256
TYPE_IDS = {"f32": UBD_TYPE_F32, "f16": UBD_TYPE_F16, "bf16": UBD_TYPE_BF16, "q8_0": UBD_TYPE_Q8_0}


class Hparams(C.Structure):
    _fields_ = [("n_layer", C.c_int32), ("n_embd", C.c_int32), ("n_head", C.c_int32),
                ("n_head_kv", C.c_int32), ("n_ff", C.c_int32), ("n_vocab", C.c_int32),
                ("n_ctx_train", C.c_int32), ("rms_eps", C.c_float), ("rope_freq_base", C.c_float),
                ("rope_type", C.c_int32)]


class TensorSrc(C.Structure):
    _fields_ = [("name", C.c_char_p), ("type", C.c_int), ("ne", C.c_int64 * 2),
                ("data", C.c_void_p), ("scales", C.c_void_p), ("on_device", C.c_int32)]


ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p)
FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p)
ABORT_FN = C.CFUNCTYPE(C.c_bool, C.c_void_p)
LOG_FN = C.CFUNCTYPE(None, C.c_int32, C.c_char_p, C.c_void_p)


class ModelParams(C.Structure):
    _fields_ = [("device", C.c_int32), ("alloc", ALLOC_FN), ("free", FREE_FN),
                ("alloc_user_data", C.c_void_p), ("stream", C.c_void_p)]


class ContextParams(C.Structure):
    _fields_ = [("n_ctx", C.c_uint32), ("n_batch", C.c_uint32), ("n_ubatch", C.c_uint32),
                ("n_seq_max", C.c_uint32), ("type_k", C.c_int), ("type_v", C.c_int),
                ("kv_unified", C.c_bool), ("abort_callback", ABORT_FN),
                ("abort_user_data", C.c_void_p), ("stream", C.c_void_p), ("graph_reuse", C.c_bool)]


class CBatch(C.Structure):
    _fields_ = [("n_tokens", C.c_int32), ("token", C.POINTER(C.c_int32)),
                ("embd", C.POINTER(C.c_float)), ("pos", C.POINTER(C.c_int32)),
                ("n_seq_id", C.POINTER(C.c_int32)),
                ("seq_id", C.POINTER(C.POINTER(C.c_int32))), ("logits", C.POINTER(C.c_int8))]


class SamplerParams(C.Structure):
    _fields_ = [("top_k", C.c_int32), ("top_p", C.c_float), ("min_p", C.c_float),
                ("temperature", C.c_float), ("penalty_last_n", C.c_int32),
                ("penalty_repeat", C.c_float), ("penalty_freq", C.c_float),
                ("penalty_present", C.c_float)]


class GgufInfo(C.Structure):
    _fields_ = [("version", C.c_uint32), ("n_files", C.c_int32), ("n_tensors", C.c_int64),
                ("n_params", C.c_double), ("file_bytes", C.c_double), ("bpw", C.c_double),
                ("file_type", C.c_int32), ("all_same", C.c_int32), ("hparams", Hparams)]


class Perf(C.Structure):
    _fields_ = [("t_load_ms", C.c_double), ("t_p_eval_ms", C.c_double), ("t_eval_ms", C.c_double),
                ("n_p_eval", C.c_int32), ("n_eval", C.c_int32), ("n_ubatch", C.c_int32),
                ("n_decode", C.c_int32), ("n_graphs", C.c_int32), ("n_reused", C.c_int32)]


# name -> (restype, argtypes); also the list of symbols include/ubd.h declares
_P = C.c_void_p
SIGNATURES = {
    "ubd_model_load": (_P, [C.POINTER(Hparams), C.POINTER(TensorSrc), C.c_int32,
                            C.POINTER(ModelParams), C.POINTER(C.c_int32)]),
    "ubd_model_free": (None, [_P]),
    "ubd_model_size": (C.c_size_t, [_P]),
    "ubd_context_default_params": (ContextParams, []),
    "ubd_init_from_model": (_P, [_P, C.POINTER(ContextParams), C.POINTER(C.c_int32)]),
    "ubd_free": (None, [_P]),
    "ubd_n_ctx": (C.c_uint32, [_P]),
    "ubd_n_batch": (C.c_uint32, [_P]),
    "ubd_n_ubatch": (C.c_uint32, [_P]),
    "ubd_batch_init": (CBatch, [C.c_int32, C.c_int32, C.c_int32]),
    "ubd_batch_free": (None, [CBatch]),
    "ubd_batch_get_one": (CBatch, [C.POINTER(C.c_int32), C.c_int32]),
    "ubd_decode": (C.c_int32, [_P, CBatch]),
    "ubd_n_outputs": (C.c_int32, [_P]),
    "ubd_get_logits": (C.POINTER(C.c_float), [_P]),
    "ubd_get_logits_ith": (C.POINTER(C.c_float), [_P, C.c_int32]),
    "ubd_get_logits_device": (C.c_void_p, [_P]),
    "ubd_sample_greedy": (C.c_int32, [_P, C.c_int32]),
    "ubd_sample_greedy_all": (C.c_int32, [_P, C.POINTER(C.c_int32), C.c_int32]),
    "ubd_greedy_chain": (C.c_int32, [_P, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32)]),
    "ubd_greedy_rows_static": (C.c_int32, [C.c_int32, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                           C.c_void_p]),
    "ubd_sampler_default_params": (SamplerParams, []),
    "ubd_sampler_init": (_P, [_P, SamplerParams]),
    "ubd_sampler_free": (None, [_P]),
    "ubd_sampler_accept": (None, [_P, C.c_int32]),
    "ubd_sampler_sample": (C.c_int32, [_P, C.c_int32, C.c_float]),
    "ubd_sampler_sample_logits": (C.c_int32, [_P, C.c_void_p, C.c_int32, C.c_float]),
    "ubd_sampler_candidates": (C.c_int32, [_P, C.POINTER(C.c_int32), C.POINTER(C.c_float), C.c_int32]),
    "ubd_synchronize": (C.c_int32, [_P]),
    "ubd_gguf_open": (_P, [C.c_char_p, C.POINTER(C.c_int32)]),
    "ubd_gguf_close": (None, [_P]),
    "ubd_gguf_version": (C.c_uint32, [_P]),
    "ubd_gguf_data_offset": (C.c_int64, [_P]),
    "ubd_gguf_n_kv": (C.c_int64, [_P]),
    "ubd_gguf_find_key": (C.c_int64, [_P, C.c_char_p]),
    "ubd_gguf_key": (C.c_char_p, [_P, C.c_int64]),
    "ubd_gguf_kv_type": (C.c_int32, [_P, C.c_int64]),
    "ubd_gguf_arr_type": (C.c_int32, [_P, C.c_int64]),
    "ubd_gguf_arr_n": (C.c_int64, [_P, C.c_int64]),
    "ubd_gguf_get_int": (C.c_int32, [_P, C.c_int64, C.c_int64, C.POINTER(C.c_int64)]),
    "ubd_gguf_get_float": (C.c_int32, [_P, C.c_int64, C.c_int64, C.POINTER(C.c_double)]),
    "ubd_gguf_get_str": (C.c_void_p, [_P, C.c_int64, C.c_int64, C.POINTER(C.c_uint64)]),
    "ubd_gguf_n_tensors": (C.c_int64, [_P]),
    "ubd_gguf_find_tensor": (C.c_int64, [_P, C.c_char_p]),
    "ubd_gguf_tensor_name": (C.c_char_p, [_P, C.c_int64]),
    "ubd_gguf_tensor_type": (C.c_int32, [_P, C.c_int64]),
    "ubd_gguf_tensor_dims": (C.c_int32, [_P, C.c_int64, C.POINTER(C.c_int64)]),
    "ubd_gguf_tensor_offset": (C.c_int64, [_P, C.c_int64]),
    "ubd_gguf_tensor_nbytes": (C.c_int64, [_P, C.c_int64]),
    "ubd_gguf_model_info": (C.c_int32, [C.c_char_p, C.POINTER(GgufInfo)]),
    "ubd_model_load_gguf": (_P, [C.c_char_p, C.POINTER(ModelParams), C.c_int32, C.POINTER(C.c_int32)]),
    "ubd_memory_seq_pos_min": (C.c_int32, [_P, C.c_int32]),
    "ubd_memory_seq_pos_max": (C.c_int32, [_P, C.c_int32]),
    "ubd_memory_seq_rm": (C.c_bool, [_P, C.c_int32, C.c_int32, C.c_int32]),
    "ubd_memory_seq_cp": (C.c_bool, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "ubd_memory_seq_keep": (C.c_bool, [_P, C.c_int32]),
    "ubd_memory_defrag": (C.c_int32, [_P]),
    "ubd_memory_cells": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_uint32), C.c_int32]),
    "ubd_get_kv_cells": (C.c_int32, [_P, C.POINTER(C.c_int32), C.c_int32]),
    "ubd_kv_fill": (C.c_int32, [_P, C.c_int32, C.c_int32, C.POINTER(C.c_void_p),
                                C.POINTER(C.c_void_p), C.c_int, C.c_int32]),
    "ubd_kv_read": (C.c_int32, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                C.POINTER(C.c_float)]),
    "ubd_debug_keep_residuals": (C.c_int32, [_P, C.c_int32]),
    "ubd_debug_get_residual": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_float), C.c_int32]),
    "ubd_debug_last_ubatch": (C.c_int32, [_P, C.POINTER(C.c_int32), C.c_int32]),
    "ubd_debug_kernel_timing": (C.c_int32, [_P, C.c_uint32]),
    "ubd_debug_kernel_class_name": (C.c_char_p, [C.c_int32]),
    "ubd_debug_kernel_stats": (C.c_int32, [_P, C.POINTER(C.c_int32), C.POINTER(C.c_double), C.c_int32]),
    "ubd_debug_set_tuning": (C.c_int32, [C.c_char_p, C.c_int32]),
    "ubd_perf_get": (None, [_P, C.POINTER(Perf)]),
    "ubd_perf_reset": (None, [_P]),
    "ubd_log_set": (None, [LOG_FN, C.c_void_p]),
    "ubd_last_error": (C.c_char_p, []),
    "ubd_planner_new": (_P, [C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32, C.c_bool, C.c_int32]),
    "ubd_planner_free": (None, [_P]),
    "ubd_planner_decode": (C.c_int32, [_P, CBatch, C.c_int32, C.c_int32]),
    "ubd_planner_n_ubatches": (C.c_int32, [_P]),
    "ubd_planner_ubatch": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                       C.POINTER(C.c_int32), C.c_int32]),
    "ubd_planner_output_row": (C.c_int32, [_P, C.c_int32]),
    "ubd_planner_n_outputs": (C.c_int32, [_P]),
    "ubd_planner_seq_pos_min": (C.c_int32, [_P, C.c_int32]),
    "ubd_planner_seq_pos_max": (C.c_int32, [_P, C.c_int32]),
    "ubd_planner_seq_rm": (C.c_bool, [_P, C.c_int32, C.c_int32, C.c_int32]),
    "ubd_planner_seq_cp": (C.c_bool, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "ubd_planner_seq_keep": (C.c_bool, [_P, C.c_int32]),
    "ubd_planner_defrag": (C.c_int32, [_P]),
    "ubd_planner_cells": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_uint32), C.c_int32]),
    "ubd_planner_n_kv": (C.c_int32, [_P, C.c_int32]),
}

_lib = None


def load_library(path=LIB_PATH):
    """Load libubd.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m llama_decode_ubatch_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def last_error():
    return load_library().ubd_last_error().decode()


def set_tuning(key, value):
    """Process-wide launch-shape knob (see ubd_debug_set_tuning)."""
    if load_library().ubd_debug_set_tuning(key.encode(), int(value)) != 0:
        raise KeyError(key)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))


def _cell_table(fn, ptr, stream, n_cells, n_seq_max):
    """(pos [n_cells], has [n_cells][n_seq_max] bool) of one stream."""
    W = (n_seq_max + 31) // 32
    pos = np.zeros(n_cells, np.int32)
    words = np.zeros(n_cells * W, np.uint32)
    n = fn(ptr, stream, pos.ctypes.data_as(C.POINTER(C.c_int32)), words.ctypes.data_as(C.POINTER(C.c_uint32)),
           n_cells * W)
    if n != n_cells:
        raise RuntimeError(f"cell table read failed: {last_error()}")
    w = words.reshape(W, n_cells)
    s = np.arange(n_seq_max)
    has = ((w[s // 32] >> (s % 32)[:, None].astype(np.uint32)) & 1).T.astype(bool)
    return pos, has


class _BatchHolder:
    """Keeps the arrays a CBatch points into alive."""

    def __init__(self, tokens, pos=None, seq_id=None, logits=None):
        self.token = _i32(tokens)
        n = self.token.size
        self.b = CBatch()
        self.b.n_tokens = n
        self.b.token = self.token.ctypes.data_as(C.POINTER(C.c_int32))
        if pos is not None:
            self.pos = _i32(pos)
            self.b.pos = self.pos.ctypes.data_as(C.POINTER(C.c_int32))
        if seq_id is not None:
            # one id per token, or a list of ids per token (several sequences)
            rows = [np.atleast_1d(np.asarray(v, np.int32)) for v in seq_id]
            self.n_seq = np.asarray([r.size for r in rows], np.int32)
            self.seq = np.ascontiguousarray(np.concatenate(rows) if rows else np.zeros(0, np.int32))
            offs = np.concatenate([[0], np.cumsum(self.n_seq)[:-1]]).astype(np.int64)
            base = self.seq.ctypes.data
            self.rows = (C.POINTER(C.c_int32) * n)(
                *[C.cast(base + 4 * int(o), C.POINTER(C.c_int32)) for o in offs])
            self.b.seq_id = C.cast(self.rows, C.POINTER(C.POINTER(C.c_int32)))
            self.b.n_seq_id = self.n_seq.ctypes.data_as(C.POINTER(C.c_int32))
        if logits is not None:
            self.logits = np.ascontiguousarray(np.asarray(logits).reshape(-1) != 0, dtype=np.int8)
            self.b.logits = self.logits.ctypes.data_as(C.POINTER(C.c_int8))


class TorchAllocator:
    """Device memory for libubd from PyTorch's caching allocator."""

    def __init__(self, torch, device):
        self.torch = torch
        self.device = device
        self.live = {}
        self.alloc_fn = ALLOC_FN(self._alloc)
        self.free_fn = FREE_FN(self._free)

    def _alloc(self, n, ud):
        try:
            t = self.torch.empty(int(n), dtype=self.torch.uint8, device=self.device)
        except Exception:  # out of memory -> NULL, reported by libubd as -2
            return None
        p = t.data_ptr()
        self.live[p] = t
        return p

    def _free(self, p, ud):
        self.live.pop(p, None)


def _stream_ptr(torch, device):
    return torch.cuda.current_stream(device).cuda_stream


class Model:
    """A loaded model.  ``tensors`` maps GGUF names to dicts as produced by
    workloads.gen.gen_tensor (NumPy host arrays) or workloads.device
    (torch CUDA tensors, passed as device pointers)."""

    def __init__(self, shape, tensors, device=0, torch_alloc=True):
        import torch
        self.lib = load_library()
        self.torch = torch
        self.shape = shape
        self.device = device
        torch.cuda.set_device(device)
        self.alloc = TorchAllocator(torch, f"cuda:{device}") if torch_alloc else None
        hp = Hparams(shape.n_layer, shape.n_embd, shape.n_head, shape.n_head_kv, shape.n_ff,
                     shape.n_vocab, shape.n_ctx_train, shape.rms_eps, shape.rope_base, 0)
        keep = []
        arr = (TensorSrc * len(tensors))()
        for i, (name, t) in enumerate(tensors.items()):
            s = arr[i]
            s.name = name.encode()
            keep.append(s.name)
            s.type = TYPE_IDS[t["type"]]
            data = t["q"] if t["type"] == "q8_0" else t["data"]
            if data.ndim == 1:
                s.ne[0], s.ne[1] = data.shape[0], 1
            else:
                s.ne[0], s.ne[1] = data.shape[1], data.shape[0]
            if isinstance(data, np.ndarray):
                data = np.ascontiguousarray(data)
                keep.append(data)
                s.data = data.ctypes.data
                s.on_device = 0
                if t["type"] == "q8_0":
                    sc = np.ascontiguousarray(t["scale"])
                    keep.append(sc)
                    s.scales = sc.ctypes.data
            else:
                s.data = data.data_ptr()
                s.on_device = 1
                if t["type"] == "q8_0":
                    s.scales = t["scale"].data_ptr()
        mp = self._params()
        st = C.c_int32(0)
        self.ptr = self.lib.ubd_model_load(C.byref(hp), arr, len(tensors), C.byref(mp), C.byref(st))
        if not self.ptr:
            raise RuntimeError(f"ubd_model_load failed ({st.value}): {last_error()}")
        self._finalizer = weakref.finalize(self, self.lib.ubd_model_free, self.ptr)

    def _params(self):
        mp = ModelParams()
        mp.device = self.device
        if self.alloc:
            mp.alloc = self.alloc.alloc_fn
            mp.free = self.alloc.free_fn
        mp.stream = _stream_ptr(self.torch, self.device)
        return mp

    @classmethod
    def from_gguf(cls, path, device=0, use_mmap=True, torch_alloc=True):
        """Load with ubd_model_load_gguf; ``shape`` then holds the
        hyperparameters the file gives."""
        import torch
        self = cls.__new__(cls)
        self.lib = load_library()
        self.torch = torch
        self.device = device
        torch.cuda.set_device(device)
        self.alloc = TorchAllocator(torch, f"cuda:{device}") if torch_alloc else None
        hp = gguf_model_info(path).hparams
        self.shape = types.SimpleNamespace(
            n_layer=hp.n_layer, n_embd=hp.n_embd, n_head=hp.n_head, n_head_kv=hp.n_head_kv, n_ff=hp.n_ff,
            n_vocab=hp.n_vocab, n_ctx_train=hp.n_ctx_train, rms_eps=hp.rms_eps, rope_base=hp.rope_freq_base)
        mp = self._params()
        st = C.c_int32(0)
        self.ptr = self.lib.ubd_model_load_gguf(str(path).encode(), C.byref(mp), int(bool(use_mmap)), C.byref(st))
        if not self.ptr:
            raise RuntimeError(f"ubd_model_load_gguf failed ({st.value}): {last_error()}")
        self._finalizer = weakref.finalize(self, self.lib.ubd_model_free, self.ptr)
        return self

    def size(self):
        return self.lib.ubd_model_size(self.ptr)

    def free(self):
        self._finalizer()


def greedy_rows_static(device, logits_ptr, ld, n_rows, n_vocab, out_ptr, stream_ptr):
    """ubd_greedy_rows_static on raw device addresses (ints); returns the
    library's status code."""
    return load_library().ubd_greedy_rows_static(device, logits_ptr, ld, n_rows, n_vocab, out_ptr, stream_ptr)


def gguf_model_info(path):
    info = GgufInfo()
    if load_library().ubd_gguf_model_info(str(path).encode(), C.byref(info)) != 0:
        raise ValueError(f"ubd_gguf_model_info failed: {last_error()}")
    return info


class Gguf:
    """Metadata and tensor records of one GGUF file (ubd_gguf_*)."""
    INT_TYPES = {0, 1, 2, 3, 4, 5, 7, 10, 11}
    FLOAT_TYPES = {6, 12}

    def __init__(self, path):
        self.lib = load_library()
        st = C.c_int32(0)
        self.ptr = self.lib.ubd_gguf_open(str(path).encode(), C.byref(st))
        if not self.ptr:
            raise ValueError(f"ubd_gguf_open failed ({st.value}): {last_error()}")
        self._finalizer = weakref.finalize(self, self.lib.ubd_gguf_close, self.ptr)
        self.version = self.lib.ubd_gguf_version(self.ptr)
        self.data_offset = self.lib.ubd_gguf_data_offset(self.ptr)

    def close(self):
        self._finalizer()

    def _elem(self, i, j, t):
        if t in self.INT_TYPES:
            v = C.c_int64()
            assert self.lib.ubd_gguf_get_int(self.ptr, i, j, C.byref(v)) == 0
            return v.value
        if t in self.FLOAT_TYPES:
            v = C.c_double()
            assert self.lib.ubd_gguf_get_float(self.ptr, i, j, C.byref(v)) == 0
            return v.value
        n = C.c_uint64()
        p = self.lib.ubd_gguf_get_str(self.ptr, i, j, C.byref(n))
        assert p
        return C.string_at(p, n.value)

    def items(self):
        """[(key, type, value)]: arrays as (element type, list), nested
        arrays as (9, count); strings as bytes."""
        out = []
        for i in range(self.lib.ubd_gguf_n_kv(self.ptr)):
            key = self.lib.ubd_gguf_key(self.ptr, i).decode("utf-8", errors="surrogateescape")
            t = self.lib.ubd_gguf_kv_type(self.ptr, i)
            if t == 9:
                et, n = self.lib.ubd_gguf_arr_type(self.ptr, i), self.lib.ubd_gguf_arr_n(self.ptr, i)
                v = (et, n) if et == 9 else (et, [self._elem(i, j, et) for j in range(n)])
            else:
                v = self._elem(i, -1, t)
            out.append((key, t, v))
        return out

    def find_key(self, key):
        return self.lib.ubd_gguf_find_key(self.ptr, key.encode())

    def tensors(self):
        out = []
        ne = (C.c_int64 * 4)()
        for i in range(self.lib.ubd_gguf_n_tensors(self.ptr)):
            nd = self.lib.ubd_gguf_tensor_dims(self.ptr, i, ne)
            name = self.lib.ubd_gguf_tensor_name(self.ptr, i).decode("utf-8", errors="surrogateescape")
            out.append(dict(name=name, dims=list(ne[:nd]),
                            type=self.lib.ubd_gguf_tensor_type(self.ptr, i),
                            offset=self.lib.ubd_gguf_tensor_offset(self.ptr, i),
                            nbytes=self.lib.ubd_gguf_tensor_nbytes(self.ptr, i)))
        return out


class Context:
    def __init__(self, model, n_ctx, n_batch=2048, n_ubatch=512, n_seq_max=1, type_k="f16",
                 type_v="f16", kv_unified=False, abort_callback=None, graph_reuse=True):
        self.lib = model.lib
        self.model = model
        torch = model.torch
        p = self.lib.ubd_context_default_params()
        p.n_ctx, p.n_batch, p.n_ubatch, p.n_seq_max = n_ctx, n_batch, n_ubatch, n_seq_max
        p.type_k, p.type_v = TYPE_IDS[type_k], TYPE_IDS[type_v]
        p.kv_unified = kv_unified
        p.graph_reuse = graph_reuse
        self._abort = None
        if abort_callback is not None:
            self._abort = ABORT_FN(lambda ud: bool(abort_callback()))
            p.abort_callback = self._abort
        p.stream = _stream_ptr(torch, model.device)
        st = C.c_int32(0)
        self.ptr = self.lib.ubd_init_from_model(model.ptr, C.byref(p), C.byref(st))
        if not self.ptr:
            raise RuntimeError(f"ubd_init_from_model failed ({st.value}): {last_error()}")
        self.n_vocab = model.shape.n_vocab
        self.n_seq_max = max(1, n_seq_max)
        self.n_stream = 1 if kv_unified else self.n_seq_max
        self.n_cells = self.lib.ubd_n_ctx(self.ptr) // self.n_stream
        self._finalizer = weakref.finalize(self, self.lib.ubd_free, self.ptr)

    def free(self):
        self._finalizer()

    @property
    def n_ctx(self):
        return self.lib.ubd_n_ctx(self.ptr)

    def decode(self, tokens, pos=None, seq_id=None, logits=None):
        h = _BatchHolder(tokens, pos, seq_id, logits)
        return self.lib.ubd_decode(self.ptr, h.b)

    def n_outputs(self):
        return self.lib.ubd_n_outputs(self.ptr)

    def logits_device_ptr(self):
        """Device address of the logits rows (ubd_get_logits_device), 0 if none."""
        return self.lib.ubd_get_logits_device(self.ptr) or 0

    def logits(self):
        n = self.n_outputs()
        p = self.lib.ubd_get_logits(self.ptr)
        if not p or n == 0:
            return None
        return np.ctypeslib.as_array(p, shape=(n, self.n_vocab)).copy()

    def logits_ith(self, i):
        p = self.lib.ubd_get_logits_ith(self.ptr, i)
        return None if not p else np.ctypeslib.as_array(p, shape=(self.n_vocab,)).copy()

    def greedy(self, i=-1):
        return self.lib.ubd_sample_greedy(self.ptr, i)

    def greedy_all(self):
        n = self.n_outputs()
        out = np.zeros(max(n, 1), np.int32)
        r = self.lib.ubd_sample_greedy_all(self.ptr, out.ctypes.data_as(C.POINTER(C.c_int32)), out.size)
        if r < 0:
            raise RuntimeError(f"ubd_sample_greedy_all failed: {last_error()}")
        return out[:r]

    def greedy_chain(self, first, n_steps, seq_id=0):
        """n_steps greedy single-token steps of one sequence, the first fed
        `first`, each later one the previous pick (ubd_greedy_chain); returns
        the picks.  Raises if no step could be done; a shorter array means a
        later step failed (see last_error())."""
        out = np.zeros(max(int(n_steps), 1), np.int32)
        r = self.lib.ubd_greedy_chain(self.ptr, int(first), int(seq_id), int(n_steps),
                                      out.ctypes.data_as(C.POINTER(C.c_int32)))
        if r < 0:
            raise RuntimeError(f"ubd_greedy_chain failed ({r}): {last_error()}")
        return out[:r]

    def synchronize(self):
        return self.lib.ubd_synchronize(self.ptr)

    def seq_pos_min(self, s):
        return self.lib.ubd_memory_seq_pos_min(self.ptr, s)

    def seq_pos_max(self, s):
        return self.lib.ubd_memory_seq_pos_max(self.ptr, s)

    def seq_rm(self, s, p0, p1):
        return self.lib.ubd_memory_seq_rm(self.ptr, s, p0, p1)

    def seq_cp(self, src, dst, p0, p1):
        return self.lib.ubd_memory_seq_cp(self.ptr, src, dst, p0, p1)

    def seq_keep(self, s):
        return self.lib.ubd_memory_seq_keep(self.ptr, s)

    def defrag(self):
        return self.lib.ubd_memory_defrag(self.ptr)

    def cells(self, stream):
        return _cell_table(self.lib.ubd_memory_cells, self.ptr, stream, self.n_cells, self.n_seq_max)

    def kv_cells(self, n_tokens):
        out = np.zeros(n_tokens, np.int32)
        r = self.lib.ubd_get_kv_cells(self.ptr, out.ctypes.data_as(C.POINTER(C.c_int32)), n_tokens)
        return None if r < 0 else out[:r]

    def kv_fill(self, seq, n_pos, k_layers, v_layers, src_type="f16"):
        """k_layers / v_layers: per-layer arrays [n_pos][n_head_kv*head_dim]
        (NumPy host arrays or torch CUDA tensors; f16 passed as uint16 /
        int16 bit patterns)."""
        on_device = not isinstance(k_layers[0], np.ndarray)
        keep = []

        def ptrs(layers):
            a = (C.c_void_p * len(layers))()
            for i, t in enumerate(layers):
                if on_device:
                    a[i] = t.data_ptr()
                else:
                    t = np.ascontiguousarray(t)
                    keep.append(t)
                    a[i] = t.ctypes.data
            return a
        ka, va = ptrs(k_layers), ptrs(v_layers)
        return self.lib.ubd_kv_fill(self.ptr, seq, n_pos, ka, va, TYPE_IDS[src_type], int(on_device))

    def kv_read(self, layer, stream, which, cell0, n):
        hp = self.model.shape
        out = np.zeros((n, hp.n_embd_kv), np.float32)
        rc = self.lib.ubd_kv_read(self.ptr, layer, stream, which, cell0, n,
                                  out.ctypes.data_as(C.POINTER(C.c_float)))
        if rc != 0:
            raise RuntimeError(f"ubd_kv_read failed: {last_error()}")
        return out

    def keep_residuals(self, enable=True):
        return self.lib.ubd_debug_keep_residuals(self.ptr, int(enable))

    def residual(self, layer, max_tokens):
        out = np.zeros((max_tokens, self.model.shape.n_embd), np.float32)
        r = self.lib.ubd_debug_get_residual(self.ptr, layer, out.ctypes.data_as(C.POINTER(C.c_float)),
                                            max_tokens)
        if r < 0:
            raise RuntimeError(f"ubd_debug_get_residual failed: {last_error()}")
        return out[:r]

    def last_ubatch(self, max_tokens):
        out = np.zeros(max_tokens, np.int32)
        r = self.lib.ubd_debug_last_ubatch(self.ptr, out.ctypes.data_as(C.POINTER(C.c_int32)), max_tokens)
        return out[:r]

    N_KERNEL_CLASSES = 16

    def kernel_timing(self, classes=None):
        """Time the named kernel classes (None: all, []: off)."""
        if classes is None:
            mask = (1 << self.N_KERNEL_CLASSES) - 1
        else:
            names = [self.lib.ubd_debug_kernel_class_name(i).decode() for i in range(self.N_KERNEL_CLASSES)]
            mask = 0
            for c in classes:
                mask |= 1 << names.index(c)
        return self.lib.ubd_debug_kernel_timing(self.ptr, mask)

    def kernel_stats(self):
        n = self.N_KERNEL_CLASSES
        la = (C.c_int32 * n)()
        ms = (C.c_double * n)()
        self.lib.ubd_debug_kernel_stats(self.ptr, la, ms, n)
        out = {}
        for i in range(n):
            if la[i]:
                out[self.lib.ubd_debug_kernel_class_name(i).decode()] = (la[i], ms[i])
        return out

    def perf(self):
        p = Perf()
        self.lib.ubd_perf_get(self.ptr, C.byref(p))
        return {f: getattr(p, f) for f, _ in Perf._fields_}


class Sampler:
    """The sampler chain on rows of a context's logits (ubd_sampler_*);
    keyword arguments override ubd_sampler_default_params()."""

    def __init__(self, ctx, **params):
        self.lib = load_library()
        self.ctx = ctx
        p = self.lib.ubd_sampler_default_params()
        for k, v in params.items():
            if not hasattr(p, k):
                raise KeyError(k)
            setattr(p, k, v)
        self.ptr = self.lib.ubd_sampler_init(ctx.ptr, p)
        if not self.ptr:
            raise ValueError(f"ubd_sampler_init failed: {last_error()}")

    def free(self):
        if self.ptr:
            self.lib.ubd_sampler_free(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def accept(self, tokens):
        for t in np.atleast_1d(tokens):
            self.lib.ubd_sampler_accept(self.ptr, int(t))

    def sample(self, i, u):
        return self.lib.ubd_sampler_sample(self.ptr, i, u)

    def sample_logits(self, logits, u):
        """logits: a float32 CUDA tensor of one row, on the context's device."""
        assert logits.dtype.itemsize == 4 and logits.is_cuda and logits.is_contiguous()
        return self.lib.ubd_sampler_sample_logits(self.ptr, logits.data_ptr(), logits.numel(), u)

    def candidates(self, cap=1024):
        ids = np.zeros(cap, np.int32)
        probs = np.zeros(cap, np.float32)
        n = self.lib.ubd_sampler_candidates(self.ptr, ids.ctypes.data_as(C.POINTER(C.c_int32)),
                                            probs.ctypes.data_as(C.POINTER(C.c_float)), cap)
        if n < 0:
            raise RuntimeError(f"ubd_sampler_candidates failed: {last_error()}")
        n = min(n, cap)
        return ids[:n], probs[:n]


class Planner:
    """The host-only planner entry points (no GPU needed)."""

    def __init__(self, n_ctx, n_batch, n_ubatch, n_seq_max, kv_unified, n_vocab):
        self.lib = load_library()
        self.ptr = self.lib.ubd_planner_new(n_ctx, n_batch, n_ubatch, n_seq_max, kv_unified, n_vocab)
        if not self.ptr:
            raise RuntimeError(f"ubd_planner_new failed: {last_error()}")
        self._finalizer = weakref.finalize(self, self.lib.ubd_planner_free, self.ptr)

    def decode(self, tokens, pos=None, seq_id=None, logits=None, fail_at=-1, fail_code=0):
        h = _BatchHolder(tokens, pos, seq_id, logits)
        return self.lib.ubd_planner_decode(self.ptr, h.b, fail_at, fail_code)

    def ubatches(self, cap=1 << 16):
        out = []
        for k in range(self.lib.ubd_planner_n_ubatches(self.ptr)):
            idx, cells, st = (np.zeros(cap, np.int32) for _ in range(3))
            n = self.lib.ubd_planner_ubatch(self.ptr, k, idx.ctypes.data_as(C.POINTER(C.c_int32)),
                                            cells.ctypes.data_as(C.POINTER(C.c_int32)),
                                            st.ctypes.data_as(C.POINTER(C.c_int32)), cap)
            out.append((idx[:n].copy(), cells[:n].copy(), st[:n].copy()))
        return out

    def output_row(self, i):
        return self.lib.ubd_planner_output_row(self.ptr, i)

    def n_outputs(self):
        return self.lib.ubd_planner_n_outputs(self.ptr)

    def seq_pos_min(self, s):
        return self.lib.ubd_planner_seq_pos_min(self.ptr, s)

    def seq_pos_max(self, s):
        return self.lib.ubd_planner_seq_pos_max(self.ptr, s)

    def seq_rm(self, s, p0, p1):
        return self.lib.ubd_planner_seq_rm(self.ptr, s, p0, p1)

    def seq_cp(self, src, dst, p0, p1):
        return self.lib.ubd_planner_seq_cp(self.ptr, src, dst, p0, p1)

    def seq_keep(self, s):
        return self.lib.ubd_planner_seq_keep(self.ptr, s)

    def defrag(self):
        return self.lib.ubd_planner_defrag(self.ptr)

    def cells(self, stream, n_cells, n_seq_max):
        return _cell_table(self.lib.ubd_planner_cells, self.ptr, stream, n_cells, n_seq_max)

    def n_kv(self, stream):
        return self.lib.ubd_planner_n_kv(self.ptr, stream)
