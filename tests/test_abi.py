"""The C ABI library loads on a GPU-less host and exports every function
include/ubd.h declares (no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ubd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"typedef[^;]*;", "", text)
    return sorted(set(re.findall(r"\b(ubd_[a-z0-9_]+)\s*\(", text)) - {"ubd_alloc_fn", "ubd_free_fn"})


def test_header_parses():
    names = declared_functions()
    assert "ubd_decode" in names and "ubd_model_load" in names and len(names) > 30


def test_library_exports_every_declared_symbol():
    from llama_decode_ubatch_amd import binding
    lib = binding.load_library()
    names = declared_functions()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the binding declares a prototype for each of them
    assert set(names) <= set(binding.SIGNATURES), set(names) - set(binding.SIGNATURES)


def test_missing_library_fails_loudly(tmp_path):
    from llama_decode_ubatch_amd import binding
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="not found"):
            binding.load_library(str(tmp_path / "libubd.so"))
    finally:
        binding._lib = saved


def test_default_params_and_errors_without_gpu():
    from llama_decode_ubatch_amd import binding
    lib = binding.load_library()
    p = lib.ubd_context_default_params()
    assert (p.n_batch, p.n_ubatch, p.n_seq_max, p.type_k, p.type_v) == (2048, 512, 1, 1, 1)
    assert p.graph_reuse is True and p.kv_unified is False
    st = ctypes.c_int32(7)
    assert not lib.ubd_model_load(None, None, 0, None, ctypes.byref(st))
    assert st.value == -1 and "missing" in binding.last_error()


def test_model_load_rejects_matrices_past_32_bit_offsets():
    """The products address each fused weight matrix with 32-bit byte
    offsets: a bf16 output matrix of 262144 x 8192 (4 GiB) is refused with
    status -1 before anything reaches the GPU (only names and shapes are
    read: the data pointers are never touched)."""
    import numpy as np
    from llama_decode_ubatch_amd import binding
    from workloads import ModelShape, tensor_specs
    big = ModelShape("big-vocab", 1, n_layer=1, n_embd=8192, n_head=64, n_head_kv=8, n_ff=28672,
                     n_vocab=262144, n_ctx_train=4096, rope_base=10000.0, wtype="bf16")
    lib = binding.load_library()
    specs = tensor_specs(big)
    dummy = np.zeros(16, np.float32)
    arr = (binding.TensorSrc * len(specs))()
    names = []
    for i, sp in enumerate(specs):
        s = arr[i]
        names.append(sp.name.encode())
        s.name = names[-1]
        s.type = binding.TYPE_IDS["f32" if sp.kind == "gain" else "bf16"]
        s.ne[0], s.ne[1] = (sp.shape[0], 1) if len(sp.shape) == 1 else (sp.shape[1], sp.shape[0])
        s.data = dummy.ctypes.data
        s.on_device = 0
    hp = binding.Hparams(big.n_layer, big.n_embd, big.n_head, big.n_head_kv, big.n_ff, big.n_vocab,
                         big.n_ctx_train, big.rms_eps, big.rope_base, 0)
    st = ctypes.c_int32(7)
    assert not lib.ubd_model_load(ctypes.byref(hp), arr, len(specs), None, ctypes.byref(st))
    assert st.value == -1 and "2 GiB" in binding.last_error()
