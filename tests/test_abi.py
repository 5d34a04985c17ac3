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
