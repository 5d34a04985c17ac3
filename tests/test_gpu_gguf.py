"""Models loaded from GGUF files (ubd_model_load_gguf) against the same
weights loaded from arrays (ubd_model_load): same kernels, same stored
values, so the logits must be bit-identical; and against the oracle
reading the same file (logits within 1e-4 of the max-norm).  Covers F32,
F16 (widened to F32 at load), BF16 and Q8_0 (GGUF blocks split on the
device) files, mmap and read loading, and a model split over three files."""
import dataclasses

import numpy as np
import pytest

from oracle import OracleContext, OracleModel, Batch
from oracle.gguf import open_model
from workloads import MODELS, gen_tensor, tensor_specs
from workloads import gguf as W

pytestmark = pytest.mark.gpu


def variants():
    m = MODELS["tiny-f32"]
    return {"f32": m, "bf16": dataclasses.replace(m, wtype="bf16", tag="tiny-bf16"),
            "q8_0": dataclasses.replace(m, wtype="q8_0", tag="tiny-q8_0")}


def f16_tensors(m):
    """The f32 model with every matrix rounded to f16 (stored as F16 in the
    file, as f32 values of the same numbers in the arrays)."""
    file_t, arr_t = {}, {}
    for s in tensor_specs(m):
        t = gen_tensor(m, s)
        if s.kind == "matrix":
            h = t["data"].astype(np.float16)
            file_t[s.name] = {"type": "f16", "data": h}
            arr_t[s.name] = {"type": "f32", "data": h.astype(np.float32)}
        else:
            file_t[s.name] = arr_t[s.name] = t
    return file_t, arr_t


def run(model, toks):
    from llama_decode_ubatch_amd import Context
    ctx = Context(model, n_ctx=256, n_batch=64, n_ubatch=16, n_seq_max=1, type_k="f32", type_v="f32")
    assert ctx.decode(toks, logits=np.ones(len(toks), np.int8)) == 0
    z = [ctx.logits()]
    for step in range(3):
        t = ctx.greedy(-1)
        assert ctx.decode([t]) == 0
        z.append(ctx.logits())
    return np.concatenate(z)


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16", "q8_0"])
def test_gguf_model_equals_array_model(tmp_path, kind):
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    m = variants()["f32" if kind == "f16" else kind]
    if kind == "f16":
        file_t, arr_t = f16_tensors(m)
    else:
        file_t = arr_t = {s.name: gen_tensor(m, s) for s in tensor_specs(m)}
    paths = W.write_model_gguf(m, str(tmp_path / kind), tensors=file_t)
    toks = np.random.default_rng(5).integers(0, m.n_vocab, 20).astype(np.int32)
    print(f"GGUF {kind}: {paths[0]}", flush=True)
    z_arr = run(Model(m, arr_t, device=0), toks)
    for use_mmap in (True, False):
        mg = Model.from_gguf(paths[0], device=0, use_mmap=use_mmap)
        assert mg.shape.n_vocab == m.n_vocab and mg.shape.n_layer == m.n_layer
        z = run(mg, toks)
        assert np.array_equal(z, z_arr), (kind, use_mmap, float(np.abs(z - z_arr).max()))
        mg.free()
    if kind in ("f32", "f16"):
        g, where = open_model(paths)
        om = OracleModel(m, lambda n: where[n].stored(n), dtype=np.float64)
        ref = OracleContext(om, n_ctx=256, n_batch=64, n_ubatch=16, type_k="f32", type_v="f32")
        assert ref.decode(Batch(toks.tolist(), logits=[1] * len(toks))) == 0
        zr = np.stack([ref.logits_ith(i) for i in range(len(toks))])
        err = float(np.abs(z_arr[:len(toks)] - zr).max() / np.abs(zr).max())
        assert err < 1e-4, err


def test_split_gguf(tmp_path):
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    m = MODELS["tiny-f32"]
    tens = {s.name: gen_tensor(m, s) for s in tensor_specs(m)}
    paths = W.write_model_gguf(m, str(tmp_path / "tiny"), n_split=3, tensors=tens)
    toks = np.arange(1, 9, dtype=np.int32)
    assert np.array_equal(run(Model.from_gguf(paths[0], device=0), toks), run(Model(m, tens, device=0), toks))


@pytest.mark.parametrize("kind", ["f32", "q8_0"])
def test_tied_output(tmp_path, kind):
    """A file without output.weight: the library uses token_embd as the
    output matrix.  Bit-identical to an array model that passes the table
    under both names (same kernels, same stored values); the f32 file also
    against the oracle reading it as a tied model."""
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    m = variants()[kind]
    tens = {s.name: gen_tensor(m, s) for s in tensor_specs(m)}
    tied = {k: v for k, v in tens.items() if k != "output.weight"}
    both = dict(tied, **{"output.weight": tens["token_embd.weight"]})
    paths = W.write_model_gguf(m, str(tmp_path / f"tied-{kind}"), tensors=tens, tied=True)
    toks = np.random.default_rng(8).integers(0, m.n_vocab, 12).astype(np.int32)
    print(f"tied GGUF {kind}: {paths[0]}", flush=True)
    z_both = run(Model(m, both, device=0), toks)
    z_arr = run(Model(m, tied, device=0), toks)
    assert np.array_equal(z_arr, z_both)
    z_file = run(Model.from_gguf(paths[0], device=0), toks)
    assert np.array_equal(z_file, z_both)
    if kind == "f32":
        g, where = open_model(paths)
        assert "output.weight" not in where
        om = OracleModel(m, lambda n: where[n].stored(n), dtype=np.float64, tied=True)
        ref = OracleContext(om, n_ctx=256, n_batch=64, n_ubatch=16, type_k="f32", type_v="f32")
        assert ref.decode(Batch(toks.tolist(), logits=[1] * len(toks))) == 0
        zr = np.stack([ref.logits_ith(i) for i in range(len(toks))])
        err = float(np.abs(z_file[:len(toks)] - zr).max() / np.abs(zr).max())
        assert err < 1e-4, err
