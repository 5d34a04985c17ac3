"""Device-side generation of the synthetic inputs (twin of gen.py).

Fills torch CUDA tensors in place through libubd_synth.so, with values
bit-identical to gen.py's host draws.  Input generation only.
"""
import ctypes
import os

import numpy as np

from . import gen
from .configs import ModelShape, Workload, tensor_specs

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libubd_synth.so")
_lib = None


def build():
    import subprocess
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "-O3", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "synth.hip"), "-o", LIB_PATH + ".tmp"]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("synth build failed:\n" + p.stdout)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
        for name, args in (("ubd_synth_table16", [vp, i64, u64, i64, vp, vp]),
                           ("ubd_synth_table32", [vp, i64, u64, i64, vp, vp]),
                           ("ubd_synth_q8_codes", [vp, i64, u64, i64, vp]),
                           ("ubd_synth_q8_scales", [vp, i64, u64, i64, vp])):
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        _lib = L
    return _lib


_TABLES = {}


def _table(torch, kind, device):
    key = (kind, device)
    if key not in _TABLES:
        if kind == "w_f32":
            t = gen.normal_table_f32(0.02)
        elif kind == "w_bf16":
            t = gen.normal_table_bf16(0.02).view(np.int16)
        elif kind == "gain":
            t = gen.gain_table_f32()
        elif kind == "kv_f16":
            t = gen.kv_table_f16().view(np.int16)
        else:
            raise KeyError(kind)
        _TABLES[key] = torch.from_numpy(np.array(t)).to(device)
    return _TABLES[key]


def _check(rc):
    if rc != 0:
        raise RuntimeError(f"synth kernel launch failed: {rc}")


def fill_tensor(torch, model: ModelShape, spec, device="cuda", literal_gains=False):
    """Generate one model tensor on the device.  Returns a dict shaped like
    gen.gen_tensor's, with torch tensors."""
    L = lib()
    stream = torch.cuda.current_stream(device).cuda_stream
    n = int(np.prod(spec.shape))
    if spec.kind == "gain":
        out = torch.empty(spec.shape, dtype=torch.float32, device=device)
        tab = _table(torch, "w_f32" if literal_gains else "gain", device)
        _check(L.ubd_synth_table32(out.data_ptr(), n, gen.tensor_key(model, spec.index, gen.SUB_VALUES), 0,
                                   tab.data_ptr(), stream))
        return {"type": "f32", "data": out}
    key = gen.tensor_key(model, spec.index, gen.SUB_VALUES)
    if model.wtype == "f32":
        out = torch.empty(spec.shape, dtype=torch.float32, device=device)
        _check(L.ubd_synth_table32(out.data_ptr(), n, key, 0, _table(torch, "w_f32", device).data_ptr(), stream))
        return {"type": "f32", "data": out}
    if model.wtype == "bf16":
        out = torch.empty(spec.shape, dtype=torch.int16, device=device)
        _check(L.ubd_synth_table16(out.data_ptr(), n, key, 0, _table(torch, "w_bf16", device).data_ptr(), stream))
        return {"type": "bf16", "data": out}
    if model.wtype == "q8_0":
        q = torch.empty(spec.shape, dtype=torch.int8, device=device)
        _check(L.ubd_synth_q8_codes(q.data_ptr(), n, key, 0, stream))
        sc = torch.empty((spec.shape[0], spec.shape[1] // 32), dtype=torch.int16, device=device)
        _check(L.ubd_synth_q8_scales(sc.data_ptr(), sc.numel(),
                                     gen.tensor_key(model, spec.index, gen.SUB_SCALES), 0, stream))
        return {"type": "q8_0", "q": q, "scale": sc}
    raise ValueError(model.wtype)


def fill_kv_block(torch, w: Workload, seq: int, layer: int, which: int, out, p0=0):
    """out: int16 CUDA tensor [n][n_embd_kv] <- f16 bits of positions p0.."""
    L = lib()
    stream = torch.cuda.current_stream(out.device).cuda_stream
    ne = w.model.n_embd_kv
    _check(L.ubd_synth_table16(out.data_ptr(), out.numel(), gen.kv_key(w, seq, layer, which), p0 * ne,
                               _table(torch, "kv_f16", out.device).data_ptr(), stream))
    return out


def model_tensors(torch, model: ModelShape, device="cuda", literal_gains=False):
    """All tensors of a model generated on the device (name -> dict)."""
    return {s.name: fill_tensor(torch, model, s, device, literal_gains) for s in tensor_specs(model)}
