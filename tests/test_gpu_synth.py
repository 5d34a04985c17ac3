"""The device-side input generator reproduces the host draws bit for bit
(so GPU-generated 8B weights and KV pre-fills are the oracle's inputs)."""
import numpy as np
import pytest

from workloads import MODELS, WORKLOADS, gen_tensor_rows, tensor_specs, kv_prefill_block, gen_tensor
from workloads import device as wdev

pytestmark = pytest.mark.gpu


def _spec(model, name):
    return next(s for s in tensor_specs(model) if s.name == name)


@pytest.mark.parametrize("model,name", [("tiny-f32", "blk.1.attn_k.weight"),
                                        ("tiny-f32", "blk.0.ffn_norm.weight"),
                                        ("8b-bf16", "blk.3.attn_v.weight"),
                                        ("8b-q8_0", "blk.2.attn_k.weight")])
def test_device_tensor_equals_host(model, name):
    import torch
    m = MODELS[model]
    sp = _spec(m, name)
    d = wdev.fill_tensor(torch, m, sp, device="cuda:0")
    torch.cuda.synchronize()
    if sp.kind == "gain" or m.wtype == "f32":
        h = gen_tensor(m, sp)
        np.testing.assert_array_equal(d["data"].cpu().numpy(), h["data"])
        return
    rows = np.array([0, 1, 17, sp.shape[0] - 1])
    h = gen_tensor_rows(m, sp, rows)
    if m.wtype == "bf16":
        np.testing.assert_array_equal(d["data"].cpu().numpy().view(np.uint16)[rows], h["data"])
    else:
        np.testing.assert_array_equal(d["q"].cpu().numpy()[rows], h["q"])
        np.testing.assert_array_equal(d["scale"].cpu().numpy().view(np.uint16)[rows], h["scale"])


def test_device_kv_block_equals_host():
    import torch
    w = WORKLOADS[4]
    out = torch.empty((300, w.model.n_embd_kv), dtype=torch.int16, device="cuda:0")
    wdev.fill_kv_block(torch, w, 3, 7, 1, out, p0=1000)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16),
                                  kv_prefill_block(w, 3, 7, 1, p0=1000, n=300))
