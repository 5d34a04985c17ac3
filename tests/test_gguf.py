"""GGUF files: pins of the oracle's reader (oracle/gguf.py) against bytes
assembled by hand here, the architecture page's Example 8 / Example 2
figures, and rejection of malformed files; then the library's reader
(ubd_gguf_*) against the oracle's on the same files (CPU only)."""
import dataclasses
import json
import os
import struct

import numpy as np
import pytest

from oracle.gguf import GGUF, GGUFError, open_model, hparams, model_info
from workloads import MODELS, gen_tensor, tensor_specs
from workloads import gguf as W

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_model_figures.json")))


def s(x: str) -> bytes:
    b = x.encode()
    return struct.pack("<Q", len(b)) + b


def hand_file(tmp_path, version=3, magic=b"GGUF", offset=0, n_dims=2, ttype=0, dup=False):
    """One 4 x 2 F32 tensor "t" and three keys, byte by byte: magic,
    version, tensor count, key count; keys (name, type, value); tensor
    record (name, dims, type, offset); zero padding to 32; data."""
    b = magic + struct.pack("<I", version) + struct.pack("<Q", 2 if dup else 1) + struct.pack("<Q", 3)
    b += s("general.architecture") + struct.pack("<I", 8) + s("llama")
    b += s("x.flag") + struct.pack("<I", 7) + b"\x01"
    b += s("x.list") + struct.pack("<I", 9) + struct.pack("<I", 5) + struct.pack("<Q", 3) + struct.pack("<3i", -1, 0, 7)
    for _ in range(2 if dup else 1):
        b += s("t") + struct.pack("<I", n_dims) + struct.pack("<Q", 4) + struct.pack("<Q", 2) * (n_dims - 1)
        b += struct.pack("<I", ttype) + struct.pack("<Q", offset)
    b += b"\0" * ((-len(b)) % 32)
    b += struct.pack("<8f", *range(8))
    p = tmp_path / "hand.gguf"
    p.write_bytes(b)
    return str(p), b


def test_hand_built_file(tmp_path):
    path, raw = hand_file(tmp_path)
    g = GGUF(path)
    assert g.version == 3 and g.keys == ["general.architecture", "x.flag", "x.list"]
    assert g.kv["general.architecture"] == (8, "llama")
    assert g.kv["x.flag"] == (7, True)
    assert g.kv["x.list"] == (9, (5, [-1, 0, 7]))
    t = g.tensors[0]
    assert (t["name"], t["dims"], t["type"], t["offset"], t["nbytes"]) == ("t", [4, 2], 0, 0, 32)
    assert g.data_start == len(raw) - 32 and g.data_start % 32 == 0
    assert g.stored("t")["data"].tolist() == [[0, 1, 2, 3], [4, 5, 6, 7]]


@pytest.mark.parametrize("kw,msg", [
    (dict(magic=b"GGUG"), "not a GGUF"),
    (dict(version=2), "version"),
    (dict(version=4), "version"),
    (dict(n_dims=5), "dimensions"),
    (dict(ttype=99), "unknown type"),
    (dict(offset=8), "misaligned"),
    (dict(offset=32), "past the end"),
    (dict(dup=True), "duplicated"),
])
def test_malformed_files_are_rejected(tmp_path, kw, msg):
    path, _ = hand_file(tmp_path, **kw)
    with pytest.raises(GGUFError, match=msg):
        GGUF(path)


def test_truncated_files_are_rejected(tmp_path):
    path, raw = hand_file(tmp_path)
    for n in range(0, len(raw) - 1, 3):
        open(path, "wb").write(raw[:n])
        with pytest.raises(GGUFError):
            GGUF(path)


@pytest.fixture(scope="module")
def tiny_files(tmp_path_factory):
    d = tmp_path_factory.mktemp("gguf")
    m = MODELS["tiny-f32"]
    one = W.write_model_gguf(m, str(d / "tiny"))
    three = W.write_model_gguf(m, str(d / "tiny_split"), n_split=3)
    q8 = dataclasses.replace(m, wtype="q8_0", tag="tiny-q8_0")
    q8p = W.write_model_gguf(q8, str(d / "tiny_q8"))
    return m, one, three, q8, q8p


def test_round_trip_and_page_example_8(tiny_files):
    m, one, three, _, _ = tiny_files
    g, where = open_model(one)
    assert len(g.tensors) == FIG["ex8_tensor_count"]
    for key, v in FIG["ex8_kv"].items():
        assert g.get(key) == v, key
    hp = hparams(g, where)
    assert (hp["n_embd"], hp["n_layer"], hp["n_head"], hp["n_head_kv"], hp["n_ff"], hp["n_vocab"]) == (
        FIG["ex8_n_embd"], FIG["ex8_n_layer"], FIG["ex8_n_head"], FIG["ex8_n_head_kv"], FIG["ex8_n_ff"],
        FIG["ex8_n_vocab"])
    info = model_info([g])
    assert round(info["n_params"] / 1e6, 2) == FIG["ex8_model_params_M"]
    assert info["file_type"] == FIG["ex8_file_type_f32"]
    assert round(info["bpw"], 2) == FIG["ex8_bpw_f32"]
    assert "GGUF V%d" % g.version == FIG["ex8_file_format"]
    for spec in tensor_specs(m)[:6]:
        want = gen_tensor(m, spec)["data"]
        assert np.array_equal(g.stored(spec.name)["data"], want), spec.name
    # the split parts hold the same tensors, each once
    g3, where3 = open_model(three)
    assert sorted(where3) == sorted(where) and g3.get("split.count") == 3
    for name in ("blk.3.ffn_down.weight", "output.weight"):
        assert where3[name].tensor_bytes(name) == where[name].tensor_bytes(name)


def test_q8_0_blocks_match_page_example_2(tiny_files):
    _, _, _, q8, q8p = tiny_files
    g, _ = open_model(q8p)
    t = g.by_name["blk.0.ffn_gate.weight"]
    assert t["nbytes"] == FIG["ex2_ffn_gate_bytes"]["q8_0"]
    assert t["nbytes"] // t["dims"][1] == FIG["ex2_ffn_gate_row_bytes_q8_0"]
    want = gen_tensor(q8, "blk.0.ffn_gate.weight")
    got = g.stored("blk.0.ffn_gate.weight")
    assert np.array_equal(got["q"], want["q"]) and np.array_equal(got["scale"], want["scale"])
    assert model_info([g])["file_type"] == "mostly Q8_0"


def test_duplicate_across_parts(tmp_path):
    rec = ("a", W.T_F32, [4], np.zeros(4, np.float32).tobytes())
    W.write_gguf(str(tmp_path / "p1.gguf"), [], [rec])
    W.write_gguf(str(tmp_path / "p2.gguf"), [], [rec])
    with pytest.raises(GGUFError, match="duplicated"):
        open_model([str(tmp_path / "p1.gguf"), str(tmp_path / "p2.gguf")])
