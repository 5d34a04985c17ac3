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


# ------------------------------------------------- the library's reader
def lib_reader(path):
    from llama_decode_ubatch_amd.binding import Gguf
    return Gguf(path)


def oracle_items(g):
    out = []
    for k in g.keys:
        t, v = g.kv[k]
        if t == 8:
            v = v.encode("utf-8", errors="surrogateescape")
        elif t == 9:
            et, items = v
            if et == 9:
                v = (9, len(items))
            elif et == 8:
                v = (8, [x.encode("utf-8", errors="surrogateescape") for x in items])
            else:
                v = (et, [int(x) if et not in (6, 12) else float(x) for x in items])
        elif t in (6, 12):
            v = float(v)
        else:
            v = int(v)
        out.append((k, t, v))
    return out


def same_as_oracle(path):
    g, c = GGUF(path), lib_reader(path)
    assert c.version == g.version and c.data_offset == g.data_start
    assert c.items() == oracle_items(g)
    ct = c.tensors()
    assert [t["name"] for t in ct] == [t["name"] for t in g.tensors]
    for a, b in zip(ct, g.tensors):
        assert (a["dims"], a["type"], a["nbytes"]) == (b["dims"], b["type"], b["nbytes"])
        assert a["offset"] == g.data_start + b["offset"]
    for t in g.tensors:
        name = t["name"].encode("utf-8", errors="surrogateescape")
        assert c.lib.ubd_gguf_find_tensor(c.ptr, name) == g.tensors.index(t)
    assert c.find_key("no.such.key") == -1
    c.close()


def test_library_reader_matches_oracle_on_hand_file(tmp_path):
    path, _ = hand_file(tmp_path)
    same_as_oracle(path)


def test_library_reader_matches_oracle_on_every_value_type(tmp_path):
    kvs = [("u8", W.U8, 250), ("i8", W.I8, -5), ("u16", W.U16, 65000), ("i16", W.I16, -32000),
           ("u32", W.U32, 4000000000), ("i32", W.I32, -2000000000), ("f32", W.F32, 1.5),
           ("bool", W.BOOL, True), ("str", W.STR, "héllo 日本"), ("empty", W.STR, ""),
           ("u64", W.U64, 2 ** 63 - 1), ("i64", W.I64, -(2 ** 62)), ("f64", W.F64, -2.5e300),
           ("arr.i16", W.ARR, (W.I16, [-1, 2, -3])), ("arr.f64", W.ARR, (W.F64, [0.25, 1e-300])),
           ("arr.str", W.ARR, (W.STR, ["a", "", "bc"])), ("arr.empty", W.ARR, (W.U8, [])),
           ("arr.nested", W.ARR, (W.ARR, [(W.I32, [1, 2]), (W.STR, ["x"])])),
           ("general.alignment", W.U32, 64)]
    recs = [("m", W.T_BF16, [64, 3], np.arange(192, dtype=np.uint16).tobytes()),
            ("v", W.T_F16, [7], np.ones(7, np.float16).tobytes()),
            ("q", W.T_Q8_0, [64, 2], bytes(range(136)))]
    p = str(tmp_path / "types.gguf")
    W.write_gguf(p, kvs, recs, alignment=64)
    same_as_oracle(p)
    g = GGUF(p)
    assert g.alignment == 64 and g.data_start % 64 == 0 and [t["offset"] % 64 for t in g.tensors] == [0, 0, 0]


@pytest.mark.parametrize("kw", [dict(magic=b"GGUG"), dict(version=2), dict(version=4), dict(n_dims=5),
                                dict(ttype=99), dict(offset=8), dict(offset=32), dict(dup=True)])
def test_library_reader_rejects_what_the_oracle_rejects(tmp_path, kw):
    from llama_decode_ubatch_amd.binding import Gguf
    path, _ = hand_file(tmp_path, **kw)
    with pytest.raises(ValueError):
        Gguf(path)


def test_library_reader_rejects_every_truncation(tmp_path):
    from llama_decode_ubatch_amd.binding import Gguf
    path, raw = hand_file(tmp_path)
    for n in range(len(raw)):
        open(path, "wb").write(raw[:n])
        with pytest.raises(ValueError):
            Gguf(path)


def test_library_reader_survives_corrupted_counts(tmp_path):
    """Random bytes written over the header and metadata: the reader either
    accepts (then agrees with the oracle) or rejects, and never reads
    outside the file."""
    from llama_decode_ubatch_amd.binding import Gguf
    path, raw = hand_file(tmp_path)
    rng = np.random.default_rng(3)
    for trial in range(300):
        b = bytearray(raw)
        for _ in range(int(rng.integers(1, 4))):
            at = int(rng.integers(4, 200))
            b[at] = int(rng.integers(0, 256))
        open(path, "wb").write(bytes(b))
        try:
            g = GGUF(path)
        except GGUFError:
            g = None
        try:
            c = Gguf(path)
        except ValueError:
            c = None
        assert (g is None) == (c is None), trial
        if g is not None:
            same_as_oracle(path)


def test_library_model_info_matches_oracle(tiny_files):
    from llama_decode_ubatch_amd.binding import gguf_model_info
    m, one, three, q8, q8p = tiny_files
    for paths in (one, three, q8p):
        g, where = open_model(paths)
        info = model_info([GGUF(p) for p in paths])
        c = gguf_model_info(paths[0])
        assert c.n_files == len(paths) and c.n_tensors == len(where)
        assert c.n_params == info["n_params"] and c.file_bytes == info["file_bytes"]
        assert abs(c.bpw - info["bpw"]) < 1e-12
        assert ("all " if c.all_same else "mostly ") + {0: "F32", 8: "Q8_0"}[c.file_type] == info["file_type"]
        hp = hparams(g, where)
        for k in ("n_layer", "n_embd", "n_head", "n_head_kv", "n_ff", "n_vocab", "n_ctx_train"):
            assert getattr(c.hparams, k) == hp[k], k
        assert c.hparams.rms_eps == np.float32(hp["rms_eps"])
        assert c.hparams.rope_freq_base == np.float32(hp["rope_freq_base"])
    assert round(gguf_model_info(one[0]).n_params / 1e6, 2) == FIG["ex8_model_params_M"]


def test_split_model_errors(tmp_path, tiny_files):
    from llama_decode_ubatch_amd.binding import gguf_model_info
    m = tiny_files[0]
    paths = W.write_model_gguf(m, str(tmp_path / "s"), n_split=2)
    os.remove(paths[1])
    with pytest.raises(ValueError):
        gguf_model_info(paths[0])
