"""The q8_0 decode products turn each int8 code into an f16 MFMA operand
without convert instructions: the weights hold each code as the byte q ^ 0x80
(= q + 128, flipped once at load), a byte permute places it under the f16
exponent byte 0x64, giving the f16 1024 + q + 128, and one packed f16
subtract of 1152 leaves q.  These tests check that
arithmetic on the host for every byte, and the permute selectors the kernel
source uses, with v_perm_b32's byte selection (selector values 0-3 pick bytes
of the second operand, 4-7 bytes of the first) modelled in Python."""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = os.path.join(ROOT, "llama_decode_ubatch_amd", "csrc", "kernels.hip")


def f16_from_bits(bits):
    return np.array(bits, dtype=np.uint16).view(np.float16)


def test_every_code_survives_the_exponent_trick():
    for b in range(256):
        q = int(np.int8(np.uint8(b)))
        v = f16_from_bits(0x6400 | (b ^ 0x80))
        assert float(v) == 1024 + q + 128
        # the subtract is exact in f16 (1024 + u and 1152 are both exact,
        # their difference is an integer of magnitude <= 128)
        d = np.float16(v) - np.float16(1152.0)
        assert d.dtype == np.float16 and float(d) == q


def v_perm_b32(src0, src1, sel):
    data = (int(src0) << 32) | int(src1)
    out = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 0xFF
        assert s < 8, "selector values past 7 produce constants, not used here"
        out |= ((data >> (8 * s)) & 0xFF) << (8 * i)
    return out


def kernel_selectors():
    text = open(KERNELS).read()
    m = re.search(r"u8x8_to_f16_1024\(uint32_t w0, uint32_t w1\) \{(.*?)\n\}", text, re.S)
    assert m, "conversion helper not found"
    calls = re.findall(r"r\[(\d)\] = __builtin_amdgcn_perm\((0x[0-9a-fA-F]+)u, (w[01]), (0x[0-9a-fA-F]+)u\);",
                       m.group(1))
    assert len(calls) == 4
    return [(int(i), int(c, 16), w, int(s, 16)) for i, c, w, s in calls]


def test_kernel_permutes_give_codes_in_element_order():
    rng = np.random.default_rng(7)
    calls = kernel_selectors()
    for _ in range(200):
        codes = rng.integers(-127, 128, size=8).astype(np.int8)
        words = codes.view(np.uint8).astype(np.uint32)
        w = {"w0": 0, "w1": 0}
        for k in range(4):
            w["w0"] |= int(words[k] ^ 0x80) << (8 * k)
            w["w1"] |= int(words[4 + k] ^ 0x80) << (8 * k)
        r = [0] * 4
        for i, const, src, sel in calls:
            r[i] = v_perm_b32(const, w[src], sel)
        halves = np.array(r, dtype=np.uint32).view(np.uint16)      # little-endian element order
        vals = f16_from_bits(halves).astype(np.float32) - 1152.0
        assert np.array_equal(vals, codes.astype(np.float32))
