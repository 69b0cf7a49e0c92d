"""Reader for tests/golden/quant_ties.txt: hand-derived quantizer results on
exact rounding ties (codes, fp16 scale and fp16 zero point)."""
import os
from dataclasses import dataclass

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_ties.txt")


@dataclass
class TieGroup:
    name: str
    bits: int
    x: np.ndarray       # float32 [32], every value exact in bf16
    s16: int
    z16: int
    codes: np.ndarray   # uint8 [32]


def _val(tok: str) -> float:
    return float.fromhex(tok) if "0x" in tok else float(tok)


def load():
    groups, cur = [], None
    with open(PATH) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            if key == "group":
                name, bits = val.split()
                cur = {"name": name, "bits": int(bits)}
                groups.append(cur)
            elif key == "x":
                cur["x"] = np.array([_val(t) for t in val.split()], np.float64)
            elif key in ("s16", "z16"):
                cur[key] = int(val, 16)
            elif key == "codes":
                cur["codes"] = np.array([int(t) for t in val.split()], np.uint8)
    out = []
    for g in groups:
        x = g["x"]
        assert x.shape == (32,) and g["codes"].shape == (32,), g["name"]
        x32 = x.astype(np.float32)
        assert np.array_equal(x32.astype(np.float64), x), g["name"]
        # exact in bf16: the low 16 bits of the fp32 pattern are zero
        assert not (x32.view(np.uint32) & 0xFFFF).any(), g["name"]
        out.append(TieGroup(g["name"], g["bits"], x32, g["s16"], g["z16"], g["codes"]))
    return out


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bf16 patterns of float32 values that are exact in bf16."""
    return (np.asarray(x32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def codes_from_page(page, slot, c_bits, content_offset=0, d_c=512):
    """Content codes of one token read back through the documented code order
    (channel 32 g + 8 j + 2 i + k: 16-byte chunk (j, g div u), word, bit
    16 k + b (4 e + i)); an independent reading of the page bytes."""
    b = c_bits
    n_groups_c = d_c // 32
    row_bytes = d_c * b // 8
    base = content_offset + slot * row_bytes
    words = np.asarray(page[base: base + row_bytes]).copy().view("<u4")
    u = 16 // b
    per_word = 4 // b
    codes = np.zeros((n_groups_c, 32), np.uint8)
    for g in range(n_groups_c):
        ld, gi = divmod(g, u)
        w_i, e = divmod(gi, per_word)
        for j in range(4):
            w = int(words[(u * b * (4 * ld + j) + 4 * w_i) // 4])
            for i in range(4):
                for k in range(2):
                    codes[g, 8 * j + 2 * i + k] = (w >> (16 * k + b * (4 * e + i))) & ((1 << b) - 1)
    return codes
