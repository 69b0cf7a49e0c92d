"""The quantizer on exact ties, against hand-derived results
(tests/golden/quant_ties.txt): codes whose quotient (x - z) / s is k + 0.5 go
to the even code, an fp16 scale and an fp16 zero point that are exactly
halfway between two fp16 values go to the even one (the rounding reading of
the RTN quantizer; the cards page's Table 1 names plain round-to-nearest).
Rounding half up or away from zero, or truncating, fails these tests."""
import numpy as np
import pytest

import oracle
from tests import golden_ties

GROUPS = golden_ties.load()


def test_golden_file_covers_every_tie_kind():
    names = {g.name for g in GROUPS}
    assert {"t4_s025", "t4_negz", "t2_ties", "t4_stie", "t4_ztie"} <= names
    # the code ties really are ties of the formula: (x - z) / s = k + 0.5 exactly
    for g in GROUPS:
        if g.name in ("t4_s025", "t4_negz", "t2_ties", "t4_ztie"):
            s = oracle.f16_bits_to_f64(g.s16)
            z = oracle.f16_bits_to_f64(g.z16)
            t = (g.x.astype(np.float64) - z) / s
            assert np.any(t - np.floor(t) == 0.5), g.name


@pytest.mark.parametrize("g", GROUPS, ids=lambda g: g.name)
def test_quantize_group_on_ties(g):
    s16, z16, q = oracle.quantize_group(g.x, g.bits)
    assert s16 == g.s16, (g.name, hex(s16))
    assert z16 == g.z16, (g.name, hex(z16))
    assert np.array_equal(q, g.codes), (g.name, q.tolist())


@pytest.mark.parametrize("c_bits", [4, 2])
def test_writer_pages_on_ties(c_bits):
    """A whole token built from the tie groups goes through the oracle writer:
    the page holds the golden codes and (scale, zero) pairs."""
    cfg = oracle.Cfg(c_bits=c_bits, n_sink=0, n_local=0)
    gs = [g for g in GROUPS if g.bits == c_bits]
    r4 = [g for g in GROUPS if g.bits == 4]
    content = [gs[i % len(gs)] for i in range(16)]
    rope = [r4[0], r4[-1]]
    c = np.concatenate([g.x for g in content])[None]
    r = np.concatenate([g.x for g in rope])[None]
    pages = np.zeros((1, oracle.page_bytes(cfg)), np.uint8)
    sink = np.zeros((1, 1, 576), np.uint16)
    local = np.zeros((1, 1, 576), np.uint16)
    oracle.write(cfg, golden_ties.bf16_bits(c), golden_ties.bf16_bits(r), np.array([0]),
                 np.array([5]), np.array([6]), np.array([[0]]), pages, sink, local)
    codes = golden_ties.codes_from_page(pages[0], 5, c_bits, oracle.page_regions(cfg)[0])
    for gi, g in enumerate(content):
        assert np.array_equal(codes[gi], g.codes), (gi, g.name)
    off = oracle.page_regions(cfg)
    sz = pages[0, off[2] + 5 * 64: off[2] + 6 * 64].copy().view("<u2").reshape(16, 2)
    for gi, g in enumerate(content):
        assert (sz[gi, 0], sz[gi, 1]) == (g.s16, g.z16), (gi, g.name)
    rsz = pages[0, off[3] + 5 * 8: off[3] + 6 * 8].copy().view("<u2").reshape(2, 2)
    for gi, g in enumerate(rope):
        assert (rsz[gi, 0], rsz[gi, 1]) == (g.s16, g.z16), (gi, g.name)
