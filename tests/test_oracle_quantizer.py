"""Pins for the oracle's quantizer, packing and page layout.

* brute force: every code is the nearest of the 2^b levels q*s + z (fp64),
  up to the fp32 evaluation of near-ties;
* representable groups round-trip exactly; constant groups give zero codes;
* hand-derived packed bytes (tests/golden) fix the code order and layout.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _levels(s16, z16, bits):
    s = oracle.f16_bits_to_f64(s16)
    z = oracle.f16_bits_to_f64(z16)
    return np.arange(1 << bits) * s + z, s


@pytest.mark.parametrize("n", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", ["normal", "outlier", "tiny", "shifted"])
def test_codes_are_nearest_level(bits, kind, n):
    rng = np.random.default_rng(10 + bits + n)
    n_bad = 0
    for trial in range(400 * 32 // n):
        x = rng.standard_normal(n)
        if kind == "outlier":
            x[rng.integers(0, n)] *= 10.0
        elif kind == "tiny":
            x *= 1e-3
        elif kind == "shifted":
            x = x * 0.1 + 5.0
        x = x.astype(np.float32)
        s16, z16, q = oracle.quantize_group(x, bits)
        lv, s = _levels(s16, z16, bits)
        assert s > 0
        d = np.abs(x.astype(np.float64)[:, None] - lv[None, :])
        best = np.argmin(d, axis=1)
        for i in range(n):
            if q[i] == best[i]:
                continue
            # only a near-tie (decided by fp32 rounding of (x - z) / s) may differ
            gap = abs(d[i, q[i]] - d[i, best[i]])
            if gap > 1e-5 * s:
                n_bad += 1
    assert n_bad == 0


@pytest.mark.parametrize("bits", [2, 4])
def test_reconstruction_error_bound(bits):
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = (rng.standard_normal(32) * rng.uniform(0.01, 20)).astype(np.float32)
        s16, z16, q = oracle.quantize_group(x, bits)
        lv, s = _levels(s16, z16, bits)
        xh = lv[q]
        # within half a step, plus the fp16 rounding of the zero point at the
        # bottom and of the scale accumulated over 2^b - 1 steps at the top
        z = oracle.f16_bits_to_f64(z16)
        slack = abs(float(x.min()) - z) + (1 << bits) * abs(
            s - (float(x.max()) - float(x.min())) / ((1 << bits) - 1))
        assert np.all(np.abs(x - xh) <= s / 2 + slack + 1e-12)


@pytest.mark.parametrize("n", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 4])
def test_representable_round_trip(bits, n):
    rng = np.random.default_rng(4 + n)
    qmax = (1 << bits) - 1
    for _ in range(200):
        e = int(rng.integers(-8, 3))
        s = 2.0 ** e
        m = int(rng.integers(-200, 200))
        z = m * s
        k = rng.integers(0, qmax + 1, n)
        k[rng.integers(0, n)] = 0
        k[rng.integers(0, n)] = qmax
        if k.min() != 0 or k.max() != qmax:
            k[0], k[1] = 0, qmax
        x = (z + k * s).astype(np.float32)
        s16, z16, q = oracle.quantize_group(x, bits)
        assert oracle.f16_bits_to_f64(s16) == s
        assert oracle.f16_bits_to_f64(z16) == z
        assert np.array_equal(q, k.astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("v", [0.0, 1.5, -3.25, 1e-3])
def test_constant_group(bits, v):
    x = np.full(32, v, np.float32)
    s16, z16, q = oracle.quantize_group(x, bits)
    assert s16 == 0
    assert z16 == int(np.float16(v).view(np.uint16))
    assert not q.any()


def test_scale_underflow_gives_zero_codes():
    # range so small that the fp16 scale rounds to zero
    x = np.full(32, 1.0, np.float32)
    x[3] = np.nextafter(np.float32(1.0), np.float32(2.0))
    s16, z16, q = oracle.quantize_group(x, 4)
    assert s16 == 0 and not q.any()


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":")
            out[k.strip()] = bytes(int(t, 16) for t in v.split())
    return out


def _write_one(cfg, c_vals, r_vals):
    def bf(v):
        import torch
        return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy(
        ).view(np.uint16).reshape(1, -1)
    B, max_pages = 1, 1
    pages = np.zeros((1, oracle.page_bytes(cfg)), np.uint8)
    D = cfg.d_c + cfg.d_r
    sink = np.zeros((B, max(cfg.n_sink, 1), D), np.uint16)
    local = np.zeros((B, max(cfg.n_local, 1), D), np.uint16)
    oracle.write(cfg, bf(c_vals), bf(r_vals), [0], [0], [1], np.zeros((1, 1), np.int32), pages,
                 sink, local)
    return pages[0]


def test_golden_packing_c4r4():
    cfg = oracle.Cfg(d_c=128, d_r=32, c_bits=4, r_bits=4, group=32, page_size=2, n_sink=0,
                     n_local=0)
    cvals = [((c % 32) + 3 * (c // 32)) % 16 * 0.5 for c in range(128)]
    rvals = [(i % 16) * 0.5 for i in range(32)]
    page = _write_one(cfg, cvals, rvals)
    g = _read_golden("pack_c4r4_tiny.txt")
    off = oracle.page_regions(cfg)
    assert off == [0, 2 * 64, 2 * 80, 2 * 96]
    assert oracle.page_bytes(cfg) == 2 * 100
    assert bytes(page[off[0]:off[0] + 64]) == g["content_codes"]
    assert bytes(page[off[1]:off[1] + 16]) == g["rope_codes"]
    assert bytes(page[off[2]:off[2] + 16]) == g["content_sz"]
    assert bytes(page[off[3]:off[3] + 4]) == g["rope_sz"]
    # slot 1 was never written
    assert not page[64:128].any()


def test_golden_packing_c2():
    cfg = oracle.Cfg(d_c=64, d_r=32, c_bits=2, r_bits=4, group=32, page_size=1, n_sink=0,
                     n_local=0)
    vals = [(c % 4) * 0.25 for c in range(32)] + [(c // 8) * 0.25 for c in range(32)]
    page = _write_one(cfg, vals, [0.0] * 32)
    g = _read_golden("pack_c2_tiny.txt")
    off = oracle.page_regions(cfg)
    assert bytes(page[off[0]:off[0] + 16]) == g["content_codes"]
    assert bytes(page[off[2]:off[2] + 8]) == g["content_sz"]


def test_golden_packing_c2r2_group64():
    """2-bit RoPE codes and a 64-channel quantization group (tests/golden)."""
    cfg = oracle.Cfg(d_c=64, d_r=64, c_bits=2, r_bits=2, group=64, page_size=1, n_sink=0,
                     n_local=0)
    cvals = [(c % 4) * 0.25 for c in range(32)] + [(c // 8) * 0.5 for c in range(32)]
    rvals = [float(c % 4) for c in range(32)] + [float(3 - c % 4) for c in range(32)]
    page = _write_one(cfg, cvals, rvals)
    g = _read_golden("pack_c2r2_g64_tiny.txt")
    off = oracle.page_regions(cfg)
    assert off == [0, 16, 32, 36] and oracle.page_bytes(cfg) == 40
    assert bytes(page[0:16]) == g["content_codes"]
    assert bytes(page[16:32]) == g["rope_codes"]
    assert bytes(page[32:36]) == g["content_sz"]
    assert bytes(page[36:40]) == g["rope_sz"]


def test_golden_packing_c4r4_group128():
    """A 128-channel group over the content and a RoPE vector narrower than
    the group, which forms one group of its own width (tests/golden)."""
    cfg = oracle.Cfg(d_c=128, d_r=64, c_bits=4, r_bits=4, group=128, page_size=1, n_sink=0,
                     n_local=0)
    cvals = [float(c % 4 + 4 * (c // 32)) for c in range(128)]
    rvals = [(c % 4) * 0.5 for c in range(32)] + [(12 + c % 4) * 0.5 for c in range(32)]
    page = _write_one(cfg, cvals, rvals)
    g = _read_golden("pack_c4r4_g128_tiny.txt")
    off = oracle.page_regions(cfg)
    assert off == [0, 64, 96, 100] and oracle.page_bytes(cfg) == 104
    assert bytes(page[0:64]) == g["content_codes"]
    assert bytes(page[64:96]) == g["rope_codes"]
    assert bytes(page[96:100]) == g["content_sz"]
    assert bytes(page[100:104]) == g["rope_sz"]


@pytest.mark.parametrize("c_bits,r_bits,group,per_token", [
    (4, 4, 64, 256 + 32 + 8 * 4 + 1 * 4), (4, 4, 128, 256 + 32 + 4 * 4 + 1 * 4),
    (4, 2, 32, 256 + 16 + 16 * 4 + 2 * 4), (2, 2, 32, 128 + 16 + 16 * 4 + 2 * 4),
    (2, 2, 128, 128 + 16 + 4 * 4 + 1 * 4), (2, 4, 64, 128 + 32 + 8 * 4 + 1 * 4)])
def test_page_sizes_of_the_variant_layouts(c_bits, r_bits, group, per_token):
    """Code bytes d * bits / 8 plus one 4-byte (scale, zero) pair per group (the
    64-channel RoPE key is one group when the group is 128), per token."""
    cfg = oracle.Cfg(c_bits=c_bits, r_bits=r_bits, group=group)
    assert oracle.page_bytes(cfg) == 64 * per_token
    cc, rc = 512 * c_bits // 8, 64 * r_bits // 8
    assert oracle.page_regions(cfg) == [0, 64 * cc, 64 * (cc + rc),
                                        64 * (cc + rc + 4 * (512 // group))]


def test_page_sizes_of_the_workload_layouts():
    # 512 content + 64 RoPE channels, groups of 32, fp16 (scale, zero) per group:
    # C4R4 = 256 + 32 + 16*4 + 2*4 = 360 B/token, C2R4 = 128 + 32 + 64 + 8 = 232 B/token
    c4 = oracle.Cfg()
    c2 = oracle.Cfg(c_bits=2)
    assert oracle.page_bytes(c4) == 64 * 360 == 23040
    assert oracle.page_bytes(c2) == 64 * 232 == 14848
    assert oracle.page_regions(c4) == [0, 16384, 18432, 22528]
    assert oracle.page_regions(c2) == [0, 8192, 10240, 14336]


@pytest.mark.parametrize("c_bits", [4, 2])
def test_code_order_as_documented(c_bits):
    """The content code row follows the order include/mla_lowbit.h states:
    channel 32 g + 8 j + 2 i + k sits in 16-byte chunk (j, g div (16 / c_bits)),
    word (g mod 4) for 4-bit or ((g mod 8) div 2) for 2-bit, at bit 16 k + 4 i
    (4-bit) or 16 k + 8 (g mod 2) + 2 i (2-bit)."""
    cfg = oracle.Cfg(c_bits=c_bits, n_sink=0, n_local=0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 512)).astype(np.float32)
    xr = rng.standard_normal((1, 64)).astype(np.float32)

    def bf16(a):
        u = a.view(np.uint32)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

    pages = np.zeros((1, oracle.page_bytes(cfg)), np.uint8)
    sink = np.zeros((1, 1, 576), np.uint16)
    local = np.zeros((1, 1, 576), np.uint16)
    oracle.write(cfg, bf16(x), bf16(xr), np.array([0]), np.array([0]), np.array([1]),
                 np.array([[0]]), pages, sink, local)
    off = oracle.page_regions(cfg)
    words = pages[0, off[0]:off[0] + 512 * c_bits // 8].copy().view("<u4")
    for g in range(16):
        xs = (bf16(x)[0, 32 * g:32 * g + 32].astype(np.uint32) << 16).view(np.float32)
        _, _, q = oracle.quantize_group(xs, c_bits)
        for j in range(4):
            for i in range(4):
                for k in range(2):
                    if c_bits == 4:
                        w, bit, m = words[4 * (4 * (g // 4) + j) + g % 4], 16 * k + 4 * i, 15
                    else:
                        w, bit, m = (words[4 * (4 * (g // 8) + j) + (g % 8) // 2],
                                     16 * k + 8 * (g % 2) + 2 * i, 3)
                    assert (int(w) >> bit) & m == q[8 * j + 2 * i + k]
