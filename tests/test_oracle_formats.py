"""Pins for the oracle's number-format helpers against library routines.

numpy's float16 cast is IEEE-754 round-to-nearest-even; torch's float32 ->
bfloat16 cast is round-to-nearest-even. Neither shares code with the oracle.
"""
import numpy as np
import torch

import oracle


def _np_f16_bits(x32: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return x32.astype(np.float16).view(np.uint16)


def test_f32_to_f16_matches_numpy_random_bits():
    rng = np.random.default_rng(0)
    # bit patterns spanning |x| from deep subnormal-in-fp16 to beyond fp16 max
    exps = rng.integers(90, 150, size=20000).astype(np.uint32)
    mans = rng.integers(0, 1 << 23, size=20000).astype(np.uint32)
    signs = rng.integers(0, 2, size=20000).astype(np.uint32)
    bits = (signs << 31) | (exps << 23) | mans
    xs = bits.view(np.float32)
    want = _np_f16_bits(xs)
    got = np.array([oracle.f32_to_f16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_f32_to_f16_ties_and_edges():
    # exact halfway cases between fp16 neighbours (normal and subnormal), the
    # overflow threshold and the smallest subnormal rounding boundaries
    cases = []
    for h in [0x0001, 0x0002, 0x03ff, 0x0400, 0x0401, 0x3c00, 0x3c01, 0x7bfe, 0x7bff]:
        lo = np.array([h], np.uint16).view(np.float16).astype(np.float64)[0]
        hi = np.array([h + 1], np.uint16).view(np.float16).astype(np.float64)[0]
        t = np.float32((lo + hi) / 2)  # exact in fp32
        cases += [t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1e9))]
    cases += [65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
              0.0, -0.0, float("inf"), -float("inf")]
    xs = np.array(cases, np.float32)
    want = _np_f16_bits(xs)
    got = np.array([oracle.f32_to_f16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want), list(zip(xs, got, want))


def test_f16_decode_all_patterns():
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_bits_to_f64(int(p)) for p in pats])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_f64_to_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                         np.array([0.0, 1.0, 1.00390625, 1.01171875, 3.3895313892515355e38])])
    xs32 = xs.astype(np.float32)
    want = torch.from_numpy(xs32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16_bits(float(x)) for x in xs32], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_widening_exact():
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x.double().numpy())
