"""Pins for the oracle's paired BF16 cache and its simulated quantize-dequantize.

BF16 cache (the unquantized baseline of Figure 5(b) and Table 9): attention
over a paged BF16 cache is textbook attention over the token rows, so it must
equal torch's scaled_dot_product_attention and logsumexp in fp64 for any page
table, and must not depend on which physical pages the table names.

QDQ (Figure 3 caption): groups that the quantizer represents exactly come back
unchanged; every value is within half a quantization step (plus the fp16
rounding of scale and zero and the final bf16 rounding) of its input; and each
value equals the decode-side dequantization of the same token's packed copy,
rounded the same way.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.oracle_helpers import oracle_cache, u16

SCALE = synth.SOFTMAX_SCALE


def _bf16_cache(cfg, inp):
    D = cfg.d_c + cfg.d_r
    pages = np.full((inp.num_pages, cfg.page_size, D), 0x7FC0, np.uint16)  # NaN canary
    oracle.bf16_write(cfg, u16(inp.c_kv), u16(inp.k_rope), inp.seq_idx.numpy(),
                      inp.pos.numpy(), inp.page_table.numpy(), pages)
    return pages


def _sdpa(q_lat, q_rope, c, r, scale):
    q = torch.cat([q_lat, q_rope], dim=-1)[None, :, None, :]
    k = torch.cat([c, r], dim=-1)[None, None].expand(1, q.shape[1], -1, -1)
    v = c[None, None].expand(1, q.shape[1], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0]
    lse = torch.logsumexp(scale * (q[0, :, 0] @ k[0, 0].T), dim=-1)
    return out.numpy(), lse.numpy()


def test_bf16_page_bytes():
    assert oracle.bf16_page_bytes(oracle.Cfg()) == 64 * 576 * 2


@pytest.mark.parametrize("lens", [[1], [64, 65], [300, 7, 129], [1000, 0, 130]])
def test_bf16_decode_equals_sdpa(lens):
    cfg = oracle.Cfg()
    H = 4
    inp = synth.build_cache_inputs(lens, H, seed=31, device="cpu")
    pages = _bf16_cache(cfg, inp)
    out, lse = oracle.bf16_decode(cfg, SCALE, u16(inp.q_lat), u16(inp.q_rope), pages,
                                  inp.page_table.numpy(), inp.seq_lens.numpy())
    for b, L in enumerate(lens):
        rows = slice(b * H, (b + 1) * H)
        if L == 0:
            assert np.all(out[rows] == 0.0) and np.all(np.isneginf(lse[rows]))
            continue
        sel = inp.seq_idx == b
        c, r = inp.c_kv[sel].double(), inp.k_rope[sel].double()
        ro, rl = _sdpa(inp.q_lat[b].double(), inp.q_rope[b].double(), c, r, SCALE)
        np.testing.assert_allclose(out[rows], ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[rows], rl, rtol=1e-12, atol=1e-12)


def test_bf16_decode_ignores_physical_page_order():
    cfg = oracle.Cfg()
    lens = [500, 200]
    inp = synth.build_cache_inputs(lens, 2, seed=32, device="cpu", spare_pages=3)
    pages = _bf16_cache(cfg, inp)
    a = oracle.bf16_decode(cfg, SCALE, u16(inp.q_lat), u16(inp.q_rope), pages,
                           inp.page_table.numpy(), inp.seq_lens.numpy())
    # move every page to a new physical id and rewrite the table to match
    perm = np.random.default_rng(0).permutation(inp.num_pages)
    moved = np.empty_like(pages)
    moved[perm] = pages
    pt = inp.page_table.numpy().copy()
    pt[pt >= 0] = perm[pt[pt >= 0]]
    b = oracle.bf16_decode(cfg, SCALE, u16(inp.q_lat), u16(inp.q_rope), moved, pt,
                           inp.seq_lens.numpy())
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_bf16_decode_selected_rows():
    cfg = oracle.Cfg()
    inp = synth.build_cache_inputs([90, 40], 3, seed=33, device="cpu")
    pages = _bf16_cache(cfg, inp)
    args = (cfg, SCALE, u16(inp.q_lat), u16(inp.q_rope), pages, inp.page_table.numpy(),
            inp.seq_lens.numpy())
    full_o, full_l = oracle.bf16_decode(*args)
    sel = [(1, 2), (0, 1)]
    o, l = oracle.bf16_decode(*args, sel=sel)
    for k, (b, h) in enumerate(sel):
        np.testing.assert_array_equal(o[k], full_o[b * 3 + h])
        assert l[k] == full_l[b * 3 + h]


def _bf16_of(x: np.ndarray) -> np.ndarray:
    """float32 values known to be bf16-representable -> their bf16 bits."""
    u = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("c_bits,r_bits,group", [(4, 4, 32), (2, 4, 32), (2, 2, 64),
                                                 (4, 2, 128)])
def test_qdq_representable_groups_are_unchanged(c_bits, r_bits, group):
    cfg = oracle.Cfg(c_bits=c_bits, r_bits=r_bits, group=group)
    rng = np.random.default_rng(7)
    n = 6

    def rows(d, bits):
        qmax = (1 << bits) - 1
        w = min(group, d)
        out = np.zeros((n, d), np.float32)
        for t in range(n):
            for g in range(d // w):
                s = 2.0 ** int(rng.integers(-6, 2))
                z = int(rng.integers(-100, 100)) * s
                k = rng.integers(0, qmax + 1, w)
                k[0], k[1] = 0, qmax
                rng.shuffle(k)
                out[t, w * g:w * g + w] = z + k * s
        return out

    xc, xr = rows(cfg.d_c, c_bits), rows(cfg.d_r, r_bits)
    oc, orr = oracle.qdq(cfg, _bf16_of(xc), _bf16_of(xr))
    np.testing.assert_array_equal(oc, _bf16_of(xc))
    np.testing.assert_array_equal(orr, _bf16_of(xr))


@pytest.mark.parametrize("c_bits", [4, 2])
def test_qdq_error_bound(c_bits):
    cfg = oracle.Cfg(c_bits=c_bits)
    inp = synth.build_cache_inputs([200], 1, seed=34, device="cpu")
    x = inp.c_kv.double().numpy()
    oc, _ = oracle.qdq(cfg, u16(inp.c_kv), u16(inp.k_rope))
    xh = oracle.bf16_bits_to_f64(oc)
    g = x.reshape(x.shape[0], -1, 32)
    rng_ = g.max(-1) - g.min(-1)
    step = rng_ / ((1 << c_bits) - 1)
    # half a step; the fp16 zero (|lo| * 2^-11) and scale (2^-11 relative,
    # times the top code) roundings; the bf16 rounding of the result (2^-8)
    bound = (step / 2 + np.abs(g.min(-1)) * 2.0 ** -11 + rng_ * 2.0 ** -11
             + np.abs(g).max(-1) * 2.0 ** -8)
    err = np.abs(xh - x).reshape(g.shape).max(-1)
    assert np.all(err <= bound + 1e-12)


@pytest.mark.parametrize("c_bits,r_bits,group", [(4, 4, 32), (2, 4, 32), (4, 2, 64),
                                                 (2, 2, 128)])
def test_qdq_matches_dequantized_packed_copy(c_bits, r_bits, group):
    """qdq(x) equals the attention-side values of x's packed copy (read back
    through the page layout), rounded to fp32 and then to bf16."""
    cfg = oracle.Cfg(c_bits=c_bits, r_bits=r_bits, group=group, n_sink=0, n_local=0)
    L = 150
    inp = synth.build_cache_inputs([L], 1, seed=35, device="cpu")
    pages, sink, local = oracle_cache(cfg, inp, 1)
    oc, orr = oracle.qdq(cfg, u16(inp.c_kv), u16(inp.k_rope))

    def rnd(v):
        return np.array([oracle.f64_to_bf16_bits(float(np.float32(e))) for e in v], np.uint16)

    for p in (0, 1, 63, 64, 149):
        kc, kr = oracle.token_values(cfg, 0, p, pages, inp.page_table.numpy(),
                                     inp.seq_lens.numpy(), sink, local)
        np.testing.assert_array_equal(oc[p], rnd(kc))
        np.testing.assert_array_equal(orr[p], rnd(kr))


def test_qdq_constant_group():
    cfg = oracle.Cfg()
    x = np.full((1, 512), 1.5, np.float32)
    r = np.full((1, 64), -0.375, np.float32)
    oc, orr = oracle.qdq(cfg, _bf16_of(x), _bf16_of(r))
    np.testing.assert_array_equal(oc, _bf16_of(x))
    np.testing.assert_array_equal(orr, _bf16_of(r))
