"""Pins for the oracle's decode (fp64 attention over the mixed BF16 / packed cache).

What fixes each part, independently of the oracle's own code:
* closed forms: one token, zero query, two tokens (sigmoid);
* every token protected (L <= 132): textbook attention, so it must equal
  torch's scaled_dot_product_attention and logsumexp in fp64;
* exactly representable cache values: quantization is lossless, so the decode
  over packed tokens must equal SDPA over the raw inputs;
* a 50-digit mpmath evaluation of the attention definition on tiny shapes;
* convexity of the output, split-K merging, and window-exit bookkeeping.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.oracle_helpers import oracle_cache, oracle_decode, oracle_decode_mq, u16

SCALE = synth.SOFTMAX_SCALE


def _inputs(lens, H, seed, **kw):
    return synth.build_cache_inputs(lens, H, seed, device="cpu", **kw)


def _dense_ref(cfg, inp, b, L):
    """Raw bf16 inputs of sequence b as fp64 (K = [c | k_rope], V = c)."""
    sel = (inp.seq_idx == b)
    c = inp.c_kv[sel].double()[:L]
    r = inp.k_rope[sel].double()[:L]
    return c, r


def _sdpa(q_lat, q_rope, c, r, scale):
    """torch SDPA (fp64, CPU) for all heads of one sequence + logsumexp."""
    q = torch.cat([q_lat, q_rope], dim=-1)[None, :, None, :]           # [1, H, 1, 576]
    k = torch.cat([c, r], dim=-1)[None, None].expand(1, q.shape[1], -1, -1)
    v = c[None, None].expand(1, q.shape[1], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0]
    lse = torch.logsumexp(scale * (q[0, :, 0] @ k[0, 0].T), dim=-1)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("L", [1, 2, 5, 64, 131, 132])
def test_all_protected_equals_sdpa(L):
    cfg = oracle.Cfg()
    H = 4
    inp = _inputs([L, max(1, L // 2)], H, seed=21)
    pages, sink, local = oracle_cache(cfg, inp, 2)
    out, lse = oracle_decode(cfg, inp, pages, sink, local, SCALE)
    for b, Lb in enumerate([L, max(1, L // 2)]):
        c, r = _dense_ref(cfg, inp, b, Lb)
        ro, rl = _sdpa(inp.q_lat[b].double(), inp.q_rope[b].double(), c, r, SCALE)
        np.testing.assert_allclose(out[b * H:(b + 1) * H], ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b * H:(b + 1) * H], rl, rtol=1e-12, atol=1e-12)


def _representable_inputs(lens, H, seed, c_bits, r_bits=4, group=32):
    """Inputs whose every quantization group (of `group` channels; the RoPE key
    is one group when narrower) is z + k*s with s a power of two and both
    extreme codes present, so the quantizer reproduces them exactly (and they
    are bf16)."""
    inp = _inputs(lens, H, seed)
    g = torch.Generator().manual_seed(seed)
    n = inp.c_kv.shape[0]

    def make(d, bits):
        qmax = (1 << bits) - 1
        w = min(group, d)
        G = d // w
        e = torch.randint(-6, 0, (n, G, 1), generator=g).double()
        s = 2.0 ** e
        m = torch.randint(-110, 100, (n, G, 1), generator=g).double()
        k = torch.randint(0, qmax + 1, (n, G, w), generator=g).double()
        k[:, :, 0] = 0
        k[:, :, 1] = qmax
        x = ((m + k) * s).reshape(n, d)
        xb = x.to(torch.bfloat16)
        assert torch.equal(xb.double(), x)
        return xb

    inp.c_kv = make(512, c_bits)
    inp.k_rope = make(64, r_bits)
    return inp


@pytest.mark.parametrize("c_bits,r_bits,group", [(4, 4, 32), (2, 4, 32), (4, 2, 32),
                                                 (2, 2, 64), (4, 4, 128), (4, 2, 64)])
def test_representable_cache_equals_unquantized(c_bits, r_bits, group):
    """Every group exactly representable: the packed copies dequantize to the
    input values, so the decode equals textbook attention on the BF16 values.
    With another group size the groups' extremes and steps would not match and
    the values would not round-trip."""
    cfg = oracle.Cfg(c_bits=c_bits, r_bits=r_bits, group=group)
    H = 3
    lens = [300, 133, 200]
    inp = _representable_inputs(lens, H, seed=5, c_bits=c_bits, r_bits=r_bits, group=group)
    pages, sink, local = oracle_cache(cfg, inp, 3)
    out, lse = oracle_decode(cfg, inp, pages, sink, local, SCALE)
    for b, L in enumerate(lens):
        c, r = _dense_ref(cfg, inp, b, L)
        ro, rl = _sdpa(inp.q_lat[b].double(), inp.q_rope[b].double(), c, r, SCALE)
        np.testing.assert_allclose(out[b * H:(b + 1) * H], ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b * H:(b + 1) * H], rl, rtol=1e-12, atol=1e-12)
        # and the packed copies alone (read every token from its page) match too
        for p in [4, 5, L - 129, L - 1, 0]:
            if p < 0:
                continue
            pt = inp.page_table.numpy()
            kc, kr = oracle.token_values(cfg, b, p, pages, pt, [10 ** 6] * 3, sink, local)
            np.testing.assert_array_equal(kc, c[p].numpy())
            np.testing.assert_array_equal(kr, r[p].numpy())


@pytest.mark.parametrize("c_bits,r_bits,group,hi", [(4, 4, 32, 0.5), (2, 2, 128, 5.0)])
def test_quantized_cache_differs_from_unquantized(c_bits, r_bits, group, hi):
    """Guard for the pin above: on ordinary data the packed tokens are lossy, so a
    decode that silently read BF16 everywhere would be caught here."""
    cfg = oracle.Cfg(c_bits=c_bits, r_bits=r_bits, group=group)
    inp = _inputs([600], 2, seed=6)
    pages, sink, local = oracle_cache(cfg, inp, 1)
    out, _ = oracle_decode(cfg, inp, pages, sink, local, SCALE)
    c, r = _dense_ref(cfg, inp, 0, 600)
    ro, _ = _sdpa(inp.q_lat[0].double(), inp.q_rope[0].double(), c, r, SCALE)
    rel = np.linalg.norm(out - ro) / np.linalg.norm(ro)
    assert 1e-3 < rel < hi  # 2-bit codes over 128-channel groups with outliers are coarse


def test_single_token_chunk_is_that_token():
    cfg = oracle.Cfg()
    H = 2
    inp = _inputs([400], H, seed=7)
    pages, sink, local = oracle_cache(cfg, inp, 1)
    pt = inp.page_table.numpy()
    ql = inp.q_lat[0].double().numpy()
    qr = inp.q_rope[0].double().numpy()
    for p in [0, 3, 4, 100, 271, 272, 399]:
        out, lse = oracle_decode(cfg, inp, pages, sink, local, SCALE, p_begin=p, p_end=p + 1)
        kc, kr = oracle.token_values(cfg, 0, p, pages, pt, [400], sink, local)
        for h in range(H):
            np.testing.assert_array_equal(out[h], kc)
            assert lse[h] == pytest.approx(SCALE * (ql[h] @ kc + qr[h] @ kr), rel=1e-13)


def test_zero_query_gives_mean_and_log_length():
    cfg = oracle.Cfg()
    L = 333
    inp = _inputs([L], 2, seed=8)
    inp.q_lat.zero_()
    inp.q_rope.zero_()
    pages, sink, local = oracle_cache(cfg, inp, 1)
    out, lse = oracle_decode(cfg, inp, pages, sink, local, SCALE)
    pt = inp.page_table.numpy()
    vals = np.stack([oracle.token_values(cfg, 0, p, pages, pt, [L], sink, local)[0]
                     for p in range(L)])
    np.testing.assert_allclose(out[0], vals.mean(0), rtol=1e-12, atol=1e-13)
    assert lse[0] == pytest.approx(math.log(L), rel=1e-14)


def test_two_tokens_sigmoid():
    cfg = oracle.Cfg()
    inp = _inputs([200], 2, seed=9)
    pages, sink, local = oracle_cache(cfg, inp, 1)
    pt = inp.page_table.numpy()
    p0, p1 = 10, 150  # one packed, one in the local window
    k0 = oracle.token_values(cfg, 0, p0, pages, pt, [200], sink, local)
    k1 = oracle.token_values(cfg, 0, p1, pages, pt, [200], sink, local)
    assert oracle.token_source(cfg, p0, 200) == 2 and oracle.token_source(cfg, p1, 200) == 1
    # a chunk [p0, p0+1) and [p1, p1+1) merged = attention over the two tokens
    o0, l0 = oracle_decode(cfg, inp, pages, sink, local, SCALE, p_begin=p0, p_end=p0 + 1)
    o1, l1 = oracle_decode(cfg, inp, pages, sink, local, SCALE, p_begin=p1, p_end=p1 + 1)
    for h in range(2):
        ql = inp.q_lat[0, h].double().numpy()
        qr = inp.q_rope[0, h].double().numpy()
        s0 = SCALE * (ql @ k0[0] + qr @ k0[1])
        s1 = SCALE * (ql @ k1[0] + qr @ k1[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        out, lse = oracle.combine(np.stack([o0[h], o1[h]]), [l0[h], l1[h]])
        np.testing.assert_allclose(out, w0 * k0[0] + (1 - w0) * k1[0], rtol=1e-12, atol=1e-13)
        assert lse == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), rel=1e-13)


def test_mpmath_definition_tiny():
    """Attention on tiny shapes against a 50-digit evaluation of the definition."""
    mpmath.mp.dps = 50
    cfg = oracle.Cfg(d_c=32, d_r=32, group=32, page_size=4, n_sink=1, n_local=2)
    for L in [1, 2, 3, 5, 8]:
        H = 2
        inp = _inputs([L], H, seed=30 + L, d_c=32, d_r=32, page=4)
        pages, sink, local = oracle_cache(cfg, inp, 1)
        out, lse = oracle_decode(cfg, inp, pages, sink, local, 0.3)
        pt = inp.page_table.numpy()
        toks = [oracle.token_values(cfg, 0, p, pages, pt, [L], sink, local) for p in range(L)]
        for h in range(H):
            ql = [mpmath.mpf(float(v)) for v in inp.q_lat[0, h].double()]
            qr = [mpmath.mpf(float(v)) for v in inp.q_rope[0, h].double()]
            sc = [mpmath.mpf("0.3") * (mpmath.fsum(a * mpmath.mpf(float(b))
                                                   for a, b in zip(ql, kc)) +
                                       mpmath.fsum(a * mpmath.mpf(float(b))
                                                   for a, b in zip(qr, kr)))
                  for kc, kr in toks]
            den = mpmath.fsum(mpmath.exp(s) for s in sc)
            ref = [mpmath.fsum(mpmath.exp(s) * mpmath.mpf(float(kc[i]))
                               for s, (kc, _) in zip(sc, toks)) / den for i in range(32)]
            np.testing.assert_allclose(out[h], [float(v) for v in ref], rtol=1e-13, atol=1e-14)
            # 0.3 is not exact in binary; the oracle uses the nearest double
            assert lse[h] == pytest.approx(float(mpmath.log(den)), rel=1e-12)


def test_output_in_convex_hull_and_empty_range():
    cfg = oracle.Cfg(c_bits=2)
    L = 500
    inp = _inputs([L], 4, seed=11)
    pages, sink, local = oracle_cache(cfg, inp, 1)
    out, lse = oracle_decode(cfg, inp, pages, sink, local, SCALE)
    pt = inp.page_table.numpy()
    vals = np.stack([oracle.token_values(cfg, 0, p, pages, pt, [L], sink, local)[0]
                     for p in range(L)])
    lo, hi = vals.min(0), vals.max(0)
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)
    o, l = oracle_decode(cfg, inp, pages, sink, local, SCALE, p_begin=L, p_end=L + 5)
    assert not o.any() and np.all(np.isneginf(l))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_merge_equals_single_pass(seed):
    cfg = oracle.Cfg()
    L = 777
    H = 3
    inp = _inputs([L], H, seed=40 + seed)
    pages, sink, local = oracle_cache(cfg, inp, 1)
    full, lfull = oracle_decode(cfg, inp, pages, sink, local, SCALE)
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, L + 1, size=int(rng.integers(1, 9))))
    bounds = [0, *cuts.tolist(), L, L]  # includes empty chunks
    parts = [oracle_decode(cfg, inp, pages, sink, local, SCALE, p_begin=a, p_end=b)
             for a, b in zip(bounds[:-1], bounds[1:])]
    for h in range(H):
        o, l = oracle.combine(np.stack([p[0][h] for p in parts]), [p[1][h] for p in parts])
        np.testing.assert_allclose(o, full[h], rtol=1e-12, atol=1e-13)
        assert l == pytest.approx(lfull[h], rel=1e-13)


def test_protected_set_boundaries():
    cfg = oracle.Cfg()
    src = lambda p, L: oracle.token_source(cfg, p, L)  # noqa: E731
    # L <= 132: every token protected
    for L in [1, 4, 5, 131, 132]:
        assert all(src(p, L) in (0, 1) for p in range(L))
    assert [src(p, 133) for p in (0, 3, 4, 5)] == [0, 0, 2, 1]
    assert [src(p, 1000) for p in (3, 4, 871, 872, 999)] == [0, 2, 2, 1, 1]
    # sink wins where the windows overlap
    assert src(2, 5) == 0


def test_window_exit_incremental_matches_bulk():
    """Write tokens one by one (lengths growing) and decode at every step near the
    window edge: each state must equal a from-scratch bulk write, and a packed copy
    never changes once written."""
    cfg = oracle.Cfg()
    H = 2
    Lmax = 140
    full = _inputs([Lmax], H, seed=12)
    D = cfg.d_c + cfg.d_r
    pages = np.zeros((full.num_pages, oracle.page_bytes(cfg)), np.uint8)
    sink = np.zeros((1, cfg.n_sink, D), np.uint16)
    local = np.zeros((1, cfg.n_local, D), np.uint16)
    pt = full.page_table.numpy()
    snapshots = {}
    for L in range(1, Lmax + 1):
        p = L - 1
        oracle.write(cfg, u16(full.c_kv[p:p + 1]), u16(full.k_rope[p:p + 1]), [0], [p], [L], pt,
                     pages, sink, local)
        snapshots[p] = pages.copy()
        if L in (1, 4, 5, 127, 128, 129, 131, 132, 133, 134, 140):
            sub = synth.CacheInputs(full.c_kv[:L], full.k_rope[:L], full.seq_idx[:L],
                                    full.pos[:L], torch.tensor([L], dtype=torch.int32),
                                    full.page_table, full.num_pages, full.q_lat, full.q_rope)
            bp, bs, bl = oracle_cache(cfg, sub, 1)
            o1, l1 = oracle_decode(cfg, sub, pages, sink, local, SCALE)
            o2, l2 = oracle_decode(cfg, sub, bp, bs, bl, SCALE)
            np.testing.assert_array_equal(o1, o2)
            np.testing.assert_array_equal(l1, l2)
            assert np.array_equal(pages, bp)
    # the packed bytes of every page slot are final as soon as the token is written
    assert np.array_equal(snapshots[Lmax - 1], pages)
    off = oracle.page_regions(cfg)
    per = [256, 32, 64, 8]  # bytes per slot in each region (C4R4)
    for p in range(Lmax):
        page = int(pt[0, p // 64])
        slot = p % 64
        for o, n in zip(off, per):
            a = o + slot * n
            assert np.array_equal(snapshots[p][page, a:a + n], pages[page, a:a + n])


@pytest.mark.parametrize("s_q", [1, 2, 3])
def test_multi_query_causal_equals_sdpa(s_q):
    """s_q query tokens over an all-protected cache (the last s_q tokens are the
    queries' own): query i attends to the first L - (s_q - 1 - i) tokens, which
    is SDPA with a bottom-right causal mask."""
    cfg = oracle.Cfg()
    H = 2
    lens = [9, 2, 1]
    inp = _inputs(lens, s_q * H, seed=61)
    pages, sink, local = oracle_cache(cfg, inp, len(lens))
    out, lse = oracle_decode_mq(cfg, inp, pages, sink, local, SCALE, s_q, H)
    for b, L in enumerate(lens):
        c, r = _dense_ref(cfg, inp, b, L)
        ql = inp.q_lat[b].double().reshape(s_q, H, -1)
        qr = inp.q_rope[b].double().reshape(s_q, H, -1)
        q = torch.cat([ql, qr], dim=-1).permute(1, 0, 2)[None]          # [1, H, s_q, 576]
        k = torch.cat([c, r], dim=-1)[None, None].expand(1, H, -1, -1)  # [1, H, L, 576]
        v = c[None, None].expand(1, H, -1, -1)
        pos = torch.arange(L)[None, :]
        lim = (L - (s_q - 1) + torch.arange(s_q))[:, None]             # exclusive limits
        mask = pos < lim                                                 # [s_q, L]
        for i in range(s_q):
            if int(lim[i]) <= 0:
                assert np.all(out[b, i] == 0) and np.all(np.isneginf(lse[b, i]))
                continue
            ro = torch.nn.functional.scaled_dot_product_attention(
                q[:, :, i:i + 1], k, v, attn_mask=mask[i:i + 1], scale=SCALE)[0, :, 0]
            s = SCALE * (q[0, :, i] @ k[0, 0].T)
            rl = torch.logsumexp(s.masked_fill(~mask[i], float("-inf")), dim=-1)
            np.testing.assert_allclose(out[b, i], ro.numpy(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, i], rl.numpy(), rtol=1e-12, atol=1e-12)


def test_compact_page_table_gives_the_same_rows():
    """A sequence decoded from a compact page table of its own (the long-context
    GPU tests and the sweep's CPU leg do this) gives the same rows as from the
    shared, shuffled page table of the whole batch: physical page ids do not
    enter the result."""
    from tests.oracle_helpers import oracle_sequence_rows
    lens = [300, 1000, 777]
    inp = synth.build_cache_inputs(lens, 4, seed=31)
    oc = oracle.Cfg(c_bits=4)
    pages, sink, local = oracle_cache(oc, inp, len(lens))
    full, full_lse = oracle.decode(oc, synth.SOFTMAX_SCALE, u16(inp.q_lat), u16(inp.q_rope), pages,
                                   inp.page_table.numpy(), inp.seq_lens.numpy(), sink, local,
                                   sel=[(1, h) for h in range(4)])
    m = inp.seq_idx == 1
    got, got_lse = oracle_sequence_rows(oc, inp.c_kv[m], inp.k_rope[m], inp.q_lat[1], inp.q_rope[1],
                                        1000, range(4), synth.SOFTMAX_SCALE)
    assert np.array_equal(full, got) and np.array_equal(full_lse, got_lse)
