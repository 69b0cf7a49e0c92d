"""GPU parity: the HIP writer and decode (called through the C ABI) against the
CPU oracle on the same seeded inputs.

* writer: packed pages, sink and local buffers bit-exact (canary-filled
  buffers, so bytes outside written slots must keep their canary value);
* decode: rel-L2 <= 2e-3, |delta| / max(1, |ref|) <= 1e-2 and lse |delta| <= 1e-3
  against the fp64 oracle, on edge lengths (all-protected, window edges, ragged
  last pages, empty sequences), both code widths and H in {16, 128}; at the
  full workload sizes on sampled (sequence, head) rows in the same launch
  configuration the bench times;
* multi-query decode (s_q query tokens per sequence, causal) against the
  oracle's per-token ranges; s_q = 1 is bit-identical to the plain decode;
* other sink / window sizes (none, a page-wide sink, a five-page window,
  single tokens), including a serving step that opens new pages.
"""
import math

import numpy as np
import pytest
import torch

import bit_mla_kv_lowbit_amd as mla
import oracle
import synth
from tests.gpu_helpers import (DEV, assert_decode_ok, gpu_cache, gpu_decode, ocfg_of, u16)
from tests.oracle_helpers import oracle_cache, oracle_decode, oracle_decode_mq, oracle_sequence_rows

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 3, 4, 5, 63, 64, 65, 131, 132, 133, 195, 196, 197, 1000, 0]


def _cfg(c_bits):
    return mla.Config(c_bits=c_bits)


@pytest.mark.parametrize("c_bits", [4, 2])
def test_writer_bit_exact_with_canaries(c_bits):
    cfg = _cfg(c_bits)
    lens = [1024, 1, 3, 4, 5, 63, 64, 65, 131, 132, 133, 197, 300]
    inp = synth.build_cache_inputs(lens, 16, seed=77 + c_bits, device="cpu", spare_pages=3)
    print(f"[case] writer c_bits={c_bits} lens={lens}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens), canary=0xA5)
    torch.cuda.synchronize()
    op, osink, olocal = oracle_cache(ocfg_of(cfg), inp, len(lens), canary=0xA5)
    assert np.array_equal(pages.cpu().numpy(), op)
    assert np.array_equal(u16(sink), osink)
    assert np.array_equal(u16(local), olocal)


def test_writer_degenerate_groups():
    """Constant groups, exact zeros and tiny ranges whose fp16 scale underflows."""
    cfg = _cfg(4)
    inp = synth.build_cache_inputs([200], 16, seed=5, device="cpu")
    c = inp.c_kv.float()
    c[0:50, 0:32] = 1.5                       # constant group
    c[50:60, 32:64] = 0.0                     # all-zero group
    c[60:70, 64:96] = 1.0
    c[60:70, 64] = 1.0078125                  # range 2^-7 / 15 is still normal fp16
    c[70:80, 96:128] = 1e-4 * torch.randn(10, 32)  # fp16-subnormal scales
    c[80:90, 128:160] = -0.0
    inp.c_kv = c.to(torch.bfloat16)
    print("[case] writer degenerate groups", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, 1)
    torch.cuda.synchronize()
    op, osink, olocal = oracle_cache(ocfg_of(cfg), inp, 1)
    assert np.array_equal(pages.cpu().numpy(), op)
    assert np.array_equal(u16(local), olocal)


@pytest.mark.parametrize("c_bits", [4, 2])
def test_writer_signed_zero_ties(c_bits):
    """+0 and -0 tie as a group's minimum (or maximum) in different 8-channel
    sub-blocks: the earlier channel decides the zero point's sign bit, as in
    the oracle's scan in channel order."""
    cfg = _cfg(c_bits)
    inp = synth.build_cache_inputs([64], 16, seed=6, device="cpu")
    c = inp.c_kv.float().abs() + 0.5                  # positive groups ...
    r = -(inp.k_rope.float().abs() + 0.5)             # ... and negative RoPE groups
    for t in range(64):
        g = t % 16
        a_, b_ = (3, 20) if t % 2 else (20, 3)        # earlier channel first or second
        c[t, 32 * g + a_] = 0.0
        c[t, 32 * g + b_] = -0.0
        r[t, 32 * (t % 2) + (5 if t % 4 < 2 else 29)] = -0.0
        r[t, 32 * (t % 2) + (29 if t % 4 < 2 else 5)] = 0.0
    inp.c_kv = c.to(torch.bfloat16)
    inp.k_rope = r.to(torch.bfloat16)
    print(f"[case] writer signed-zero ties c_bits={c_bits}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, 1)
    torch.cuda.synchronize()
    op, osink, olocal = oracle_cache(ocfg_of(cfg), inp, 1)
    assert np.array_equal(pages.cpu().numpy(), op)


@pytest.mark.parametrize("c_bits", [4, 2])
def test_writer_exact_ties(c_bits):
    """Groups whose code quotients, fp16 scale or fp16 zero point lie exactly on
    a rounding tie (hand-derived results in tests/golden/quant_ties.txt): the
    GPU writer's pages are bit-identical to the oracle's and hold the golden
    codes and (scale, zero) pairs, ties going to the even value."""
    from tests import golden_ties
    groups = golden_ties.load()
    gs = [g for g in groups if g.bits == c_bits]
    r4 = [g for g in groups if g.bits == 4]
    cfg = _cfg(c_bits)
    n = 64
    content = [[gs[(i + t) % len(gs)] for i in range(16)] for t in range(n)]
    rope = [[r4[t % len(r4)], r4[(t + 1) % len(r4)]] for t in range(n)]
    c = np.stack([np.concatenate([g.x for g in row]) for row in content])
    r = np.stack([np.concatenate([g.x for g in row]) for row in rope])
    inp = synth.build_cache_inputs([n], 16, seed=8, device="cpu")
    inp.c_kv = torch.from_numpy(c).to(torch.bfloat16)
    inp.k_rope = torch.from_numpy(r).to(torch.bfloat16)
    print(f"[case] writer exact ties c_bits={c_bits}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, 1, canary=0x3C)
    torch.cuda.synchronize()
    op, osink, olocal = oracle_cache(ocfg_of(cfg), inp, 1, canary=0x3C)
    gp = pages.cpu().numpy()
    assert np.array_equal(gp, op)
    assert np.array_equal(u16(sink), osink)
    assert np.array_equal(u16(local), olocal)
    oc = ocfg_of(cfg)
    off = oracle.page_regions(oc)
    pid = int(inp.page_table[0, 0])
    for t in range(n):
        codes = golden_ties.codes_from_page(gp[pid], t, c_bits, off[0])
        sz = gp[pid, off[2] + 64 * t: off[2] + 64 * (t + 1)].copy().view("<u2").reshape(16, 2)
        for gi, g in enumerate(content[t]):
            assert np.array_equal(codes[gi], g.codes), (t, gi, g.name)
            assert (int(sz[gi, 0]), int(sz[gi, 1])) == (g.s16, g.z16), (t, gi, g.name)
        rsz = gp[pid, off[3] + 8 * t: off[3] + 8 * (t + 1)].copy().view("<u2").reshape(2, 2)
        for gi, g in enumerate(rope[t]):
            assert (int(rsz[gi, 0]), int(rsz[gi, 1])) == (g.s16, g.z16), (t, gi, g.name)


@pytest.mark.parametrize("c_bits", [4, 2])
@pytest.mark.parametrize("H", [16, 128])
def test_decode_edge_lengths(c_bits, H):
    cfg = _cfg(c_bits)
    inp = synth.build_cache_inputs(EDGE_LENS, H, seed=300 + H + c_bits, device="cpu")
    print(f"[case] decode edges c_bits={c_bits} H={H}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(EDGE_LENS))
    out, lse = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, len(EDGE_LENS))
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out, lse, ref, ref_lse, label=f"edges c{c_bits} H{H}")
    # the empty sequence gives zeros and -inf
    b0 = EDGE_LENS.index(0)
    assert not out[b0].float().abs().sum().item()
    assert torch.isneginf(lse[b0]).all()


@pytest.mark.parametrize("c_bits,H", [(4, 16), (2, 16), (4, 128)])
def test_decode_full_and_short_rows_in_one_batch(c_bits, H):
    """Sequences that fill their page-table row next to shorter ones: the
    decode first reads the page ids of the range a full row would give and
    reads them again when the length says otherwise, so both cases (and an
    empty sequence) meet in one launch."""
    lens = [4096, 4000, 4096, 64, 4033, 4096, 0, 4095]
    cfg = _cfg(c_bits)
    inp = synth.build_cache_inputs(lens, H, seed=77 + H + c_bits, device="cpu")
    assert inp.page_table.shape[1] * 64 == max(lens)
    print(f"[case] decode full/short rows c_bits={c_bits} H={H}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens))
    out, lse = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, len(lens))
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out, lse, ref, ref_lse, label=f"full/short rows c{c_bits} H{H}")
    assert torch.isneginf(lse[lens.index(0)]).all()


def test_decode_single_range_writes_output_directly():
    """64 short sequences at H = 128 (1..300 tokens): most of them fall inside
    one chunk of the length-aware split, whose workgroup writes out / lse
    itself; the rest are merged from their chunk partials."""
    cfg = _cfg(4)
    lens = [(37 * b) % 300 + 1 for b in range(64)]
    inp = synth.build_cache_inputs(lens, 128, seed=61, device="cpu")
    # the H = 128 workspace: per-sequence chunk bounds (int2, padded to 256 B)
    # and (128 chunks + 64 sequences) partial slots of 128 rows (lse + 512 fp16)
    assert mla.decode_workspace_bytes(cfg, 64, 128, inp.page_table.shape[1]) == \
        512 + (128 + 64) * 128 * 1028
    print("[case] decode single range B64 H128", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens))
    out, lse = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, len(lens))
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out, lse, ref, ref_lse, label="single range")


@pytest.mark.parametrize("H", [16, 128])
def test_decode_rescales_when_scores_jump(H):
    """RoPE keys of later tokens scaled up so their scores exceed the running
    reference max by far more than the lazy-rescale threshold (2^8)
    mid-sequence and inside one page range: the reference max moves, O and l
    are rescaled. Token 1500 sits in the second half of a 32-token step, so at
    H = 128 one token block of that step moves its max and the other does not.
    Only the RoPE part is scaled: the content latent is also the value, and
    larger values would only test the fp16 rounding of the value tile."""
    cfg = _cfg(4)
    lens = [3000, 700]
    inp = synth.build_cache_inputs(lens, H, seed=23, device="cpu")
    k = inp.k_rope.float()
    # tokens 1500.. of sequence 0 and 400.. of sequence 1 (packed and window)
    big = torch.zeros(k.shape[0], dtype=torch.bool)
    big[1500:3000] = True
    big[3000 + 400:] = True
    k[big] *= 12.0
    inp.k_rope = k.to(torch.bfloat16)
    # the jump, in log2 units, of every head of sequence 0 (from the unquantized
    # inputs) is well past the threshold
    S = (inp.q_lat[0].float() @ inp.c_kv[:3000].float().T
         + inp.q_rope[0].float() @ k[:3000].T) * (synth.SOFTMAX_SCALE / math.log(2.0))
    jump = S[:, 1500:].max(1).values - S[:, :1500].max(1).values
    assert jump.min().item() > 10.0, jump.min().item()
    print(f"[case] decode score jumps H={H}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens))
    out, lse = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, len(lens))
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out, lse, ref, ref_lse, label=f"score jumps H{H}")


def test_decode_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    cfg = _cfg(wl.c_bits)
    inp, _ = synth.workload_inputs(wl, device="cpu")
    print("[case] tiny workload", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, wl.B)
    out, lse = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, wl.B)
    assert np.array_equal(pages.cpu().numpy(), op)
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out, lse, ref, ref_lse, label="tiny")


def test_decode_deterministic():
    cfg = _cfg(4)
    inp = synth.build_cache_inputs([3000, 700], 16, seed=9, device="cpu")
    pages, sink, local = gpu_cache(cfg, inp, 2)
    o1, l1 = gpu_decode(cfg, inp, pages, sink, local)
    o2, l2 = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_graph_replay_matches_eager():
    """A decode captured in a HIP graph and replayed several times, with eager
    work on the same buffers between replays, gives the eager result each time."""
    cfg = _cfg(4)
    inp = synth.build_cache_inputs([5000, 130, 2100], 16, seed=13, device="cpu")
    pages, sink, local = gpu_cache(cfg, inp, 3)
    g = lambda t: t.to(DEV)  # noqa: E731
    ql, qr, pt, sl = g(inp.q_lat), g(inp.q_rope), g(inp.page_table), g(inp.seq_lens)
    ws = torch.empty(max(16, mla.decode_workspace_bytes(cfg, 3, 16, pt.shape[1])),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(3, 16, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(3, 16, dtype=torch.float32, device=DEV)

    def run(stream=None):
        mla.decode(cfg, ql, qr, pages, pt, sl, sink, local, synth.SOFTMAX_SCALE, out=out,
                   lse=lse, workspace=ws, stream=stream)

    run()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        run(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for k in range(4):
        out.fill_(7.0)
        lse.fill_(-1.0)
        ws.fill_(0xFF)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {k}"
        assert torch.equal(lse, ref_l), f"replay {k}"
        run()  # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))


def test_writer_drops_tokens_outside_the_table():
    """Tokens of no sequence or beyond the page table are not written; the
    valid ones are bit-exact."""
    cfg = _cfg(4)
    oc = ocfg_of(cfg)
    inp = synth.build_cache_inputs([200, 64], 16, seed=17, device="cpu")
    B, max_pages = 2, inp.page_table.shape[1]
    op, osink, olocal = oracle_cache(oc, inp, B)
    n = inp.seq_idx.numel()
    bad_seq = torch.tensor([B, -1, 0, 1, 0], dtype=torch.int32)
    bad_pos = torch.tensor([5, 5, max_pages * 64, -3, 1 << 30], dtype=torch.int32)
    pick = torch.tensor([3, 7, 11, 100, 150])
    c_kv = torch.cat([inp.c_kv, inp.c_kv[pick]])
    k_rope = torch.cat([inp.k_rope, inp.k_rope[pick]])
    seq_idx = torch.cat([inp.seq_idx, bad_seq])
    pos = torch.cat([inp.pos, bad_pos])
    pages, sink, local = mla.allocate_cache(cfg, B, inp.num_pages, DEV)
    g = lambda t: t.to(DEV)  # noqa: E731
    mla.write(cfg, g(c_kv), g(k_rope), g(seq_idx), g(pos), g(inp.seq_lens), g(inp.page_table),
              pages, sink, local)
    torch.cuda.synchronize()
    assert n + 5 == seq_idx.numel()
    assert np.array_equal(pages.cpu().numpy(), op)
    assert np.array_equal(u16(sink), osink)
    assert np.array_equal(u16(local), olocal)


def test_serving_steps_across_the_window_edge():
    """Fused write+decode steps one token at a time as the sequences cross the
    sink/local boundaries; each step equals a from-scratch oracle build."""
    cfg = _cfg(4)
    oc = ocfg_of(cfg)
    H = 16
    start = [120, 1, 60]
    n_steps = 16
    final = [s + n_steps for s in start]
    full = synth.build_cache_inputs(final, H, seed=41, device="cpu")
    B = len(start)
    pages, sink, local = mla.allocate_cache(cfg, B, full.num_pages, DEV)
    # bulk-write the first `start[b]` tokens
    keep = torch.cat([torch.arange(s) + sum(final[:b]) for b, s in enumerate(start)])
    pt = full.page_table.to(DEV)
    mla.write(cfg, full.c_kv[keep].to(DEV), full.k_rope[keep].to(DEV),
              full.seq_idx[keep].to(DEV), full.pos[keep].to(DEV),
              torch.tensor(start, dtype=torch.int32, device=DEV), pt, pages, sink, local)
    q_lat, q_rope = full.q_lat.to(DEV), full.q_rope.to(DEV)
    for k in range(n_steps):
        L = [s + k + 1 for s in start]
        idx = torch.tensor([sum(final[:b]) + s + k for b, s in enumerate(start)])
        seq_lens = torch.tensor(L, dtype=torch.int32)
        out, lse = mla.write_decode(cfg, full.c_kv[idx].to(DEV), full.k_rope[idx].to(DEV),
                                    (seq_lens - 1).to(DEV), q_lat, q_rope, pages, pt,
                                    seq_lens.to(DEV), sink, local, synth.SOFTMAX_SCALE)
        torch.cuda.synchronize()
        # from-scratch oracle at these lengths
        sel = torch.cat([torch.arange(l) + sum(final[:b]) for b, l in enumerate(L)])
        sub = synth.CacheInputs(full.c_kv[sel], full.k_rope[sel], full.seq_idx[sel],
                                full.pos[sel], seq_lens, full.page_table, full.num_pages,
                                full.q_lat, full.q_rope)
        op, osink, olocal = oracle_cache(oc, sub, B)
        ref, ref_lse = oracle_decode(oc, sub, op, osink, olocal, synth.SOFTMAX_SCALE)
        assert_decode_ok(out, lse, ref, ref_lse, label=f"step {k} L={L}")
        # every packed copy written so far is bit-exact (window exits re-quantize nothing)
        assert np.array_equal(pages.cpu().numpy(), op)


def _full_workload(name, n_seq, n_head, seed_rows=0):
    wl = synth.WORKLOADS[name]
    cfg = _cfg(wl.c_bits)
    oc = ocfg_of(cfg)
    print(f"[case] full workload {name}: generating on the GPU", flush=True)
    inp, step = synth.workload_inputs(wl, device=DEV)
    pages, sink, local = mla.allocate_cache(cfg, wl.B, inp.num_pages, DEV)
    pre_lens = inp.seq_lens
    mla.write(cfg, inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, pre_lens, inp.page_table, pages,
              sink, local)
    if step is None:
        out, lse = mla.decode(cfg, inp.q_lat, inp.q_rope, pages, inp.page_table, pre_lens, sink,
                              local, synth.SOFTMAX_SCALE)
        lens = pre_lens
    else:
        out, lse = mla.write_decode(cfg, step.c_kv, step.k_rope, step.pos, inp.q_lat, inp.q_rope,
                                    pages, inp.page_table, step.seq_lens, sink, local,
                                    synth.SOFTMAX_SCALE)
        lens = step.seq_lens
    torch.cuda.synchronize()
    print(f"[case] full workload {name}: GPU done, oracle on sampled rows", flush=True)
    # sampled sequences: shortest, longest and random others
    lens_h = lens.cpu().numpy()
    rng = np.random.default_rng(seed_rows)
    seqs = {int(np.argmin(lens_h)), int(np.argmax(lens_h))}
    while len(seqs) < min(n_seq, wl.B):
        seqs.add(int(rng.integers(0, wl.B)))
    seqs = sorted(seqs)
    rows = [(b, int(h)) for b in seqs for h in sorted(rng.choice(wl.H, n_head, replace=False))]
    # oracle cache for the sampled sequences only (same page ids)
    mask = torch.zeros(inp.seq_idx.numel(), dtype=torch.bool, device=DEV)
    for b in seqs:
        mask |= inp.seq_idx == b
    sub = synth.CacheInputs(inp.c_kv[mask].cpu(), inp.k_rope[mask].cpu(), inp.seq_idx[mask].cpu(),
                            inp.pos[mask].cpu(), pre_lens.cpu(), inp.page_table.cpu(),
                            inp.num_pages, inp.q_lat.cpu(), inp.q_rope.cpu())
    op, osink, olocal = oracle_cache(oc, sub, wl.B)
    if step is not None:
        sb = np.array(seqs, np.int32)
        oracle.write(oc, u16(step.c_kv[seqs]), u16(step.k_rope[seqs]), sb,
                     step.pos.cpu().numpy()[sb], step.seq_lens.cpu().numpy(),
                     inp.page_table.cpu().numpy(), op, osink, olocal)
    ref, ref_lse = oracle.decode(oc, synth.SOFTMAX_SCALE, u16(inp.q_lat), u16(inp.q_rope), op,
                                 inp.page_table.cpu().numpy(), lens_h, osink, olocal, sel=rows)
    assert_decode_ok(out, lse, ref, ref_lse, rows=rows, label=f"{name} rows={len(rows)}")
    # the sampled sequences' pages and BF16 buffers are bit-exact
    pt = inp.page_table.cpu().numpy()
    for b in seqs:
        ids = pt[b, :(int(lens_h[b]) + 63) // 64]
        assert np.array_equal(pages[torch.from_numpy(ids).long().to(DEV)].cpu().numpy(), op[ids])
        assert np.array_equal(u16(sink[b]), osink[b])
        assert np.array_equal(u16(local[b]), olocal[b])


def test_full_v2lite_sampled():
    _full_workload("v2lite", n_seq=3, n_head=16)


def test_full_v3_sampled():
    _full_workload("v3", n_seq=4, n_head=6)


def test_full_c2r4_sampled():
    _full_workload("c2r4", n_seq=2, n_head=4)


def test_full_serve_sampled():
    _full_workload("serve", n_seq=4, n_head=4)


MQ_LENS = [1, 2, 3, 4, 5, 64, 65, 66, 131, 132, 133, 134, 197, 1000, 0, 5000]


@pytest.mark.parametrize("c_bits,s_q,H", [(4, 2, 16), (4, 4, 16), (2, 2, 16), (4, 2, 128)])
def test_decode_multi_query(c_bits, s_q, H):
    """s_q query tokens per sequence (multi-token prediction verification):
    query i attends to p < L - (s_q - 1 - i); lengths shorter than s_q, window
    edges and ragged pages."""
    cfg = _cfg(c_bits)
    inp = synth.build_cache_inputs(MQ_LENS, s_q * H, seed=500 + s_q + H + c_bits, device="cpu")
    print(f"[case] multi-query c_bits={c_bits} s_q={s_q} H={H}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(MQ_LENS))
    g = lambda t: t.to(DEV)  # noqa: E731
    B = len(MQ_LENS)
    ql = g(inp.q_lat).view(B, s_q, H, -1)
    qr = g(inp.q_rope).view(B, s_q, H, -1)
    out, lse = mla.decode_mq(cfg, ql, qr, pages, g(inp.page_table), g(inp.seq_lens), sink, local,
                             synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, B)
    ref, ref_lse = oracle_decode_mq(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE, s_q, H)
    assert_decode_ok(out.reshape(B * s_q * H, -1), lse.reshape(-1), ref.reshape(-1, 512),
                     ref_lse.reshape(-1), label=f"mq c{c_bits} s_q{s_q} H{H}")


def test_decode_multi_query_one_token_is_decode():
    cfg = _cfg(4)
    inp = synth.build_cache_inputs([3000, 131, 0], 16, seed=71, device="cpu")
    pages, sink, local = gpu_cache(cfg, inp, 3)
    o1, l1 = gpu_decode(cfg, inp, pages, sink, local)
    g = lambda t: t.to(DEV)  # noqa: E731
    o2, l2 = mla.decode_mq(cfg, g(inp.q_lat)[:, None], g(inp.q_rope)[:, None], pages,
                           g(inp.page_table), g(inp.seq_lens), sink, local, synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2[:, 0].view(torch.int16))
    assert torch.equal(l1, l2[:, 0])


PROT_LENS = [0, 1, 5, 63, 64, 65, 130, 300, 1000, 3000]


@pytest.mark.parametrize("c_bits,n_sink,n_local", [(4, 0, 0), (4, 0, 128), (4, 4, 0),
                                                   (4, 64, 256), (4, 1, 1), (2, 16, 200)])
def test_protection_settings(c_bits, n_sink, n_local):
    """Other sink / window sizes the ABI accepts (no sink, no window, a sink that
    fills a page, a 256-token window over five pages, single tokens): writer
    bytes, plain and multi-query decode, and one serving step."""
    cfg = mla.Config(c_bits=c_bits, n_sink=n_sink, n_local=n_local)
    oc = ocfg_of(cfg)
    H, B = 16, len(PROT_LENS)
    inp = synth.build_cache_inputs(PROT_LENS, 2 * H, seed=900 + n_sink + n_local + c_bits,
                                   device="cpu")
    print(f"[case] protection c_bits={c_bits} n_sink={n_sink} n_local={n_local}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, B, canary=0x3C)
    torch.cuda.synchronize()
    op, osink, olocal = oracle_cache(oc, inp, B, canary=0x3C)
    assert np.array_equal(pages.cpu().numpy(), op)
    assert np.array_equal(u16(sink), osink)
    assert np.array_equal(u16(local), olocal)
    g = lambda t: t.to(DEV)  # noqa: E731
    # multi-query decode (s_q = 2, H = 16 each), then the plain decode of all 32 rows
    out, lse = mla.decode_mq(cfg, g(inp.q_lat).view(B, 2, H, -1), g(inp.q_rope).view(B, 2, H, -1),
                             pages, g(inp.page_table), g(inp.seq_lens), sink, local,
                             synth.SOFTMAX_SCALE)
    out1, lse1 = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode_mq(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE, 2, H)
    assert_decode_ok(out.reshape(-1, 512), lse.reshape(-1), ref.reshape(-1, 512),
                     ref_lse.reshape(-1), label=f"prot mq s{n_sink} l{n_local}")
    r1, rl1 = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out1, lse1, r1, rl1, label=f"prot s{n_sink} l{n_local}")
    # one serving step: a new token at position L of every sequence
    new_lens = [L + 1 for L in PROT_LENS]
    step_inp = synth.build_cache_inputs(new_lens, 2 * H, seed=901 + n_sink + n_local,
                                        device="cpu")
    pt = torch.tensor(np.array(
        [np.pad(inp.page_table[b].numpy(), (0, 1), constant_values=-1) for b in range(B)]))
    extra = [b for b, L in enumerate(PROT_LENS) if L % 64 == 0]  # needs a new page
    num_pages = inp.num_pages
    for b in extra:
        pt[b, PROT_LENS[b] // 64] = num_pages
        num_pages += 1
    pages2 = torch.full((num_pages, pages.shape[1]), 0x3C, dtype=torch.uint8, device=DEV)
    pages2[:inp.num_pages] = pages
    sel = torch.tensor([int(np.flatnonzero(step_inp.seq_idx.numpy() == b)[-1]) if new_lens[b] else 0
                        for b in range(B)])
    c_new, r_new = step_inp.c_kv[sel], step_inp.k_rope[sel]
    pos = torch.tensor(PROT_LENS, dtype=torch.int32)
    lens_new = torch.tensor(new_lens, dtype=torch.int32)
    out2, lse2 = mla.write_decode(cfg, g(c_new), g(r_new), g(pos), g(inp.q_lat), g(inp.q_rope),
                                  pages2, g(pt), g(lens_new), sink, local, synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    op2 = np.full((num_pages, op.shape[1]), 0x3C, np.uint8)
    op2[:inp.num_pages] = op
    oracle.write(oc, u16(c_new), u16(r_new), np.arange(B, dtype=np.int32), pos.numpy(),
                 lens_new.numpy(), pt.numpy(), op2, osink, olocal)
    assert np.array_equal(pages2.cpu().numpy(), op2)
    assert np.array_equal(u16(sink), osink)
    assert np.array_equal(u16(local), olocal)
    r2, rl2 = oracle.decode(oc, synth.SOFTMAX_SCALE, u16(inp.q_lat), u16(inp.q_rope), op2,
                            pt.numpy(), lens_new.numpy(), osink, olocal)
    assert_decode_ok(out2, lse2, r2, rl2, label=f"prot step s{n_sink} l{n_local}")


def test_ranges_longer_than_256_pages():
    """B32 H256 (one round of workgroups holds one range per sequence and head
    block) at 20000 tokens: each workgroup takes a 313-page range, beyond the
    first 256 page ids its threads stage; packed and BF16 caches."""
    B, H, L = 32, 256, 20000
    cfg = _cfg(4)
    oc = ocfg_of(cfg)
    print("[case] ranges beyond 256 pages: B32 H256 L20000", flush=True)
    inp = synth.build_cache_inputs([L] * B, H, seed=77, device=DEV)
    pages, sink, local = mla.allocate_cache(cfg, B, inp.num_pages, DEV)
    mla.write(cfg, inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.seq_lens, inp.page_table,
              pages, sink, local)
    out, lse = mla.decode(cfg, inp.q_lat, inp.q_rope, pages, inp.page_table, inp.seq_lens, sink,
                          local, synth.SOFTMAX_SCALE)
    p16 = mla.allocate_bf16_cache(inp.num_pages, DEV)
    mla.bf16_write(inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.page_table, p16)
    o16, l16 = mla.bf16_decode(inp.q_lat, inp.q_rope, p16, inp.page_table, inp.seq_lens,
                               synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    assert mla.binding.lib() is not None
    rows = [(b, h) for b in (0, 31) for h in (0, 17, 128, 255)]
    seqs = [0, 31]
    mask = torch.zeros(inp.seq_idx.numel(), dtype=torch.bool, device=DEV)
    for b in seqs:
        mask |= inp.seq_idx == b
    sub = synth.CacheInputs(inp.c_kv[mask].cpu(), inp.k_rope[mask].cpu(), inp.seq_idx[mask].cpu(),
                            inp.pos[mask].cpu(), inp.seq_lens.cpu(), inp.page_table.cpu(),
                            inp.num_pages, inp.q_lat.cpu(), inp.q_rope.cpu())
    op, osink, olocal = oracle_cache(oc, sub, B)
    ref, ref_lse = oracle.decode(oc, synth.SOFTMAX_SCALE, u16(inp.q_lat), u16(inp.q_rope), op,
                                 inp.page_table.cpu().numpy(), inp.seq_lens.cpu().numpy(), osink,
                                 olocal, sel=rows)
    assert_decode_ok(out, lse, ref, ref_lse, rows=rows, label="313-page ranges")
    ob = np.zeros((inp.num_pages, 64, 576), np.uint16)
    oracle.bf16_write(oracle.Cfg(), u16(sub.c_kv), u16(sub.k_rope), sub.seq_idx.numpy(),
                      sub.pos.numpy(), sub.page_table.numpy(), ob)
    r16, rl16 = oracle.bf16_decode(oracle.Cfg(), synth.SOFTMAX_SCALE, u16(inp.q_lat),
                                   u16(inp.q_rope), ob, inp.page_table.cpu().numpy(),
                                   inp.seq_lens.cpu().numpy(), sel=rows)
    assert_decode_ok(o16, l16, r16, rl16, rows=rows, label="313-page ranges, bf16")


@pytest.mark.parametrize("B,L", [(8, 1048576), (32, 486400)])
def test_long_context_sweep_sampled(B, L):
    """The context sweep's launch at its longest contexts (H = 16, one bulk
    write, the default workspace): B8 at 1M tokens (one round of workgroups,
    page ranges just past 256 pages) and B32 at 486,400 tokens (one round, ranges
    of about 475 pages, near the 512-item cap). The first and last sequences,
    every head, against the oracle."""
    H = 16
    cfg = _cfg(4)
    oc = ocfg_of(cfg)
    print(f"[case] long-context sweep B{B} H{H} L{L}", flush=True)
    inp = synth.bulk_cache_inputs(B, L, H, seed=2100 + B, device=DEV)
    pages, sink, local = mla.allocate_cache(cfg, B, inp.num_pages, DEV)
    mla.write(cfg, inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.seq_lens, inp.page_table,
              pages, sink, local)
    out, lse = mla.decode(cfg, inp.q_lat, inp.q_rope, pages, inp.page_table, inp.seq_lens, sink,
                          local, synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    del pages, sink, local
    for b in (0, B - 1):
        ref, ref_lse = oracle_sequence_rows(oc, inp.c_kv[b * L:(b + 1) * L], inp.k_rope[b * L:(b + 1) * L],
                                            inp.q_lat[b], inp.q_rope[b], L, range(H),
                                            synth.SOFTMAX_SCALE)
        assert_decode_ok(out, lse, ref, ref_lse, rows=[(b, h) for h in range(H)],
                         label=f"sweep B{B} L{L} seq {b}")


VARIANTS = [(4, 2, 32), (2, 2, 32), (4, 4, 64), (2, 4, 128), (4, 2, 128), (2, 2, 64)]


@pytest.mark.parametrize("c_bits,r_bits,group", VARIANTS)
def test_variant_writer_bit_exact(c_bits, r_bits, group):
    """Other bit widths and group sizes (2-bit RoPE codes, groups of 64 and 128
    channels): pages, sink and local buffers bit-exact with the oracle, canary
    bytes outside the written slots kept; degenerate groups included."""
    cfg = mla.Config(c_bits=c_bits, r_bits=r_bits, group=group)
    lens = [700, 1, 5, 64, 65, 133, 197]
    inp = synth.build_cache_inputs(lens, 16, seed=90 + c_bits + r_bits + group, device="cpu",
                                   spare_pages=2)
    c = inp.c_kv.float()
    c[0:20, 0:128] = 1.5                           # constant groups of every size
    c[20:30, 128:256] = -0.0
    c[30:40, 256:384] = 1e-4 * torch.randn(10, 128)  # fp16-subnormal scales
    inp.c_kv = c.to(torch.bfloat16)
    print(f"[case] variant writer c{c_bits} r{r_bits} g{group}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens), canary=0x5A)
    torch.cuda.synchronize()
    op, osink, olocal = oracle_cache(ocfg_of(cfg), inp, len(lens), canary=0x5A)
    assert np.array_equal(pages.cpu().numpy(), op)
    assert np.array_equal(u16(sink), osink)
    assert np.array_equal(u16(local), olocal)


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("c_bits,r_bits,group", VARIANTS)
def test_variant_decode(c_bits, r_bits, group, H):
    """The decode over the variant formats (16-head blocks and the 128-head
    path) against the oracle: edge lengths, several pages and a ragged tail."""
    cfg = mla.Config(c_bits=c_bits, r_bits=r_bits, group=group)
    lens = [1, 131, 133, 197, 1000, 2500, 0, 4099]
    inp = synth.build_cache_inputs(lens, H, seed=110 + c_bits + r_bits + group + H, device="cpu")
    print(f"[case] variant decode c{c_bits} r{r_bits} g{group} H{H}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens))
    out, lse = gpu_decode(cfg, inp, pages, sink, local)
    torch.cuda.synchronize()
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, len(lens))
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out, lse, ref, ref_lse, label=f"variant c{c_bits} r{r_bits} g{group} H{H}")
