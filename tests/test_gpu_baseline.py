"""GPU parity for the paired BF16 cache and the simulated quantize-dequantize,
called through the C ABI, against the CPU oracle on the same seeded inputs.

* BF16 writer: pages bit-exact (canary-filled pool, so bytes outside written
  slots keep their canary);
* BF16 decode: rel-L2 <= 2e-3, |delta| / max(1, |ref|) <= 1e-2, lse |delta| <= 1e-3
  against the fp64 oracle on edge lengths (1, ragged last pages, empty), H in
  {16, 128}, and on sampled rows of the V2-Lite-shaped workload in the launch
  configuration the bench times;
* QDQ: bf16 outputs bit-exact for both content code widths, including
  degenerate groups.
"""
import numpy as np
import pytest
import torch

import bit_mla_kv_lowbit_amd as mla
import oracle
import synth
from tests.gpu_helpers import DEV, assert_decode_ok, ocfg_of, u16

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 63, 64, 65, 127, 128, 129, 1000, 0, 4097]


def _gpu_bf16_cache(inp, canary=None):
    pages = mla.allocate_bf16_cache(inp.num_pages, DEV)
    if canary is not None:
        pages.view(torch.int16).fill_(canary)
    g = lambda t: t.to(DEV)  # noqa: E731
    mla.bf16_write(g(inp.c_kv), g(inp.k_rope), g(inp.seq_idx), g(inp.pos), g(inp.page_table),
                   pages)
    return pages


def _oracle_bf16_cache(inp, canary=0):
    oc = oracle.Cfg()
    pages = np.full((inp.num_pages, 64, 576), canary, np.uint16)
    oracle.bf16_write(oc, u16(inp.c_kv), u16(inp.k_rope), inp.seq_idx.cpu().numpy(),
                      inp.pos.cpu().numpy(), inp.page_table.cpu().numpy(), pages)
    return pages


def test_bf16_writer_bit_exact_with_canaries():
    lens = [130, 1, 64, 65, 700]
    inp = synth.build_cache_inputs(lens, 16, seed=41, device="cpu", spare_pages=2)
    print(f"[case] bf16 writer lens={lens}", flush=True)
    pages = _gpu_bf16_cache(inp, canary=0x5A5A)
    torch.cuda.synchronize()
    assert np.array_equal(u16(pages), _oracle_bf16_cache(inp, canary=0x5A5A))


@pytest.mark.parametrize("H", [16, 128])
def test_bf16_decode_edge_lengths(H):
    inp = synth.build_cache_inputs(EDGE_LENS, H, seed=420 + H, device="cpu")
    print(f"[case] bf16 decode edges H={H}", flush=True)
    pages = _gpu_bf16_cache(inp)
    g = lambda t: t.to(DEV)  # noqa: E731
    out, lse = mla.bf16_decode(g(inp.q_lat), g(inp.q_rope), pages, g(inp.page_table),
                               g(inp.seq_lens), synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    op = _oracle_bf16_cache(inp)
    ref, ref_lse = oracle.bf16_decode(oracle.Cfg(), synth.SOFTMAX_SCALE, u16(inp.q_lat),
                                      u16(inp.q_rope), op, inp.page_table.numpy(),
                                      inp.seq_lens.numpy())
    assert_decode_ok(out, lse, ref, ref_lse, label=f"bf16 edges H{H}")
    b0 = EDGE_LENS.index(0)
    assert not out[b0].float().abs().sum().item()


@pytest.mark.parametrize("name", ["v2lite", "v3"])
def test_bf16_decode_full_sampled(name):
    """The V2-Lite-shaped (B8 H16 L32768) and V3-shaped (B32 H128 L8192, the
    64-head kernel) batches as a BF16 cache, in the bench's launch
    configuration; sampled sequences and heads against the oracle."""
    wl = synth.WORKLOADS[name]
    print(f"[case] bf16 full {name}: generating on the GPU", flush=True)
    inp, _ = synth.workload_inputs(wl, device=DEV)
    pages = mla.allocate_bf16_cache(inp.num_pages, DEV)
    mla.bf16_write(inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.page_table, pages)
    out, lse = mla.bf16_decode(inp.q_lat, inp.q_rope, pages, inp.page_table, inp.seq_lens,
                               synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    print(f"[case] bf16 full {name}: GPU done, oracle on sampled rows", flush=True)
    rng = np.random.default_rng(3)
    seqs = [0, 5]
    rows = [(b, int(h)) for b in seqs for h in sorted(rng.choice(wl.H, 6, replace=False))]
    ref, ref_lse = oracle.bf16_decode(oracle.Cfg(), synth.SOFTMAX_SCALE, u16(inp.q_lat),
                                      u16(inp.q_rope), u16(pages), inp.page_table.cpu().numpy(),
                                      inp.seq_lens.cpu().numpy(), sel=rows)
    assert_decode_ok(out, lse, ref, ref_lse, rows=rows, label=f"bf16 {name}")
    # the sampled sequences' pages hold exactly their token rows
    op = np.zeros((inp.num_pages, 64, 576), np.uint16)
    mask = torch.zeros(inp.seq_idx.numel(), dtype=torch.bool, device=DEV)
    for b in seqs:
        mask |= inp.seq_idx == b
    oracle.bf16_write(oracle.Cfg(), u16(inp.c_kv[mask]), u16(inp.k_rope[mask]),
                      inp.seq_idx[mask].cpu().numpy(), inp.pos[mask].cpu().numpy(),
                      inp.page_table.cpu().numpy(), op)
    pt = inp.page_table.cpu().numpy()
    for b in seqs:
        ids = torch.from_numpy(pt[b]).long().to(DEV)
        assert np.array_equal(u16(pages[ids]), op[pt[b]])


@pytest.mark.parametrize("c_bits", [4, 2])
def test_qdq_bit_exact(c_bits):
    cfg = mla.Config(c_bits=c_bits)
    inp = synth.build_cache_inputs([777], 1, seed=50 + c_bits, device="cpu")
    c = inp.c_kv.float()
    c[0:20, 0:32] = 2.5                          # constant group
    c[20:30, 32:64] = 0.0                        # zero group
    c[30:40, 64:96] = 1e-4 * torch.randn(10, 32)  # fp16-subnormal scales
    c[40:50, 96:128] = 300.0 * torch.randn(10, 32)  # wide range
    inp.c_kv = c.to(torch.bfloat16)
    print(f"[case] qdq c_bits={c_bits}", flush=True)
    oc_, or_ = mla.qdq(cfg, inp.c_kv.to(DEV), inp.k_rope.to(DEV))
    torch.cuda.synchronize()
    rc, rr = oracle.qdq(ocfg_of(cfg), u16(inp.c_kv), u16(inp.k_rope))
    assert np.array_equal(u16(oc_), rc)
    assert np.array_equal(u16(or_), rr)


@pytest.mark.parametrize("c_bits,r_bits,group", [(4, 2, 32), (2, 2, 64), (4, 4, 128),
                                                 (2, 4, 64), (4, 2, 128)])
def test_qdq_bit_exact_variants(c_bits, r_bits, group):
    """QDQ at other bit widths and group sizes (groups of 64 / 128 channels are
    spread over 8 / 16 lanes): bit-exact with the oracle, ragged token count."""
    cfg = mla.Config(c_bits=c_bits, r_bits=r_bits, group=group)
    inp = synth.build_cache_inputs([203], 1, seed=60 + group + r_bits, device="cpu")
    c = inp.c_kv.float()
    c[0:20, 0:128] = 2.5
    c[20:30, 128:256] = 1e-4 * torch.randn(10, 128)
    inp.c_kv = c.to(torch.bfloat16)
    print(f"[case] qdq c{c_bits} r{r_bits} g{group}", flush=True)
    oc_, or_ = mla.qdq(cfg, inp.c_kv.to(DEV), inp.k_rope.to(DEV))
    torch.cuda.synchronize()
    rc, rr = oracle.qdq(ocfg_of(cfg), u16(inp.c_kv), u16(inp.k_rope))
    assert np.array_equal(u16(oc_), rc)
    assert np.array_equal(u16(or_), rr)


def test_qdq_in_place():
    cfg = mla.C4R4
    inp = synth.build_cache_inputs([300], 1, seed=57, device="cpu")
    rc, rr = oracle.qdq(ocfg_of(cfg), u16(inp.c_kv), u16(inp.k_rope))
    c, r = inp.c_kv.to(DEV), inp.k_rope.to(DEV)
    mla.qdq(cfg, c, r, out_c=c, out_r=r)
    torch.cuda.synchronize()
    assert np.array_equal(u16(c), rc)
    assert np.array_equal(u16(r), rr)


def _replay_check(run, outs, label):
    """Capture run() in a HIP graph; replay it 4 times, with the outputs
    scribbled over and an eager run() between replays; every replay must give
    the eager result."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        run(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for k in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0x5A)
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"{label} replay {k}"
        run()
        torch.cuda.synchronize()


def test_graph_replay_bf16_decode_mq_and_qdq():
    inp = synth.build_cache_inputs([3000, 70, 1500], 32, seed=88, device="cpu")
    g = lambda t: t.to(DEV)  # noqa: E731
    ql, qr, pt, sl = g(inp.q_lat), g(inp.q_rope), g(inp.page_table), g(inp.seq_lens)
    B, max_pages = 3, pt.shape[1]
    print("[case] graph replay: bf16 decode, multi-query decode, qdq", flush=True)

    pages16 = _gpu_bf16_cache(inp)
    ws = torch.empty(max(16, mla.bf16_decode_workspace_bytes(B, 32, max_pages)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(B, 32, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, 32, dtype=torch.float32, device=DEV)
    _replay_check(lambda stream=None: mla.bf16_decode(ql, qr, pages16, pt, sl,
                                                      synth.SOFTMAX_SCALE, out=out, lse=lse,
                                                      workspace=ws, stream=stream),
                  (out, lse), "bf16 decode")

    cfg = mla.C4R4
    pages, sink, local = mla.allocate_cache(cfg, B, inp.num_pages, DEV)
    mla.write(cfg, g(inp.c_kv), g(inp.k_rope), g(inp.seq_idx), g(inp.pos), sl, pt, pages, sink,
              local)
    ws2 = torch.empty(max(16, mla.decode_workspace_bytes(cfg, B, 32, max_pages)),
                      dtype=torch.uint8, device=DEV)
    out2 = torch.empty(B, 2, 16, 512, dtype=torch.bfloat16, device=DEV)
    lse2 = torch.empty(B, 2, 16, dtype=torch.float32, device=DEV)
    ql2, qr2 = ql.view(B, 2, 16, -1), qr.view(B, 2, 16, -1)
    _replay_check(lambda stream=None: mla.decode_mq(cfg, ql2, qr2, pages, pt, sl, sink, local,
                                                    synth.SOFTMAX_SCALE, out=out2, lse=lse2,
                                                    workspace=ws2, stream=stream),
                  (out2, lse2), "multi-query decode")

    c, r = g(inp.c_kv), g(inp.k_rope)
    oc, orr = torch.empty_like(c), torch.empty_like(r)
    _replay_check(lambda stream=None: mla.qdq(cfg, c, r, out_c=oc, out_r=orr, stream=stream),
                  (oc, orr), "qdq")
