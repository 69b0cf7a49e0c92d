"""mla_lowbit_decode_noalloc (the decode for callers that cannot allocate:
its workspace is the library's static device scratch) against
mla_lowbit_decode on the same inputs, through the C ABI: two calls in a row,
the second on a smaller batch, each bit-identical to the workspace decode and
within the parity tolerance of the fp64 oracle. Also: a shape whose workspace
exceeds the scratch is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import bit_mla_kv_lowbit_amd as mla
from bit_mla_kv_lowbit_amd import binding
import synth
from tests.gpu_helpers import DEV, assert_decode_ok, gpu_cache, ocfg_of
from tests.oracle_helpers import oracle_cache, oracle_decode


def _run(cfg, lens, H, seed):
    inp = synth.build_cache_inputs(lens, H, seed=seed, device="cpu")
    print(f"[case] noalloc c_bits={cfg.c_bits} H={H} lens={lens}", flush=True)
    pages, sink, local = gpu_cache(cfg, inp, len(lens))
    g = lambda t: t.to(DEV)  # noqa: E731
    q, qr, pt, sl = g(inp.q_lat), g(inp.q_rope), g(inp.page_table), g(inp.seq_lens)
    B = len(lens)
    # outputs start filled with a pattern the decode must overwrite everywhere
    out_n = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    lse_n = torch.full((B, H), 7.0, dtype=torch.float32, device=DEV)
    mla.decode_noalloc(cfg, q, qr, pages, pt, sl, sink, local, synth.SOFTMAX_SCALE, out_n, lse_n)
    out_w, lse_w = mla.decode(cfg, q, qr, pages, pt, sl, sink, local, synth.SOFTMAX_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_w)
    assert torch.equal(lse_n, lse_w)
    oc = ocfg_of(cfg)
    op, osink, olocal = oracle_cache(oc, inp, B)
    ref, ref_lse = oracle_decode(oc, inp, op, osink, olocal, synth.SOFTMAX_SCALE)
    assert_decode_ok(out_n, lse_n, ref, ref_lse, label=f"noalloc H{H} lens={lens}")


@pytest.mark.gpu
@pytest.mark.parametrize("c_bits", [4, 2])
def test_noalloc_two_calls_second_smaller(c_bits):
    cfg = mla.Config(c_bits=c_bits)
    # first call: a batch whose sequences split into several page ranges
    _run(cfg, [9000, 4096, 131, 0, 2500, 7000], 128 if c_bits == 4 else 16, seed=910 + c_bits)
    # second call on the same scratch: fewer sequences, fewer heads, shorter
    _run(cfg, [700, 65, 1], 16, seed=920 + c_bits)


def test_noalloc_refuses_oversized_shape_before_launch():
    c = mla.C4R4.c()
    B, H, max_pages = 64, 1024, 4096
    need = mla.decode_workspace_bytes(mla.C4R4, B, H, max_pages)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    rc = mla.lib().mla_lowbit_decode_noalloc(ctypes.byref(c), B, H, 0.1, fake, fake, fake, fake,
                                             max_pages, fake, fake, fake, fake, fake, None)
    assert rc == binding.ESCRATCH
    assert "scratch" in binding.strerror(rc)
