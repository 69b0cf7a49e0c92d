"""Helpers for the GPU parity tests: run both paths on the same seeded inputs."""
import numpy as np
import torch

import bit_mla_kv_lowbit_amd as mla
import oracle
import synth
from tests.oracle_helpers import oracle_cache, u16

DEV = torch.device("cuda:0")

# decode tolerance against the fp64 oracle (bf16 outputs): rel-L2 over the
# whole output, |delta| / max(1, |ref|) per element, absolute on the lse
TOL_REL_L2 = 2e-3
TOL_MAX = 1e-2
TOL_LSE = 1e-3


def ocfg_of(cfg: mla.Config) -> oracle.Cfg:
    return oracle.Cfg(cfg.d_c, cfg.d_r, cfg.c_bits, cfg.r_bits, cfg.group, cfg.page_size,
                      cfg.n_sink, cfg.n_local)


def gpu_cache(cfg, inp, B, canary=None):
    """GPU writer over every token of inp (inputs moved to the device). With a
    canary byte, every buffer starts filled with it instead of zeros."""
    pages, sink, local = mla.allocate_cache(cfg, B, inp.num_pages, DEV)
    if canary is not None:
        pages.fill_(canary)
        pat = int(np.array([canary * 257], np.uint16).view(np.int16)[0])
        sink.view(torch.int16).fill_(pat)
        local.view(torch.int16).fill_(pat)
    g = lambda t: t.to(DEV)  # noqa: E731
    mla.write(cfg, g(inp.c_kv), g(inp.k_rope), g(inp.seq_idx), g(inp.pos), g(inp.seq_lens),
              g(inp.page_table), pages, sink, local)
    return pages, sink, local


def gpu_decode(cfg, inp, pages, sink, local, scale=synth.SOFTMAX_SCALE):
    g = lambda t: t.to(DEV)  # noqa: E731
    out, lse = mla.decode(cfg, g(inp.q_lat), g(inp.q_rope), pages, g(inp.page_table),
                          g(inp.seq_lens), sink, local, scale)
    return out, lse


def compare_decode(out, lse, ref, ref_lse, rows=None):
    """Returns (rel_l2, max_rel_abs, lse_abs); rows selects (b, h) pairs of out."""
    got = out.float().cpu().numpy()
    gl = lse.cpu().numpy()
    if rows is not None:
        got = np.stack([got[b, h] for b, h in rows])
        gl = np.array([gl[b, h] for b, h in rows])
    else:
        got = got.reshape(ref.shape)
        gl = gl.reshape(-1)
    both_empty = np.isneginf(ref_lse) & np.isneginf(gl)
    assert np.array_equal(np.isneginf(ref_lse), np.isneginf(gl)), "empty rows differ"
    with np.errstate(invalid="ignore"):  # -inf - -inf on empty rows, masked out
        dl = np.abs(np.where(both_empty, 0.0, gl - ref_lse))
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    mx = np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))) if ref.size else 0.0
    return float(rel), float(mx), float(dl.max() if dl.size else 0.0)


def assert_decode_ok(out, lse, ref, ref_lse, rows=None, label=""):
    rel, mx, dl = compare_decode(out, lse, ref, ref_lse, rows)
    print(f"[parity] {label} rel_l2={rel:.3e} max_rel_abs={mx:.3e} lse_abs={dl:.3e}", flush=True)
    assert rel <= TOL_REL_L2, (label, rel)
    assert mx <= TOL_MAX, (label, mx)
    assert dl <= TOL_LSE, (label, dl)
