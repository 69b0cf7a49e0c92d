"""Test-side helpers: build the oracle's host cache from synthetic inputs."""
import numpy as np
import torch

import oracle


def u16(t: torch.Tensor) -> np.ndarray:
    """Raw bit pattern of a bf16/fp16 tensor as a uint16 numpy array (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def cfg_for(c_bits: int = 4, **kw) -> oracle.Cfg:
    return oracle.Cfg(c_bits=c_bits, **kw)


def oracle_cache(cfg: oracle.Cfg, inp, B: int, canary=None):
    """Run the oracle writer over every token of `inp` into fresh host buffers
    (zeroed, or filled with a canary byte)."""
    D = cfg.d_c + cfg.d_r
    fill = 0 if canary is None else canary
    pages = np.full((inp.num_pages, oracle.page_bytes(cfg)), fill, np.uint8)
    sink = np.full((B, max(cfg.n_sink, 1), D), fill * 257, np.uint16)
    local = np.full((B, max(cfg.n_local, 1), D), fill * 257, np.uint16)
    oracle.write(cfg, u16(inp.c_kv), u16(inp.k_rope), inp.seq_idx.cpu().numpy(),
                 inp.pos.cpu().numpy(), inp.seq_lens.cpu().numpy(),
                 inp.page_table.cpu().numpy(), pages, sink, local)
    return pages, sink, local


def oracle_decode(cfg, inp, pages, sink, local, scale, sel=None, p_begin=0, p_end=-1):
    return oracle.decode(cfg, scale, u16(inp.q_lat), u16(inp.q_rope), pages,
                         inp.page_table.cpu().numpy(), inp.seq_lens.cpu().numpy(), sink, local,
                         sel=sel, p_begin=p_begin, p_end=p_end)


def oracle_decode_mq(cfg, inp, pages, sink, local, scale, s_q: int, H: int):
    """Multi-query decode by the oracle: q_lat / q_rope hold B x (s_q * H) rows
    (query token i = rows i*H .. i*H + H - 1); query token i of sequence b
    attends to tokens p < seq_lens[b] - (s_q - 1 - i). Returns (out [B, s_q, H,
    d_c], lse [B, s_q, H])."""
    lens = inp.seq_lens.cpu().numpy()
    B = len(lens)
    out = np.zeros((B, s_q, H, cfg.d_c))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        for i in range(s_q):
            end = max(0, int(lens[b]) - (s_q - 1 - i))
            sel = [(b, i * H + h) for h in range(H)]
            o, l = oracle_decode(cfg, inp, pages, sink, local, scale, sel=sel, p_begin=0,
                                 p_end=end)
            out[b, i], lse[b, i] = o, l
    return out, lse


def oracle_sequence_rows(cfg, c_kv, k_rope, q_lat_b, q_rope_b, L: int, heads, scale):
    """Oracle decode of one sequence whose tokens 0..L-1 are c_kv / k_rope (in
    order), written into a compact page table of its own (the physical page ids
    do not enter the result). q_lat_b / q_rope_b: [H, d] of that sequence.
    Returns (out [len(heads), d_c], lse [len(heads)])."""
    n_pages = max(1, -(-L // cfg.page_size))
    pt = np.arange(n_pages, dtype=np.int32)[None]
    lens = np.array([L], np.int32)
    D = cfg.d_c + cfg.d_r
    pages = np.zeros((n_pages, oracle.page_bytes(cfg)), np.uint8)
    sink = np.zeros((1, max(cfg.n_sink, 1), D), np.uint16)
    local = np.zeros((1, max(cfg.n_local, 1), D), np.uint16)
    oracle.write(cfg, u16(c_kv), u16(k_rope), np.zeros(L, np.int32),
                 np.arange(L, dtype=np.int32), lens, pt, pages, sink, local)
    return oracle.decode(cfg, scale, u16(q_lat_b[None]), u16(q_rope_b[None]), pages, pt, lens,
                         sink, local, sel=[(0, int(h)) for h in heads])
