"""Seeded synthetic inputs for the low-bit MLA cache writer and decode.

This module only draws inputs; it holds none of the method's arithmetic
(no quantization, packing or attention). Both the GPU path and the CPU oracle
are fed from the tensors it returns.

Value recipe (the workloads' statement: latent c_kv ~ N(0,1) with 8 random
channels scaled x10, k_rope ~ N(0,1) rotated by RoPE with theta = 10000 at the
token's position, q_lat / q_rope ~ N(0,1), everything stored as bf16, softmax
scale 1/sqrt(192)):
  * c_kv: fp32 N(0,1); 8 distinct channel indices, drawn once per seed and
    shared by every token and sequence, are multiplied by 10; then rounded to
    bf16 (round-to-nearest-even).
  * k_rope: fp32 N(0,1) pairs (2i, 2i+1) rotated by the angle p * theta_i with
    theta_i = 10000^(-2i/d_r) and p the token position counted from 0; the
    angle and its cos/sin are taken in fp64, the rotation in fp32; then bf16.
  * q_lat, q_rope: N(0,1) rounded to bf16.
  * page table: every sequence gets ceil(len / 64) pages drawn from one random
    permutation of the physical pool (so logical neighbours are scattered);
    unused entries are -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

D_C, D_R = 512, 64
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)
PAGE = 64


@dataclass
class Workload:
    """One decode workload: B sequences, H query heads, content code width."""
    name: str
    B: int
    H: int
    c_bits: int
    lens: Optional[List[int]] = None   # cached tokens per sequence (after the write)
    len_range: Optional[tuple] = None  # (lo, hi): lengths before the step, uniform
    step_write: bool = False           # one new token per sequence is written, then decoded
    seed: int = 0
    desc: str = ""

    def lengths(self) -> List[int]:
        """Tokens attended per sequence (after any step write)."""
        if self.lens is not None:
            return list(self.lens)
        g = torch.Generator().manual_seed(self.seed + 7)
        lo, hi = self.len_range
        pre = torch.randint(lo, hi + 1, (self.B,), generator=g).tolist()
        return [int(x) + (1 if self.step_write else 0) for x in pre]


WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=16, c_bits=4, lens=[1024], seed=1000,
                     desc="Tiny C4R4 decode: B1 H16 L1024"),
    "v2lite": Workload("v2lite", B=8, H=16, c_bits=4, lens=[32768] * 8, seed=1001,
                       desc="DeepSeek-V2-Lite-shaped C4R4 decode: B8 H16 L32768"),
    "v3": Workload("v3", B=32, H=128, c_bits=4, lens=[8192] * 32, seed=1002,
                   desc="DeepSeek-V3-shaped C4R4 decode: B32 H128 L8192"),
    "c2r4": Workload("c2r4", B=8, H=16, c_bits=2, lens=[131072] * 8, seed=1003,
                     desc="C2R4 long-context decode: B8 H16 L131072"),
    "serve": Workload("serve", B=64, H=128, c_bits=4, len_range=(1024, 131072), step_write=True,
                      seed=1004, desc="Serving step: B64 H128 L~U[1024,131072]+1, write+decode"),
}


def outlier_channels(seed: int, d_c: int = D_C, n: int = 8) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed * 31 + 5)
    return torch.randperm(d_c, generator=g)[:n]


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def latent_tokens(n: int, seed: int, device="cpu", d_c: int = D_C, outliers=None) -> torch.Tensor:
    """[n, d_c] bf16 content latents with x10 outlier channels."""
    g = _gen(device, seed)
    x = torch.randn(n, d_c, generator=g, device=device, dtype=torch.float32)
    if outliers is not None and len(outliers):
        x[:, outliers.to(device)] *= 10.0
    return x.to(torch.bfloat16)


def rope_keys(positions: torch.Tensor, seed: int, device="cpu", d_r: int = D_R,
              theta: float = 10000.0) -> torch.Tensor:
    """[n, d_r] bf16 RoPE keys: N(0,1) pairs rotated at each token's position."""
    n = positions.numel()
    g = _gen(device, seed)
    x = torch.randn(n, d_r, generator=g, device=device, dtype=torch.float32)
    i = torch.arange(d_r // 2, device=device, dtype=torch.float64)
    inv = theta ** (-2.0 * i / d_r)
    ang = positions.to(device=device, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    x0, x1 = x[:, 0::2], x[:, 1::2]
    y = torch.empty_like(x)
    y[:, 0::2] = x0 * cos - x1 * sin
    y[:, 1::2] = x0 * sin + x1 * cos
    return y.to(torch.bfloat16)


def queries(B: int, H: int, seed: int, device="cpu", d_c: int = D_C, d_r: int = D_R):
    g = _gen(device, seed)
    q_lat = torch.randn(B, H, d_c, generator=g, device=device).to(torch.bfloat16)
    q_rope = torch.randn(B, H, d_r, generator=g, device=device).to(torch.bfloat16)
    return q_lat, q_rope


def page_table(lens: List[int], seed: int, page: int = PAGE, spare: int = 0):
    """Shuffled page table [B, max_pages] int32 (-1 = unused) and the pool size."""
    need = [max(1, -(-L // page)) for L in lens]
    max_pages = max(need)
    total = sum(need) + spare
    g = torch.Generator().manual_seed(seed * 17 + 3)
    perm = torch.randperm(total, generator=g)
    pt = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    k = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[k:k + n].to(torch.int32)
        k += n
    return pt, total


@dataclass
class CacheInputs:
    """Tokens to write (in order), lengths after the writes, and the page table."""
    c_kv: torch.Tensor       # [n, d_c] bf16
    k_rope: torch.Tensor     # [n, d_r] bf16
    seq_idx: torch.Tensor    # [n] int32
    pos: torch.Tensor        # [n] int32
    seq_lens: torch.Tensor   # [B] int32 (after these writes)
    page_table: torch.Tensor  # [B, max_pages] int32
    num_pages: int
    q_lat: torch.Tensor = field(default=None)   # [B, H, d_c] bf16
    q_rope: torch.Tensor = field(default=None)  # [B, H, d_r] bf16


def sequence_tokens(b: int, start: int, stop: int, seed: int, device="cpu", d_c: int = D_C,
                    d_r: int = D_R, outliers=None):
    """Tokens [start, stop) of sequence b: the stream for each (seed, b) is split into
    fixed 4096-token chunks so any sub-range is reproducible on its own."""
    CH = 4096
    outs_c, outs_r = [], []
    c0 = start // CH
    for c in range(c0, -(-stop // CH)):
        lo, hi = c * CH, (c + 1) * CH
        s = seed * 1_000_003 + b * 10_007 + c
        pos = torch.arange(lo, hi, dtype=torch.int64)
        xc = latent_tokens(CH, s, device, d_c, outliers)
        xr = rope_keys(pos, s + 500_000_000, device, d_r)
        a, z = max(start, lo) - lo, min(stop, hi) - lo
        outs_c.append(xc[a:z])
        outs_r.append(xr[a:z])
    return torch.cat(outs_c), torch.cat(outs_r)


def build_cache_inputs(lens: List[int], H: int, seed: int, device="cpu", d_c: int = D_C,
                       d_r: int = D_R, page: int = PAGE, outliers=True, spare_pages: int = 0,
                       table_lens: Optional[List[int]] = None):
    """All tokens 0..L_b-1 of every sequence, in sequence order, plus queries.
    The page table covers table_lens (default: lens) tokens per sequence."""
    outl = outlier_channels(seed, d_c) if outliers else None
    cs, rs, si, ps = [], [], [], []
    for b, L in enumerate(lens):
        if L == 0:
            continue
        c, r = sequence_tokens(b, 0, L, seed, device, d_c, d_r, outl)
        cs.append(c)
        rs.append(r)
        si.append(torch.full((L,), b, dtype=torch.int32, device=device))
        ps.append(torch.arange(L, dtype=torch.int32, device=device))
    pt, total = page_table(table_lens if table_lens is not None else lens, seed, page,
                           spare_pages)
    q_lat, q_rope = queries(len(lens), H, seed + 99, device, d_c, d_r)
    empty_c = torch.zeros(0, d_c, dtype=torch.bfloat16, device=device)
    empty_r = torch.zeros(0, d_r, dtype=torch.bfloat16, device=device)
    empty_i = torch.zeros(0, dtype=torch.int32, device=device)
    return CacheInputs(
        c_kv=torch.cat(cs) if cs else empty_c,
        k_rope=torch.cat(rs) if rs else empty_r,
        seq_idx=torch.cat(si) if si else empty_i,
        pos=torch.cat(ps) if ps else empty_i,
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        page_table=pt.to(device),
        num_pages=total,
        q_lat=q_lat,
        q_rope=q_rope,
    )


@dataclass
class StepTokens:
    """One new token per sequence for a serving step (written at position pos[b])."""
    c_kv: torch.Tensor    # [B, d_c] bf16
    k_rope: torch.Tensor  # [B, d_r] bf16
    pos: torch.Tensor     # [B] int32
    seq_lens: torch.Tensor  # [B] int32, lengths after the step


def workload_inputs(wl: Workload, device="cpu"):
    """Bulk cache contents of a workload (tokens present before the step) and, for
    a serving step, the new tokens. Returns (CacheInputs, StepTokens or None)."""
    lens = wl.lengths()
    if not wl.step_write:
        return build_cache_inputs(lens, wl.H, wl.seed, device), None
    pre = [L - 1 for L in lens]
    inp = build_cache_inputs(pre, wl.H, wl.seed, device, table_lens=lens)
    outl = outlier_channels(wl.seed)
    cs, rs = [], []
    for b, p in enumerate(pre):
        c, r = sequence_tokens(b, p, p + 1, wl.seed, device, outliers=outl)
        cs.append(c)
        rs.append(r)
    step = StepTokens(torch.cat(cs), torch.cat(rs),
                      torch.tensor(pre, dtype=torch.int32, device=device),
                      torch.tensor(lens, dtype=torch.int32, device=device))
    return inp, step


def bulk_cache_inputs(B: int, L: int, H: int, seed: int, device="cpu", outliers=True):
    """B sequences of L tokens each, drawn in one shot (same value recipe as
    build_cache_inputs, not its chunked streams): for large sweeps where the
    chunk loop would dominate. Tokens are in sequence order."""
    outl = outlier_channels(seed) if outliers else None
    n = B * L
    c_kv = latent_tokens(n, seed, device, outliers=outl)
    pos = torch.arange(L, dtype=torch.int32, device=device).repeat(B)
    k_rope = rope_keys(pos, seed + 500_000_000, device)
    seq_idx = torch.arange(B, dtype=torch.int32, device=device).repeat_interleave(L)
    pt, total = page_table([L] * B, seed)
    q_lat, q_rope = queries(B, H, seed + 99, device)
    return CacheInputs(c_kv=c_kv, k_rope=k_rope, seq_idx=seq_idx, pos=pos,
                       seq_lens=torch.full((B,), L, dtype=torch.int32, device=device),
                       page_table=pt.to(device), num_pages=total, q_lat=q_lat, q_rope=q_rope)
