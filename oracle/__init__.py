"""ctypes shim over the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the GPU path and never imports it.

Every function takes and returns numpy arrays. bf16 and fp16 values travel as
their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (always when force, else only if missing)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d_c", "d_r", "c_bits", "r_bits", "group", "page_size", "n_sink", "n_local")]


@dataclass(frozen=True)
class Cfg:
    d_c: int = 512
    d_r: int = 64
    c_bits: int = 4
    r_bits: int = 4
    group: int = 32
    page_size: int = 64
    n_sink: int = 4
    n_local: int = 128

    def c(self) -> _Cfg:
        return _Cfg(self.d_c, self.d_r, self.c_bits, self.r_bits, self.group, self.page_size,
                    self.n_sink, self.n_local)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, f64 = ctypes.c_int, ctypes.c_double
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = f64
        L.orc_f64_to_bf16.argtypes = [f64]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_quantize_group.argtypes = [P, i32, i32, P, P, P]
        L.orc_quantize_group.restype = None
        L.orc_page_bytes.argtypes = [P]
        L.orc_page_bytes.restype = ctypes.c_size_t
        L.orc_page_regions.argtypes = [P, P]
        L.orc_page_regions.restype = None
        L.orc_write.argtypes = [P, i32, P, P, P, P, P, P, i32, i32, P, ctypes.c_int64, P, P]
        L.orc_write.restype = i32
        L.orc_token_source.argtypes = [P, i32, i32]
        L.orc_token_source.restype = i32
        L.orc_token_values.argtypes = [P, i32, i32, P, P, i32, P, P, P, P, P]
        L.orc_token_values.restype = i32
        L.orc_decode.argtypes = [P, i32, i32, f64, P, P, P, P, i32, P, P, P, i32, P, P, i32, i32,
                                 P, P]
        L.orc_decode.restype = i32
        L.orc_combine.argtypes = [i32, i32, P, P, P, P]
        L.orc_combine.restype = None
        L.orc_bf16_page_bytes.argtypes = [P]
        L.orc_bf16_page_bytes.restype = ctypes.c_size_t
        L.orc_bf16_write.argtypes = [P, i32, P, P, P, P, P, i32, i32, P, ctypes.c_int64]
        L.orc_bf16_write.restype = i32
        L.orc_bf16_decode.argtypes = [P, i32, i32, f64, P, P, P, P, i32, P, i32, P, P, P, P]
        L.orc_bf16_decode.restype = i32
        L.orc_qdq.argtypes = [P, i32, P, P, P, P]
        L.orc_qdq.restype = i32
        L.orc_set_num_threads.argtypes = [i32]
        L.orc_set_num_threads.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype in (np.int16, np.float16):
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(ctypes.c_float(x)))


def f16_bits_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(ctypes.c_uint16(h)))


def f64_to_bf16_bits(x: float) -> int:
    return int(lib().orc_f64_to_bf16(ctypes.c_double(x)))


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns (no arithmetic beyond a shift)."""
    b = _u16(b)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantize_group(x, bits: int):
    """Returns (s16 bits, z16 bits, codes uint8[n]) for one group of fp32 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    q = np.zeros(x.size, np.uint8)
    lib().orc_quantize_group(_p(x), x.size, bits, _p(s), _p(z), _p(q))
    return int(s[0]), int(z[0]), q


def page_bytes(cfg: Cfg) -> int:
    c = cfg.c()
    return int(lib().orc_page_bytes(ctypes.byref(c)))


def page_regions(cfg: Cfg):
    c = cfg.c()
    off = np.zeros(4, np.uint64)
    lib().orc_page_regions(ctypes.byref(c), _p(off))
    return [int(v) for v in off]


def write(cfg: Cfg, c_kv, k_rope, seq_idx, pos, seq_lens, page_table, pages: np.ndarray,
          sink: np.ndarray, local: np.ndarray) -> None:
    """Fused writer into host buffers (pages uint8 [num_pages, page_bytes], sink/local
    uint16 [B, n, d_c + d_r]); modifies them in place."""
    c = cfg.c()
    c_kv, k_rope = _u16(c_kv), _u16(k_rope)
    seq_idx, pos, seq_lens, page_table = map(_i32, (seq_idx, pos, seq_lens, page_table))
    B, max_pages = page_table.shape
    assert pages.dtype == np.uint8 and pages.flags["C_CONTIGUOUS"]
    assert sink.dtype == np.uint16 and local.dtype == np.uint16
    num_pages = pages.shape[0]
    rc = lib().orc_write(ctypes.byref(c), int(seq_idx.size), _p(c_kv), _p(k_rope), _p(seq_idx),
                         _p(pos), _p(seq_lens), _p(page_table), B, max_pages, _p(pages),
                         num_pages, _p(sink), _p(local))
    if rc != 0:
        raise ValueError(f"orc_write rejected its arguments ({rc})")


def token_source(cfg: Cfg, p: int, L: int) -> int:
    c = cfg.c()
    return int(lib().orc_token_source(ctypes.byref(c), p, L))


def token_values(cfg: Cfg, b: int, p: int, pages, page_table, seq_lens, sink, local):
    c = cfg.c()
    page_table, seq_lens = _i32(page_table), _i32(seq_lens)
    kc = np.zeros(cfg.d_c, np.float64)
    kr = np.zeros(cfg.d_r, np.float64)
    rc = lib().orc_token_values(ctypes.byref(c), b, p, _p(pages), _p(page_table),
                                page_table.shape[1], _p(seq_lens), _p(_u16(sink)), _p(_u16(local)),
                                _p(kc), _p(kr))
    if rc != 0:
        raise ValueError("orc_token_values rejected its arguments")
    return kc, kr


def decode(cfg: Cfg, scale: float, q_lat, q_rope, pages, page_table, seq_lens, sink, local,
           sel=None, p_begin: int = 0, p_end: int = -1):
    """fp64 decode. q_lat [B,H,d_c], q_rope [B,H,d_r] bf16 bits. sel: optional list of
    (b, h). Returns (out [rows, d_c] fp64, lse [rows] fp64)."""
    c = cfg.c()
    q_lat, q_rope = _u16(q_lat), _u16(q_rope)
    B, H = q_lat.shape[0], q_lat.shape[1]
    page_table, seq_lens = _i32(page_table), _i32(seq_lens)
    if sel is None:
        n_sel, sb, sh = 0, np.zeros(1, np.int32), np.zeros(1, np.int32)
        rows = B * H
    else:
        sel = np.asarray(sel, dtype=np.int32).reshape(-1, 2)
        n_sel, sb, sh = sel.shape[0], _i32(sel[:, 0]), _i32(sel[:, 1])
        rows = n_sel
    out = np.zeros((rows, cfg.d_c), np.float64)
    lse = np.zeros(rows, np.float64)
    rc = lib().orc_decode(ctypes.byref(c), B, H, float(scale), _p(q_lat), _p(q_rope), _p(pages),
                          _p(page_table), page_table.shape[1], _p(seq_lens), _p(_u16(sink)),
                          _p(_u16(local)), n_sel, _p(sb), _p(sh), int(p_begin), int(p_end),
                          _p(out), _p(lse))
    if rc != 0:
        raise ValueError(f"orc_decode rejected its arguments ({rc})")
    return out, lse


def combine(o_s, lse_s):
    """Merge partials o_s [n, d], lse_s [n] of one row."""
    o_s = np.ascontiguousarray(np.asarray(o_s, np.float64))
    lse_s = np.ascontiguousarray(np.asarray(lse_s, np.float64))
    n, d = o_s.shape
    out = np.zeros(d, np.float64)
    lse = np.zeros(1, np.float64)
    lib().orc_combine(n, d, _p(o_s), _p(lse_s), _p(out), _p(lse))
    return out, float(lse[0])


def _sel(B: int, H: int, sel):
    if sel is None:
        return 0, np.zeros(1, np.int32), np.zeros(1, np.int32), B * H
    sel = np.asarray(sel, dtype=np.int32).reshape(-1, 2)
    return sel.shape[0], _i32(sel[:, 0]), _i32(sel[:, 1]), sel.shape[0]


def bf16_page_bytes(cfg: Cfg) -> int:
    c = cfg.c()
    return int(lib().orc_bf16_page_bytes(ctypes.byref(c)))


def bf16_write(cfg: Cfg, c_kv, k_rope, seq_idx, pos, page_table, pages: np.ndarray) -> None:
    """Copy token rows into a BF16 paged cache (pages uint16 [num_pages, page_size,
    d_c + d_r]), in place."""
    c = cfg.c()
    c_kv, k_rope = _u16(c_kv), _u16(k_rope)
    seq_idx, pos, page_table = map(_i32, (seq_idx, pos, page_table))
    B, max_pages = page_table.shape
    assert pages.dtype == np.uint16 and pages.flags["C_CONTIGUOUS"]
    rc = lib().orc_bf16_write(ctypes.byref(c), int(seq_idx.size), _p(c_kv), _p(k_rope),
                              _p(seq_idx), _p(pos), _p(page_table), B, max_pages, _p(pages),
                              pages.shape[0])
    if rc != 0:
        raise ValueError(f"orc_bf16_write rejected its arguments ({rc})")


def bf16_decode(cfg: Cfg, scale: float, q_lat, q_rope, pages, page_table, seq_lens, sel=None):
    """fp64 attention over a BF16 paged cache. Returns (out [rows, d_c], lse [rows])."""
    c = cfg.c()
    q_lat, q_rope = _u16(q_lat), _u16(q_rope)
    B, H = q_lat.shape[0], q_lat.shape[1]
    page_table, seq_lens = _i32(page_table), _i32(seq_lens)
    n_sel, sb, sh, rows = _sel(B, H, sel)
    out = np.zeros((rows, cfg.d_c), np.float64)
    lse = np.zeros(rows, np.float64)
    rc = lib().orc_bf16_decode(ctypes.byref(c), B, H, float(scale), _p(q_lat), _p(q_rope),
                               _p(_u16(pages)), _p(page_table), page_table.shape[1],
                               _p(seq_lens), n_sel, _p(sb), _p(sh), _p(out), _p(lse))
    if rc != 0:
        raise ValueError(f"orc_bf16_decode rejected its arguments ({rc})")
    return out, lse


def qdq(cfg: Cfg, c_kv, k_rope):
    """Simulated quantize-dequantize of token rows; returns bf16 bits (out_c, out_r)."""
    c = cfg.c()
    c_kv, k_rope = _u16(c_kv), _u16(k_rope)
    n = c_kv.shape[0]
    out_c = np.zeros((n, cfg.d_c), np.uint16)
    out_r = np.zeros((n, cfg.d_r), np.uint16)
    rc = lib().orc_qdq(ctypes.byref(c), n, _p(c_kv), _p(k_rope), _p(out_c), _p(out_r))
    if rc != 0:
        raise ValueError(f"orc_qdq rejected its arguments ({rc})")
    return out_c, out_r
