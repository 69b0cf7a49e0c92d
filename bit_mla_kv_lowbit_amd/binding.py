"""ctypes binding over libmla_lowbit.so (declarations: include/mla_lowbit.h).

Argument marshalling only: every step of the write and decode runs in the HIP
kernels. There is no CPU fallback; a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_lowbit.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ELAUNCH, ESCRATCH = 0, -1, -2, -3, -4, -5

# static device scratch of mla_lowbit_decode_noalloc (MLA_LOWBIT_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class MlaLowbitError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed with {code}: {strerror(code)}")


class _CCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d_c", "d_r", "c_bits", "r_bits", "group", "page_size", "n_sink", "n_local")]


@dataclass(frozen=True)
class Config:
    """Cache geometry (mla_lowbit_config)."""
    d_c: int = 512
    d_r: int = 64
    c_bits: int = 4
    r_bits: int = 4
    group: int = 32
    page_size: int = 64
    n_sink: int = 4
    n_local: int = 128

    def c(self) -> _CCfg:
        return _CCfg(self.d_c, self.d_r, self.c_bits, self.r_bits, self.group, self.page_size,
                     self.n_sink, self.n_local)


C4R4 = Config(c_bits=4)
C2R4 = Config(c_bits=2)

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.mla_lowbit_version.argtypes = []
        L.mla_lowbit_version.restype = i32
        L.mla_lowbit_strerror.argtypes = [i32]
        L.mla_lowbit_strerror.restype = ctypes.c_char_p
        L.mla_lowbit_check_config.argtypes = [P]
        L.mla_lowbit_check_config.restype = i32
        L.mla_lowbit_page_bytes.argtypes = [P]
        L.mla_lowbit_page_bytes.restype = sz
        L.mla_lowbit_decode_workspace_bytes.argtypes = [P, i32, i32, i32]
        L.mla_lowbit_decode_workspace_bytes.restype = sz
        L.mla_lowbit_write.argtypes = [P, i32, P, P, P, P, P, P, i32, i32, P, P, P, P]
        L.mla_lowbit_write.restype = i32
        L.mla_lowbit_decode.argtypes = [P, i32, i32, ctypes.c_float, P, P, P, P, i32, P, P, P, P, P,
                                        P, sz, P]
        L.mla_lowbit_decode.restype = i32
        L.mla_lowbit_write_decode.argtypes = [P, i32, i32, ctypes.c_float, P, P, P, P, P, P, P, i32,
                                              P, P, P, P, P, P, sz, P]
        L.mla_lowbit_write_decode.restype = i32
        L.mla_lowbit_decode_noalloc.argtypes = [P, i32, i32, ctypes.c_float, P, P, P, P, i32, P,
                                                P, P, P, P, P]
        L.mla_lowbit_decode_noalloc.restype = i32
        L.mla_lowbit_decode_mq.argtypes = [P, i32, i32, i32, ctypes.c_float, P, P, P, P, i32,
                                           P, P, P, P, P, P, sz, P]
        L.mla_lowbit_decode_mq.restype = i32
        L.mla_lowbit_qdq.argtypes = [P, i32, P, P, P, P, P]
        L.mla_lowbit_qdq.restype = i32
        L.mla_bf16_page_bytes.argtypes = []
        L.mla_bf16_page_bytes.restype = sz
        L.mla_bf16_decode_workspace_bytes.argtypes = [i32, i32, i32]
        L.mla_bf16_decode_workspace_bytes.restype = sz
        L.mla_bf16_write.argtypes = [i32, P, P, P, P, P, i32, i32, P, P]
        L.mla_bf16_write.restype = i32
        L.mla_bf16_decode.argtypes = [i32, i32, ctypes.c_float, P, P, P, P, i32, P, P, P, P, sz, P]
        L.mla_bf16_decode.restype = i32
        _lib = L
    return _lib


def strerror(code: int) -> str:
    try:
        return lib().mla_lowbit_strerror(code).decode()
    except RuntimeError:
        return f"error {code}"


def version() -> int:
    return lib().mla_lowbit_version()


def page_bytes(cfg: Config) -> int:
    c = cfg.c()
    return int(lib().mla_lowbit_page_bytes(ctypes.byref(c)))


def decode_workspace_bytes(cfg: Config, B: int, H: int, max_pages: int) -> int:
    c = cfg.c()
    return int(lib().mla_lowbit_decode_workspace_bytes(ctypes.byref(c), B, H, max_pages))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != OK:
        raise MlaLowbitError(fn, rc)


def _want(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _expect(t, name, dtype, shape):
    """t must be a tensor of `dtype` and exactly `shape` (None: any size).
    The C ABI sees only pointers, so these checks are what keeps a kernel
    from reading or writing past a caller's buffer."""
    _want(t, dtype, name)
    if len(t.shape) != len(shape) or any(
            want is not None and int(got) != want for got, want in zip(t.shape, shape)):
        raise ValueError(f"{name} must have shape {tuple('*' if x is None else x for x in shape)}"
                         f", got {tuple(t.shape)}")


def _check_cache(cfg: "Config", B: int, pages, sink, local, page_table, seq_lens):
    """Packed pages uint8 [num_pages, page_bytes]; sink / local bf16
    [B, n_sink | n_local, d_c + d_r] (unused, may be None, when the count is 0);
    page_table int32 [B, max_pages]; seq_lens int32 [B]."""
    pb = page_bytes(cfg)
    if pb == 0:
        c = cfg.c()
        raise MlaLowbitError("mla_lowbit_check_config", lib().mla_lowbit_check_config(ctypes.byref(c)))
    _expect(pages, "pages", torch.uint8, (None, pb))
    D = cfg.d_c + cfg.d_r
    if cfg.n_sink > 0:
        _expect(sink, "sink", torch.bfloat16, (B, cfg.n_sink, D))
    if cfg.n_local > 0:
        _expect(local, "local", torch.bfloat16, (B, cfg.n_local, D))
    _expect(page_table, "page_table", torch.int32, (B, None))
    if page_table.shape[1] < 1:
        raise ValueError("page_table needs at least one column")
    _expect(seq_lens, "seq_lens", torch.int32, (B,))


def _outputs(out, lse, shape, dev):
    """Allocate or check out (bf16 [*shape, d_c]) and lse (fp32 shape)."""
    if out is None:
        out = torch.empty(*shape, 512, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(*shape, dtype=torch.float32, device=dev)
    _expect(out, "out", torch.bfloat16, (*shape, 512))
    _expect(lse, "lse", torch.float32, tuple(shape))
    return out, lse


def _workspace(workspace, need, dev):
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _want(workspace, torch.uint8, "workspace")
    return workspace


def allocate_cache(cfg: Config, B: int, num_pages: int, device="cuda"):
    """Zeroed device buffers for a cache: pages uint8 [num_pages, page_bytes],
    sink / local bf16 [B, n, d_c + d_r]."""
    D = cfg.d_c + cfg.d_r
    pages = torch.zeros(num_pages, page_bytes(cfg), dtype=torch.uint8, device=device)
    sink = torch.zeros(B, max(cfg.n_sink, 1), D, dtype=torch.bfloat16, device=device)
    local = torch.zeros(B, max(cfg.n_local, 1), D, dtype=torch.bfloat16, device=device)
    return pages, sink, local


def write(cfg: Config, c_kv, k_rope, seq_idx, pos, seq_lens, page_table, pages, sink, local,
          stream=None) -> None:
    """mla_lowbit_write: quantize + pack every token, keep BF16 copies of protected ones."""
    _want(seq_idx, torch.int32, "seq_idx")
    n = int(seq_idx.numel())
    _expect(seq_idx, "seq_idx", torch.int32, (n,))
    _expect(c_kv, "c_kv", torch.bfloat16, (n, cfg.d_c))
    _expect(k_rope, "k_rope", torch.bfloat16, (n, cfg.d_r))
    _expect(pos, "pos", torch.int32, (n,))
    _want(page_table, torch.int32, "page_table")
    B, max_pages = page_table.shape
    _check_cache(cfg, B, pages, sink, local, page_table, seq_lens)
    c = cfg.c()
    rc = lib().mla_lowbit_write(ctypes.byref(c), n, _ptr(c_kv), _ptr(k_rope), _ptr(seq_idx),
                                _ptr(pos), _ptr(seq_lens), _ptr(page_table), B, max_pages,
                                _ptr(pages), _ptr(sink), _ptr(local), _stream(stream))
    _check("mla_lowbit_write", rc)


def decode(cfg: Config, q_lat, q_rope, pages, page_table, seq_lens, sink, local, scale: float,
           out=None, lse=None, workspace=None, stream=None):
    """mla_lowbit_decode. Returns (out bf16 [B,H,d_c], lse fp32 [B,H])."""
    _want(q_lat, torch.bfloat16, "q_lat")
    if q_lat.dim() != 3:
        raise ValueError("q_lat must be [B, H, d_c]")
    B, H, _ = q_lat.shape
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, cfg.d_c))
    _expect(q_rope, "q_rope", torch.bfloat16, (B, H, cfg.d_r))
    _check_cache(cfg, B, pages, sink, local, page_table, seq_lens)
    max_pages = page_table.shape[1]
    dev = q_lat.device
    out, lse = _outputs(out, lse, (B, H), dev)
    workspace = _workspace(workspace, decode_workspace_bytes(cfg, B, H, max_pages), dev)
    c = cfg.c()
    rc = lib().mla_lowbit_decode(ctypes.byref(c), B, H, float(scale), _ptr(q_lat), _ptr(q_rope),
                                 _ptr(pages), _ptr(page_table), max_pages, _ptr(seq_lens),
                                 _ptr(sink), _ptr(local), _ptr(out), _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_lowbit_decode", rc)
    return out, lse


def decode_noalloc(cfg: Config, q_lat, q_rope, pages, page_table, seq_lens, sink, local,
                   scale: float, out, lse, stream=None):
    """mla_lowbit_decode_noalloc: mla_lowbit_decode with the library's static
    device scratch in place of a workspace. out (bf16 [B, H, d_c]) and lse
    (fp32 [B, H]) must be given; the call allocates nothing. Calls that overlap
    on one GPU share the scratch and race."""
    _want(q_lat, torch.bfloat16, "q_lat")
    if q_lat.dim() != 3:
        raise ValueError("q_lat must be [B, H, d_c]")
    B, H, _ = q_lat.shape
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, cfg.d_c))
    _expect(q_rope, "q_rope", torch.bfloat16, (B, H, cfg.d_r))
    _check_cache(cfg, B, pages, sink, local, page_table, seq_lens)
    if out is None or lse is None:
        raise ValueError("decode_noalloc allocates nothing: pass out and lse")
    _expect(out, "out", torch.bfloat16, (B, H, cfg.d_c))
    _expect(lse, "lse", torch.float32, (B, H))
    c = cfg.c()
    rc = lib().mla_lowbit_decode_noalloc(ctypes.byref(c), B, H, float(scale), _ptr(q_lat),
                                         _ptr(q_rope), _ptr(pages), _ptr(page_table),
                                         page_table.shape[1], _ptr(seq_lens), _ptr(sink),
                                         _ptr(local), _ptr(out), _ptr(lse), _stream(stream))
    _check("mla_lowbit_decode_noalloc", rc)
    return out, lse


def decode_mq(cfg: Config, q_lat, q_rope, pages, page_table, seq_lens, sink, local,
              scale: float, out=None, lse=None, workspace=None, stream=None):
    """mla_lowbit_decode_mq: q_lat [B, s_q, H, d_c], q_rope [B, s_q, H, d_r]; query token i
    attends to tokens p < seq_lens[b] - (s_q - 1 - i). Returns (out [B, s_q, H, d_c] bf16,
    lse [B, s_q, H] fp32)."""
    _want(q_lat, torch.bfloat16, "q_lat")
    _want(q_rope, torch.bfloat16, "q_rope")
    if q_lat.dim() != 4 or q_lat.shape[3] != cfg.d_c:
        raise ValueError("q_lat must be [B, s_q, H, d_c]")
    B, s_q, H, _ = q_lat.shape
    if q_rope.shape != (B, s_q, H, cfg.d_r):
        raise ValueError("q_rope must be [B, s_q, H, d_r]")
    _check_cache(cfg, B, pages, sink, local, page_table, seq_lens)
    max_pages = page_table.shape[1]
    dev = q_lat.device
    out, lse = _outputs(out, lse, (B, s_q, H), dev)
    workspace = _workspace(workspace, decode_workspace_bytes(cfg, B, s_q * H, max_pages), dev)
    c = cfg.c()
    rc = lib().mla_lowbit_decode_mq(ctypes.byref(c), B, s_q, H, float(scale), _ptr(q_lat),
                                    _ptr(q_rope), _ptr(pages), _ptr(page_table), max_pages,
                                    _ptr(seq_lens), _ptr(sink), _ptr(local), _ptr(out),
                                    _ptr(lse), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check("mla_lowbit_decode_mq", rc)
    return out, lse


def write_decode(cfg: Config, c_kv, k_rope, pos, q_lat, q_rope, pages, page_table, seq_lens,
                 sink, local, scale: float, out=None, lse=None, workspace=None, stream=None):
    """mla_lowbit_write_decode: one new token per sequence (c_kv [B, d_c], k_rope
    [B, d_r], pos [B]), then decode."""
    _want(q_lat, torch.bfloat16, "q_lat")
    if q_lat.dim() != 3:
        raise ValueError("q_lat must be [B, H, d_c]")
    B, H, _ = q_lat.shape
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, cfg.d_c))
    _expect(q_rope, "q_rope", torch.bfloat16, (B, H, cfg.d_r))
    _expect(c_kv, "c_kv", torch.bfloat16, (B, cfg.d_c))
    _expect(k_rope, "k_rope", torch.bfloat16, (B, cfg.d_r))
    _expect(pos, "pos", torch.int32, (B,))
    _check_cache(cfg, B, pages, sink, local, page_table, seq_lens)
    max_pages = page_table.shape[1]
    dev = q_lat.device
    out, lse = _outputs(out, lse, (B, H), dev)
    workspace = _workspace(workspace, decode_workspace_bytes(cfg, B, H, max_pages), dev)
    c = cfg.c()
    rc = lib().mla_lowbit_write_decode(ctypes.byref(c), B, H, float(scale), _ptr(c_kv),
                                       _ptr(k_rope), _ptr(pos), _ptr(q_lat), _ptr(q_rope),
                                       _ptr(pages), _ptr(page_table), max_pages, _ptr(seq_lens),
                                       _ptr(sink), _ptr(local), _ptr(out), _ptr(lse),
                                       _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    _check("mla_lowbit_write_decode", rc)
    return out, lse


def qdq(cfg: Config, c_kv, k_rope, out_c=None, out_r=None, stream=None):
    """mla_lowbit_qdq: simulated quantize-dequantize of token rows (bf16 in, bf16 out)."""
    _want(c_kv, torch.bfloat16, "c_kv")
    _want(k_rope, torch.bfloat16, "k_rope")
    n = int(c_kv.shape[0])
    if c_kv.shape != (n, cfg.d_c) or k_rope.shape != (n, cfg.d_r):
        raise ValueError("c_kv / k_rope shapes do not match the config")
    if out_c is None:
        out_c = torch.empty_like(c_kv)
    if out_r is None:
        out_r = torch.empty_like(k_rope)
    if out_c.shape != c_kv.shape or out_r.shape != k_rope.shape:
        raise ValueError("out_c / out_r must match c_kv / k_rope")
    c = cfg.c()
    rc = lib().mla_lowbit_qdq(ctypes.byref(c), n, _ptr(c_kv), _ptr(k_rope), _ptr(out_c),
                              _ptr(out_r), _stream(stream))
    _check("mla_lowbit_qdq", rc)
    return out_c, out_r


def bf16_page_bytes() -> int:
    return int(lib().mla_bf16_page_bytes())


def bf16_decode_workspace_bytes(B: int, H: int, max_pages: int) -> int:
    return int(lib().mla_bf16_decode_workspace_bytes(B, H, max_pages))


def allocate_bf16_cache(num_pages: int, device="cuda", d_c: int = 512, d_r: int = 64,
                        page_size: int = 64):
    """Zeroed BF16 paged cache: bf16 [num_pages, page_size, d_c + d_r]."""
    return torch.zeros(num_pages, page_size, d_c + d_r, dtype=torch.bfloat16, device=device)


def bf16_write(c_kv, k_rope, seq_idx, pos, page_table, pages, stream=None) -> None:
    """mla_bf16_write: copy token rows into the BF16 paged cache."""
    _want(seq_idx, torch.int32, "seq_idx")
    n = int(seq_idx.numel())
    _expect(seq_idx, "seq_idx", torch.int32, (n,))
    _expect(c_kv, "c_kv", torch.bfloat16, (n, 512))
    _expect(k_rope, "k_rope", torch.bfloat16, (n, 64))
    _expect(pos, "pos", torch.int32, (n,))
    _expect(pages, "pages", torch.bfloat16, (None, 64, 576))
    _expect(page_table, "page_table", torch.int32, (None, None))
    B, max_pages = page_table.shape
    rc = lib().mla_bf16_write(n, _ptr(c_kv), _ptr(k_rope), _ptr(seq_idx), _ptr(pos),
                              _ptr(page_table), B, max_pages, _ptr(pages), _stream(stream))
    _check("mla_bf16_write", rc)


def bf16_decode(q_lat, q_rope, pages, page_table, seq_lens, scale: float, out=None, lse=None,
                workspace=None, stream=None):
    """mla_bf16_decode. Returns (out bf16 [B,H,512], lse fp32 [B,H])."""
    _want(q_lat, torch.bfloat16, "q_lat")
    _want(q_rope, torch.bfloat16, "q_rope")
    if q_lat.dim() != 3 or q_lat.shape[2] != 512:
        raise ValueError("q_lat must be [B, H, 512]")
    B, H, d_c = q_lat.shape
    if q_rope.shape != (B, H, 64):
        raise ValueError("q_rope must be [B, H, 64]")
    _expect(pages, "pages", torch.bfloat16, (None, 64, 576))
    _expect(page_table, "page_table", torch.int32, (B, None))
    _expect(seq_lens, "seq_lens", torch.int32, (B,))
    max_pages = page_table.shape[1]
    dev = q_lat.device
    out, lse = _outputs(out, lse, (B, H), dev)
    workspace = _workspace(workspace, bf16_decode_workspace_bytes(B, H, max_pages), dev)
    rc = lib().mla_bf16_decode(B, H, float(scale), _ptr(q_lat), _ptr(q_rope), _ptr(pages),
                               _ptr(page_table), max_pages, _ptr(seq_lens), _ptr(out), _ptr(lse),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check("mla_bf16_decode", rc)
    return out, lse
