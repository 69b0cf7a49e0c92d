"""C-ABI library checks that need no GPU: it loads, exports every symbol that
include/mla_lowbit.h declares, answers the size queries, and rejects bad
arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import bit_mla_kv_lowbit_amd as mla
from bit_mla_kv_lowbit_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_lowbit.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_(?:lowbit|bf16)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["mla_lowbit_write", "mla_lowbit_decode", "mla_lowbit_write_decode",
              "mla_lowbit_page_bytes", "mla_lowbit_decode_workspace_bytes",
              "mla_lowbit_strerror", "mla_lowbit_version", "mla_lowbit_check_config",
              "mla_lowbit_qdq", "mla_lowbit_decode_mq", "mla_bf16_page_bytes", "mla_bf16_decode_workspace_bytes",
              "mla_bf16_write", "mla_bf16_decode"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    for n in _declared():
        assert hasattr(L, n), n


def test_size_queries():
    assert mla.page_bytes(mla.C4R4) == 23040
    assert mla.page_bytes(mla.C2R4) == 14848
    assert mla.page_bytes(mla.Config(group=64)) == 64 * 324
    assert mla.page_bytes(mla.Config(c_bits=2, r_bits=2, group=128)) == 64 * 164
    assert mla.page_bytes(mla.Config(group=48)) == 0
    ws = mla.decode_workspace_bytes(mla.C4R4, 8, 16, 512)
    assert ws > 0 and ws % 4 == 0
    assert mla.decode_workspace_bytes(mla.C4R4, 8, 24, 512) == 0  # H not a multiple of 16
    assert mla.decode_workspace_bytes(mla.C4R4, 8, 16, 0) == 0
    assert mla.version() >= 100
    assert "workspace" in binding.strerror(binding.EWORKSPACE)


@pytest.mark.parametrize("c_bits,r_bits,group", [(c, r, g) for c in (4, 2) for r in (4, 2)
                                                 for g in (32, 64, 128)])
def test_variant_page_bytes_match_the_oracle(c_bits, r_bits, group):
    import oracle
    cfg = mla.Config(c_bits=c_bits, r_bits=r_bits, group=group)
    c = cfg.c()
    assert mla.lib().mla_lowbit_check_config(ctypes.byref(c)) == binding.OK
    assert mla.page_bytes(cfg) == oracle.page_bytes(oracle.Cfg(c_bits=c_bits, r_bits=r_bits,
                                                               group=group))


@pytest.mark.parametrize("bad", [dict(d_c=256), dict(d_r=32), dict(c_bits=3), dict(r_bits=3),
                                 dict(group=16), dict(group=256), dict(page_size=32), dict(n_sink=65),
                                 dict(n_local=257), dict(n_sink=-1)])
def test_unsupported_configs(bad):
    c = mla.Config(**bad).c()
    assert mla.lib().mla_lowbit_check_config(ctypes.byref(c)) == binding.EUNSUPPORTED


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def _decode_call(cfg=mla.C4R4, B=2, H=16, scale=0.1, ws_bytes=1 << 40, **over):
    args = dict(q_lat=_fake(), q_rope=_fake(), pages=_fake(), page_table=_fake(),
                seq_lens=_fake(), sink=_fake(), local=_fake(), out=_fake(), lse=_fake(),
                ws=_fake())
    args.update(over)
    c = cfg.c()
    return mla.lib().mla_lowbit_decode(ctypes.byref(c), B, H, scale, args["q_lat"],
                                       args["q_rope"], args["pages"], args["page_table"], 4,
                                       args["seq_lens"], args["sink"], args["local"], args["out"],
                                       args["lse"], args["ws"], ws_bytes, None)


def test_decode_validation_errors():
    # each call fails host-side validation, so nothing is launched
    assert _decode_call(H=24) == binding.EINVAL
    assert _decode_call(H=0) == binding.EINVAL
    assert _decode_call(B=-1) == binding.EINVAL
    assert _decode_call(scale=0.0) == binding.EINVAL
    assert _decode_call(scale=float("nan")) == binding.EINVAL
    assert _decode_call(q_lat=None) == binding.EINVAL
    assert _decode_call(out=_fake(0x10008)) == binding.EINVAL  # misaligned
    assert _decode_call(ws_bytes=16) == binding.EWORKSPACE
    assert _decode_call(cfg=mla.Config(c_bits=3)) == binding.EUNSUPPORTED
    # zero sequences is a valid no-op
    assert _decode_call(B=0) == binding.OK


def test_write_validation_errors():
    c = mla.C4R4.c()
    L = mla.lib()

    def call(n=4, B=2, max_pages=4, c_kv=_fake(), pages=_fake(), sink=_fake(), cfg=c):
        return L.mla_lowbit_write(ctypes.byref(cfg), n, c_kv, _fake(), _fake(), _fake(), _fake(),
                                  _fake(), B, max_pages, pages, sink, _fake(), None)

    assert call(n=-1) == binding.EINVAL
    assert call(c_kv=None) == binding.EINVAL
    assert call(pages=_fake(0x10004)) == binding.EINVAL
    assert call(sink=None) == binding.EINVAL
    assert call(max_pages=0) == binding.EINVAL
    assert call(B=0) == binding.EINVAL
    assert call(cfg=mla.Config(r_bits=3).c()) == binding.EUNSUPPORTED
    assert call(n=0) == binding.OK  # nothing to write


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding._ptr(t)


def test_bf16_size_queries():
    assert mla.bf16_page_bytes() == 64 * 576 * 2
    assert mla.bf16_decode_workspace_bytes(8, 16, 512) == mla.decode_workspace_bytes(
        mla.C4R4, 8, 16, 512)
    assert mla.bf16_decode_workspace_bytes(8, 24, 512) == 0
    assert mla.bf16_decode_workspace_bytes(8, 16, 0) == 0


def test_bf16_validation_errors():
    L = mla.lib()

    def dec(B=2, H=16, scale=0.1, ws_bytes=1 << 40, q_lat=_fake(), out=_fake()):
        return L.mla_bf16_decode(B, H, scale, q_lat, _fake(), _fake(), _fake(), 4, _fake(), out,
                                 _fake(), _fake(), ws_bytes, None)

    assert dec(H=24) == binding.EINVAL
    assert dec(B=-1) == binding.EINVAL
    assert dec(scale=-1.0) == binding.EINVAL
    assert dec(q_lat=None) == binding.EINVAL
    assert dec(out=_fake(0x10002)) == binding.EINVAL
    assert dec(ws_bytes=8) == binding.EWORKSPACE
    assert dec(B=0) == binding.OK

    def wr(n=4, B=2, max_pages=4, pages=_fake(), seq_idx=_fake()):
        return L.mla_bf16_write(n, _fake(), _fake(), seq_idx, _fake(), _fake(), B, max_pages,
                                pages, None)

    assert wr(n=-1) == binding.EINVAL
    assert wr(pages=None) == binding.EINVAL
    assert wr(seq_idx=None) == binding.EINVAL
    assert wr(max_pages=0) == binding.EINVAL
    assert wr(B=0) == binding.EINVAL
    assert wr(n=0) == binding.OK


def test_qdq_validation_errors():
    L = mla.lib()

    def call(cfg=mla.C4R4, n=4, out_c=_fake()):
        c = cfg.c()
        return L.mla_lowbit_qdq(ctypes.byref(c), n, _fake(), _fake(), out_c, _fake(), None)

    assert call(n=-1) == binding.EINVAL
    assert call(out_c=None) == binding.EINVAL
    assert call(out_c=_fake(0x10004)) == binding.EINVAL
    assert call(cfg=mla.Config(c_bits=8)) == binding.EUNSUPPORTED
    assert call(n=0) == binding.OK


def test_decode_mq_validation_errors():
    L = mla.lib()

    def call(B=2, s_q=2, H=16, ws_bytes=1 << 40, q_lat=_fake()):
        c = mla.C4R4.c()
        return L.mla_lowbit_decode_mq(ctypes.byref(c), B, s_q, H, 0.1, q_lat, _fake(), _fake(),
                                      _fake(), 4, _fake(), _fake(), _fake(), _fake(), _fake(),
                                      _fake(), ws_bytes, None)

    assert call(s_q=0) == binding.EINVAL
    assert call(H=8) == binding.EINVAL  # s_q * H = 16, but a head block would span two tokens
    assert call(H=24) == binding.EINVAL
    assert call(q_lat=None) == binding.EINVAL
    assert call(ws_bytes=16) == binding.EWORKSPACE
    assert call(B=0) == binding.OK


def test_binding_shape_checks():
    """The binding rejects mismatched shapes before it touches the GPU."""
    import torch
    bf = torch.bfloat16
    i32 = torch.int32
    pt = torch.zeros(2, 4, dtype=i32)
    sl = torch.zeros(2, dtype=i32)
    with pytest.raises(ValueError):  # q_lat must be 4-D for the multi-query call
        mla.decode_mq(mla.C4R4, torch.zeros(2, 16, 512, dtype=bf), torch.zeros(2, 16, 64, dtype=bf),
                      None, pt, sl, None, None, 0.1)
    with pytest.raises(ValueError):  # q_rope shape differs from q_lat's
        mla.decode_mq(mla.C4R4, torch.zeros(2, 2, 16, 512, dtype=bf),
                      torch.zeros(2, 1, 16, 64, dtype=bf), None, pt, sl, None, None, 0.1)
    with pytest.raises(ValueError):  # BF16 pages must be [num_pages, 64, 576]
        mla.bf16_decode(torch.zeros(2, 16, 512, dtype=bf), torch.zeros(2, 16, 64, dtype=bf),
                        torch.zeros(4, 64, 512, dtype=bf), pt, sl, 0.1)
    with pytest.raises(ValueError):  # token rows must be [n, 512] / [n, 64]
        mla.bf16_write(torch.zeros(3, 512, dtype=bf), torch.zeros(3, 32, dtype=bf),
                       torch.zeros(3, dtype=i32), torch.zeros(3, dtype=i32), pt,
                       torch.zeros(4, 64, 576, dtype=bf))
    with pytest.raises(ValueError):  # QDQ outputs must match the inputs
        mla.qdq(mla.C4R4, torch.zeros(3, 512, dtype=bf), torch.zeros(3, 64, dtype=bf),
                out_c=torch.zeros(2, 512, dtype=bf))


def _bad_shape(fn, *a, match="must have shape", **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_binding_checks_every_tensor_of_decode_and_write():
    """Every tensor a call hands to the C ABI is checked for dtype and shape on
    the host first (CPU tensors here: a check that passed would go on to the
    device-pointer check, whose message differs)."""
    import torch
    bf, i32, u8, f32 = torch.bfloat16, torch.int32, torch.uint8, torch.float32
    cfg = mla.C4R4
    B, H, P = 2, 16, 4
    good = dict(q_lat=torch.zeros(B, H, 512, dtype=bf), q_rope=torch.zeros(B, H, 64, dtype=bf),
                pages=torch.zeros(8, 23040, dtype=u8), page_table=torch.zeros(B, P, dtype=i32),
                seq_lens=torch.zeros(B, dtype=i32), sink=torch.zeros(B, 4, 576, dtype=bf),
                local=torch.zeros(B, 128, 576, dtype=bf))

    def dec(**over):
        a = dict(good, **over)
        return mla.decode(cfg, a["q_lat"], a["q_rope"], a["pages"], a["page_table"],
                          a["seq_lens"], a["sink"], a["local"], 0.1, out=a.get("out"),
                          lse=a.get("lse"), workspace=a.get("workspace"))

    # all shapes right: the first failure is the device check of the first pointer
    with pytest.raises(ValueError, match="GPU"):
        dec(out=torch.zeros(B, H, 512, dtype=bf), lse=torch.zeros(B, H, dtype=f32),
            workspace=torch.zeros(16, dtype=u8))
    _bad_shape(dec, q_rope=torch.zeros(B, H, 32, dtype=bf))
    _bad_shape(dec, q_rope=torch.zeros(B, H + 16, 64, dtype=bf))
    _bad_shape(dec, pages=torch.zeros(8, 14848, dtype=u8))            # C2R4 pages for C4R4
    _bad_shape(dec, page_table=torch.zeros(B + 1, P, dtype=i32))
    _bad_shape(dec, seq_lens=torch.zeros(B - 1, dtype=i32))
    _bad_shape(dec, sink=torch.zeros(B, 2, 576, dtype=bf))
    _bad_shape(dec, local=torch.zeros(B - 1, 128, 576, dtype=bf))
    _bad_shape(dec, out=torch.zeros(B, H, 256, dtype=bf))
    _bad_shape(dec, lse=torch.zeros(B, H + 1, dtype=f32))
    with pytest.raises(TypeError):
        dec(lse=torch.zeros(B, H, dtype=bf))
    with pytest.raises(TypeError):
        dec(seq_lens=torch.zeros(B, dtype=torch.int64))
    with pytest.raises(TypeError):
        dec(q_rope=torch.zeros(B, H, 64, dtype=torch.float16))
    with pytest.raises(TypeError):
        dec(pages=torch.zeros(8, 23040 // 2, dtype=torch.int16))
    with pytest.raises(TypeError):
        dec(sink=None)

    def wd(**over):
        a = dict(good, c_kv=torch.zeros(B, 512, dtype=bf), k_rope=torch.zeros(B, 64, dtype=bf),
                 pos=torch.zeros(B, dtype=i32))
        a.update(over)
        return mla.write_decode(cfg, a["c_kv"], a["k_rope"], a["pos"], a["q_lat"], a["q_rope"],
                                a["pages"], a["page_table"], a["seq_lens"], a["sink"],
                                a["local"], 0.1)

    _bad_shape(wd, c_kv=torch.zeros(B + 1, 512, dtype=bf))
    _bad_shape(wd, k_rope=torch.zeros(B, 32, dtype=bf))
    _bad_shape(wd, pos=torch.zeros(B + 1, dtype=i32))
    _bad_shape(wd, seq_lens=torch.zeros(B + 1, dtype=i32))
    with pytest.raises(TypeError):
        wd(pos=torch.zeros(B, dtype=torch.int64))

    n = 3

    def wr(**over):
        a = dict(good, c_kv=torch.zeros(n, 512, dtype=bf), k_rope=torch.zeros(n, 64, dtype=bf),
                 seq_idx=torch.zeros(n, dtype=i32), pos=torch.zeros(n, dtype=i32))
        a.update(over)
        return mla.write(cfg, a["c_kv"], a["k_rope"], a["seq_idx"], a["pos"], a["seq_lens"],
                         a["page_table"], a["pages"], a["sink"], a["local"])

    with pytest.raises(ValueError, match="GPU"):
        wr()
    _bad_shape(wr, pos=torch.zeros(n + 1, dtype=i32))
    _bad_shape(wr, c_kv=torch.zeros(n, 256, dtype=bf))
    _bad_shape(wr, seq_lens=torch.zeros(B + 2, dtype=i32))
    _bad_shape(wr, local=torch.zeros(B, 64, 576, dtype=bf))
    _bad_shape(wr, pages=torch.zeros(8, 23041, dtype=u8))
    with pytest.raises(binding.MlaLowbitError):  # unsupported config: refused before shapes
        mla.decode(mla.Config(group=48), good["q_lat"], good["q_rope"], good["pages"],
                   good["page_table"], good["seq_lens"], good["sink"], good["local"], 0.1)


def test_binding_checks_bf16_and_mq_outputs():
    import torch
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    B, H = 2, 16
    pages = torch.zeros(4, 64, 576, dtype=bf)
    pt = torch.zeros(B, 4, dtype=i32)
    sl = torch.zeros(B, dtype=i32)
    q, qr = torch.zeros(B, H, 512, dtype=bf), torch.zeros(B, H, 64, dtype=bf)
    _bad_shape(mla.bf16_decode, q, qr, pages, torch.zeros(B + 1, 4, dtype=i32), sl, 0.1)
    _bad_shape(mla.bf16_decode, q, qr, pages, pt, torch.zeros(B + 1, dtype=i32), 0.1)
    _bad_shape(mla.bf16_decode, q, qr, pages, pt, sl, 0.1, out=torch.zeros(B, H, 64, dtype=bf))
    _bad_shape(mla.bf16_decode, q, qr, pages, pt, sl, 0.1, lse=torch.zeros(B, dtype=f32))
    qm, qrm = torch.zeros(B, 2, H, 512, dtype=bf), torch.zeros(B, 2, H, 64, dtype=bf)
    p8 = torch.zeros(4, 23040, dtype=torch.uint8)
    sink, local = torch.zeros(B, 4, 576, dtype=bf), torch.zeros(B, 128, 576, dtype=bf)
    _bad_shape(mla.decode_mq, mla.C4R4, qm, qrm, p8, pt, sl, sink, local, 0.1,
               out=torch.zeros(B, H, 512, dtype=bf))
    _bad_shape(mla.decode_mq, mla.C4R4, qm, qrm, p8, pt, torch.zeros(B, 1, dtype=i32), sink,
               local, 0.1)


def test_noalloc_rejects_bad_arguments_before_the_device():
    c = mla.C4R4.c()
    L = mla.lib()

    def call(B=2, H=16, max_pages=4, q_lat=_fake(), out=_fake(), scale=0.1):
        return L.mla_lowbit_decode_noalloc(ctypes.byref(c), B, H, scale, q_lat, _fake(), _fake(),
                                           _fake(), max_pages, _fake(), _fake(), _fake(), out,
                                           _fake(), None)

    assert call(H=24) == binding.EINVAL
    assert call(q_lat=None) == binding.EINVAL
    assert call(out=_fake(0x10002)) == binding.EINVAL
    assert call(scale=-1.0) == binding.EINVAL
    assert call(B=0) == binding.OK
    assert call(B=64, H=1024, max_pages=4096) == binding.ESCRATCH
