"""The C-ABI library builds, loads and exports every symbol include/vc.h declares
(no compute: these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "compressed_kv_draft_amd", "libvc.so")
HDR = os.path.join(ROOT, "include", "vc.h")


def declared_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(vc_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("vc_draft_attn", "vc_verify_attn", "vc_accept", "vc_prefetch_full_kv",
                 "vc_quantize_kv", "vc_debug_dequant", "vc_argmax", "vc_draft_ws_bytes",
                 "vc_verify_ws_bytes", "vc_last_error", "vc_version"):
        assert want in names, want


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libvc.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_the_header():
    # the Python binding declares argtypes for every C entry point (parsed, not imported:
    # importing it would need a GPU runtime)
    src = open(os.path.join(ROOT, "compressed_kv_draft_amd", "_lib.py")).read()
    for n in declared_functions():
        assert f'"{n}"' in src, n


def test_host_validation_without_gpu(lib):
    """Argument checks run on the host before anything is enqueued."""
    lib.vc_last_error.restype = ctypes.c_char_p
    lib.vc_version.restype = ctypes.c_int
    assert lib.vc_version() >= 1
    f = lib.vc_draft_attn
    f.restype = ctypes.c_int
    rc = f(None, None, None, None, None, 1, 4, 1, 64, ctypes.c_float(0.125), None, ctypes.c_size_t(0), None)
    assert rc == -1
    assert b"null" in lib.vc_last_error()
    g = lib.vc_argmax
    g.restype = ctypes.c_int
    assert g(None, 1, 10, None, None) == -1
    h = lib.vc_accept
    h.restype = ctypes.c_int
    assert h(None, None, 1, 2, 3, None, None, None) == -1
    # chunked verify: the slot count is a host-side plan (deterministic, positive
    # for a valid range, 0 otherwise); the range and merge calls reject bad input
    rp = lib.vc_verify_range_parts
    rp.restype = ctypes.c_int
    n = rp(8, 64, 8, 128, 33, 0, 4096)
    assert n >= 1 and n == rp(8, 64, 8, 128, 33, 0, 4096)
    assert rp(8, 64, 8, 128, 33, 4096, 4096) == 0 and rp(8, 64, 8, 96, 33, 0, 4096) == 0
    r = lib.vc_verify_attn_range
    r.restype = ctypes.c_int
    assert r(None, None, None, 4096, 33, 0, 4096, None, 8, 64, 8, 128, ctypes.c_float(0.088), None) == -1
    m = lib.vc_verify_merge
    m.restype = ctypes.c_int
    assert m(None, 0, 8, 64, 33, 128, None, None) == -1
    # rollover quantiser: descriptor checks and range checks against the source
    # and the cache capacity all come before any launch
    qb = lib.vc_quantize_blocks
    qb.restype = ctypes.c_int
    assert qb(None, None, 1, 1, 64, 128, 0, 1, None, 0, None) == -1

    class Desc(ctypes.Structure):
        _fields_ = [("kind", ctypes.c_int), ("bits", ctypes.c_int), ("n_quant", ctypes.c_int)] + \
                   [(f, ctypes.c_void_p) for f in ("k_codes", "v_codes", "k_meta", "v_meta", "k_full", "v_full")] + \
                   [("L_full", ctypes.c_int), ("L_cap", ctypes.c_int), ("keep_idx", ctypes.c_void_p),
                    ("n_keep", ctypes.c_int), ("q_cap", ctypes.c_int)]
    d = Desc(kind=1, bits=2, n_quant=64, q_cap=128)
    ref = ctypes.byref(d)
    assert qb(None, None, 1, 1, 256, 128, 0, 0, ref, 4, None) == 0            # empty append at the end
    assert qb(None, None, 1, 1, 256, 128, 0, 1, ref, 4, None) == -1           # past the capacity
    assert b"outside" in lib.vc_last_error()
    assert qb(None, None, 1, 1, 256, 128, 240, 1, ref, 2, None) == -1         # past the source rows
    assert qb(None, None, 1, 1, 256, 128, 0, 1, ref, 2, None) == -1           # null sources
    assert qb(None, None, 1, 1, 256, 96, 0, 1, ref, 2, None) == -2           # D=96 unsupported
    d.q_cap = 100
    assert qb(None, None, 1, 1, 256, 128, 0, 1, ref, 0, None) == -1           # capacity not a multiple of 32
    d.kind = 2
    assert qb(None, None, 1, 1, 256, 128, 0, 1, ref, 0, None) == -1
    # canonical <-> internal QUANT conversion: every check precedes the launch
    pk, up = lib.vc_pack_quant, lib.vc_unpack_quant
    pk.restype = up.restype = ctypes.c_int
    q = Desc(kind=1, bits=4, n_quant=64, q_cap=128)
    qr = ctypes.byref(q)
    assert pk(None, None, None, None, 1, 1, 64, 128, None, 0, None) == -1      # null descriptor
    assert up(None, 1, 1, 128, None, None, None, None, None) == -1
    assert pk(None, None, None, None, 1, 1, 0, 128, qr, 4, None) == 0          # nothing to convert
    assert pk(None, None, None, None, 1, 1, 64, 128, qr, 0, None) == -1        # null canonical arrays
    assert b"null" in lib.vc_last_error()
    assert pk(None, None, None, None, 1, 1, 48, 128, qr, 0, None) == -1        # rows not whole blocks
    assert pk(None, None, None, None, 1, 1, 64, 128, qr, 3, None) == -1        # blocks past the capacity
    assert b"outside" in lib.vc_last_error()
    assert pk(None, None, None, None, 1, 1, 64, 96, qr, 0, None) == -2         # D=96 unsupported
    assert pk(None, None, None, None, 0, 1, 64, 128, qr, 0, None) == -1        # B = 0
    q.bits = 3
    assert pk(None, None, None, None, 1, 1, 64, 128, qr, 0, None) == -1        # bits not 2 or 4
    q.bits, q.kind = 4, 2
    assert up(qr, 1, 1, 128, None, None, None, None, None) == -1               # not a QUANT cache
    # workspace sizes: 0 for shapes no call accepts, a positive size otherwise
    dw, vw = lib.vc_draft_ws_bytes, lib.vc_verify_ws_bytes
    dw.restype = vw.restype = ctypes.c_size_t
    assert dw(8, 32, 8, 128, 32768) >= 256 and dw(0, 32, 8, 128, 32768) == 0 and dw(8, 32, 8, 128, -1) == 0
    assert vw(8, 32, 8, 128, 33, 32768) >= 256 and vw(8, 30, 8, 128, 33, 32768) == 0
    assert vw(8, 32, 8, 128, 0, 32768) == 0


def test_no_oracle_in_product_path():
    """The product package never imports the oracle, and the oracle never imports the product."""
    pkg = os.path.join(ROOT, "compressed_kv_draft_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"\boracle\b", txt.replace("no CPU fallback", "")) or fn.endswith(".md"), fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith(".py"):
            assert "compressed_kv_draft_amd" not in open(os.path.join(ROOT, "oracle", fn)).read(), fn
