"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function include/*.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import tree_verify_mla_02_amd as kdt
from tree_verify_mla_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names.update(re.findall(r"\b(kdt_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for need in ("kdt_build_visibility", "kdt_tree_verify_attn", "kdt_tree_verify_workspace_size"):
        assert need in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = kdt.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.kdt_version() == 1


def test_status_strings():
    lib = kdt.load()
    assert lib.kdt_status_string(0) == b"KDT_OK"
    assert lib.kdt_status_string(2) == b"KDT_ERR_UNSUPPORTED"
    assert lib.kdt_status_string(99) == b"KDT_ERR_UNKNOWN"


def test_visibility_rejects_bad_arguments_on_host():
    lib = kdt.load()
    assert lib.kdt_build_visibility(None, 1, 4, None, None, None) == _lib.KDT_ERR_INVALID_ARG
    assert b"NULL" in lib.kdt_last_error()
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: the call fails before any launch
    assert lib.kdt_build_visibility(fake, 1, 257, fake, None, None) == _lib.KDT_ERR_UNSUPPORTED
    assert lib.kdt_build_visibility(fake, 1, 0, fake, None, None) == _lib.KDT_ERR_UNSUPPORTED
    assert lib.kdt_build_visibility(fake, 0, 4, fake, None, None) == _lib.KDT_ERR_INVALID_ARG
    assert lib.kdt_build_visibility(ctypes.c_void_p((1 << 20) + 2), 1, 4, fake, None, None) == _lib.KDT_ERR_MISALIGNED


def test_prepare_rejects_bad_arguments_on_host():
    lib = kdt.load()
    d = _lib.VerifyDesc(batch=1, num_nodes=8, num_heads=4, d_latent=512, d_rope=64, dtype=_lib.KDT_BF16,
                        max_cache_len=16, total_cache_len=16, q_lat_stride=512, q_rope_stride=64, ckv_stride=576,
                        krope_stride=576, tree_ckv_stride=576, tree_krope_stride=576)
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every call fails before any launch
    assert lib.kdt_tree_verify_prepare(None, fake, fake, ctypes.byref(d), fake, 1 << 20, None, None) == \
        _lib.KDT_ERR_INVALID_ARG
    assert lib.kdt_tree_verify_prepare(fake, fake, None, ctypes.byref(d), fake, 1 << 20, None, None) == \
        _lib.KDT_ERR_INVALID_ARG
    assert lib.kdt_tree_verify_prepare(ctypes.c_void_p((1 << 20) + 2), fake, fake, ctypes.byref(d), fake, 1 << 20,
                                       None, None) == _lib.KDT_ERR_MISALIGNED
    assert lib.kdt_tree_verify_prepare(fake, ctypes.c_void_p((1 << 20) + 4), fake, ctypes.byref(d), fake, 1 << 20,
                                       None, None) == _lib.KDT_ERR_MISALIGNED
    d.num_nodes = 300
    assert lib.kdt_tree_verify_prepare(fake, fake, fake, ctypes.byref(d), fake, 1 << 20, None, None) == \
        _lib.KDT_ERR_UNSUPPORTED


@pytest.mark.parametrize("field,value,code", [
    ("num_nodes", 0, _lib.KDT_ERR_UNSUPPORTED), ("num_nodes", 300, _lib.KDT_ERR_UNSUPPORTED),
    ("batch", 0, _lib.KDT_ERR_INVALID_ARG), ("num_heads", 0, _lib.KDT_ERR_INVALID_ARG),
    ("d_latent", 256, _lib.KDT_ERR_UNSUPPORTED), ("dtype", 7, _lib.KDT_ERR_UNSUPPORTED),
    ("ckv_stride", 500, _lib.KDT_ERR_INVALID_ARG), ("ckv_stride", 570, _lib.KDT_ERR_MISALIGNED), ("q_lat_stride", 516, _lib.KDT_ERR_MISALIGNED),
    ("max_cache_len", -1, _lib.KDT_ERR_INVALID_ARG),
    # the plan's 32-bit split counts take lengths up to 2^30 keys; beyond int32 the length is invalid
    ("max_cache_len", (1 << 30) + 1, _lib.KDT_ERR_UNSUPPORTED), ("max_cache_len", 1 << 31, _lib.KDT_ERR_INVALID_ARG),
])
def test_desc_validation_on_host(field, value, code):
    d = _lib.VerifyDesc(batch=1, num_nodes=8, num_heads=4, d_latent=512, d_rope=64, dtype=_lib.KDT_BF16,
                        max_cache_len=16, total_cache_len=16, q_lat_stride=512, q_rope_stride=64, ckv_stride=576,
                        krope_stride=576, tree_ckv_stride=576, tree_krope_stride=576)
    setattr(d, field, value)
    lib = kdt.load()
    assert lib.kdt_tree_verify_num_splits(ctypes.byref(d)) == -1
    assert lib.kdt_tree_verify_workspace_size(ctypes.byref(d)) == 0
    assert lib.kdt_last_status() == code
    assert lib.kdt_tree_verify_attn(*([None] * 8), ctypes.c_float(1.0), None, ctypes.byref(d), None, 0, None,
                                    None) == code


def test_tree_accept_rejects_bad_arguments_on_host():
    lib = kdt.load()
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every call fails before any launch
    args = [fake] * 4 + [1, 8] + [fake] * 3 + [None]   # valid as given (never launched here)
    bad = list(args)
    bad[1] = None
    assert lib.kdt_tree_accept(*bad) == _lib.KDT_ERR_INVALID_ARG
    bad = list(args)
    bad[5] = 257
    assert lib.kdt_tree_accept(*bad) == _lib.KDT_ERR_UNSUPPORTED
    bad = list(args)
    bad[4] = 0
    assert lib.kdt_tree_accept(*bad) == _lib.KDT_ERR_INVALID_ARG
    bad = list(args)
    bad[6] = ctypes.c_void_p((1 << 20) + 2)
    assert lib.kdt_tree_accept(*bad) == _lib.KDT_ERR_MISALIGNED


def test_kv_compact_rejects_bad_arguments_on_host():
    lib = kdt.load()
    d = _lib.VerifyDesc(batch=2, num_nodes=8, num_heads=4, d_latent=512, d_rope=64, dtype=_lib.KDT_BF16,
                        max_cache_len=16, total_cache_len=32, q_lat_stride=512, q_rope_stride=64, ckv_stride=576,
                        krope_stride=576, tree_ckv_stride=576, tree_krope_stride=576)
    a, b2 = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)   # never dereferenced

    def call(ckv=a, krope=a, lens=a, tc=a, tr=a, path=a, acc=a, oc=b2, orope=b2, nl=a, cap=64, desc=d):
        return lib.kdt_kv_compact(ckv, krope, lens, tc, tr, path, acc, oc, orope, nl, cap, ctypes.byref(desc),
                                  None, None)
    assert call(lens=None) == _lib.KDT_ERR_INVALID_ARG
    assert call(nl=None) == _lib.KDT_ERR_INVALID_ARG
    assert call(cap=-1) == _lib.KDT_ERR_INVALID_ARG
    assert call(tc=ctypes.c_void_p((1 << 20) + 8)) == _lib.KDT_ERR_MISALIGNED
    assert call(acc=ctypes.c_void_p((1 << 20) + 2)) == _lib.KDT_ERR_MISALIGNED
    assert call(oc=a, orope=b2) == _lib.KDT_ERR_INVALID_ARG          # in place for one part only
    assert call(oc=a, orope=a) == _lib.KDT_ERR_INVALID_ARG           # in place with batch 2
    assert b"batch 1" in lib.kdt_last_error()
    d.num_nodes = 300
    assert call() == _lib.KDT_ERR_UNSUPPORTED


def test_build_tree_rejects_bad_arguments_on_host():
    lib = kdt.load()
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every call fails before any launch

    def call(lp=fake, cand=fake, B=1, D=8, K=8, N=64, par=fake, tok=None, dep=None, rk=None):
        return lib.kdt_build_tree(lp, cand, B, D, K, N, par, tok, dep, rk, None)
    assert call(lp=None) == _lib.KDT_ERR_INVALID_ARG
    assert call(par=None) == _lib.KDT_ERR_INVALID_ARG
    assert call(B=0) == _lib.KDT_ERR_INVALID_ARG
    assert call(D=0) == _lib.KDT_ERR_INVALID_ARG
    assert call(K=0) == _lib.KDT_ERR_INVALID_ARG
    assert call(D=2, K=4097) == _lib.KDT_ERR_UNSUPPORTED
    assert call(N=0) == _lib.KDT_ERR_UNSUPPORTED
    assert call(N=257) == _lib.KDT_ERR_UNSUPPORTED
    assert call(tok=ctypes.c_void_p((1 << 20) + 2)) == _lib.KDT_ERR_MISALIGNED


def test_noalloc_rejects_bad_desc_on_host():
    """The allocation-free entry point validates the batch before it looks at its scratch array."""
    lib = kdt.load()
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced
    f = lib.kdt_tree_verify_attn_noalloc
    f.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
    assert f(*([fake] * 8), ctypes.c_float(1.0), fake, None, None, None) == _lib.KDT_ERR_INVALID_ARG
    assert b"desc" in lib.kdt_last_error()
