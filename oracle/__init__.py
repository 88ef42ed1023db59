"""fp64 CPU oracle for tree-verify MLA-absorb attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it, and it
shares no code with the HIP path: the arithmetic lives in ``kdt_oracle.c`` (plain C,
fp64, built with gcc) and in ``bruteforce.py`` (an independent numpy formulation).

Inputs are widened exactly to fp64 (bf16 -> fp64 and fp32 -> fp64 are exact) and the
scale is the fp32 value the GPU receives.  Each pinned property of these functions is
listed in the header of ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdt_oracle.c")
_LIB = os.path.join(_HERE, "libkdt_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, strict IEEE: no -ffast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.kdt_oracle_visibility.restype = ctypes.c_int64
        lib.kdt_oracle_visibility.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p]
        lib.kdt_oracle_attention.restype = None
        lib.kdt_oracle_attention.argtypes = ([ctypes.c_void_p] * 8 +
                                             [ctypes.c_int64] * 5 +
                                             [ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_int])
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def visibility(parents) -> "tuple[np.ndarray, int]":
    """Ancestor bitmasks [B, N, W] uint64 and the count of invalid rows."""
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    B, N = par.shape
    W = (N + 63) // 64
    masks = np.zeros((B, N, W), dtype=np.uint64)
    bad = _load().kdt_oracle_visibility(_ptr(par), B, N, _ptr(masks))
    return masks, int(bad)


def attention(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, masks, cache_lens, scale: float,
              rows: Optional[Sequence[int]] = None, threads: int = 0) -> np.ndarray:
    """Outputs [B, N, H, d_c] (rows=None) or [len(rows), d_c] for flat row ids (b*N+i)*H+h."""
    ql, qr = _f64(q_lat), _f64(q_rope)
    B, N, H, dc = ql.shape
    dr = qr.shape[-1]
    ck, kr = _f64(ckv).reshape(-1, dc), _f64(krope).reshape(-1, dr)
    tc, tr = _f64(tree_ckv).reshape(B * N, dc), _f64(tree_krope).reshape(B * N, dr)
    m = np.ascontiguousarray(np.asarray(masks, dtype=np.uint64))
    lens = np.ascontiguousarray(np.asarray(cache_lens, dtype=np.int32))
    assert m.shape[:2] == (B, N) and lens.shape == (B,)
    assert ck.shape[0] >= int(lens.astype(np.int64).sum())
    s = float(np.float32(scale))
    if rows is None:
        out = np.zeros((B, N, H, dc), dtype=np.float64)
        r_arr, nr = np.zeros(1, np.int64), -1
    else:
        r_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        assert r_arr.size == 0 or (r_arr.min() >= 0 and r_arr.max() < B * N * H)
        out = np.zeros((r_arr.size, dc), dtype=np.float64)
        nr = r_arr.size
        if nr == 0:
            return out
    _load().kdt_oracle_attention(_ptr(ql), _ptr(qr), _ptr(ck), _ptr(kr), _ptr(tc), _ptr(tr),
                                 _ptr(m), _ptr(lens), B, N, H, dc, dr, s, _ptr(r_arr), nr,
                                 _ptr(out), int(threads))
    return out


def run(inp, rows=None, threads: int = 0):
    """Masks and attention for a ``workloads.Inputs`` batch."""
    masks, bad = visibility(inp.parents.numpy())
    out = attention(inp.q_lat, inp.q_rope, inp.ckv, inp.krope, inp.tree_ckv, inp.tree_krope,
                    masks, inp.cache_lens.numpy(), inp.scale, rows=rows, threads=threads)
    return masks, out, bad
