"""ctypes binding of libkdt (include/kdt.h).  Argument marshalling only.

Every computation runs in the HIP kernels of libkdt.so; torch only provides device memory
and the current stream.  When the library is missing the calls raise -- there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdt.so")

KDT_OK, KDT_ERR_INVALID_ARG, KDT_ERR_UNSUPPORTED, KDT_ERR_MISALIGNED, KDT_ERR_WORKSPACE, KDT_ERR_HIP = range(6)
KDT_DEV_BAD_PARENT, KDT_DEV_CACHE_LEN, KDT_DEV_BAD_ACCEPT = 1, 2, 4
KDT_BF16, KDT_F32 = 0, 1

EXPORTS = [
    "kdt_build_visibility", "kdt_tree_verify_workspace_size", "kdt_tree_verify_attn",
    "kdt_tree_verify_plan", "kdt_tree_verify_prepare", "kdt_tree_verify_attend", "kdt_tree_verify_combine",
    "kdt_tree_verify_num_splits", "kdt_status_string", "kdt_last_error", "kdt_last_status", "kdt_version",
    "kdt_tree_accept", "kdt_kv_compact", "kdt_build_tree", "kdt_tree_verify_attn_noalloc",
    "kdt_tree_verify_prepare_attend", "kdt_tree_verify_prepare_attend_launches",
]


class VerifyDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_nodes", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("max_cache_len", ctypes.c_int64), ("total_cache_len", ctypes.c_int64),
        ("q_lat_stride", ctypes.c_int64), ("q_rope_stride", ctypes.c_int64),
        ("ckv_stride", ctypes.c_int64), ("krope_stride", ctypes.c_int64),
        ("tree_ckv_stride", ctypes.c_int64), ("tree_krope_stride", ctypes.c_int64),
    ]


class KdtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_status_name(code)}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libkdt.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tree_verify_mla_02_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(VerifyDesc)
    lib.kdt_build_visibility.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.kdt_tree_verify_workspace_size.argtypes = [dp]
    lib.kdt_tree_verify_workspace_size.restype = sz
    lib.kdt_tree_verify_num_splits.argtypes = [dp]
    lib.kdt_tree_verify_attn.argtypes = [vp] * 8 + [ctypes.c_float, vp, dp, vp, sz, vp, vp]
    lib.kdt_tree_verify_plan.argtypes = [vp, dp, vp, sz, vp, vp]
    lib.kdt_tree_verify_prepare.argtypes = [vp, vp, vp, dp, vp, sz, vp, vp]
    lib.kdt_tree_verify_attend.argtypes = [vp] * 7 + [ctypes.c_float, vp, dp, vp, sz, vp]
    lib.kdt_tree_verify_combine.argtypes = [vp, dp, vp, sz, vp]
    lib.kdt_tree_verify_prepare_attend.argtypes = [vp] * 9 + [ctypes.c_float, vp, dp, vp, sz, vp, vp]
    lib.kdt_tree_verify_prepare_attend_launches.argtypes = [dp]
    lib.kdt_tree_accept.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.kdt_kv_compact.argtypes = [vp] * 10 + [i64, dp, vp, vp]
    lib.kdt_build_tree.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.kdt_status_string.restype = ctypes.c_char_p
    lib.kdt_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("kdt_tree_verify_workspace_size", "kdt_status_string", "kdt_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _status_name(code: int) -> str:
    try:
        return load().kdt_status_string(code).decode()
    except Exception:
        return f"status {code}"


def _check(code: int):
    if code != KDT_OK:
        raise KdtError(code, load().kdt_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _row_stride(t: torch.Tensor, name: str) -> int:
    """Elements between consecutive rows of a tensor whose last dim is contiguous."""
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    lead = t.shape[:-1]
    if len(lead) == 0 or t.numel() == 0:
        return t.shape[-1]
    # rows must be evenly spaced: every leading dim collapses into one row index
    stride = t.stride(-2) if t.dim() >= 2 else t.shape[-1]
    expect = stride
    for d in range(t.dim() - 2, -1, -1):
        if t.shape[d] > 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: rows are not evenly spaced (strides {t.stride()})")
        expect *= t.shape[d]
    return stride


def make_desc(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, max_cache_len: int,
              total_cache_len: Optional[int] = None) -> VerifyDesc:
    B, N, H, dc = q_lat.shape
    dr = q_rope.shape[-1]
    if q_lat.dtype == torch.bfloat16:
        dtype = KDT_BF16
    elif q_lat.dtype == torch.float32:
        dtype = KDT_F32
    else:
        raise ValueError(f"unsupported dtype {q_lat.dtype}")
    for t, n in ((q_rope, "q_rope"), (ckv, "ckv"), (krope, "krope"), (tree_ckv, "tree_ckv"), (tree_krope, "tree_krope")):
        if t.dtype != q_lat.dtype:
            raise ValueError(f"{n} has dtype {t.dtype}, expected {q_lat.dtype}")
    d = VerifyDesc()
    d.batch, d.num_nodes, d.num_heads, d.d_latent, d.d_rope, d.dtype = B, N, H, dc, dr, dtype
    d.max_cache_len = int(max_cache_len)
    d.total_cache_len = int(ckv.shape[0] if total_cache_len is None else total_cache_len)
    d.q_lat_stride = _row_stride(q_lat, "q_lat")
    d.q_rope_stride = _row_stride(q_rope, "q_rope")
    d.ckv_stride = _row_stride(ckv, "ckv")
    d.krope_stride = _row_stride(krope, "krope")
    d.tree_ckv_stride = _row_stride(tree_ckv, "tree_ckv")
    d.tree_krope_stride = _row_stride(tree_krope, "tree_krope")
    return d


def workspace_size(desc: VerifyDesc) -> int:
    n = load().kdt_tree_verify_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise KdtError(load().kdt_last_status(), load().kdt_last_error().decode())
    return n


def num_splits(desc: VerifyDesc) -> int:
    n = load().kdt_tree_verify_num_splits(ctypes.byref(desc))
    if n < 0:
        raise KdtError(load().kdt_last_status(), load().kdt_last_error().decode())
    return n


def alloc_workspace(desc: VerifyDesc, device=None) -> torch.Tensor:
    # torch's caching allocator hands out 512-byte aligned blocks
    return torch.empty(workspace_size(desc), dtype=torch.uint8, device=device or "cuda")


def build_visibility(parents: torch.Tensor, out: Optional[torch.Tensor] = None,
                     dev_status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """parents [B, N] int32 (device) -> ancestor bitmasks [B, N, ceil(N/64)] (int64 view of uint64)."""
    if parents.dtype != torch.int32 or not parents.is_contiguous() or parents.dim() != 2:
        raise ValueError("parents must be a contiguous [B, N] int32 tensor")
    B, N = parents.shape
    W = (N + 63) // 64
    if out is None:
        out = torch.empty((B, N, W), dtype=torch.int64, device=parents.device)
    _check(load().kdt_build_visibility(_ptr(parents), B, N, _ptr(out), _ptr(dev_status), _stream(stream)))
    return out


def tree_verify_attn(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, bitmask, cache_lens, scale: float, *,
                     max_cache_len: int, out=None, workspace=None, dev_status=None,
                     total_cache_len: Optional[int] = None, stream=None) -> torch.Tensor:
    """Tree-verify MLA-absorb attention; returns out [B, N, H, d_c] fp32.

    max_cache_len is a host-side upper bound on cache_lens (required: reading it back from the
    device would synchronise the host)."""
    desc = make_desc(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, max_cache_len, total_cache_len)
    B, N, H, dc = q_lat.shape
    if out is None:
        out = torch.empty((B, N, H, dc), dtype=torch.float32, device=q_lat.device)
    if workspace is None:
        workspace = alloc_workspace(desc, q_lat.device)
    _check(load().kdt_tree_verify_attn(
        _ptr(q_lat), _ptr(q_rope), _ptr(ckv), _ptr(krope), _ptr(tree_ckv), _ptr(tree_krope), _ptr(bitmask),
        _ptr(cache_lens), ctypes.c_float(scale), _ptr(out), ctypes.byref(desc), _ptr(workspace),
        workspace.numel(), _ptr(dev_status), _stream(stream)))
    return out


def plan(cache_lens, desc: VerifyDesc, workspace, dev_status=None, stream=None):
    _check(load().kdt_tree_verify_plan(_ptr(cache_lens), ctypes.byref(desc), _ptr(workspace), workspace.numel(),
                                       _ptr(dev_status), _stream(stream)))


def prepare(parents, cache_lens, desc: VerifyDesc, workspace, masks_out: Optional[torch.Tensor] = None,
            dev_status=None, stream=None) -> torch.Tensor:
    """Masks [B, N, ceil(N/64)] (int64 view of uint64) and the plan in `workspace`, one launch."""
    if parents.dtype != torch.int32 or not parents.is_contiguous() or parents.dim() != 2:
        raise ValueError("parents must be a contiguous [B, N] int32 tensor")
    B, N = parents.shape
    if masks_out is None:
        masks_out = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=parents.device)
    _check(load().kdt_tree_verify_prepare(_ptr(parents), _ptr(masks_out), _ptr(cache_lens), ctypes.byref(desc),
                                          _ptr(workspace), workspace.numel(), _ptr(dev_status), _stream(stream)))
    return masks_out


def attend(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, bitmask, scale, out, desc: VerifyDesc, workspace,
           stream=None):
    _check(load().kdt_tree_verify_attend(_ptr(q_lat), _ptr(q_rope), _ptr(ckv), _ptr(krope), _ptr(tree_ckv),
                                         _ptr(tree_krope), _ptr(bitmask), ctypes.c_float(scale), _ptr(out),
                                         ctypes.byref(desc), _ptr(workspace), workspace.numel(), _stream(stream)))


def combine(out, desc: VerifyDesc, workspace, stream=None):
    _check(load().kdt_tree_verify_combine(_ptr(out), ctypes.byref(desc), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))


def prepare_attend(parents, cache_lens, q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, scale, out,
                   desc: VerifyDesc, workspace, masks_out: Optional[torch.Tensor] = None, dev_status=None,
                   stream=None) -> torch.Tensor:
    """prepare + attend in one call (one launch for a one-request bf16 batch); combine
    follows as after attend.  Returns the masks [B, N, ceil(N/64)] (int64 view of uint64)."""
    if parents.dtype != torch.int32 or not parents.is_contiguous() or parents.dim() != 2:
        raise ValueError("parents must be a contiguous [B, N] int32 tensor")
    B, N = parents.shape
    if masks_out is None:
        masks_out = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=parents.device)
    _check(load().kdt_tree_verify_prepare_attend(
        _ptr(parents), _ptr(masks_out), _ptr(cache_lens), _ptr(q_lat), _ptr(q_rope), _ptr(ckv), _ptr(krope),
        _ptr(tree_ckv), _ptr(tree_krope), ctypes.c_float(scale), _ptr(out), ctypes.byref(desc), _ptr(workspace),
        workspace.numel(), _ptr(dev_status), _stream(stream)))
    return masks_out


def prepare_attend_launches(desc: VerifyDesc) -> int:
    """Kernel launches prepare_attend makes for `desc`: 1 or 2."""
    n = load().kdt_tree_verify_prepare_attend_launches(ctypes.byref(desc))
    if n < 0:
        raise KdtError(load().kdt_last_status(), load().kdt_last_error().decode())
    return n


def _int32_2d(t, name):
    if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 2:
        raise ValueError(f"{name} must be a contiguous [B, N] int32 tensor")


def tree_accept(parents, tokens, target_next, root_next, path=None, accept_len=None, bonus=None, stream=None):
    """Greedy acceptance: (path [B, N], accept_len [B], bonus [B]), int32 on the device."""
    for t, n in ((parents, "parents"), (tokens, "tokens"), (target_next, "target_next")):
        _int32_2d(t, n)
    B, N = parents.shape
    if tokens.shape != (B, N) or target_next.shape != (B, N):
        raise ValueError("parents, tokens and target_next must have the same [B, N] shape")
    if root_next.dtype != torch.int32 or root_next.shape != (B,) or not root_next.is_contiguous():
        raise ValueError("root_next must be a contiguous [B] int32 tensor")
    dev = parents.device
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
    _check(load().kdt_tree_accept(_ptr(parents), _ptr(tokens), _ptr(target_next), _ptr(root_next), B, N,
                                  _ptr(path), _ptr(accept_len), _ptr(bonus), _stream(stream)))
    return path, accept_len, bonus


def build_tree(logp, cand, num_nodes: int, parents=None, tokens=None, depth=None, rank=None, stream=None):
    """Best-first draft tree from per-depth top-K log probabilities.

    logp [B, D, K] float32 and cand [B, D, K] int32 on the device; returns (parents, tokens,
    depth, rank), each [B, num_nodes] int32 (-2 in rows a too small tree cannot fill)."""
    if logp.dtype != torch.float32 or logp.dim() != 3 or not logp.is_contiguous():
        raise ValueError("logp must be a contiguous [B, D, K] float32 tensor")
    if cand.dtype != torch.int32 or cand.shape != logp.shape or not cand.is_contiguous():
        raise ValueError("cand must be a contiguous int32 tensor shaped like logp")
    B, D, K = logp.shape
    outs = []
    for t in (parents, tokens, depth, rank):
        if t is None:
            t = torch.empty((B, num_nodes), dtype=torch.int32, device=logp.device)
        _int32_2d(t, "tree output")
        outs.append(t)
    _check(load().kdt_build_tree(_ptr(logp), _ptr(cand), B, D, K, int(num_nodes), *[_ptr(t) for t in outs],
                                 _stream(stream)))
    return tuple(outs)


def kv_compact(ckv, krope, cache_lens, tree_ckv, tree_krope, path, accept_len, desc: VerifyDesc, ckv_out,
               krope_out, new_lens=None, capacity_rows: Optional[int] = None, dev_status=None, stream=None):
    """Commit the accepted tree rows after each request's committed rows (into ckv_out /
    krope_out, same row strides as the source); returns new_lens [B] int32."""
    if new_lens is None:
        new_lens = torch.empty(desc.batch, dtype=torch.int32, device=cache_lens.device)
    if capacity_rows is None:
        es = ckv_out.element_size()
        capacity_rows = (ckv_out.untyped_storage().nbytes() - ckv_out.storage_offset() * es) // (desc.ckv_stride * es)
    _check(load().kdt_kv_compact(_ptr(ckv), _ptr(krope), _ptr(cache_lens), _ptr(tree_ckv), _ptr(tree_krope),
                                 _ptr(path), _ptr(accept_len), _ptr(ckv_out), _ptr(krope_out), _ptr(new_lens),
                                 int(capacity_rows), ctypes.byref(desc), _ptr(dev_status), _stream(stream)))
    return new_lens


# ---------------------------------------------------------------- allocation-free variant
def _load_noalloc():
    lib = load()
    f = lib.kdt_tree_verify_attn_noalloc
    if f.argtypes is None:
        f.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(VerifyDesc),
                                              ctypes.c_void_p, ctypes.c_void_p]
        f.restype = ctypes.c_int
    return f


def tree_verify_attn_noalloc(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, bitmask, cache_lens, scale: float, *,
                             max_cache_len: int, out, dev_status=None, total_cache_len: Optional[int] = None,
                             desc: Optional[VerifyDesc] = None, stream=None) -> torch.Tensor:
    """kdt_tree_verify_attn_noalloc (include/kdt_noalloc.h): the verify attention with the
    library's static per-device scratch array as its workspace.  `out` must be given (nothing is
    allocated); returns it."""
    if desc is None:
        desc = make_desc(q_lat, q_rope, ckv, krope, tree_ckv, tree_krope, max_cache_len, total_cache_len)
    _check(_load_noalloc()(
        _ptr(q_lat), _ptr(q_rope), _ptr(ckv), _ptr(krope), _ptr(tree_ckv), _ptr(tree_krope), _ptr(bitmask),
        _ptr(cache_lens), ctypes.c_float(scale), _ptr(out), ctypes.byref(desc), _ptr(dev_status), _stream(stream)))
    return out
