"""ctypes binding of libsa.so: argument marshalling only.

Every function has the name of the C entry point it calls and the same arguments.
Buffers may be torch tensors on the GPU (their data pointer is passed; their size,
dtype and contiguity are checked here, since the C side only sees pointers) or raw
integer device addresses (passed unchecked). A nonzero status raises :class:`SaError`.
The library is required: importing this module without a built ``libsa.so`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_LIBRARY names another build of the same library (e.g. one whose host code carries
# address and undefined-behaviour sanitizers); by default the in-tree libsa.so
LIB_PATH = os.environ.get("SA_LIBRARY") or os.path.join(_HERE, "libsa.so")

SA_OK = 0
SA_ERR_NULL = -1
SA_ERR_SHAPE = -2
SA_ERR_CSR = -3
SA_ERR_DTYPE = -4
SA_ERR_UNSUPPORTED = -5
SA_ERR_ALIGN = -6
SA_ERR_HIP = -7
SA_ERR_WORKSPACE = -8

SA_F32 = 0
SA_BF16 = 1
SA_FLAG_VALIDATE = 1

EXPORTS = ("sa_plan_bytes", "sa_plan_bytes_segments", "sa_plan_build", "sa_sddmm", "sa_sparse_softmax", "sa_spmm",
           "sa_fused_forward", "sa_fused_backward", "sa_fused_backward_noalloc",
           "sa_transpose_workspace_bytes", "sa_csr_transpose",
           "sa_gather_entries", "sa_gather_order_build", "sa_gather_entries_ordered",
           "sa_sparse_softmax_backward", "sa_bias_grad", "sa_mask_workspace_bytes", "sa_coo_to_csr",
           "sa_key_mask_from_lengths", "sa_varlen_row_ptr", "sa_varlen_col_idx", "sa_topk_mask",
           "sa_block_cover_row_ptr", "sa_block_cover_col_idx", "sa_block_cover_bits",
           "sa_fused_backward_cover", "sa_validate_csr",
           "sa_status_string", "sa_last_hip_error_string")


class sa_problem(ctypes.Structure):
    """Mirror of ``struct sa_problem`` in include/sa.h (field order and sizes are ABI)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("n", ctypes.c_int32), ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("block", ctypes.c_int32),
        ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
        ("nnz", ctypes.c_int64),
        ("scale", ctypes.c_float), ("key_mask_heads", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("key_mask", ctypes.c_void_p), ("plan", ctypes.c_void_p),
        ("seqlen_k", ctypes.c_void_p),
        ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class sa_block_cover(ctypes.Structure):
    """Mirror of ``struct sa_block_cover`` in include/sa.h."""
    _fields_ = [
        ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
        ("t_row_ptr", ctypes.c_void_p), ("t_col_idx", ctypes.c_void_p),
        ("bits", ctypes.c_void_p), ("bits_t", ctypes.c_void_p), ("nnz", ctypes.c_int64),
    ]


def _load():
    # torch provides the device memory and streams, so the library must run on torch's HIP
    # runtime: importing torch first maps its libamdhip64 (SONAME libamdhip64.so.7), which
    # the loader then reuses for libsa.so's dependency instead of mapping a second runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python masked_scaled_dot_amd/build.py` "
            "(hipcc for gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(sa_problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    sig = {
        "sa_plan_bytes": (sz, [P]),
        "sa_plan_bytes_segments": (sz, [P, i64]),
        "sa_plan_build": (ctypes.c_int, [P, vp, sz, vp]),
        "sa_sddmm": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "sa_sparse_softmax": (ctypes.c_int, [P, vp, vp, vp]),
        "sa_spmm": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "sa_fused_forward": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp]),
        "sa_fused_backward": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "sa_fused_backward_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "sa_transpose_workspace_bytes": (sz, [P]),
        "sa_csr_transpose": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
        "sa_gather_entries": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "sa_gather_order_build": (ctypes.c_int, [P, vp, vp, vp, sz, vp]),
        "sa_mask_workspace_bytes": (sz, [i32, i64]),
        "sa_coo_to_csr": (ctypes.c_int, [i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sa_key_mask_from_lengths": (ctypes.c_int, [i32, i32, vp, vp, vp]),
        "sa_varlen_row_ptr": (ctypes.c_int, [i32, i32, vp, i32, vp, vp, sz, vp]),
        "sa_varlen_col_idx": (ctypes.c_int, [i32, i32, vp, i32, vp, vp, i64, vp]),
        "sa_topk_mask": (ctypes.c_int, [i32, i32, vp, vp, vp, vp]),
        "sa_gather_entries_ordered": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp]),
        "sa_sparse_softmax_backward": (ctypes.c_int, [P, vp, vp, ctypes.c_float, vp, vp]),
        "sa_bias_grad": (ctypes.c_int, [P, vp, ctypes.c_float, vp, vp]),
        "sa_validate_csr": (ctypes.c_int, [P, vp]),
        "sa_block_cover_row_ptr": (ctypes.c_int, [P, vp, vp]),
        "sa_block_cover_col_idx": (ctypes.c_int, [P, vp, i64, vp, vp]),
        "sa_block_cover_bits": (ctypes.c_int, [P, ctypes.POINTER(sa_block_cover), vp]),
        "sa_fused_backward_cover": (ctypes.c_int, [P, ctypes.POINTER(sa_block_cover), vp, vp, vp, vp, vp,
                                                   vp, vp, vp, vp, vp, vp, vp]),
        "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "sa_last_hip_error_string": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


class SaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = f" [{_lib.sa_last_hip_error_string().decode()}]" if status == SA_ERR_HIP else ""
        super().__init__(f"{where}: {sa_status_string(status)} ({status}){detail}")


def sa_status_string(status: int) -> str:
    return _lib.sa_status_string(int(status)).decode()


# ------------------------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _is_tensor(x) -> bool:
    return type(x).__module__.startswith("torch") and hasattr(x, "data_ptr")


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if _is_tensor(x):
        return x.data_ptr() or None
    return int(x) or None


def _check(x, what: str, numel: int, dtype=None):
    """Size / dtype / layout checks for torch tensors (raw addresses are trusted)."""
    if x is None or not _is_tensor(x):
        return
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if x.numel() < numel:
        raise ValueError(f"{what} has {x.numel()} elements, needs {numel}")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{what} has dtype {x.dtype}, needs {dtype}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        torch = _torch()
        if torch.cuda.is_available() and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream or None
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream or None
    return int(stream) or None


class Problem:
    """Holds an ``sa_problem`` plus references to the tensors it points into."""

    def __init__(self, B, H, n, d, dtype=SA_BF16, row_ptr=None, col_idx=None, nnz=None, block=1,
                 scale=1.0, bias=None, key_mask=None, key_mask_heads=1, plan=None, flags=0,
                 seqlen_k=None):
        self._keep = (row_ptr, col_idx, bias, key_mask, plan)
        self._seqlen_k = seqlen_k
        if nnz is None:
            nnz = 0 if col_idx is None else (col_idx.numel() if _is_tensor(col_idx) else 0)
        self.c = sa_problem(B=B, H=H, n=n, d=d, dtype=dtype, block=block,
                            row_ptr=_ptr(row_ptr), col_idx=_ptr(col_idx), nnz=nnz,
                            scale=scale, key_mask_heads=key_mask_heads,
                            bias=_ptr(bias), key_mask=_ptr(key_mask), plan=_ptr(plan),
                            seqlen_k=_ptr(seqlen_k), flags=flags, reserved=0)
        torch = _torch()
        if row_ptr is not None:
            rows = n if block == 1 else (n + block - 1) // block
            _check(row_ptr, "row_ptr", rows + 1, torch.int32)
            _check(col_idx, "col_idx", nnz, torch.int32)
        _check(bias, "bias", H * n * n, torch.float32)
        _check(key_mask, "key_mask", B * key_mask_heads * n, torch.float32)
        _check(seqlen_k, "seqlen_k", B, torch.int32)

    # convenience sizes
    @property
    def BH(self):
        return self.c.B * self.c.H

    def qkv_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.c.dtype == SA_BF16 else torch.float32

    def set_plan(self, plan):
        self._keep = self._keep[:4] + (plan,)
        self.c.plan = _ptr(plan)


def _p(prob):
    return ctypes.byref(prob.c if isinstance(prob, Problem) else prob)


def _c(prob) -> sa_problem:
    return prob.c if isinstance(prob, Problem) else prob


def _raise(st, where):
    if st != SA_OK:
        raise SaError(st, where)


def sa_plan_bytes(prob) -> int:
    return int(_lib.sa_plan_bytes(_p(prob)))


def sa_plan_bytes_segments(prob, max_segments: int) -> int:
    return int(_lib.sa_plan_bytes_segments(_p(prob), int(max_segments)))


def sa_plan_build(prob, plan, plan_bytes: Optional[int] = None, stream=None):
    if plan_bytes is None:
        plan_bytes = plan.numel() * plan.element_size() if _is_tensor(plan) else sa_plan_bytes(prob)
    _raise(_lib.sa_plan_build(_p(prob), _ptr(plan), plan_bytes, _stream(stream)), "sa_plan_build")


def sa_sddmm(prob, q, k, scores, stream=None):
    c = _c(prob)
    qkv = _dtype_of(c)
    _check(q, "q", c.B * c.H * c.n * c.d, qkv)
    _check(k, "k", c.B * c.H * c.n * c.d, qkv)
    _check(scores, "scores", c.B * c.H * c.nnz, _torch().float32)
    _raise(_lib.sa_sddmm(_p(prob), _ptr(q), _ptr(k), _ptr(scores), _stream(stream)), "sa_sddmm")


def sa_sparse_softmax(prob, scores, weights, stream=None):
    c = _c(prob)
    f32 = _torch().float32
    _check(scores, "scores", c.B * c.H * c.nnz, f32)
    _check(weights, "weights", c.B * c.H * c.nnz, f32)
    _raise(_lib.sa_sparse_softmax(_p(prob), _ptr(scores), _ptr(weights), _stream(stream)),
           "sa_sparse_softmax")


def sa_spmm(prob, weights, v, out, stream=None):
    c = _c(prob)
    f32 = _torch().float32
    _check(weights, "weights", c.B * c.H * c.nnz, f32)
    _check(v, "v", c.B * c.H * c.n * c.d, _dtype_of(c))
    _check(out, "out", c.B * c.H * c.n * c.d, f32)
    _raise(_lib.sa_spmm(_p(prob), _ptr(weights), _ptr(v), _ptr(out), _stream(stream)), "sa_spmm")


def sa_fused_forward(prob, q, k, v, out, lse=None, stream=None):
    c = _c(prob)
    qkv, f32 = _dtype_of(c), _torch().float32
    for x, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(x, name, c.B * c.H * c.n * c.d, qkv)
    _check(out, "out", c.B * c.H * c.n * c.d, f32)
    _check(lse, "lse", c.B * c.H * c.n, f32)
    _raise(_lib.sa_fused_forward(_p(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _stream(stream)), "sa_fused_forward")


def sa_fused_backward(prob, q, k, v, out, lse, dout, dq, dk, dv, workspace, dscores=None,
                      t_row_ptr=None, t_col_idx=None, stream=None):
    c = _c(prob)
    qkv, f32 = _dtype_of(c), _torch().float32
    N = c.B * c.H * c.n * c.d
    for x, name in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(x, name, N, qkv)
    for x, name in ((out, "out"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(x, name, N, f32)
    _check(lse, "lse", c.B * c.H * c.n, f32)
    _check(workspace, "workspace", c.B * c.H * c.n, f32)
    _check(dscores, "dscores", c.B * c.H * c.n * c.n, f32)
    if c.row_ptr:
        nb = (c.n + 63) // 64
        _check(t_row_ptr, "t_row_ptr", nb + 1, _torch().int32)
        _check(t_col_idx, "t_col_idx", c.nnz, _torch().int32)
    _raise(_lib.sa_fused_backward(_p(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                  _ptr(dout), _ptr(t_row_ptr), _ptr(t_col_idx), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(dscores), _ptr(workspace), _stream(stream)),
           "sa_fused_backward")


def sa_fused_backward_noalloc(prob, q, k, v, out, lse, dout, dq, dk, dv, dscores=None,
                              t_row_ptr=None, t_col_idx=None, stream=None):
    """sa_fused_backward with the library's fixed device scratch instead of a workspace."""
    c = _c(prob)
    qkv, f32 = _dtype_of(c), _torch().float32
    N = c.B * c.H * c.n * c.d
    for x, name in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(x, name, N, qkv)
    for x, name in ((out, "out"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(x, name, N, f32)
    _check(lse, "lse", c.B * c.H * c.n, f32)
    _check(dscores, "dscores", c.B * c.H * c.n * c.n, f32)
    if c.row_ptr:
        nb = (c.n + 63) // 64
        _check(t_row_ptr, "t_row_ptr", nb + 1, _torch().int32)
        _check(t_col_idx, "t_col_idx", c.nnz, _torch().int32)
    _raise(_lib.sa_fused_backward_noalloc(_p(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                          _ptr(dout), _ptr(t_row_ptr), _ptr(t_col_idx), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(dscores), _stream(stream)),
           "sa_fused_backward_noalloc")


def sa_transpose_workspace_bytes(prob) -> int:
    return int(_lib.sa_transpose_workspace_bytes(_p(prob)))


def sa_csr_transpose(prob, row_ptr_t, col_idx_t, perm, workspace, stream=None):
    c = _c(prob)
    i32 = _torch().int32
    _check(row_ptr_t, "row_ptr_t", c.n + 1, i32)
    _check(col_idx_t, "col_idx_t", c.nnz, i32)
    _check(perm, "perm", c.nnz, i32)
    nbytes = workspace.numel() * workspace.element_size() if _is_tensor(workspace) else 0
    _raise(_lib.sa_csr_transpose(_p(prob), _ptr(row_ptr_t), _ptr(col_idx_t), _ptr(perm),
                                 _ptr(workspace), nbytes, _stream(stream)), "sa_csr_transpose")


def sa_gather_entries(prob, perm, src, dst, stream=None):
    c = _c(prob)
    f32 = _torch().float32
    _check(perm, "perm", c.nnz, _torch().int32)
    _check(src, "src", c.B * c.H * c.nnz, f32)
    _check(dst, "dst", c.B * c.H * c.nnz, f32)
    _raise(_lib.sa_gather_entries(_p(prob), _ptr(perm), _ptr(src), _ptr(dst), _stream(stream)),
           "sa_gather_entries")


def sa_gather_order_build(prob, perm, order, workspace, stream=None):
    c = _c(prob)
    i32 = _torch().int32
    _check(perm, "perm", c.nnz, i32)
    _check(order, "order", 2 * c.nnz, i32)
    nbytes = workspace.numel() * workspace.element_size() if _is_tensor(workspace) else 0
    _raise(_lib.sa_gather_order_build(_p(prob), _ptr(perm), _ptr(order), _ptr(workspace), nbytes,
                                      _stream(stream)), "sa_gather_order_build")


def sa_gather_entries_ordered(prob, order, src_a, dst_a, src_b=None, dst_b=None, stream=None):
    c = _c(prob)
    f32 = _torch().float32
    _check(order, "order", 2 * c.nnz, _torch().int32)
    for x, name in ((src_a, "src_a"), (dst_a, "dst_a"), (src_b, "src_b"), (dst_b, "dst_b")):
        _check(x, name, c.B * c.H * c.nnz, f32)
    _raise(_lib.sa_gather_entries_ordered(_p(prob), _ptr(order), _ptr(src_a), _ptr(dst_a),
                                          _ptr(src_b), _ptr(dst_b), _stream(stream)),
           "sa_gather_entries_ordered")


def sa_sparse_softmax_backward(prob, weights, dweights, out_scale, dscores, stream=None):
    c = _c(prob)
    f32 = _torch().float32
    for x, name in ((weights, "weights"), (dweights, "dweights"), (dscores, "dscores")):
        _check(x, name, c.B * c.H * c.nnz, f32)
    _raise(_lib.sa_sparse_softmax_backward(_p(prob), _ptr(weights), _ptr(dweights),
                                           float(out_scale), _ptr(dscores), _stream(stream)),
           "sa_sparse_softmax_backward")


def sa_mask_workspace_bytes(n, nnz) -> int:
    return int(_lib.sa_mask_workspace_bytes(int(n), int(nnz)))


def _nbytes(x):
    return x.numel() * x.element_size() if _is_tensor(x) else 0


def sa_coo_to_csr(n, rows, cols, row_ptr, col_idx, counts, workspace, stream=None):
    """CSR of the set of (rows[k], cols[k]) pairs inside [0, n); counts gets {stored,
    dropped out of range, merged repeats}."""
    i32 = _torch().int32
    nnz = rows.numel() if _is_tensor(rows) else 0
    _check(rows, "rows", nnz, i32)
    _check(cols, "cols", nnz, i32)
    _check(row_ptr, "row_ptr", n + 1, i32)
    _check(col_idx, "col_idx", nnz, i32)
    _check(counts, "counts", 3, i32)
    _raise(_lib.sa_coo_to_csr(int(n), int(nnz), _ptr(rows), _ptr(cols), _ptr(row_ptr), _ptr(col_idx),
                              _ptr(counts), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "sa_coo_to_csr")


def sa_key_mask_from_lengths(B, n, seqlen_k, key_mask, stream=None):
    _check(seqlen_k, "seqlen_k", B, _torch().int32)
    _check(key_mask, "key_mask", B * n, _torch().float32)
    _raise(_lib.sa_key_mask_from_lengths(int(B), int(n), _ptr(seqlen_k), _ptr(key_mask),
                                         _stream(stream)), "sa_key_mask_from_lengths")


def sa_varlen_row_ptr(B, total, cu_seqlens, window, row_ptr, workspace, stream=None):
    i32 = _torch().int32
    _check(cu_seqlens, "cu_seqlens", B + 1, i32)
    _check(row_ptr, "row_ptr", total + 1, i32)
    _raise(_lib.sa_varlen_row_ptr(int(B), int(total), _ptr(cu_seqlens), int(window), _ptr(row_ptr),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "sa_varlen_row_ptr")


def sa_varlen_col_idx(B, total, cu_seqlens, window, row_ptr, col_idx, stream=None):
    i32 = _torch().int32
    _check(cu_seqlens, "cu_seqlens", B + 1, i32)
    _check(row_ptr, "row_ptr", total + 1, i32)
    _check(col_idx, "col_idx", 0, i32)
    cap = col_idx.numel() if _is_tensor(col_idx) else 0
    _raise(_lib.sa_varlen_col_idx(int(B), int(total), _ptr(cu_seqlens), int(window), _ptr(row_ptr),
                                  _ptr(col_idx), int(cap), _stream(stream)), "sa_varlen_col_idx")


def sa_bias_grad(prob, dscores, factor, dbias, stream=None):
    c = _c(prob)
    f32 = _torch().float32
    per_head = c.nnz if c.row_ptr else c.n * c.n  # the dense pattern: [B*H, n, n]
    _check(dscores, "dscores", c.B * c.H * per_head, f32)
    _check(dbias, "dbias", c.H * c.n * c.n, f32)
    _raise(_lib.sa_bias_grad(_p(prob), _ptr(dscores), float(factor), _ptr(dbias), _stream(stream)),
           "sa_bias_grad")


def sa_topk_mask(n, k, scores, row_ptr, col_idx, stream=None):
    """Each row keeps the k columns of largest score (ascending in col_idx)."""
    torch = _torch()
    kk = max(0, min(int(k), int(n)))
    _check(scores, "scores", n * n, torch.float32)
    _check(row_ptr, "row_ptr", n + 1, torch.int32)
    _check(col_idx, "col_idx", n * kk, torch.int32)
    _raise(_lib.sa_topk_mask(int(n), int(k), _ptr(scores), _ptr(row_ptr), _ptr(col_idx),
                             _stream(stream)), "sa_topk_mask")


def sa_validate_csr(prob, stream=None) -> int:
    """Returns the status (SA_OK or SA_ERR_CSR); raises on argument errors."""
    st = _lib.sa_validate_csr(_p(prob), _stream(stream))
    if st not in (SA_OK, SA_ERR_CSR):
        _raise(st, "sa_validate_csr")
    return st


def sa_block_cover_row_ptr(prob, cover_row_ptr, stream=None):
    c = _c(prob)
    _check(cover_row_ptr, "cover_row_ptr", (c.n + 63) // 64 + 1, _torch().int32)
    _raise(_lib.sa_block_cover_row_ptr(_p(prob), _ptr(cover_row_ptr), _stream(stream)),
           "sa_block_cover_row_ptr")


def sa_block_cover_col_idx(prob, cover_row_ptr, cover_nnz, cover_col_idx, stream=None):
    c = _c(prob)
    _check(cover_row_ptr, "cover_row_ptr", (c.n + 63) // 64 + 1, _torch().int32)
    _check(cover_col_idx, "cover_col_idx", int(cover_nnz), _torch().int32)
    _raise(_lib.sa_block_cover_col_idx(_p(prob), _ptr(cover_row_ptr), int(cover_nnz), _ptr(cover_col_idx),
                                       _stream(stream)), "sa_block_cover_col_idx")


class BlockCover:
    """The arrays of a block cover (device tensors, owned here) and their C struct."""

    def __init__(self, row_ptr, col_idx, t_row_ptr, t_col_idx, bits, bits_t, nnz):
        self.row_ptr, self.col_idx, self.t_row_ptr, self.t_col_idx = row_ptr, col_idx, t_row_ptr, t_col_idx
        self.bits, self.bits_t, self.nnz = bits, bits_t, int(nnz)
        self.c = sa_block_cover(_ptr(row_ptr), _ptr(col_idx), _ptr(t_row_ptr), _ptr(t_col_idx),
                                _ptr(bits), _ptr(bits_t), self.nnz)


def sa_block_cover_bits(prob, cover, stream=None):
    n = cover.nnz * 64
    _check(cover.bits, "bits", n, _torch().int64)
    _check(cover.bits_t, "bits_t", n, _torch().int64)
    _raise(_lib.sa_block_cover_bits(_p(prob), ctypes.byref(cover.c), _stream(stream)), "sa_block_cover_bits")


def block_cover(prob, device="cuda", stream=None) -> BlockCover:
    """Runs the four once-per-mask steps of the block cover in order (sa_block_cover_row_ptr,
    sa_block_cover_col_idx, sa_csr_transpose over the cover, sa_block_cover_bits) on `stream`
    (torch's current stream when None); reads the cover's size back to the host in between,
    after synchronising that stream. The arrays are allocated while that stream is current,
    so torch's allocator orders their reuse after the work queued on it."""
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    if not hasattr(s, "cuda_stream"):
        s = torch.cuda.ExternalStream(int(s))
    with torch.cuda.stream(s):
        c = _c(prob)
        nb = (c.n + 63) // 64
        rp = torch.zeros(nb + 1, dtype=torch.int32, device=device)
        sa_block_cover_row_ptr(prob, rp, s)
        s.synchronize()
        nnz = int(rp[nb].item()) if nb else 0
        ci = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
        sa_block_cover_col_idx(prob, rp, nnz, ci, s)
        grid = Problem(1, 1, nb, 32, SA_F32, rp, ci[:nnz], nnz)
        trp = torch.zeros(nb + 1, dtype=torch.int32, device=device)
        tci = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
        perm = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
        ws = torch.empty(max(sa_transpose_workspace_bytes(grid), 1), dtype=torch.uint8, device=device)
        sa_csr_transpose(grid, trp, tci[:nnz], perm[:nnz], ws, stream=s)
        bits = torch.empty(max(nnz, 1) * 64, dtype=torch.int64, device=device)
        bits_t = torch.empty_like(bits)
        cover = BlockCover(rp, ci, trp, tci, bits, bits_t, nnz)
        sa_block_cover_bits(prob, cover, s)
    return cover


def sa_fused_backward_cover(prob, cover, q, k, v, out, lse, dout, dq, dk, dv, workspace, dscores=None,
                            stream=None):
    c = _c(prob)
    qkv, f32 = _dtype_of(c), _torch().float32
    N = c.B * c.H * c.n * c.d
    for x, name in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(x, name, N, qkv)
    for x, name in ((out, "out"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(x, name, N, f32)
    _check(lse, "lse", c.B * c.H * c.n, f32)
    _check(workspace, "workspace", c.B * c.H * c.n, f32)
    _check(dscores, "dscores", c.B * c.H * c.n * c.n, f32)
    _raise(_lib.sa_fused_backward_cover(_p(prob), ctypes.byref(cover.c), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dscores),
                                        _ptr(workspace), _stream(stream)), "sa_fused_backward_cover")


def _dtype_of(c: sa_problem):
    torch = _torch()
    return torch.bfloat16 if c.dtype == SA_BF16 else torch.float32


def raw(name: str):
    """The raw ctypes function of an exported symbol (for ABI tests)."""
    return getattr(_lib, name)
