"""C-ABI checks that need no GPU: the library loads, exports every entry point declared in
include/sa.h, the ctypes struct mirrors the C layout, and host-side argument checks
return their status codes before any device work (fake non-NULL pointers are never
dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


def _ensure_built():
    if not os.path.exists(os.path.join(ROOT, "masked_scaled_dot_amd", "libsa.so")):
        import __graft_entry__
        __graft_entry__._build_module().build()


_ensure_built()
import masked_scaled_dot_amd as sa  # noqa: E402
from masked_scaled_dot_amd import _lib  # noqa: E402

FAKE = 0x10000  # aligned, never dereferenced by the paths tested here


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    declared = _declared()
    assert set(declared) == set(sa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (sa_\w+)", out))
    assert set(declared) <= exported
    for name in declared:
        assert getattr(ctypes.CDLL(sa.LIB_PATH), name) is not None


def test_struct_layout_matches_c(tmp_path):
    fields = [f[0] for f in _lib.sa_problem._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(sa_problem, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "sa.h"\n'
                   'int main(void) {\n  printf("size %zu\\n", sizeof(sa_problem));\n'
                   f"{body}\n  return 0;\n}}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(_lib.sa_problem)
    for f in fields:
        assert int(got[f]) == getattr(_lib.sa_problem, f).offset, f


def _prob(**kw):
    base = dict(B=1, H=2, n=100, d=64, dtype=sa.SA_BF16, block=1, row_ptr=FAKE, col_idx=FAKE,
                nnz=500, scale=0.125, key_mask_heads=1, bias=None, key_mask=None, plan=None,
                flags=0, reserved=0)
    base.update(kw)
    return _lib.sa_problem(**base)


def _call(name, p, *ptrs):
    fn = _lib.raw(name)
    return fn(ctypes.byref(p) if p is not None else None, *ptrs)


PIPE = [("sa_sddmm", 4), ("sa_sparse_softmax", 3), ("sa_spmm", 4), ("sa_fused_forward", 6)]


@pytest.mark.parametrize("name,nargs", PIPE)
def test_null_problem(name, nargs):
    assert _call(name, None, *([FAKE] * (nargs - 1)), None) == sa.SA_ERR_NULL


@pytest.mark.parametrize("name,nargs", PIPE)
@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, sa.SA_ERR_DTYPE),
    ("d", 48, sa.SA_ERR_UNSUPPORTED),
    ("d", 256, sa.SA_ERR_UNSUPPORTED),
    ("block", 32, sa.SA_ERR_UNSUPPORTED),
    ("nnz", -1, sa.SA_ERR_SHAPE),
    ("nnz", 100 * 100 + 1, sa.SA_ERR_SHAPE),
    ("n", -5, sa.SA_ERR_SHAPE),
    ("flags", 8, sa.SA_ERR_UNSUPPORTED),
    ("reserved", 1, sa.SA_ERR_UNSUPPORTED),
    ("scale", float("nan"), sa.SA_ERR_SHAPE),
    ("col_idx", None, sa.SA_ERR_NULL),
])
def test_descriptor_errors(name, nargs, field, value, status):
    p = _prob(**{field: value})
    assert _call(name, p, *([FAKE] * (nargs - 2)), None, None) == status


@pytest.mark.parametrize("name,nargs", PIPE[:3])
def test_non_csr_patterns_rejected_by_pipeline_calls(name, nargs):
    assert _call(name, _prob(row_ptr=None), *([FAKE] * (nargs - 1)), None) == sa.SA_ERR_UNSUPPORTED
    assert _call(name, _prob(block=64, nnz=4), *([FAKE] * (nargs - 1)), None) == sa.SA_ERR_UNSUPPORTED


def test_key_mask_heads_broadcast_rule():
    # the key mask's head dimension is 1 or H (AlphaFold2 PR, mask shape list)
    for kmh, st in ((1, None), (2, None), (3, sa.SA_ERR_SHAPE), (0, sa.SA_ERR_SHAPE)):
        p = _prob(key_mask=FAKE, key_mask_heads=kmh, n=0, nnz=0)   # n=0: valid calls do nothing
        got = _call("sa_sddmm", p, FAKE, FAKE, FAKE, None)
        assert got == (sa.SA_OK if st is None else st)


@pytest.mark.parametrize("name,nargs", PIPE)
def test_null_buffers(name, nargs):
    for i in range(nargs - 1 - (1 if name == "sa_fused_forward" else 0)):
        ptrs = [FAKE] * (nargs - 1)
        ptrs[i] = None
        assert _call(name, _prob(), *ptrs, None) == sa.SA_ERR_NULL, i


@pytest.mark.parametrize("name,nargs", PIPE)
def test_misaligned_buffers(name, nargs):
    for i in range(nargs - 1 - (1 if name == "sa_fused_forward" else 0)):
        ptrs = [FAKE] * (nargs - 1)
        ptrs[i] = FAKE + 2
        assert _call(name, _prob(), *ptrs, None) == sa.SA_ERR_ALIGN, i


@pytest.mark.parametrize("name,nargs", PIPE)
def test_empty_problems_do_nothing(name, nargs):
    for field in ("B", "H", "n"):
        p = _prob(**{field: 0}, nnz=0)
        assert _call(name, p, *([None] * (nargs - 1)), None) == sa.SA_OK


def test_plan_bytes_and_build_checks():
    p = _prob(n=4096, nnz=1052026)
    # bad descriptors size to 0; a valid one needs the device (it reads row_ptr)
    assert _lib.raw("sa_plan_bytes")(ctypes.byref(_prob(row_ptr=None))) == 0
    assert _lib.raw("sa_plan_bytes")(ctypes.byref(_prob(block=64, nnz=4))) == 0
    assert _lib.raw("sa_plan_bytes")(ctypes.byref(_prob(n=0, nnz=0))) == 4 * 16
    assert _lib.raw("sa_plan_build")(ctypes.byref(p), None, 1 << 20, None) == sa.SA_ERR_NULL
    # header, row entries (4 words each), per tile: info, far columns, 13 x 64 block records of
    # 4 words
    minimal = 4 * (16 + 4 * 4096 + (8 + 64 + 13 * 64 * 4) * 64)
    assert _lib.raw("sa_plan_build")(ctypes.byref(p), FAKE, minimal - 4, None) == sa.SA_ERR_WORKSPACE
    # the plan is read 16 bytes at a time: a buffer off that alignment is refused, by the build
    # and by every call that carries it, before any device access
    assert _lib.raw("sa_plan_build")(ctypes.byref(p), FAKE + 4, minimal, None) == sa.SA_ERR_ALIGN
    q = _prob(n=4096, nnz=1052026)
    q.plan = FAKE + 8
    assert _lib.raw("sa_sddmm")(ctypes.byref(q), FAKE, FAKE, FAKE, None) == sa.SA_ERR_ALIGN


def test_validate_requires_a_pattern():
    assert _lib.raw("sa_validate_csr")(ctypes.byref(_prob(row_ptr=None)), None) == sa.SA_ERR_NULL


def test_status_strings():
    for code in range(0, -9, -1):
        s = sa.sa_status_string(code)
        assert s.startswith("SA_")
    assert "unknown" in sa.sa_status_string(-99)


def test_binding_checks_tensor_sizes():
    import torch
    rp = torch.zeros(101, dtype=torch.int32)
    ci = torch.zeros(10, dtype=torch.int32)
    with pytest.raises(ValueError):
        sa.Problem(1, 1, 100, 64, sa.SA_BF16, rp, ci, nnz=20)
    prob = sa.Problem(1, 1, 100, 64, sa.SA_BF16, rp, ci, nnz=10)
    small = torch.zeros(5)
    with pytest.raises(ValueError):
        sa.sa_sparse_softmax(prob, small, small)


def test_single_hip_runtime_shared_with_torch():
    """The library must run on the HIP runtime that owns torch's memory and streams."""
    maps = open("/proc/self/maps").read().splitlines()
    hip = sorted({ln.split()[-1] for ln in maps if "libamdhip64" in ln})
    assert len(hip) == 1, hip


# ---- backward-pass entry points (host checks only)

BWD = [("sa_gather_entries", 4), ("sa_csr_transpose", 6)]


def test_backward_calls_reject_bad_descriptors():
    f = _lib.raw
    for p, st in ((None, sa.SA_ERR_NULL), (_prob(row_ptr=None), sa.SA_ERR_UNSUPPORTED),
                  (_prob(block=64, nnz=4), sa.SA_ERR_UNSUPPORTED), (_prob(dtype=7), sa.SA_ERR_DTYPE)):
        ref = ctypes.byref(p) if p is not None else None
        assert f("sa_gather_entries")(ref, FAKE, FAKE, FAKE + 64, None) == st
        assert f("sa_sparse_softmax_backward")(ref, FAKE, FAKE, 1.0, FAKE, None) == st
        if p is None or p.row_ptr:  # the dense pattern is valid for the bias gradient
            assert f("sa_bias_grad")(ref, FAKE, 1.0, FAKE, None) == st
        assert f("sa_csr_transpose")(ref, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == st
        assert f("sa_gather_order_build")(ref, FAKE, FAKE, FAKE, 1 << 30, None) == st
        assert f("sa_gather_entries_ordered")(ref, FAKE, FAKE, FAKE + 64, None, None, None) == st
        if p is not None:
            assert f("sa_transpose_workspace_bytes")(ref) == 0


def test_backward_calls_check_buffers_and_arguments():
    f, p = _lib.raw, ctypes.byref(_prob())
    assert f("sa_gather_entries")(p, None, FAKE, FAKE + 64, None) == sa.SA_ERR_NULL
    assert f("sa_gather_entries")(p, FAKE, FAKE, FAKE, None) == sa.SA_ERR_SHAPE  # in place
    assert f("sa_sparse_softmax_backward")(p, FAKE, None, 1.0, FAKE, None) == sa.SA_ERR_NULL
    assert f("sa_sparse_softmax_backward")(p, FAKE, FAKE, float("inf"), FAKE, None) == sa.SA_ERR_SHAPE
    assert f("sa_bias_grad")(p, None, 1.0, FAKE, None) == sa.SA_ERR_NULL
    assert f("sa_bias_grad")(p, FAKE, float("nan"), FAKE, None) == sa.SA_ERR_SHAPE
    assert f("sa_csr_transpose")(p, None, FAKE, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_NULL
    assert f("sa_csr_transpose")(p, FAKE, FAKE, FAKE, None, 1 << 30, None) == sa.SA_ERR_NULL
    assert f("sa_csr_transpose")(p, FAKE, FAKE, FAKE, FAKE, 64, None) == sa.SA_ERR_WORKSPACE
    # keys and values are sorted out of place: at least 2 x (8 + 4) bytes per entry
    assert f("sa_transpose_workspace_bytes")(p) >= 24 * 500
    assert f("sa_gather_order_build")(p, FAKE, None, FAKE, 1 << 30, None) == sa.SA_ERR_NULL
    assert f("sa_gather_order_build")(p, FAKE, FAKE, FAKE, 64, None) == sa.SA_ERR_WORKSPACE
    g = f("sa_gather_entries_ordered")
    A, B, C, D = FAKE, FAKE + 64, FAKE + 128, FAKE + 192
    assert g(p, None, A, B, None, None, None) == sa.SA_ERR_NULL
    assert g(p, FAKE, A, B, C, None, None) == sa.SA_ERR_NULL  # src_b without dst_b
    assert g(p, FAKE, A, A, None, None, None) == sa.SA_ERR_SHAPE
    for aliased in ((A, B, C, B), (A, B, B, C), (A, B, C, A), (A, B, C, C)):
        assert g(p, FAKE, *aliased, None) == sa.SA_ERR_SHAPE, aliased
    for field in ("B", "H"):
        q = ctypes.byref(_prob(**{field: 0}, nnz=0))
        assert g(q, None, None, None, None, None, None) == sa.SA_OK
        assert f("sa_gather_entries")(q, None, None, None, None) == sa.SA_OK
        assert f("sa_sparse_softmax_backward")(q, None, None, 1.0, None, None) == sa.SA_OK


# ---- mask construction entry points (host checks only)

def test_mask_calls_check_sizes_and_buffers():
    f = _lib.raw
    ws = f("sa_mask_workspace_bytes")
    assert ws(-1, 10) == 0 and ws(10, -1) == 0 and ws(10, 1 << 31) == 0
    assert ws(4096, 1000) >= 2 * 8 * 1000  # keys sorted out of place
    coo = f("sa_coo_to_csr")
    assert coo(-1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_SHAPE
    assert coo(10, 1 << 31, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_SHAPE
    assert coo(10, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_NULL
    assert coo(10, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == sa.SA_ERR_NULL
    assert coo(10, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == sa.SA_ERR_WORKSPACE
    km = f("sa_key_mask_from_lengths")
    assert km(-1, 4, FAKE, FAKE, None) == sa.SA_ERR_SHAPE
    assert km(2, 4, None, FAKE, None) == sa.SA_ERR_NULL
    assert km(0, 4, None, None, None) == sa.SA_OK
    rp, ci = f("sa_varlen_row_ptr"), f("sa_varlen_col_idx")
    assert rp(2, -1, FAKE, -1, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_SHAPE
    assert rp(2, 100000, FAKE, -1, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_SHAPE  # 1e10 pairs
    assert rp(0, 10, FAKE, -1, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_SHAPE  # no sequence
    assert rp(2, 10, None, -1, FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_NULL
    assert rp(2, 10, FAKE, -1, FAKE, FAKE, 8, None) == sa.SA_ERR_WORKSPACE
    assert ci(2, 10, FAKE, -1, FAKE, FAKE, -1, None) == sa.SA_ERR_SHAPE
    assert ci(2, 10, FAKE, -1, None, FAKE, 100, None) == sa.SA_ERR_NULL
    assert ci(2, 10, FAKE, -1, FAKE, FAKE, 0, None) == sa.SA_OK  # nothing to write


def test_fused_backward_checks():
    f = _lib.raw("sa_fused_backward")
    # q k v out lse dout t_row_ptr t_col_idx dq dk dv dscores workspace stream
    args = [FAKE] * 12 + [FAKE, None]
    dense = _prob(row_ptr=None, col_idx=None, nnz=0)
    assert f(ctypes.byref(_prob()), *args) == sa.SA_ERR_UNSUPPORTED            # element CSR
    bsr = list(args)
    bsr[6] = None                                                            # no transposed pattern
    assert f(ctypes.byref(_prob(block=64, nnz=4)), *bsr) == sa.SA_ERR_NULL
    assert f(ctypes.byref(_prob(row_ptr=None, col_idx=None, nnz=0, dtype=sa.SA_F32)), *args) \
        == sa.SA_ERR_UNSUPPORTED                                             # fp32 inputs
    bad = list(args)
    bad[12] = None                                                           # no workspace
    assert f(ctypes.byref(dense), *bad) == sa.SA_ERR_NULL
    bad = list(args)
    bad[11] = None                                                           # dscores is optional
    bad[1] = FAKE + 4                                                        # misaligned k
    assert f(ctypes.byref(dense), *bad) == sa.SA_ERR_ALIGN
    assert f(None, *args) == sa.SA_ERR_NULL
    big = _prob(row_ptr=None, col_idx=None, nnz=0, n=30000, bias=FAKE)  # bias head past 2 GB
    assert f(ctypes.byref(big), *args) == sa.SA_ERR_UNSUPPORTED


# ---- block cover and the fused backward over it (host checks only)

def test_block_cover_calls_check_arguments():
    f = _lib.raw
    good = _prob()
    for p, st in ((None, sa.SA_ERR_NULL), (_prob(row_ptr=None), sa.SA_ERR_UNSUPPORTED),
                  (_prob(block=64, nnz=4), sa.SA_ERR_UNSUPPORTED), (_prob(n=(1 << 22) + 1), sa.SA_ERR_SHAPE)):
        ref = ctypes.byref(p) if p is not None else None
        assert f("sa_block_cover_row_ptr")(ref, FAKE, None) == st
        assert f("sa_block_cover_col_idx")(ref, FAKE, 1, FAKE, None) == st
    p = ctypes.byref(good)
    assert f("sa_block_cover_row_ptr")(p, None, None) == sa.SA_ERR_NULL
    assert f("sa_block_cover_col_idx")(p, FAKE, 1, None, None) == sa.SA_ERR_NULL
    assert f("sa_block_cover_col_idx")(p, FAKE, -1, FAKE, None) == sa.SA_ERR_SHAPE
    assert f("sa_block_cover_col_idx")(p, FAKE, 5, FAKE, None) == sa.SA_ERR_SHAPE  # > (ceil(100/64))^2
    c = _lib.sa_block_cover(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4)
    assert f("sa_block_cover_bits")(p, None, None) == sa.SA_ERR_NULL
    for field in ("row_ptr", "col_idx", "t_row_ptr", "t_col_idx", "bits", "bits_t"):
        bad = _lib.sa_block_cover(**{k: (None if k == field else FAKE) for k in
                                     ("row_ptr", "col_idx", "t_row_ptr", "t_col_idx", "bits", "bits_t")}, nnz=4)
        assert f("sa_block_cover_bits")(p, ctypes.byref(bad), None) == sa.SA_ERR_NULL, field
    c.nnz = 5
    assert f("sa_block_cover_bits")(p, ctypes.byref(c), None) == sa.SA_ERR_SHAPE


def test_fused_backward_cover_checks_arguments():
    f = _lib.raw("sa_fused_backward_cover")
    c = ctypes.byref(_lib.sa_block_cover(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4))
    bufs = [FAKE] * 10
    assert f(None, c, *bufs, FAKE, None) == sa.SA_ERR_NULL
    for p, st in ((_prob(row_ptr=None), sa.SA_ERR_UNSUPPORTED), (_prob(block=64, nnz=4), sa.SA_ERR_UNSUPPORTED),
                  (_prob(dtype=sa.SA_F32), sa.SA_ERR_UNSUPPORTED), (_prob(dtype=7), sa.SA_ERR_DTYPE)):
        assert f(ctypes.byref(p), c, *bufs, FAKE, None) == st
    p = ctypes.byref(_prob())
    assert f(p, None, *bufs, FAKE, None) == sa.SA_ERR_NULL
    for i in range(10):
        args = list(bufs)
        if i == 9:  # dscores is optional; the workspace is not
            assert f(p, c, *args, None, None) == sa.SA_ERR_NULL
            continue
        args[i] = None
        assert f(p, c, *args, FAKE, None) == sa.SA_ERR_NULL, i
    assert f(p, c, *([FAKE + 8] + bufs[1:]), FAKE, None) == sa.SA_ERR_ALIGN


def test_plan_size_is_host_only_bound():
    """sa_plan_bytes needs no device access (a descriptor whose row_ptr points nowhere valid
    still gets a size) and grows with the head count and size, not with the pattern's content."""
    fake = FAKE
    a = sa.Problem(1, 12, 4096, 64, sa.SA_BF16, fake, fake, 1_052_026)
    b = sa.Problem(1, 12, 4096, 128, sa.SA_BF16, fake, fake, 1_052_026)
    assert 0 < sa.sa_plan_bytes(a) < sa.sa_plan_bytes(b)
