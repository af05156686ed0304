"""GPU test of sa_fused_backward_noalloc (the fused backward whose row-sum scratch is the
library's fixed device array instead of a caller workspace): two calls in a row through the
C ABI, the second on a smaller problem, each compared with sa_fused_backward given its own
workspace on the same inputs. Both entry points run the same kernels, so the gradients must
agree bit for bit. Also: sizes beyond the fixed scratch and device validation are refused."""
import numpy as np
import pytest
import torch

import gen
import masked_scaled_dot_amd as sa
from masked_scaled_dot_amd import _lib
from gpu_util import DEV, DevProblem, say

pytestmark = pytest.mark.gpu


def _grads(dp, p, fn):
    N = (p.BH, p.n, p.d)
    out = torch.empty(N, device=DEV)
    lse = torch.empty(p.BH, p.n, device=DEV)
    sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, out, lse)
    g = torch.Generator(device="cpu").manual_seed(p.n)
    dO = torch.randn(N, generator=g).to(DEV, torch.bfloat16)
    dq, dk, dv = (torch.full(N, float("nan"), device=DEV) for _ in range(3))
    ds = torch.full((p.BH, p.n, p.n), float("nan"), device=DEV)
    fn(dp.prob, dp.q, dp.k, dp.v, out, lse, dO, dq, dk, dv, ds)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (dq, dk, dv, ds)]


def _with_workspace(prob, q, k, v, out, lse, dO, dq, dk, dv, ds):
    ws = torch.full((prob.BH * prob.c.n,), float("nan"), device=DEV)
    sa.sa_fused_backward(prob, q, k, v, out, lse, dO, dq, dk, dv, ws, dscores=ds)


def _noalloc(prob, q, k, v, out, lse, dO, dq, dk, dv, ds):
    sa.sa_fused_backward_noalloc(prob, q, k, v, out, lse, dO, dq, dk, dv, dscores=ds)


def test_noalloc_matches_workspace_entry_point_twice():
    for B, n in ((8, 384), (3, 97)):  # the second call is smaller than the first
        p = gen.make("evoformer_l384", B=B, n=n)
        say(f"noalloc fused backward: B={B} H={p.H} n={n}")
        dp = DevProblem(p)
        ref = _grads(dp, p, _with_workspace)
        got = _grads(dp, p, _noalloc)
        for name, a, b in zip(("dq", "dk", "dv", "dscores"), got, ref):
            assert np.isfinite(a).all(), name
            assert np.array_equal(a, b), f"{name} differs from sa_fused_backward (B={B}, n={n})"


def test_noalloc_refuses_sizes_and_validation():
    # B*H*n row sums beyond the 16 MiB scratch: 4 Mi floats + one head of n = 4096
    p = sa.Problem(1025, 1, 4096, 32, sa.SA_BF16, scale=0.5)
    x = torch.empty(16, device=DEV)
    st = _lib.raw("sa_fused_backward_noalloc")(_lib.ctypes.byref(p.c), *([x.data_ptr()] * 12), None)
    assert st == sa.SA_ERR_WORKSPACE
    q = gen.make("evoformer_l384", B=1, n=64)
    dp = DevProblem(q, flags=sa.SA_FLAG_VALIDATE)
    st = _lib.raw("sa_fused_backward_noalloc")(_lib.ctypes.byref(dp.prob.c), *([x.data_ptr()] * 12), None)
    assert st == sa.SA_ERR_UNSUPPORTED
