"""GPU parity of the fused backward over an element CSR pattern, run on its block cover
(sa_block_cover_* and sa_fused_backward_cover).

The cover (block CSR, its transpose and both word layouts) is compared bit for bit with the
oracle's (oracle.cover, pinned in test_oracle_cover_pins.py). The gradients of the fused
element-CSR forward (sa_fused_forward: O and lse on the GPU) are compared with torch autograd
in fp64 of the masked definition (oracle.backward.grads_autograd with the CSR pattern) on
the same bf16-rounded inputs, at the bf16 tolerances: a windowed pattern with global tokens,
random rows with bias and key mask, the Evoformer-style dense pattern as element CSR
(d = 32), d = 128 with a ragged last tile, rows without entries, and at full size
(12 heads, n = 4096) sampled heads.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import masked_scaled_dot_amd as sa
from oracle import backward as obw
from oracle import cover as ocv
from gpu_util import DEV, DevProblem, check, say

pytestmark = pytest.mark.gpu


def _bf16(x):
    bits = gen.bf16_round_bits(np.asarray(x, np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV), gen.bf16_bits_to_f32(bits)


def _element_csr(p):
    rp, ci = p.element_csr()
    return dataclasses.replace(p, row_ptr=rp.astype(np.int32), col_idx=ci.astype(np.int32), block=1)


def _empty_rows(p, rows):
    """The pattern of p with the given rows emptied."""
    keep = [(r, p.col_idx[p.row_ptr[r]:p.row_ptr[r + 1]]) for r in range(p.n)]
    cols = [c if r not in rows else c[:0] for r, c in keep]
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = np.concatenate(cols).astype(np.int32)
    return dataclasses.replace(p, row_ptr=rp, col_idx=ci)


CASES = {
    "window_global_d64": lambda: gen.make("longformer_n4096", n=700, H=3, window=40),
    "random_bias_keymask": lambda: gen.make("random_n8192", n=300, H=2, B=2, kmin=1, kmax=120,
                                            bias=True, key_mask=True, pmax=40),
    "evoformer_dense_d32": lambda: _element_csr(gen.make("evoformer_l384", B=2, H=2, n=96)),
    "random_d128_ragged": lambda: gen.make("random_n8192", n=64 * 3 + 29, H=2, d=128, kmin=1, kmax=60),
    "empty_rows": lambda: _empty_rows(gen.make("longformer_n4096", n=300, H=2, window=20),
                                      {0, 5, 63, 64, 200, 299}),
}


def _check_cover(p, cover):
    want = ocv.block_cover(p.n, p.row_ptr, p.col_idx)
    nnz = cover.nnz
    assert nnz == len(want["col_idx"])
    for name in ("row_ptr", "t_row_ptr"):
        assert np.array_equal(getattr(cover, name).cpu().numpy(), want[name]), name
    for name in ("col_idx", "t_col_idx"):
        assert np.array_equal(getattr(cover, name)[:nnz].cpu().numpy(), want[name]), name
    for name in ("bits", "bits_t"):
        got = getattr(cover, name)[:nnz * 64].cpu().numpy().view(np.uint64).reshape(nnz, 64)
        assert np.array_equal(got, want[name]), name


def _run(p, plan, seed, dscores=False):
    dp = DevProblem(p, plan=plan)
    cover = sa.block_cover(dp.prob, device=DEV)
    N = (p.BH, p.n, p.d)
    out = torch.empty(N, device=DEV)
    lse = torch.empty(p.BH, p.n, device=DEV)
    sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, out, lse)
    dO, dO_host = _bf16(np.random.default_rng(seed).standard_normal(N))
    dq, dk, dv = (torch.full(N, float("nan"), device=DEV) for _ in range(3))
    ds = torch.zeros((p.BH, p.n, p.n), device=DEV) if dscores else None
    ws = torch.empty(p.BH * p.n, device=DEV)
    sa.sa_fused_backward_cover(dp.prob, cover, dp.q, dp.k, dp.v, out, lse, dO, dq, dk, dv, ws, dscores=ds)
    torch.cuda.synchronize()
    return dp, cover, dO_host, dict(dQ=dq, dK=dk, dV=dv, dS=ds)


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_backward_cover_parity(name):
    p = CASES[name]()
    plan = name != "random_d128_ragged"
    say(f"fused backward over the block cover {name}: B={p.B} H={p.H} n={p.n} d={p.d} nnz={p.nnz} "
        f"bias={p.bias is not None} mask={p.key_mask is not None} plan={plan}")
    dp, cover, dO_host, got = _run(p, plan, 31, dscores=p.bias is not None)
    _check_cover(p, cover)
    ref = obw.grads_autograd(p.q, p.k, p.v, dp.scale, p.H, ("csr", p.row_ptr, p.col_idx), dO_host,
                             **dp.oracle_args())
    for g in ("dQ", "dK", "dV"):
        check(got[g].cpu().numpy(), ref[g], p.dtype, g)
    if p.bias is not None:
        dbias = torch.full((p.H, p.n, p.n), float("nan"), device=DEV)
        dense = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16, None, None, 0, scale=dp.scale)
        sa.sa_bias_grad(dense, got["dS"], 1.0, dbias)
        torch.cuda.synchronize()
        check(dbias.cpu().numpy(), ref["dBias"], p.dtype, "dBias")


def test_fused_backward_cover_full_size_sampled_heads():
    """The Longformer-style workload at full size (12 heads, n = 4096, d = 64): the cover
    bit for bit against the oracle's, and dQ, dK, dV of sampled heads against autograd of
    those heads alone (a head's gradients depend only on its own q, k, v and dO)."""
    p = gen.make("longformer_n4096")
    say(f"fused backward over the block cover, full size: BH={p.BH} n={p.n} nnz={p.nnz}")
    dp, cover, dO_host, got = _run(p, True, 32)
    _check_cover(p, cover)
    got = {g: got[g].cpu().numpy() for g in ("dQ", "dK", "dV")}
    assert all(np.isfinite(x).all() for x in got.values())
    for t in (0, 7, p.BH - 1):
        ref = obw.grads_autograd(p.q[t:t + 1], p.k[t:t + 1], p.v[t:t + 1], dp.scale, 1,
                                 ("csr", p.row_ptr, p.col_idx), dO_host[t:t + 1])
        for g in ("dQ", "dK", "dV"):
            check(got[g][t:t + 1], ref[g], p.dtype, f"{g} head {t}")
