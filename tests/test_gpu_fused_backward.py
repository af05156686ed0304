"""GPU parity of the backward of the fused dense forward (sa_fused_backward).

The forward runs on the GPU (sa_fused_forward: O and lse), the backward recomputes the
weights from lse; dQ, dK, dV and dS (summed over the batches into the bias gradient by
sa_bias_grad) are compared with torch autograd in fp64 of the dense definition
(oracle.backward.grads_autograd, pinned in test_oracle_backward_pins.py) on the same
bf16-rounded inputs, at the bf16 tolerances. Cases cover d = 32, 64, 128, a ragged last tile,
bias with and without a key mask, key lengths, a batch whose keys are all masked, and block
CSR (with the transposed block pattern from sa_csr_transpose).
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import masked_scaled_dot_amd as sa
from oracle import backward as obw
from oracle import mask as omask
from gpu_util import DEV, DevProblem, check, say

pytestmark = pytest.mark.gpu


def _bf16(x):
    bits = gen.bf16_round_bits(np.asarray(x, np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV), gen.bf16_bits_to_f32(bits)


def _all_masked_batch(p):
    km = p.key_mask.copy()
    km[-1] = -np.inf
    return dataclasses.replace(p, key_mask=km)


CASES = {
    "d32_bias_mask_ragged": (lambda: gen.make("evoformer_l384", B=2, H=2, n=96), None),
    "d64_bias_mask": (lambda: gen.make("evoformer_l384", B=2, H=2, n=130, d=64), None),
    "d128_bias_only": (lambda: dataclasses.replace(gen.make("evoformer_l384", B=1, H=2, n=70, d=128),
                                                   key_mask=None), None),
    "d64_plain": (lambda: dataclasses.replace(gen.make("evoformer_l384", B=2, H=1, n=200, d=64),
                                              bias=None, key_mask=None), None),
    "d32_seqlen_k": (lambda: dataclasses.replace(gen.make("evoformer_l384", B=3, H=2, n=150),
                                                 key_mask=None), [150, 77, 1]),
    "d32_batch_all_masked": (lambda: _all_masked_batch(gen.make("evoformer_l384", B=2, H=2, n=64)), None),
}


def _block_transpose(p):
    """The transposed block pattern (block-rows of each block-column) by sa_csr_transpose on
    a descriptor over the block grid."""
    nb = (p.n + 63) // 64
    rp = torch.from_numpy(p.row_ptr).to(DEV)
    ci = torch.from_numpy(p.col_idx).to(DEV)
    prob = sa.Problem(1, 1, nb, 32, sa.SA_BF16, rp, ci, p.nnz)
    rpt = torch.empty(nb + 1, dtype=torch.int32, device=DEV)
    cit = torch.empty(max(p.nnz, 1), dtype=torch.int32, device=DEV)
    perm = torch.empty_like(cit)
    ws = torch.empty(max(sa.sa_transpose_workspace_bytes(prob), 1), dtype=torch.uint8, device=DEV)
    sa.sa_csr_transpose(prob, rpt, cit[:p.nnz], perm[:p.nnz], ws)
    return rpt, cit


CASES.update({
    "bsr_d128_ragged": (lambda: gen.make("bsr_n16384", n=64 * 6 + 21, H=2, extra=3), None),
    "bsr_d64_bias_mask": (lambda: gen.make("bsr_n16384", n=64 * 5 + 7, H=2, d=64, extra=2,
                                           bias=True, key_mask=True, pmax=40), None),
})


def _pattern(p):
    return ("dense",) if p.row_ptr is None else ("bsr", p.row_ptr, p.col_idx, 64)


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_backward_parity(name):
    make, lens = CASES[name]
    p = make()
    say(f"fused backward {name}: B={p.B} H={p.H} n={p.n} d={p.d} bias={p.bias is not None} "
        f"mask={p.key_mask is not None} lens={lens}")
    dp = DevProblem(p)
    sl = None
    if lens is not None:
        sl = torch.tensor(np.asarray(lens, np.int32), device=DEV)
        dp.prob = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16, None, None, 0, scale=p.scale,
                             bias=dp.bias, key_mask=dp.key_mask, seqlen_k=sl)
    N = (p.BH, p.n, p.d)
    out = torch.empty(N, device=DEV)
    lse = torch.empty(p.BH, p.n, device=DEV)
    sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, out, lse)
    dO, dO_host = _bf16(np.random.default_rng(21).standard_normal(N))
    dq, dk, dv = (torch.full(N, float("nan"), device=DEV) for _ in range(3))
    ds = torch.full((p.BH, p.n, p.n), float("nan") if p.row_ptr is None else 0.0, device=DEV)
    ws = torch.empty(p.BH * p.n, device=DEV)
    rpt, cit = _block_transpose(p) if p.row_ptr is not None else (None, None)
    sa.sa_fused_backward(dp.prob, dp.q, dp.k, dp.v, out, lse, dO, dq, dk, dv, ws, dscores=ds,
                         t_row_ptr=rpt, t_col_idx=cit)
    torch.cuda.synchronize()
    km = p.key_mask
    if lens is not None:
        km = omask.key_mask_from_lengths(lens, p.n)[:, None, :] + (0 if km is None else km)
    ref = obw.grads_autograd(p.q, p.k, p.v, p.scale, p.H, _pattern(p), dO_host, bias=p.bias,
                             key_mask=km)
    check(dq.cpu().numpy(), ref["dQ"], p.dtype, "dQ")
    check(dk.cpu().numpy(), ref["dK"], p.dtype, "dK")
    check(dv.cpu().numpy(), ref["dV"], p.dtype, "dV")
    if p.bias is not None:
        dbias = torch.full((p.H, p.n, p.n), float("nan"), device=DEV)
        dense = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16, None, None, 0, scale=p.scale)
        sa.sa_bias_grad(dense, ds, 1.0, dbias)
        torch.cuda.synchronize()
        check(dbias.cpu().numpy(), ref["dBias"], p.dtype, "dBias")


def test_fused_backward_full_size_sampled_heads():
    """The Evoformer-style workload at full size (32 x 8 heads, n = 384, d = 32, bias and key
    padding): dQ, dK and dV of sampled heads against autograd of those heads alone (a head's
    gradients depend on its own q, k, v, dO, its bias head and its batch's key mask)."""
    p = gen.make("evoformer_l384")
    say(f"fused backward full size: BH={p.BH} n={p.n} d={p.d}")
    dp = DevProblem(p)
    N = (p.BH, p.n, p.d)
    out = torch.empty(N, device=DEV)
    lse = torch.empty(p.BH, p.n, device=DEV)
    sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, out, lse)
    dO, dO_host = _bf16(np.random.default_rng(22).standard_normal(N))
    dq, dk, dv = (torch.full(N, float("nan"), device=DEV) for _ in range(3))
    ws = torch.empty(p.BH * p.n, device=DEV)
    sa.sa_fused_backward(dp.prob, dp.q, dp.k, dp.v, out, lse, dO, dq, dk, dv, ws)
    torch.cuda.synchronize()
    got = {"dQ": dq.cpu().numpy(), "dK": dk.cpu().numpy(), "dV": dv.cpu().numpy()}
    assert all(np.isfinite(x).all() for x in got.values())
    for t in (0, 77, p.BH - 1):
        b, h = divmod(t, p.H)
        ref = obw.grads_autograd(p.q[t:t + 1], p.k[t:t + 1], p.v[t:t + 1], p.scale, 1, ("dense",),
                                 dO_host[t:t + 1], bias=p.bias[h:h + 1], key_mask=p.key_mask[b:b + 1])
        for name in ("dQ", "dK", "dV"):
            check(got[name][t:t + 1], ref[name], p.dtype, f"{name} head {t}")


def test_fused_backward_graph_replay_matches_eager():
    """The fused forward and backward captured as one HIP graph reproduce the eager results
    bit for bit on every replay (no state is kept between calls)."""
    p = gen.make("evoformer_l384", B=2, H=2, n=130, d=64)
    dp = DevProblem(p)
    N = (p.BH, p.n, p.d)
    out = torch.empty(N, device=DEV)
    lse = torch.empty(p.BH, p.n, device=DEV)
    dO, _ = _bf16(np.random.default_rng(23).standard_normal(N))
    dq, dk, dv = (torch.empty(N, device=DEV) for _ in range(3))
    ws = torch.empty(p.BH * p.n, device=DEV)

    def run():
        sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, out, lse)
        sa.sa_fused_backward(dp.prob, dp.q, dp.k, dp.v, out, lse, dO, dq, dk, dv, ws)

    run()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, lse, dq, dk, dv)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for x in (out, lse, dq, dk, dv):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs from the eager result"
        run()
