"""GPU parity of the backward of the fused dense forward (sa_fused_backward).

The forward runs on the GPU (sa_fused_forward: O and lse), the backward recomputes the
weights from lse; dQ, dK, dV and dS (summed over the batches into the bias gradient by
sa_bias_grad) are compared with torch autograd in fp64 of the dense definition
(oracle.backward.grads_autograd, pinned in test_oracle_backward_pins.py) on the same
bf16-rounded inputs, at the bf16 tolerances. Cases cover d = 32, 64, 128, a ragged last tile,
bias with and without a key mask, key lengths, and a batch whose keys are all masked.
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
    ds = torch.full((p.BH, p.n, p.n), float("nan"), device=DEV)
    ws = torch.empty(p.BH * p.n, device=DEV)
    sa.sa_fused_backward(dp.prob, dp.q, dp.k, dp.v, out, lse, dO, dq, dk, dv, ws, dscores=ds)
    torch.cuda.synchronize()
    km = p.key_mask
    if lens is not None:
        km = omask.key_mask_from_lengths(lens, p.n)[:, None, :] + (0 if km is None else km)
    ref = obw.grads_autograd(p.q, p.k, p.v, p.scale, p.H, ("dense",), dO_host, bias=p.bias,
                             key_mask=km)
    check(dq.cpu().numpy(), ref["dQ"], p.dtype, "dQ")
    check(dk.cpu().numpy(), ref["dK"], p.dtype, "dK")
    check(dv.cpu().numpy(), ref["dV"], p.dtype, "dV")
    if p.bias is not None:
        dbias = torch.full((p.H, p.n, p.n), float("nan"), device=DEV)
        sa.sa_bias_grad(dp.prob, ds, 1.0, dbias)
        torch.cuda.synchronize()
        check(dbias.cpu().numpy(), ref["dBias"], p.dtype, "dBias")
