"""Test-side helpers for GPU parity: move a generated problem to the device, run the
library through its C ABI, and compare with the oracle at the stated tolerances."""
import numpy as np
import torch

import masked_scaled_dot_amd as sa

DEV = torch.device("cuda:0")

# Tolerances: fp32 inputs max-abs <= 1e-5; bf16 inputs (fp32 accumulate) max-abs <= 1e-2
# and mean-abs <= 1e-3, for weights and context alike.
TOL = {"f32": (1e-5, None), "bf16": (1e-2, 1e-3)}


def say(msg):
    print(msg, flush=True)


def qkv_tensor(p, which):
    bits = getattr(p, which + "_bits")
    if p.dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(getattr(p, which)).to(DEV)


class DevProblem:
    """Device copies of a gen.Problem plus the sa.Problem descriptor pointing at them."""

    def __init__(self, p, scale=None, flags=0, with_bias=True, with_mask=True, plan=False):
        self.p = p
        self.q, self.k, self.v = (qkv_tensor(p, w) for w in ("q", "k", "v"))
        self.row_ptr = None if p.row_ptr is None else torch.from_numpy(p.row_ptr).to(DEV)
        self.col_idx = None if p.col_idx is None else torch.from_numpy(p.col_idx).to(DEV)
        self.bias = torch.from_numpy(p.bias).to(DEV) if (p.bias is not None and with_bias) else None
        self.key_mask = torch.from_numpy(np.ascontiguousarray(p.key_mask)).to(DEV) \
            if (p.key_mask is not None and with_mask) else None
        self.scale = p.scale if scale is None else scale
        self.prob = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16 if p.dtype == "bf16" else sa.SA_F32,
                               self.row_ptr, self.col_idx, p.nnz, block=p.block, scale=self.scale,
                               bias=self.bias, key_mask=self.key_mask,
                               key_mask_heads=p.key_mask_heads, flags=flags)
        self.plan = None
        if plan:
            self.build_plan()

    def build_plan(self):
        # room for every long-row segment of the pattern (rows over 1024 entries take
        # ceil(len / 256) each), so that the split paths run even on patterns with many
        lens = np.diff(self.p.row_ptr.astype(np.int64))
        segs = int(((lens[lens > 1024] + 255) // 256).sum())
        nbytes = sa.sa_plan_bytes_segments(self.prob, max(segs, 1024))
        assert nbytes > 0
        self.plan = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=DEV)
        sa.sa_plan_build(self.prob, self.plan)
        self.prob.set_plan(self.plan)
        return self.plan

    def pipeline(self):
        p = self.p
        scores = torch.full((p.BH * p.nnz,), float("nan"), device=DEV)
        weights = torch.full_like(scores, float("nan"))
        out = torch.full((p.BH, p.n, p.d), float("nan"), device=DEV)
        sa.sa_sddmm(self.prob, self.q, self.k, scores)
        sa.sa_sparse_softmax(self.prob, scores, weights)
        sa.sa_spmm(self.prob, weights, self.v, out)
        torch.cuda.synchronize()
        return (scores.view(p.BH, p.nnz).cpu().numpy(), weights.view(p.BH, p.nnz).cpu().numpy(),
                out.cpu().numpy())

    def fused(self, want_lse=True):
        p = self.p
        out = torch.full((p.BH, p.n, p.d), float("nan"), device=DEV)
        lse = torch.full((p.BH, p.n), float("nan"), device=DEV) if want_lse else None
        sa.sa_fused_forward(self.prob, self.q, self.k, self.v, out, lse)
        torch.cuda.synchronize()
        return out.cpu().numpy(), (lse.cpu().numpy() if want_lse else None)

    def oracle_args(self):
        p = self.p
        return dict(bias=p.bias if self.bias is not None else None,
                    key_mask=p.key_mask if self.key_mask is not None else None,
                    km_heads=p.key_mask_heads)


def check(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    # -inf references (masked scores, empty-row lse) must be reproduced exactly
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finite/inf pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{what}: infinite values differ"
    err = np.abs(got[fin] - ref[fin])
    if err.size == 0:
        return 0.0, 0.0
    mx, mean = float(err.max()), float(err.mean())
    tmax, tmean = TOL[dtype]
    assert mx <= tmax, f"{what}: max-abs {mx:.3e} > {tmax}"
    if tmean is not None:
        assert mean <= tmean, f"{what}: mean-abs {mean:.3e} > {tmean}"
    return mx, mean
