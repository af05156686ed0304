"""GPU parity at the full workload sizes, on whole outputs.

Every element of the scores, weights and context of the three-step pipeline, and of
the context and lse of the fused forward, is compared with the fp64 oracle (the CSR
evaluation of the three steps, ``oracle.attention_csr``, whose agreement with the dense
definition is pinned on the CPU) at the tolerances of the method: max-abs <= 1e-2 and
mean-abs <= 1e-3 for bf16 inputs with fp32 accumulation. The block-sparse workload is
checked on two whole heads (the first and the last) of its 16. Each check prints one
``PARITY`` line with the workload, kernel, output and the max-abs / mean-abs error.

Also here: the fused forward over element CSR with a bias head larger than 2 GiB (n =
23232), which must not take the tile kernels whose bias offsets are 32-bit.
"""
import functools

import numpy as np
import pytest
import torch

import gen
import masked_scaled_dot_amd as sa
import oracle
from gpu_util import DEV, DevProblem, check, say

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def workload(name):
    return gen.make(name)


@functools.lru_cache(maxsize=1)
def reference(name, heads=None):
    """fp64 oracle of the workload (element pattern), optionally for a subset of heads."""
    p = workload(name)
    rp, ci = p.element_csr()
    sl = slice(None) if heads is None else list(heads)
    q, k, v = p.q[sl], p.k[sl], p.v[sl]
    H = p.H
    if heads is not None:
        # the oracle flattens heads as t = b*H + h; a subset keeps H so that bias / key mask
        # rows still index by h = t % H (the subsets used here have B = 1)
        assert p.B == 1
    km = p.key_mask
    return oracle.attention_csr(q, k, v, rp, ci, p.scale, H, bias=p.bias, key_mask=km,
                                km_heads=p.key_mask_heads)


def report(name, kernel, what, got, ref, dtype):
    mx, mean = check(got, ref, dtype, f"{name} {kernel} {what}")
    say(f"PARITY {name} {kernel} {what} max_abs={mx:.3e} mean_abs={mean:.3e} n_values={np.size(ref)}")


def _element(p):
    if p.row_ptr is not None and p.block == 1:
        return p
    import copy
    rp, ci = p.element_csr()
    e = copy.copy(p)
    e.row_ptr, e.col_idx, e.block = rp.astype(np.int32), ci.astype(np.int32), 1
    return e


@pytest.mark.parametrize("name", ["longformer_n4096", "random_n8192", "evoformer_l384"])
def test_full_whole_outputs(name):
    """Element CSR workloads: the pipeline (with its row plan) and the fused forward (with
    and without the plan); the dense workload: the fused forward."""
    p = workload(name)
    ref = reference(name)
    if p.row_ptr is not None:
        say(f"full pipeline (whole outputs) {name}: BH={p.BH} n={p.n} nnz/head={p.nnz}")
        dp = DevProblem(p, plan=True)
        S, W, O = dp.pipeline()
        report(name, "sddmm", "scores", S, ref["S"], p.dtype)
        report(name, "softmax", "weights", W, ref["W"], p.dtype)
        report(name, "spmm", "context", O, ref["O"], p.dtype)
        del S, W, O
        plans = (True, False)
    else:
        plans = (False,)
    for plan in plans:
        say(f"full fused (whole outputs) {name}: BH={p.BH} n={p.n} plan={plan}")
        dp = DevProblem(p, plan=plan)
        O, lse = dp.fused()
        kern = "fused" + ("_plan" if plan else "")
        report(name, kern, "context", O, ref["O"], p.dtype)
        report(name, kern, "lse", lse, ref["lse"], p.dtype)


def test_full_block_sparse_two_whole_heads():
    name = "bsr_n16384"
    p = workload(name)
    heads = (0, p.BH - 1)
    say(f"full block-sparse {name}: BH={p.BH} n={p.n}; heads {heads} compared whole")
    dp = DevProblem(p)
    O, lse = dp.fused()
    ref = reference(name, heads)
    report(name, "fused_bsr", "context", O[list(heads)], ref["O"], p.dtype)
    report(name, "fused_bsr", "lse", lse[list(heads)], ref["lse"], p.dtype)
    assert np.all(np.isfinite(O))
    del dp, O, lse
    torch.cuda.empty_cache()
    # the three-step pipeline on the element expansion of the same pattern (every head runs;
    # the two heads are compared whole)
    pe = _element(p)
    say(f"full pipeline on the element expansion {name}: nnz/head={pe.nnz}")
    dpe = DevProblem(pe, plan=True)
    S, W, Oe = dpe.pipeline()
    report(name, "sddmm", "scores", S[list(heads)], ref["S"], p.dtype)
    report(name, "softmax", "weights", W[list(heads)], ref["W"], p.dtype)
    report(name, "spmm", "context", Oe[list(heads)], ref["O"], p.dtype)
    del S, W, Oe
    # the fused forward on the element expansion with its plan: every tile is whole blocks
    say(f"full fused forward on the element expansion {name} (plan, whole-block tiles)")
    Of, lsef = dpe.fused()
    report(name, "fused_plan_blocks", "context", Of[list(heads)], ref["O"], p.dtype)
    report(name, "fused_plan_blocks", "lse", lsef[list(heads)], ref["lse"], p.dtype)


class _SampledBiasRows:
    """Stands in for a [1, n, n] bias array of which only some rows are held on the host:
    ``bias[0, i:i+1, :]`` returns row i (the only form of indexing the oracle uses)."""

    def __init__(self, rows):
        self.rows = rows

    def __getitem__(self, key):
        h, rows, cols = key
        assert h == 0 and rows.stop == rows.start + 1 and cols == slice(None)
        return self.rows[rows.start][None, :]


def test_fused_element_csr_bias_beyond_32bit_offsets():
    """A bias head of n * n * 4 > 2 GiB bytes (n = 23232) with an element-CSR plan: the
    result must match the oracle on sampled rows, i.e. the bias is read at every row."""
    n, H, d, w = 23232, 1, 64, 16
    rows = [list(range(max(0, i - w), min(n, i + w + 1))) for i in range(n)]
    rp, ci = gen.csr_from_rows(rows)
    rng = np.random.default_rng(23232)
    x = rng.standard_normal((3, H, n, d)).astype(np.float32)
    bits = gen.bf16_round_bits(x).reshape(x.shape)
    q, k, v = (gen.bf16_bits_to_f32(bits[i]).reshape(H, n, d) for i in range(3))
    g = torch.Generator(device=DEV).manual_seed(7)
    bias_d = torch.randn((H, n, n), generator=g, device=DEV, dtype=torch.float32)
    say(f"element CSR + bias of {bias_d.numel() * 4 / 2**30:.2f} GiB: n={n} window={w}")
    prob_np = gen.Problem(name="bias_2gib", B=1, H=H, n=n, d=d, dtype="bf16", q=q, k=k, v=v,
                          row_ptr=rp, col_idx=ci, scale=1 / np.sqrt(d), q_bits=bits[0],
                          k_bits=bits[1], v_bits=bits[2])
    dp = DevProblem(prob_np, plan=True)
    dp.bias = bias_d
    dp.prob = sa.Problem(1, H, n, d, sa.SA_BF16, dp.row_ptr, dp.col_idx, prob_np.nnz,
                         scale=prob_np.scale, bias=bias_d)
    dp.prob.set_plan(dp.plan)
    O, lse = dp.fused()
    rng2 = np.random.default_rng(1)
    sample = sorted(set([0, n - 1, n // 2, 23170, 23171] + rng2.integers(0, n, 60).tolist()))
    bias_rows = dict(zip(sample, bias_d[0, sample].cpu().numpy()))
    ref = oracle.attention_rows(q, k, v, prob_np.scale, H, ("csr", rp, ci), [(0, i) for i in sample],
                                bias=_SampledBiasRows(bias_rows))
    ref_o, ref_l = ref["O"], ref["lse"]
    report("bias_2gib", "fused_csr_plan", "context (sampled rows)",
           np.stack([O[0, i] for i in sample]), np.stack(ref_o), "bf16")
    report("bias_2gib", "fused_csr_plan", "lse (sampled rows)",
           np.array([lse[0, i] for i in sample]), np.array(ref_l), "bf16")
