"""GPU parity of the CSR pipeline's backward pass (gradients with respect to q, k, v).

The library's pieces run through the C ABI: the pattern transpose, SDDMM of dO with V,
the softmax gradient, per-entry gathers and SpMM over the pattern and its transpose. The
results are compared with the fp64 chain-rule oracle (oracle.backward.grads_csr, pinned in
test_oracle_backward_pins.py) at the forward's tolerances; the transposed pattern is
checked bit-exactly against a host sort. At the full Longformer-style size, where the
oracle's row loops are too slow, identities of the exact gradients are checked instead.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import masked_scaled_dot_amd as sa
from oracle import backward as obw
from gpu_util import DEV, DevProblem, check, say

pytestmark = pytest.mark.gpu


def _grad_out(p, seed):
    """dO in the problem's dtype (bf16 values are rounded once, and the oracle reads the
    same values widened)."""
    x = np.random.default_rng(seed).standard_normal((p.BH, p.n, p.d)).astype(np.float32)
    if p.dtype == "bf16":
        bits = gen.bf16_round_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV), gen.bf16_bits_to_f32(bits)
    return torch.from_numpy(x).to(DEV), x


def _host_transpose(row_ptr, col_idx, n):
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    order = np.lexsort((rows, col_idx))  # by column, then row
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, col_idx.astype(np.int64) + 1, 1)
    return np.cumsum(rp).astype(np.int32), rows[order].astype(np.int32), order.astype(np.int32)


class Backward:
    """The backward pass of the CSR pipeline, one C-ABI call per step."""

    def __init__(self, dp, plan=True):
        self.dp = dp
        p = dp.p
        self.nnz = p.nnz
        self.rpt = torch.empty(p.n + 1, dtype=torch.int32, device=DEV)
        self.cit = torch.empty(max(p.nnz, 1), dtype=torch.int32, device=DEV)
        self.perm = torch.empty(max(p.nnz, 1), dtype=torch.int32, device=DEV)
        ws = torch.empty(max(sa.sa_transpose_workspace_bytes(dp.prob), 1), dtype=torch.uint8, device=DEV)
        sa.sa_csr_transpose(dp.prob, self.rpt, self.cit[:p.nnz], self.perm[:p.nnz], ws)
        # the ordered gather runs with the plan, the plain one without: both take part
        self.order = None
        if plan and p.nnz:
            self.order = torch.empty(2 * p.nnz, dtype=torch.int32, device=DEV)
            sa.sa_gather_order_build(dp.prob, self.perm[:p.nnz], self.order, ws)
        dtype = sa.SA_BF16 if p.dtype == "bf16" else sa.SA_F32
        # dW = dO . v at the pattern: SDDMM at scale 1 without additive terms
        self.prob_dw = sa.Problem(p.B, p.H, p.n, p.d, dtype, dp.row_ptr, dp.col_idx, p.nnz, scale=1.0)
        self.prob_t = sa.Problem(p.B, p.H, p.n, p.d, dtype, self.rpt, self.cit[:p.nnz], p.nnz, scale=dp.scale)
        if plan:
            for prob in (self.prob_dw, self.prob_t):
                buf = torch.zeros((sa.sa_plan_bytes(prob) + 3) // 4, dtype=torch.int32, device=DEV)
                sa.sa_plan_build(prob, buf)
                prob.set_plan(buf)

    def run(self, W, dO):
        dp, p = self.dp, self.dp.p
        dW = torch.empty(p.BH * p.nnz, device=DEV)
        dS = torch.empty_like(dW)
        Wt, dSt = torch.empty_like(dW), torch.empty_like(dW)
        dQ, dK, dV = (torch.empty(p.BH, p.n, p.d, device=DEV) for _ in range(3))
        sa.sa_sddmm(self.prob_dw, dO, dp.v, dW)
        sa.sa_sparse_softmax_backward(dp.prob, W, dW, dp.scale, dS)
        sa.sa_spmm(dp.prob, dS, dp.k, dQ)
        if self.order is not None:
            sa.sa_gather_entries_ordered(dp.prob, self.order, dS, dSt, W, Wt)
        else:
            sa.sa_gather_entries(dp.prob, self.perm[:p.nnz], dS, dSt)
            sa.sa_gather_entries(dp.prob, self.perm[:p.nnz], W, Wt)
        sa.sa_spmm(self.prob_t, dSt, dp.q, dK)
        sa.sa_spmm(self.prob_t, Wt, dO, dV)
        got = dict(dW=dW, dS=dS, dQ=dQ, dK=dK, dV=dV)
        if dp.bias is not None:  # dS above carries the scale; the bias enters S unscaled
            got["dBias"] = torch.zeros(p.H, p.n, p.n, device=DEV)
            sa.sa_bias_grad(dp.prob, dS, 1.0 / dp.scale, got["dBias"])
        return got


def _element_csr(p):
    rp, ci = p.element_csr()
    return dataclasses.replace(p, row_ptr=rp.astype(np.int32), col_idx=ci.astype(np.int32), block=1)


def _forward_weights(dp):
    p = dp.p
    S = torch.empty(p.BH * p.nnz, device=DEV)
    W = torch.empty_like(S)
    sa.sa_sddmm(dp.prob, dp.q, dp.k, S)
    sa.sa_sparse_softmax(dp.prob, S, W)
    return W


CASES = {
    "window_f32": lambda: gen.make("window_n128"),
    "longformer_bf16": lambda: gen.make("longformer_n4096", n=700, H=3, window=40),
    "longformer_long_rows": lambda: gen.make("longformer_n4096", n=2500, H=2, window=100),
    "random_bf16": lambda: gen.make("random_n8192", n=1000, H=2, kmin=1, kmax=300),
    "random_bias_keymask": lambda: gen.make("random_n8192", n=300, H=2, B=2, kmin=1, kmax=120,
                                            bias=True, key_mask=True, pmax=40),
    # the Evoformer-style dense pattern with pair bias and key padding, as element CSR
    "evoformer_dense_bias": lambda: _element_csr(gen.make("evoformer_l384", B=3, H=2, n=96)),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("plan", [False, True], ids=["rows", "plan"])
def test_backward_parity(name, plan):
    p = CASES[name]()
    say(f"backward {name} plan={plan}: BH={p.BH} n={p.n} d={p.d} nnz={p.nnz} {p.dtype}")
    dp = DevProblem(p, plan=plan)
    bw = Backward(dp, plan=plan)
    torch.cuda.synchronize()
    rpt, cit, perm = _host_transpose(p.row_ptr, p.col_idx, p.n)
    assert np.array_equal(bw.rpt.cpu().numpy(), rpt)
    assert np.array_equal(bw.cit[:p.nnz].cpu().numpy(), cit)
    assert np.array_equal(bw.perm[:p.nnz].cpu().numpy(), perm)
    dO, dO_host = _grad_out(p, 11)
    W = _forward_weights(dp)
    got = bw.run(W, dO)
    torch.cuda.synchronize()
    ref = obw.grads_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, dp.scale, p.H, dO_host, **dp.oracle_args())
    check(got["dW"].view(p.BH, p.nnz).cpu().numpy(), ref["dW"], p.dtype, "dW")
    check(got["dS"].view(p.BH, p.nnz).cpu().numpy(), dp.scale * ref["dS"], p.dtype, "scale*dS")
    for g in ("dQ", "dK", "dV"):
        check(got[g].cpu().numpy(), ref[g], p.dtype, g)
    if "dBias" in got:
        check(got["dBias"].cpu().numpy(), ref["dBias"], p.dtype, "dBias")


ORDER_CASES = dict(CASES, longformer_full=lambda: gen.make("longformer_n4096"))


@pytest.mark.parametrize("name", sorted(ORDER_CASES))
def test_ordered_gather_equals_permutation(name):
    """The block read order: every block of 4096 transposed positions lists its sources
    ascending with a permutation of its slots, and the ordered gather (one array or two)
    equals dst[t, k] = src[t, perm[k]] bit for bit, including the ragged last block."""
    p = ORDER_CASES[name]()
    say(f"ordered gather {name}: BH={p.BH} nnz={p.nnz}")
    dp = DevProblem(p, plan=False)
    bw = Backward(dp, plan=True)
    nnz = p.nnz
    perm = bw.perm[:nnz].long()
    order = bw.order.cpu().numpy().astype(np.int64)
    src_o, slot = order[:nnz], order[nnz:]
    perm_h = perm.cpu().numpy()
    for b0 in range(0, nnz, 4096):
        b1 = min(nnz, b0 + 4096)
        assert np.all(np.diff(src_o[b0:b1]) > 0)
        assert np.array_equal(np.sort(slot[b0:b1]), np.arange(b1 - b0))
        assert np.array_equal(perm_h[b0 + slot[b0:b1]], src_o[b0:b1])
    g = torch.Generator(device=DEV).manual_seed(3)
    a = torch.randn(p.BH * nnz, device=DEV, generator=g)
    b = torch.randn(p.BH * nnz, device=DEV, generator=g)
    want_a = a.view(p.BH, nnz)[:, perm].reshape(-1)
    want_b = b.view(p.BH, nnz)[:, perm].reshape(-1)
    da, db = torch.full_like(a, float("nan")), torch.full_like(b, float("nan"))
    sa.sa_gather_entries_ordered(dp.prob, bw.order, a, da, b, db)
    torch.cuda.synchronize()
    assert torch.equal(da, want_a) and torch.equal(db, want_b)
    da.fill_(float("nan"))
    sa.sa_gather_entries_ordered(dp.prob, bw.order, b, da)
    plain = torch.full_like(a, float("nan"))
    sa.sa_gather_entries(dp.prob, bw.perm[:nnz], b, plain)
    torch.cuda.synchronize()
    assert torch.equal(da, want_b) and torch.equal(plain, want_b)


def test_backward_full_size_identities():
    """Longformer-style workload at full size (12 heads, n=4096): for the exact gradients,
    sum_j dS[i, j] = 0 on every row, sum_j dV[j] = sum_i dO[i] over rows with a finite
    score, and sum_i q_i . dQ_i = sum_j k_j . dK_j (both equal scale * sum dS[i,j] q_i . k_j)."""
    p = gen.make("longformer_n4096")
    say(f"backward identities longformer_n4096: BH={p.BH} nnz={p.nnz}")
    dp = DevProblem(p, plan=True)
    bw = Backward(dp, plan=True)
    dO, _ = _grad_out(p, 5)
    W = _forward_weights(dp)
    got = bw.run(W, dO)
    torch.cuda.synchronize()
    rp = torch.from_numpy(p.row_ptr.astype(np.int64)).to(DEV)
    rows = torch.repeat_interleave(torch.arange(p.n, device=DEV), rp[1:] - rp[:-1])
    dS = got["dS"].view(p.BH, p.nnz).double()
    row_sum = torch.zeros(p.BH, p.n, device=DEV, dtype=torch.float64).index_add_(1, rows, dS)
    assert float(row_sum.abs().max()) < 1e-4
    dV_sum = got["dV"].double().sum(dim=1)
    dO_sum = dO.double().sum(dim=1)  # every row of this pattern has finite scores
    assert float((dV_sum - dO_sum).abs().max()) < 1e-2
    lhs = (dp.q.double() * got["dQ"].double()).sum()
    rhs = (dp.k.double() * got["dK"].double()).sum()
    assert abs(float(lhs - rhs)) <= 1e-4 * max(1.0, abs(float(lhs)))


def test_backward_graph_replay_matches_eager():
    """The backward pass captured as one HIP graph (SDDMM, softmax gradient, SpMM, ordered
    gather, transposed SpMMs with their long-row merge counters): every replay, with eager
    work in between, reproduces the eager gradients bit for bit."""
    p = CASES["longformer_long_rows"]()
    say(f"backward graph replay: BH={p.BH} n={p.n} nnz={p.nnz}")
    dp = DevProblem(p, plan=True)
    bw = Backward(dp, plan=True)
    dO, _ = _grad_out(p, 13)
    W = _forward_weights(dp)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in bw.run(W, dO).items()}
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = bw.run(W, dO)
    for rep in range(3):
        for x in got.values():
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x in got.items():
            assert torch.equal(x, ref[name]), f"replay {rep}: {name} differs from the eager result"
        bw.run(W, dO)  # eager work between replays
