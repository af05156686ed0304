"""GPU parity of mask construction: COO -> CSR, key mask from key lengths, and the pattern
of packed variable-length batches, against oracle.mask (pinned in test_oracle_mask_pins.py).

Patterns and key masks are integer / exact results and are compared bit for bit. At full
size the COO input is a generated pattern scattered back as shuffled pairs with repeats
and pairs outside the matrix, so the expected CSR is the generator's own. A packed batch is
also run through the pipeline and the fused forward and compared with the oracle's
attention over the same pattern.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import masked_scaled_dot_amd as sa
from oracle import dense as odense
from oracle import mask as omask
from gpu_util import DEV, DevProblem, check, say

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def _coo_to_csr(n, rows, cols):
    nnz = len(rows)
    R, C = _i32(rows), _i32(cols)
    row_ptr = torch.full((n + 1,), -7, dtype=torch.int32, device=DEV)
    col_idx = torch.full((max(nnz, 1),), -7, dtype=torch.int32, device=DEV)
    counts = torch.full((3,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(sa.sa_mask_workspace_bytes(n, nnz), 1), dtype=torch.uint8, device=DEV)
    sa.sa_coo_to_csr(n, R, C, row_ptr, col_idx[:nnz], counts, ws)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy()
    return rp, col_idx.cpu().numpy()[:rp[-1]], tuple(counts.cpu().numpy().tolist())


def _small_coo(seed, n, nnz, lo=-3, hi=None):
    rng = np.random.default_rng(seed)
    hi = n + 3 if hi is None else hi
    return rng.integers(lo, hi, nnz), rng.integers(lo, hi, nnz)


SMALL = {
    "hand": (4, [2, 0, 2, 5, 0, 1, -1, 2], [1, 3, 1, 0, 0, 2, 1, 0]),
    "random_dups": (1000, *_small_coo(1, 1000, 20000)),
    "dense_small": (37, *_small_coo(2, 37, 5000)),  # nearly every pair, many repeats
    "all_outside": (10, [10, -1, 11], [0, 3, 99]),
    "empty": (5, [], []),
    "one_row": (1, [0, 0, 0, 1], [0, 0, 0, 0]),
    "no_rows": (0, [0, 1], [0, 0]),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_coo_to_csr_small(name):
    n, rows, cols = SMALL[name]
    say(f"coo_to_csr {name}: n={n} pairs={len(rows)}")
    got = _coo_to_csr(n, np.asarray(rows), np.asarray(cols))
    want = omask.coo_to_csr(n, rows, cols)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])
    assert got[2] == tuple(want[2])


@pytest.mark.parametrize("name", ["longformer_n4096", "random_n8192"])
def test_coo_to_csr_full_size_round_trip(name):
    p = gen.make(name, H=1)
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    cols = p.col_idx.astype(np.int64)
    rng = np.random.default_rng(9)
    extra = rng.integers(0, len(rows), 100_000)
    R = np.concatenate([rows, rows[extra], [-1, p.n, 5]])
    C = np.concatenate([cols, cols[extra], [0, 0, p.n]])
    order = rng.permutation(len(R))
    say(f"coo_to_csr round trip {name}: n={p.n} pairs={len(R)}")
    rp, ci, counts = _coo_to_csr(p.n, R[order], C[order])
    assert np.array_equal(rp, p.row_ptr)
    assert np.array_equal(ci, p.col_idx)
    assert counts == (len(rows), 3, 100_000)


def test_key_mask_from_lengths():
    lens = np.array([0, 1, 383, 384, 500, -4, 200], np.int32)
    B, n = len(lens), 384
    km = torch.full((B, n), float("nan"), device=DEV)
    sa.sa_key_mask_from_lengths(B, n, _i32(lens), km)
    torch.cuda.synchronize()
    assert np.array_equal(km.cpu().numpy(), omask.key_mask_from_lengths(lens, n))


def test_key_mask_from_lengths_reproduces_the_padding_mask():
    """The key-padding mask of the Evoformer-style workload (the last p_b keys masked) is
    exactly the mask of the lengths n - p_b, and the fused forward gives the same bits."""
    p = gen.make("evoformer_l384", B=4, H=2)
    lens = np.isfinite(p.key_mask[:, 0, :]).sum(axis=1).astype(np.int32)
    assert np.array_equal(p.key_mask[:, 0, :], omask.key_mask_from_lengths(lens, p.n))
    km = torch.empty((p.B, 1, p.n), device=DEV)
    sa.sa_key_mask_from_lengths(p.B, p.n, _i32(lens), km)
    dp = DevProblem(p)
    ref, ref_lse = dp.fused()
    dp2 = DevProblem(p)
    dp2.key_mask = km
    dp2.prob = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16, None, None, 0, scale=p.scale,
                          bias=dp2.bias, key_mask=km, key_mask_heads=1)
    got, got_lse = dp2.fused()
    assert np.array_equal(got, ref) and np.array_equal(got_lse, ref_lse)


VARLEN = {
    "full": ([0, 5, 6, 14, 14, 300, 301, 700], 700, -1),
    "window": ([0, 200, 260, 700, 1000], 1000, 16),
    "trailing_tokens": ([0, 64, 100], 130, -1),
    "one_sequence": ([0, 513], 513, -1),
}


def _varlen(cu, total, window):
    cu_d = _i32(cu)
    B = len(cu) - 1
    row_ptr = torch.full((total + 1,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(sa.sa_mask_workspace_bytes(total, 0), dtype=torch.uint8, device=DEV)
    sa.sa_varlen_row_ptr(B, total, cu_d, window, row_ptr, ws)
    nnz = int(row_ptr[total].item())
    col_idx = torch.full((max(nnz, 1),), -7, dtype=torch.int32, device=DEV)
    sa.sa_varlen_col_idx(B, total, cu_d, window, row_ptr, col_idx[:nnz])
    torch.cuda.synchronize()
    return row_ptr.cpu().numpy(), col_idx.cpu().numpy()[:nnz]


@pytest.mark.parametrize("name", sorted(VARLEN))
def test_varlen_pattern(name):
    cu, total, window = VARLEN[name]
    say(f"varlen {name}: total={total} sequences={len(cu) - 1} window={window}")
    rp, ci = _varlen(cu, total, window)
    want_rp, want_ci = omask.varlen_csr(cu, total, window)
    assert np.array_equal(rp, want_rp)
    assert np.array_equal(ci, want_ci)


@pytest.mark.parametrize("name", ["full", "window"])
def test_varlen_attention(name):
    """A packed batch (B = 1, n = total tokens) through the pipeline and the fused forward,
    against the oracle's attention over the same pattern."""
    cu, total, window = VARLEN[name]
    rp, ci = _varlen(cu, total, window)
    p = gen.make("longformer_n4096", n=total, H=2)
    p = dataclasses.replace(p, row_ptr=rp, col_idx=ci)
    say(f"varlen attention {name}: total={total} nnz={p.nnz}")
    ref = odense.attention_dense(p.q, p.k, p.v, p.scale, p.H, ("csr", rp, ci))
    for plan in (False, True):
        dp = DevProblem(p, plan=plan)
        _, W, O = dp.pipeline()
        check(O, ref["O"], p.dtype, f"pipeline O plan={plan}")
        Of, lse = dp.fused()
        check(Of, ref["O"], p.dtype, f"fused O plan={plan}")
        check(lse, ref["lse"], p.dtype, f"fused lse plan={plan}")


# ---- key lengths read by the kernels (sa_problem.seqlen_k)

def _with_lengths(dp, lens, use_key_mask=True):
    p = dp.p
    sl = _i32(lens)
    km = dp.key_mask if use_key_mask else None
    dp.prob = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16 if p.dtype == "bf16" else sa.SA_F32,
                         dp.row_ptr, dp.col_idx, p.nnz, block=p.block, scale=dp.scale,
                         bias=dp.bias, key_mask=km, key_mask_heads=p.key_mask_heads,
                         seqlen_k=sl)
    if dp.plan is not None:
        dp.prob.set_plan(dp.plan)
    return dp


def _oracle_with_lengths(p, lens, use_key_mask=True):
    km = omask.key_mask_from_lengths(lens, p.n)[:, None, :]
    if use_key_mask and p.key_mask is not None:
        km = km + p.key_mask  # both masks apply
    return odense.attention_dense(p.q, p.k, p.v, p.scale, p.H, _pattern(p), bias=p.bias,
                                  key_mask=km, km_heads=1)


def _pattern(p):
    if p.row_ptr is None:
        return ("dense",)
    if p.block == 64:
        return ("bsr", p.row_ptr, p.col_idx, 64)
    return ("csr", p.row_ptr, p.col_idx)


SEQLEN = {
    # name: (problem, lengths per batch, keep the generator's key mask too)
    "dense_bias": (lambda: gen.make("evoformer_l384", B=5, H=2), [384, 0, 1, 200, 320], False),
    "dense_bias_and_mask": (lambda: gen.make("evoformer_l384", B=3, H=2), [300, 64, 384], True),
    "dense_ragged_n": (lambda: gen.make("evoformer_l384", B=2, H=2, n=200), [130, 200], False),
    "dense_f32": (lambda: gen.make("evoformer_l384", B=2, H=2, n=160, dtype="f32"), [100, 7], False),
    "bsr": (lambda: gen.make("bsr_n16384", n=640, H=2, d=64, extra=3), [500], False),
    # lengths that end in the first key half of a block (its second half all masked), at a
    # block boundary, inside the ragged last block, and 0
    "bsr_d128_half_blocks": (lambda: gen.make("bsr_n16384", n=64 * 6 + 21, H=2, B=4, d=128, extra=3),
                             [340, 320, 400, 0], False),
    "bsr_d32_half_blocks": (lambda: gen.make("bsr_n16384", n=64 * 5, H=1, B=2, d=32, extra=2), [275, 1], False),
    "csr": (lambda: gen.make("longformer_n4096", n=700, H=2, window=40), [650], False),
    "csr_with_key_mask": (lambda: gen.make("random_n8192", n=300, H=2, B=2, kmin=1, kmax=120,
                                           bias=True, key_mask=True, pmax=40), [250, 299], True),
    # a global-token column past the length: the plan's far columns (the gathered block and
    # the few-columns epilogue) must mask it
    "csr_far_cols_past_length": (lambda: gen.make("longformer_n4096", n=700, H=2, window=40,
                                                  global_tokens=(0, 1, 690)), [650], False),
    # rows longer than the plan's split threshold (segments) with a length
    "csr_long_rows": (lambda: gen.make("longformer_n4096", n=2500, H=2, window=100), [1800], False),
    # the element expansion of a block pattern (the plan's whole-block tiles)
    "csr_whole_blocks": (lambda: _element(gen.make("bsr_n16384", n=640, H=2, d=64, extra=3)), [500], False),
}


def _element(p):
    import copy
    rp, ci = p.element_csr()
    e = copy.copy(p)
    e.row_ptr, e.col_idx, e.block = rp.astype(np.int32), ci.astype(np.int32), 1
    return e


@pytest.mark.parametrize("plan", [False, True], ids=["rows", "plan"])
@pytest.mark.parametrize("name", sorted(SEQLEN))
def test_seqlen_k_fused(name, plan):
    make, lens, keep_km = SEQLEN[name]
    p = make()
    if plan and (p.row_ptr is None or p.block != 1):
        pytest.skip("plans are for element CSR")
    say(f"seqlen_k fused {name} plan={plan}: B={p.B} H={p.H} n={p.n} lens={lens}")
    dp = _with_lengths(DevProblem(p, plan=plan), lens, keep_km)
    ref = _oracle_with_lengths(p, lens, keep_km)
    O, lse = dp.fused()
    check(O, ref["O"], p.dtype, "O")
    check(lse, ref["lse"], p.dtype, "lse")


@pytest.mark.parametrize("plan", [False, True], ids=["rows", "plan"])
@pytest.mark.parametrize("name", ["csr", "csr_with_key_mask", "csr_far_cols_past_length", "csr_long_rows"])
def test_seqlen_k_pipeline(name, plan):
    """SDDMM reads the key lengths (masked scores are exactly -inf); softmax and SpMM then
    need nothing more."""
    make, lens, keep_km = SEQLEN[name]
    p = make()
    say(f"seqlen_k pipeline {name} plan={plan}: B={p.B} H={p.H} n={p.n} lens={lens}")
    dp = _with_lengths(DevProblem(p, plan=plan), lens, keep_km)
    ref = _oracle_with_lengths(p, lens, keep_km)
    S, W, O = dp.pipeline()
    check(O, ref["O"], p.dtype, "O")
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    for t in range(p.BH):
        masked = p.col_idx >= lens[t // p.H]
        assert np.all(S[t][masked] == -np.inf) and np.all(W[t][masked] == 0)
    assert rows.size == p.nnz


def test_seqlen_k_dense_equals_key_mask_vector():
    """The Evoformer-style workload's key padding given as lengths instead of its mask
    vector: the dense tiles skip the blocks past the length and give the same result."""
    p = gen.make("evoformer_l384", B=4, H=2)
    lens = np.isfinite(p.key_mask[:, 0, :]).sum(axis=1).astype(np.int32)
    ref_O, ref_lse = DevProblem(p).fused()
    got_O, got_lse = _with_lengths(DevProblem(p), lens, use_key_mask=False).fused()
    np.testing.assert_allclose(got_O, ref_O, atol=1e-6, rtol=0)
    np.testing.assert_allclose(got_lse, ref_lse, atol=1e-6, rtol=0)


# ---- masks generated from scores: the k largest of every row

def _topk(S, k):
    n = S.shape[0]
    kk = max(0, min(k, n))
    Sd = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).to(DEV)
    rp = torch.full((n + 1,), -7, dtype=torch.int32, device=DEV)
    ci = torch.full((max(n * kk, 1),), -7, dtype=torch.int32, device=DEV)
    sa.sa_topk_mask(n, k, Sd, rp, ci[:n * kk])
    torch.cuda.synchronize()
    return rp.cpu().numpy(), ci.cpu().numpy()[:n * kk]


def _topk_case(name):
    seeds = {"normal": 1, "ties": 2, "specials": 3, "k_past_n": 4, "k_zero": 5, "one_row": 6,
             "ragged_n": 7, "empty": 8}
    rng = np.random.default_rng(seeds[name])
    if name == "normal":
        return rng.standard_normal((300, 300)).astype(np.float32), 17
    if name == "ties":
        return rng.integers(0, 6, (200, 200)).astype(np.float32), 50
    if name == "specials":
        S = rng.standard_normal((64, 64)).astype(np.float32)
        pick = rng.random(S.shape)
        S[pick < 0.1] = np.nan
        S[(pick >= 0.1) & (pick < 0.2)] = -np.inf
        S[(pick >= 0.2) & (pick < 0.25)] = np.inf
        S[(pick >= 0.25) & (pick < 0.35)] = -0.0
        S[(pick >= 0.35) & (pick < 0.45)] = 0.0
        return S, 10
    if name == "k_past_n":
        return rng.standard_normal((33, 33)).astype(np.float32), 40
    if name == "k_zero":
        return rng.standard_normal((20, 20)).astype(np.float32), 0
    if name == "one_row":
        return np.array([[2.5]], np.float32), 1
    if name == "empty":
        return np.zeros((0, 0), np.float32), 4
    if name == "ragged_n":
        return rng.standard_normal((777, 777)).astype(np.float32), 100
    raise KeyError(name)


@pytest.mark.parametrize("name", ["normal", "ties", "specials", "k_past_n", "k_zero", "one_row", "ragged_n",
                                  "empty"])
def test_topk_mask(name):
    S, k = _topk_case(name)
    say(f"topk {name}: n={S.shape[0]} k={k}")
    rp, ci = _topk(S, k)
    want_rp, want_ci = omask.topk_rows(S, k)
    assert np.array_equal(rp, want_rp)
    assert np.array_equal(ci, want_ci)


def test_topk_mask_full_size_sampled_rows_and_attention():
    """n = 4096, k = 256 from bf16-rounded q.k scores of one head: sampled rows bit-exact
    against the oracle, every row sorted and of k distinct columns, and attention over the
    generated mask (pipeline with a plan) against the oracle's on sampled rows."""
    p = gen.make("longformer_n4096", H=1)
    S = (p.q[0].astype(np.float64) @ p.k[0].astype(np.float64).T).astype(np.float32)
    rp, ci = _topk(S, 256)
    rows = np.random.default_rng(1).choice(p.n, 24, replace=False)
    want_rp, want_ci = omask.topk_rows(S[rows], 256)
    got = np.concatenate([ci[256 * r:256 * r + 256] for r in rows])
    assert np.array_equal(got, want_ci)
    C = ci.reshape(p.n, 256)
    assert np.all(np.diff(C, axis=1) > 0) and C.min() >= 0 and C.max() < p.n
    assert np.array_equal(rp, np.arange(p.n + 1) * 256)
    pt = dataclasses.replace(p, row_ptr=rp.astype(np.int32), col_idx=ci.astype(np.int32))
    dp = DevProblem(pt, plan=True)
    _, W, O = dp.pipeline()
    pairs = [(0, int(r)) for r in rows]
    ref = odense.attention_rows(pt.q, pt.k, pt.v, pt.scale, pt.H, ("csr", pt.row_ptr, pt.col_idx), pairs)
    check(np.stack([O[t, i] for t, i in pairs]), ref["O"], pt.dtype, "context (sampled rows)")
