"""GPU parity: every entry point against the fp64 oracle, through the C ABI.

Small cases are compared element by element with the whole oracle output; they span
several tiles and a ragged tail. Full-size workloads are compared on sampled rows that
the oracle evaluates one by one, plus invariants over every row.
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


def _elementwise(p):
    """The same problem with its pattern expanded to element CSR (for the pipeline calls)."""
    if p.row_ptr is not None and p.block == 1:
        return p
    import copy
    rp, ci = p.element_csr()
    e = copy.copy(p)
    e.row_ptr, e.col_idx, e.block = rp.astype(np.int32), ci.astype(np.int32), 1
    return e


def _pattern(p):
    if p.row_ptr is None:
        return ("dense",)
    if p.block == 64:
        return ("bsr", p.row_ptr, p.col_idx, 64)
    return ("csr", p.row_ptr, p.col_idx)


def _empty_block_rows(p, rows):
    """p (a block-sparse pattern) with the given block-rows emptied."""
    import copy
    rp, ci = p.row_ptr.astype(np.int64), p.col_idx
    lens = np.diff(rp)
    keep = np.ones(len(ci), bool)
    for r in rows:
        keep[rp[r]:rp[r + 1]] = False
        lens[r] = 0
    e = copy.copy(p)
    e.col_idx = ci[keep].astype(np.int32)
    e.row_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return e


SMALL = {
    "window_n128_f32": lambda: gen.make("window_n128"),
    "window_f32_d64_ragged": lambda: gen.make("window_n128", n=131, d=64, H=2),
    "window_f32_d128": lambda: gen.make("window_n128", n=77, d=128, window=30),
    "longformer_bf16_d64": lambda: gen.make("longformer_n4096", n=700, H=3, window=40),
    "longformer_bf16_d32": lambda: gen.make("longformer_n4096", n=333, H=2, d=32, window=20),
    "longformer_bf16_d128": lambda: gen.make("longformer_n4096", n=257, H=2, d=128, window=60),
    "random_bf16_long_rows": lambda: gen.make("random_n8192", n=1000, H=2, kmin=1, kmax=900),
    "random_f32_d32": lambda: gen.make("random_n8192", n=500, H=2, d=32, dtype="f32", kmin=1, kmax=200),
    "bsr_bf16_d128_ragged": lambda: gen.make("bsr_n16384", n=64 * 6 + 21, H=2, extra=3),
    "bsr_bf16_d64": lambda: gen.make("bsr_n16384", n=64 * 8, H=2, d=64, extra=2),
    "bsr_f32_d32": lambda: gen.make("bsr_n16384", n=64 * 5, H=1, d=32, dtype="f32", extra=2),
    # block-rows 1 and 6 (the ragged last one) store no block: their outputs are zero
    "bsr_bf16_d32_empty_rows": lambda: _empty_block_rows(gen.make("bsr_n16384", n=64 * 6 + 5, H=2, d=32,
                                                                  extra=2), (1, 6)),
    "evoformer_bf16_odd": lambda: gen.make("evoformer_l384", B=3, H=2, n=97),
    "evoformer_bf16": lambda: gen.make("evoformer_l384", B=2, H=8, n=384),
    "evoformer_f32_d64": lambda: gen.make("evoformer_l384", B=2, H=2, n=130, d=64, dtype="f32"),
    "evoformer_bf16_d64": lambda: gen.make("evoformer_l384", B=2, H=2, n=130, d=64),
    "evoformer_bf16_d128_bias": lambda: gen.make("evoformer_l384", B=1, H=2, n=70, d=128, key_mask=False),
    "evoformer_bf16_d32_mask_only": lambda: gen.make("evoformer_l384", B=3, H=2, n=200, bias=False),
    "random_bias_keymask": lambda: gen.make("random_n8192", n=300, H=2, B=2, kmin=1, kmax=120,
                                            bias=True, key_mask=True, pmax=40),
    # rows longer than the plan's split threshold (1024 entries): global-token rows, random
    "longformer_long_rows": lambda: gen.make("longformer_n4096", n=2500, H=2, window=100),
    # the same with eight heads: each XCD's segment workgroups take the segments of its own heads
    "longformer_long_rows_8heads": lambda: gen.make("longformer_n4096", n=1300, H=8, window=60),
    "random_long_rows": lambda: gen.make("random_n8192", n=2100, H=2, kmin=1, kmax=1800),
    "longformer_bias_keymask": lambda: gen.make("longformer_n4096", n=600, H=2, B=2, window=50,
                                                bias=True, key_mask=True, pmax=100),
}


@functools.lru_cache(maxsize=None)
def small(name):
    return SMALL[name]()


@pytest.mark.parametrize("plan", [False, True], ids=["rows", "plan"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_pipeline_parity_small(name, plan):
    p = _elementwise(small(name))
    say(f"pipeline {name} plan={plan}: BH={p.BH} n={p.n} d={p.d} nnz={p.nnz} {p.dtype}")
    dp = DevProblem(p, plan=plan)
    S, W, O = dp.pipeline()
    ref = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H, **dp.oracle_args())
    check(S, ref["S"], p.dtype, "scores")
    check(W, ref["W"], p.dtype, "weights")
    refd = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, _pattern(small(name)),
                                  want_weights=False, **dp.oracle_args())
    check(O, refd["O"], p.dtype, "context")
    # the pattern and indices are the caller's and come back untouched, bit for bit
    assert np.array_equal(dp.row_ptr.cpu().numpy(), p.row_ptr)
    assert np.array_equal(dp.col_idx.cpu().numpy(), p.col_idx)


@pytest.mark.parametrize("plan", [False, True], ids=["rows", "plan"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_fused_parity_small(name, plan):
    p = small(name)
    if plan and (p.row_ptr is None or p.block != 1):
        pytest.skip("the row plan applies to element CSR only")
    say(f"fused {name} plan={plan}: BH={p.BH} n={p.n} d={p.d} block={p.block} dense={p.row_ptr is None}")
    dp = DevProblem(p, plan=plan)
    O, lse = dp.fused()
    ref = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, _pattern(p), want_weights=False,
                                 **dp.oracle_args())
    eo = check(O, ref["O"], p.dtype, "context")
    el = check(lse, ref["lse"], p.dtype, "lse")
    say(f"PARITY {name} fused{'_plan' if plan else ''} context max_abs={eo[0]:.3e} mean_abs={eo[1]:.3e}"
        f" lse max_abs={el[0]:.3e}")


def _extreme_problem(kind, d):
    import copy
    if kind == "bsr":  # block-rows of 1 to 6 blocks, the last one ragged
        n = 64 * 6 + 37
        base = gen.make("bsr_n16384", n=n, H=2, d=d, extra=0)
        rng = np.random.default_rng(77 + d)
        nb = (n + 63) // 64
        rows = [sorted(set(rng.choice(nb, size=int(rng.integers(1, 6)), replace=False).tolist() + [r]))
                for r in range(nb)]
        p = copy.copy(base)
        p.row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
        p.col_idx = np.concatenate([np.asarray(r, np.int32) for r in rows])
        return p, False
    if kind == "csr_plan":  # window + global tokens: banded matrix-core tiles and far columns
        return gen.make("longformer_n4096", n=64 * 5 + 11, H=2, d=d, window=40), True
    # dense, too long for the LDS-resident kernel at d = 128: the 64-query tile
    return gen.make("evoformer_l384", B=1, H=2, n=64 * 5 + 3, d=d, bias=False, key_mask=False), False


@pytest.mark.parametrize("kind,d", [("bsr", 32), ("bsr", 64), ("bsr", 128), ("csr_plan", 64),
                                    ("csr_plan", 128), ("dense", 128)])
@pytest.mark.parametrize("scale", [2.0, 0.02])
def test_fused_extreme_scales(kind, d, scale):
    """The matrix-core fused tiles under extreme score ranges: a large scale puts the scores
    of one row hundreds of log2 units apart (most weights underflow to 0, a row's weight sits
    on one key, the running maximum moves far past its lazy threshold from block to block), a
    tiny scale keeps every weight near 1."""
    p, plan = _extreme_problem(kind, d)
    dp = DevProblem(p, scale=scale, plan=plan)
    O, lse = dp.fused()
    ref = oracle.attention_dense(p.q, p.k, p.v, scale, p.H, _pattern(p), want_weights=False,
                                 **dp.oracle_args())
    eo = check(O, ref["O"], p.dtype, "context")
    el = check(lse, ref["lse"], p.dtype, "lse")
    say(f"PARITY extreme_scales {kind} d={d} scale={scale} context max_abs={eo[0]:.3e}"
        f" mean_abs={eo[1]:.3e} lse max_abs={el[0]:.3e}")


# element CSR patterns whose tiles are whole 64x64 blocks (expansions of block-sparse
# patterns): the fused forward with a plan computes such tiles as block-sparse tiles
BLOCKY = {
    "bsr_bf16_d128_ragged": lambda: small("bsr_bf16_d128_ragged"),
    "bsr_bf16_d64": lambda: small("bsr_bf16_d64"),
    "bsr_bf16_d32_bias_keymask": lambda: gen.make("bsr_n16384", n=64 * 5 + 9, H=2, B=2, d=32, extra=2,
                                                  bias=True, key_mask=True, pmax=50),
    "bsr_bf16_d64_bias": lambda: gen.make("bsr_n16384", n=64 * 7, H=2, d=64, extra=3, bias=True),
}


def _drop_entry(p, row):
    """p with the last entry of ``row`` removed (its tile is no longer whole blocks)."""
    import copy
    rp, ci = p.row_ptr.astype(np.int64), p.col_idx
    keep = np.ones(len(ci), bool)
    keep[rp[row + 1] - 1] = False
    e = copy.copy(p)
    e.col_idx = ci[keep].astype(np.int32)
    e.row_ptr = (rp - (np.arange(len(rp)) > row)).astype(np.int32)
    return e


@pytest.mark.parametrize("mixed", [False, True], ids=["whole", "one_tile_csr"])
@pytest.mark.parametrize("name", sorted(BLOCKY))
def test_fused_plan_whole_block_tiles(name, mixed):
    """Element expansion of a block-sparse pattern through the fused forward with a plan:
    whole-block tiles run as block-sparse tiles, the rest as CSR tiles; all against the
    oracle. ``one_tile_csr`` drops one entry of row 70, so tile 1 takes the CSR path."""
    pb = BLOCKY[name]()
    p = _elementwise(pb)
    if mixed:
        p = _drop_entry(p, 70)
    dp = DevProblem(p, plan=True)
    h = dp.plan.cpu().numpy()
    T = h[4]
    words = h[h[11]:h[11] + 8 * T].reshape(-1, 8)
    nblock = int((words[:, 5] > 0).sum())
    say(f"fused whole-block tiles {name} mixed={mixed}: n={p.n} d={p.d} tiles={T} block tiles={nblock}"
        f" bias={p.bias is not None} key_mask={p.key_mask is not None}")
    assert nblock >= 1
    if mixed:
        assert words[1, 5] == 0
    O, lse = dp.fused()
    ref = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, ("csr", p.row_ptr, p.col_idx),
                                 want_weights=False, **dp.oracle_args())
    eo = check(O, ref["O"], p.dtype, "context")
    el = check(lse, ref["lse"], p.dtype, "lse")
    say(f"PARITY {name}{'_mixed' if mixed else ''} fused_plan_blocks context max_abs={eo[0]:.3e}"
        f" mean_abs={eo[1]:.3e} lse max_abs={el[0]:.3e}")
    if not mixed:  # the same tiles through the block-sparse entry point
        O2, lse2 = DevProblem(pb).fused()
        check(O, O2, p.dtype, "context vs block-sparse call")


def test_fused_without_lse_and_scale_one():
    p = small("longformer_bf16_d64")
    dp = DevProblem(p, scale=1.0)
    O, _ = dp.fused(want_lse=False)
    ref = oracle.attention_dense(p.q, p.k, p.v, 1.0, p.H, _pattern(p), want_weights=False)
    check(O, ref["O"], p.dtype, "context scale=1")
    S, W, O2 = dp.pipeline()
    check(O2, ref["O"], p.dtype, "pipeline context scale=1")


# ------------------------------------------------------------------------------ edge cases

def _custom(rows, n, d, dtype, H=1, B=1, seed=5, key_mask=None):
    rp, ci = gen.csr_from_rows(rows)
    rng = np.random.default_rng(seed)
    qkv = []
    for _ in range(3):
        x = rng.standard_normal((B * H, n, d)).astype(np.float32)
        bits = gen.bf16_round_bits(x) if dtype == "bf16" else None
        qkv.append((gen.bf16_bits_to_f32(bits).reshape(x.shape) if bits is not None else x,
                    None if bits is None else bits.reshape(x.shape)))
    return gen.Problem(name="custom", B=B, H=H, n=n, d=d, dtype=dtype, q=qkv[0][0], k=qkv[1][0],
                       v=qkv[2][0], row_ptr=rp, col_idx=ci, scale=1 / np.sqrt(d),
                       key_mask=key_mask, q_bits=qkv[0][1], k_bits=qkv[1][1], v_bits=qkv[2][1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_and_fully_masked_rows(dtype):
    n, d = 70, 64
    rng = np.random.default_rng(3)
    rows = [sorted(rng.choice(n, size=int(rng.integers(1, 20)), replace=False).tolist())
            for _ in range(n)]
    for i in (0, 5, 69):
        rows[i] = []
    rows[7] = [3]                    # key 3 is masked for batch 1 -> row 7 fully masked there
    km = np.zeros((2, 1, n), np.float32)
    km[1, 0, 3] = -np.inf
    km[0, 0, 40:] = -np.inf
    p = _custom(rows, n, d, dtype, H=2, B=2, key_mask=km)
    dp = DevProblem(p)
    S, W, O = dp.pipeline()
    ref = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H, key_mask=km)
    check(S, ref["S"], dtype, "scores")
    check(W, ref["W"], dtype, "weights")
    check(O, ref["O"], dtype, "context")
    for t in range(p.BH):
        for i in (0, 5, 69):
            assert np.all(O[t, i] == 0)
    assert np.all(O[2:, 7] == 0) and np.all(W[2:, p.row_ptr[7]] == 0)
    Of, lse = dp.fused()
    check(Of, ref["O"], dtype, "fused context")
    check(lse, ref["lse"], dtype, "fused lse")
    assert lse[2, 7] == -np.inf and lse[0, 0] == -np.inf


@pytest.mark.parametrize("bias", [True, False], ids=["bias", "mask_only"])
@pytest.mark.parametrize("n,d", [(1000, 32), (600, 64)])
def test_dense_tile_skips_masked_key_blocks(n, d, bias):
    """Dense pattern with heads too large to keep in LDS (the tile kernel): key blocks whose
    key-mask values are all -inf are skipped -- an interior block, the padded tail, and a
    batch whose keys are all masked (its rows give O = 0 and lse = -inf)."""
    import dataclasses
    p = gen.make("evoformer_l384", B=3, H=2, n=n, d=d, bias=bias)
    km = np.zeros((3, 1, n), np.float32)
    km[0, 0, 128:192] = -np.inf        # one whole interior key block
    km[0, 0, 70:75] = -np.inf          # part of a block
    km[1, 0, n - 300:] = -np.inf       # a tail longer than four blocks
    km[2, 0, :] = -np.inf              # every key
    p = dataclasses.replace(p, key_mask=km, key_mask_heads=1)
    say(f"dense tile with masked key blocks: n={n} d={d} bias={bias}")
    dp = DevProblem(p)
    O, lse = dp.fused()
    ref = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, ("dense",), want_weights=False,
                                 **dp.oracle_args())
    eo = check(O, ref["O"], p.dtype, "context")
    el = check(lse, ref["lse"], p.dtype, "lse")
    assert np.all(O[4:6] == 0) and np.all(lse[4:6] == -np.inf)  # batch 2: heads 4 and 5
    say(f"PARITY dense_tile_masked_blocks_n{n}_d{d} fused context max_abs={eo[0]:.3e} mean_abs={eo[1]:.3e}"
        f" lse max_abs={el[0]:.3e}")


@pytest.mark.parametrize("bias", [True, False], ids=["bias", "mask_only"])
@pytest.mark.parametrize("n,d", [(384, 32), (200, 64)])
def test_dense_resident_skips_leading_key_blocks(n, d, bias):
    """Dense pattern whose heads fit in LDS: a key-padding mask hides all of key block 0 in
    batch 0 (the first visited block is block 1) and all of block 1 plus a few single keys in
    batch 1; batch 2 keeps every key. Context and lse match the oracle."""
    import dataclasses
    p = gen.make("evoformer_l384", B=3, H=2, n=n, d=d, bias=bias)
    km = np.zeros((3, 1, n), np.float32)
    km[0, 0, :64] = -np.inf
    km[0, 0, 100:131] = -np.inf
    km[1, 0, 64:128] = -np.inf
    km[1, 0, [3, 17, n - 1]] = -np.inf
    p = dataclasses.replace(p, key_mask=km, key_mask_heads=1)
    say(f"dense resident, leading key blocks masked: n={n} d={d} bias={bias}")
    dp = DevProblem(p)
    O, lse = dp.fused()
    ref = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, ("dense",), want_weights=False,
                                 **dp.oracle_args())
    eo = check(O, ref["O"], p.dtype, "context")
    el = check(lse, ref["lse"], p.dtype, "lse")
    say(f"PARITY dense_resident_leading_blocks_n{n}_d{d} fused context max_abs={eo[0]:.3e}"
        f" mean_abs={eo[1]:.3e} lse max_abs={el[0]:.3e}")


@pytest.mark.parametrize("n,d", [(384, 32), (200, 64), (97, 128)])
def test_dense_running_max_jumps(n, d):
    """Dense pattern with a pair bias that moves each row's maximum in steps across the 32-key
    units: a first unit hundreds below the rest (its exponentials underflow against any early
    reference), rises of 3-6 (under the slack the running maximum allows, but enough to lift
    a unit's sum of weights past it), and jumps of 12-60 in later units. Every step of the
    online softmax (first reference, no move, move and rescale) is taken; context and lse
    match the oracle."""
    import dataclasses
    p = gen.make("evoformer_l384", B=2, H=2, n=n, d=d)
    rng = np.random.default_rng(77)
    steps = np.array([-200.0, -5.0, 0.0, 3.0, 6.0, 12.0, 60.0])
    units = (n + 31) // 32
    shift = np.cumsum(rng.choice(steps, size=(p.H, n, units)), axis=2)
    shift[:, :, 0] = -300.0
    bias = p.bias + np.repeat(shift, 32, axis=2)[:, :, :n].astype(np.float32)
    p = dataclasses.replace(p, bias=bias.astype(np.float32))
    say(f"dense running-max jumps: n={n} d={d}")
    dp = DevProblem(p)
    O, lse = dp.fused()
    ref = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, ("dense",), want_weights=False,
                                 **dp.oracle_args())
    eo = check(O, ref["O"], p.dtype, "context")
    el = check(lse, ref["lse"], p.dtype, "lse")
    say(f"PARITY dense_running_max_jumps_n{n}_d{d} fused context max_abs={eo[0]:.3e} mean_abs={eo[1]:.3e}"
        f" lse max_abs={el[0]:.3e}")


TINY_N = [1, 2, 5, 31, 33, 63, 65]


@pytest.mark.parametrize("n", TINY_N)
def test_tiny_sizes(n):
    """Degenerate sizes, one case each through every path: the dense pattern with bias and key
    mask (resident kernel at d = 32, 64, 128; the vector path in fp32), a window pattern
    through the pipeline and the fused forward with and without a plan, and a block CSR of
    one ragged block-row."""
    cases = [("dense_d32", gen.make("evoformer_l384", B=2, H=2, n=n, pmax=n)),
             ("dense_d64", gen.make("evoformer_l384", B=1, H=2, n=n, d=64)),
             ("dense_d128", gen.make("evoformer_l384", B=1, H=1, n=n, d=128)),
             ("dense_f32", gen.make("evoformer_l384", B=1, H=2, n=n, dtype="f32")),
             ("window_bf16", gen.make("window_n128", n=n, H=2, d=64, dtype="bf16", window=3)),
             ("window_f32", gen.make("window_n128", n=n, H=1, window=3)),
             ("bsr", gen.make("bsr_n16384", n=n, H=2, d=64, extra=2))]
    for name, p in cases:
        say(f"tiny n={n} {name}")
        pat = _pattern(p)
        for plan in ((False, True) if p.row_ptr is not None and p.block == 1 else (False,)):
            dp = DevProblem(p, plan=plan)
            O, lse = dp.fused()
            ref = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, pat, want_weights=False,
                                         **dp.oracle_args())
            check(O, ref["O"], p.dtype, f"{name} fused context plan={plan}")
            check(lse, ref["lse"], p.dtype, f"{name} fused lse plan={plan}")
            if p.row_ptr is not None and p.block == 1:
                S, W, Op = dp.pipeline()
                refc = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H,
                                            **dp.oracle_args())
                check(W, refc["W"], p.dtype, f"{name} weights plan={plan}")
                check(Op, refc["O"], p.dtype, f"{name} pipeline context plan={plan}")


@pytest.mark.parametrize("name", ["longformer_long_rows", "random_long_rows"])
def test_plan_without_segment_room(name):
    """A plan sized for no long-row segments (sa_plan_bytes_segments(p, 0)) is built without
    them (header word 7 = 0); every kernel then computes the long rows whole, and the outputs
    still match the oracle."""
    p = small(name)
    dp = DevProblem(p)
    nbytes = sa.sa_plan_bytes_segments(dp.prob, 0)
    assert 0 < nbytes < sa.sa_plan_bytes(dp.prob)
    plan = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=DEV)
    sa.sa_plan_build(dp.prob, plan)
    dp.prob.set_plan(plan)
    dp.plan = plan
    hdr = plan[:16].cpu().numpy()
    assert hdr[7] == 0 and hdr[6] > 0, hdr  # segments counted but not written
    say(f"plan without segment room: {name} n={p.n} segments={hdr[6]}")
    S, W, O = dp.pipeline()
    ref = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H, **dp.oracle_args())
    check(S, ref["S"], p.dtype, "scores")
    check(W, ref["W"], p.dtype, "weights")
    check(O, ref["O"], p.dtype, "context")
    Of, lse = dp.fused()
    refd = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, _pattern(p), want_weights=False,
                                  **dp.oracle_args())
    check(Of, refd["O"], p.dtype, "fused context")
    check(lse, refd["lse"], p.dtype, "fused lse")


@pytest.mark.parametrize("kind", ["bsr", "dense_key_mask"])
def test_rows_beyond_the_lds_block_list(kind):
    """n = 33,280 (520 key blocks): more block-columns than the tile kernel keeps in LDS (512).
    Block CSR: block-row 0 holds all 520 blocks, block-row 1 the first and the last, the others
    their diagonal block. Dense with a key-padding mask: the list of visited key blocks does
    not fit either, and every block is visited. Rows sampled from each kind of block-row are
    compared with the oracle."""
    import copy
    n, nb = 33280, 520
    if kind == "bsr":
        base = gen.make("bsr_n16384", n=n, H=1, d=32, extra=0)
        rows = [list(range(nb)), [0, nb - 1]] + [[r] for r in range(2, nb)]
        p = copy.copy(base)
        p.row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
        p.col_idx = np.concatenate([np.asarray(r, np.int32) for r in rows])
        picks = [0, 31, 63, 64, 100, 127, 128, 20000, n - 1]
    else:
        p = gen.make("evoformer_l384", B=1, H=1, n=n, d=32, bias=False, pmax=200)
        picks = [0, 1, 16000, 33000, n - 1]
    say(f"rows beyond the LDS block list: {kind} n={n} nnz={p.nnz}")
    dp = DevProblem(p)
    O, lse = dp.fused()
    pairs = [(0, i) for i in picks]
    ref = oracle.attention_rows(p.q, p.k, p.v, p.scale, p.H, _pattern(p), pairs, **dp.oracle_args())
    check(O[0, picks], ref["O"], p.dtype, f"{kind} context")
    check(lse[0, picks], ref["lse"], p.dtype, f"{kind} lse")


def test_block_sparse_tiles_in_several_rounds():
    """Block CSR with more (head, block-row) tiles than the device runs at once (4500 tiles at
    n = 95,987, three heads: the tiles run in several rounds), whose block-rows cycle through
    every shape a tile can have: empty, one block, two blocks, 25 blocks, and 3-9 random ones;
    the last block is ragged. Rows sampled from each kind of block-row in every head are
    compared with the oracle; every row of an empty block-row must give O = 0 and lse = -inf."""
    import copy
    nb = 1500
    n = 64 * nb - 13
    base = gen.make("bsr_n16384", n=n, H=3, d=32, extra=0)
    rng = np.random.default_rng(2024)
    rows = []
    for r in range(nb):
        kind = r % 7
        if kind == 0 and r != nb - 1:
            cols = []
        elif kind == 1:
            cols = [r]
        elif kind == 2:
            cols = [max(r - 1, 0), r] if r > 0 else [0, 1]
        elif kind == 3:
            cols = rng.choice(nb, size=25, replace=False).tolist()
        else:
            cols = rng.choice(nb, size=int(rng.integers(3, 10)), replace=False).tolist() + [r]
        rows.append(sorted(set(cols)))
    p = copy.copy(base)
    p.row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    p.col_idx = np.concatenate([np.asarray(r, np.int32) for r in rows])
    say(f"block CSR, tiles in several rounds: n={n} H={p.H} block nnz={p.nnz}")
    dp = DevProblem(p)
    O, lse = dp.fused()
    picks = []
    for br in [0, 1, 2, 3, 4, 5, 6, 700, 701, 702, 703, 704, 1493, 1494, 1495, 1496, nb - 1]:
        picks += [64 * br, min(64 * br + 37, n - 1), min(64 * br + 63, n - 1)]
    pairs = [(t, i) for t in range(p.H) for i in picks]
    ref = oracle.attention_rows(p.q, p.k, p.v, p.scale, p.H, _pattern(p), pairs, **dp.oracle_args())
    got_o = np.stack([O[t, i] for t, i in pairs])
    got_l = np.array([lse[t, i] for t, i in pairs])
    eo = check(got_o, ref["O"], p.dtype, "context")
    el = check(got_l, ref["lse"], p.dtype, "lse")
    empty = np.concatenate([np.arange(64 * br, min(64 * br + 64, n)) for br in range(nb) if not rows[br]])
    assert np.all(O[:, empty] == 0) and np.all(lse[:, empty] == -np.inf)
    live = np.setdiff1d(np.arange(n), empty)
    assert np.all(np.isfinite(O[:, live])) and np.all(np.isfinite(lse[:, live]))
    say(f"PARITY bsr_tiles_in_several_rounds fused context max_abs={eo[0]:.3e} mean_abs={eo[1]:.3e}"
        f" lse max_abs={el[0]:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_diagonal_only_rows_are_exact(dtype):
    n, d = 300, 32
    p = _custom([[i] for i in range(n)], n, d, dtype, H=3)
    dp = DevProblem(p)
    S, W, O = dp.pipeline()
    assert np.array_equal(W, np.ones_like(W))
    assert np.array_equal(O, p.v)
    Of, lse = dp.fused()
    assert np.array_equal(Of, p.v)


def test_zero_queries_give_uniform_weights():
    p = _elementwise(small("random_bf16_long_rows"))
    dp = DevProblem(p)
    dp.q.zero_()
    S, W, O = dp.pipeline()
    lens = np.diff(p.row_ptr)
    row_of = np.repeat(np.arange(p.n), lens)
    np.testing.assert_allclose(W, np.broadcast_to(1.0 / lens[row_of], W.shape), rtol=2e-6, atol=0)
    assert np.all(S == 0)


@pytest.mark.parametrize("name", ["longformer_bf16_d64", "longformer_long_rows"])
def test_determinism_bitwise(name):
    p = _elementwise(small(name))
    for plan in (False, True):
        dp = DevProblem(p, plan=plan)
        a = dp.pipeline()
        b = dp.pipeline()
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        assert np.array_equal(dp.fused()[0], dp.fused()[0])


def test_softmax_alone_long_rows_and_infinities():
    rows_len = [0, 1, 3, 64, 65, 511, 512, 513, 1000, 4096, 5000, 0, 7]
    rows_len += [0] * (5001 - len(rows_len))          # a square (n, n) mask: n >= longest row
    rp = np.zeros(len(rows_len) + 1, np.int32)
    rp[1:] = np.cumsum(rows_len)
    nnz = int(rp[-1])
    BH = 3
    S = gen.random_scores(BH, nnz, seed=9, spread=4.0)
    S[0, rp[3]:rp[3] + 10] = -np.inf                  # part of a row masked
    S[1, rp[8]:rp[9]] = -np.inf                        # a whole long row masked
    S[2, rp[2]:rp[3]] = -np.inf                        # a whole short row masked
    n = len(rows_len)
    prob = sa.Problem(1, BH, n, 32, sa.SA_F32, torch.from_numpy(rp).to(DEV),
                      torch.zeros(nnz, dtype=torch.int32, device=DEV), nnz)
    s_dev = torch.from_numpy(S).to(DEV)
    w_dev = torch.full_like(s_dev, float("nan"))
    sa.sa_sparse_softmax(prob, s_dev, w_dev)
    ref = oracle.sparse_softmax(S, rp)
    check(w_dev.cpu().numpy(), ref, "f32", "softmax")
    sa.sa_sparse_softmax(prob, s_dev, s_dev)          # in place
    check(s_dev.cpu().numpy(), ref, "f32", "softmax in place")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 32), ("bf16", 128), ("f32", 128)])
def test_spmm_alone(dtype, d):
    p = _elementwise(gen.make("random_n8192", n=400, H=2, d=d, dtype=dtype, kmin=0 + 1, kmax=300))
    dp = DevProblem(p)
    Wn = gen.random_weights(p.BH, p.nnz, seed=11)
    w_dev = torch.from_numpy(Wn).to(DEV)
    out = torch.full((p.BH, p.n, p.d), float("nan"), device=DEV)
    sa.sa_spmm(dp.prob, w_dev, dp.v, out)
    ref = oracle.spmm(Wn, p.row_ptr, p.col_idx, p.v)
    # unnormalised weights in [0,1): compare relative to the row's weight mass
    got = out.cpu().numpy()
    mass = np.zeros((p.BH, p.n))
    for i in range(p.n):
        mass[:, i] = Wn[:, p.row_ptr[i]:p.row_ptr[i + 1]].sum(axis=1)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert np.all(np.abs(got - ref) <= tol * np.maximum(mass, 1.0)[:, :, None])


# ------------------------------------------------------------------------------ validation / plan

def test_validate_csr():
    p = small("longformer_bf16_d32")
    dp = DevProblem(p)
    assert sa.sa_validate_csr(dp.prob) == sa.SA_OK
    bad_cols = p.col_idx.copy()
    bad_cols[10], bad_cols[11] = bad_cols[11], bad_cols[10]          # unsorted row
    for rp, ci in ((p.row_ptr, bad_cols),
                   (p.row_ptr, np.where(np.arange(p.nnz) == 5, p.n + 3, p.col_idx).astype(np.int32)),
                   (np.where(np.arange(p.n + 1) == 50, p.row_ptr[52], p.row_ptr).astype(np.int32),
                    p.col_idx)):
        rp_d = torch.from_numpy(rp).to(DEV)
        ci_d = torch.from_numpy(ci).to(DEV)
        prob = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16, rp_d, ci_d, p.nnz, scale=p.scale)
        assert sa.sa_validate_csr(prob) == sa.SA_ERR_CSR
        probv = sa.Problem(p.B, p.H, p.n, p.d, sa.SA_BF16, rp_d, ci_d, p.nnz, scale=p.scale,
                           flags=sa.SA_FLAG_VALIDATE)
        scores = torch.empty(p.BH * p.nnz, device=DEV)
        with pytest.raises(sa.SaError) as ei:
            sa.sa_sddmm(probv, dp.q, dp.k, scores)
        assert ei.value.status == sa.SA_ERR_CSR
        # without validation a malformed CSR still runs without invalid accesses
        sa.sa_sddmm(prob, dp.q, dp.k, scores)
        torch.cuda.synchronize()


def _host_plan(p, BH, d):
    """The plan's contents computed on the host from its definition (core ranges, tiles,
    long-row segments)."""
    rp, ci, n = p.row_ptr.astype(np.int64), p.col_idx, p.n
    rows = np.zeros((n, 2), np.int64)
    for i in range(n):
        a, b = rp[i], rp[i + 1]
        L = b - a
        if 0 < L <= 1024:
            med, half = ci[(a + b) // 2], (L + 1) // 2
            lo = a + np.searchsorted(ci[a:b], med - half, "left")
            hi = a + np.searchsorted(ci[a:b], med + half, "right")
            rows[i] = lo, hi
        else:
            rows[i] = a, a
    tiles, fars, blks = [], [], []
    for t0 in range(0, n, 64):
        lo, hi, core, farcols, banded = None, None, 0, [], 1
        for i in range(t0, min(n, t0 + 64)):
            a, b = rp[i], rp[i + 1]
            if b - a > 1024:
                continue
            if rows[i, 1] > rows[i, 0]:
                c0, c1 = ci[rows[i, 0]], ci[rows[i, 1] - 1]
                lo = c0 if lo is None else min(lo, c0)
                hi = c1 if hi is None else max(hi, c1)
                core += rows[i, 1] - rows[i, 0]
                if c1 - c0 != rows[i, 1] - rows[i, 0] - 1:  # core columns not consecutive
                    banded = 0
            farcols += list(ci[a:rows[i, 0]]) + list(ci[rows[i, 1]:b])
        uniq = sorted(set(farcols))
        ok = len(farcols) <= 1024 and len(uniq) <= 64
        kb0, kb1 = (0, 0) if hi is None else (lo // 64, hi // 64 + 1)
        nblk = (kb1 - kb0) + (1 if uniq else 0)
        mfma = ok and nblk > 0 and kb1 - kb0 <= 12 and core + len(farcols) >= 0.25 * 64 * 64 * nblk
        blocks = _whole_blocks(rp, ci, n, t0)
        nbk = len(blocks) if blocks and not mfma else 0
        tiles.append((kb0, kb1, int(mfma), len(uniq) if ok else 0, banded, nbk, 0, 0))
        fars.append(uniq if ok else None)
        blks.append(blocks if nbk else None)
    segs = []
    lr = 0
    for i in range(n):
        a, b = rp[i], rp[i + 1]
        L = b - a
        if L > 1024:
            ns = -(-L // 256)
            for s_ in range(ns):
                segs.append((i, a + L * s_ // ns, a + L * (s_ + 1) // ns, lr, s_, ns, 0, 0))
            lr += 1
    return rows, np.array(tiles), fars, np.array(segs, dtype=np.int64).reshape(-1, 8), lr, blks


def _whole_blocks(rp, ci, n, t0):
    """Block-columns of tile t0 when its rows (at most 1024 entries each) all hold the same
    columns and these are whole 64-key blocks (the block that holds key n - 1 may be cut at
    n); else None."""
    lists = [ci[rp[i]:rp[i + 1]] for i in range(t0, min(n, t0 + 64))]
    first = lists[0]
    if len(first) == 0 or len(first) > 1024 or any(not np.array_equal(x, first) for x in lists):
        return None
    blocks = sorted(set(int(c) // 64 for c in first))
    full = np.concatenate([np.arange(64 * b, min(64 * b + 64, n)) for b in blocks])
    return blocks if np.array_equal(full, first) else None


@pytest.mark.parametrize("name", ["longformer_long_rows", "random_long_rows", "window_n128_f32",
                                  "bsr_bf16_d128_ragged"])
def test_plan_build_matches_host(name):
    p = _elementwise(small(name))
    dp = DevProblem(p)
    plan = dp.build_plan()
    torch.cuda.synchronize()
    h = plan.cpu().numpy().astype(np.int64)
    rows, tiles, fars, segs, L, blks = _host_plan(p, p.BH, p.d)
    assert h[0] == 0x53415032 and h[1] == p.n and h[2] == p.nnz and h[7] == 1
    assert h[4] == len(tiles) and h[5] == L and h[6] == len(segs)
    assert h[8] == p.BH and h[9] == p.d
    rows4 = np.zeros((p.n, 4), np.int64)
    rows4[:, :2] = rows
    rows4[:, 2] = [p.col_idx[lo] if hi > lo else 0 for lo, hi in rows]  # column of the first core entry
    assert h[10] == 16 and h[11] == 16 + 4 * p.n                   # offsets from n alone
    assert np.array_equal(h[h[10]:h[10] + 4 * p.n].reshape(-1, 4), rows4)
    T = len(tiles)
    assert np.array_equal(h[h[11]:h[11] + 8 * T].reshape(-1, 8), tiles)
    far_base = h[11] + 8 * T
    for ti, uniq in enumerate(fars):
        if uniq:
            assert list(h[far_base + 64 * ti:far_base + 64 * ti + len(uniq)]) == uniq
    # block records of a matrix-core tile: per key block and row, the first entry in the
    # block and the 64-bit mask of key slots present; the gathered block's slots are the
    # positions of the tile's far columns
    blk_base = h[11] + (8 + 64) * T
    per_tile = 13 * 64 * 4
    for ti in range(T):
        if tiles[ti, 5]:  # whole-block tile: its block-columns open its record space
            nbk = tiles[ti, 5]
            assert list(h[blk_base + per_tile * ti: blk_base + per_tile * ti + nbk]) == blks[ti]
        if not tiles[ti, 2]:
            continue
        kb0, kb1 = tiles[ti, 0], tiles[ti, 1]
        rec = h[blk_base + per_tile * ti: blk_base + per_tile * (ti + 1)].reshape(13, 64, 4)
        for r in range(64):
            i = ti * 64 + r
            if i >= p.n or p.row_ptr[i + 1] - p.row_ptr[i] > 1024:
                assert all(rec[j, r, 1] == 0 and rec[j, r, 2] == 0 for j in range(kb1 - kb0))
                continue
            lo, hi = rows[i]
            core = p.col_idx[lo:hi].astype(np.int64)
            for j in range(kb1 - kb0):
                k0 = (kb0 + j) * 64
                first = lo + int(np.searchsorted(core, k0))
                m = 0
                for c in core[(core >= k0) & (core < k0 + 64)]:
                    m |= 1 << int(c - k0)
                got = tuple(int(x) & 0xffffffff for x in rec[j, r])
                assert got == (first, m & 0xffffffff, m >> 32, 0), (ti, r, j)
            if fars[ti]:
                a, b = p.row_ptr[i], p.row_ptr[i + 1]
                far_cols = list(p.col_idx[a:lo]) + list(p.col_idx[hi:b])
                m = 0
                for c in far_cols:
                    m |= 1 << fars[ti].index(int(c))
                got = tuple(int(x) & 0xffffffff for x in rec[kb1 - kb0, r])
                aux = (lo - a) + 65536 * (hi - lo)
                assert got == (a, m & 0xffffffff, m >> 32, aux), (ti, r)
    if name == "longformer_long_rows":
        assert tiles[20, 2] == 1 and fars[20] == [0, 1]      # global-token columns gathered
        assert tiles[20, 4] == 1                             # window rows: banded
    if name == "bsr_bf16_d128_ragged":                       # every tile is whole blocks
        assert all(tiles[ti, 5] > 0 or tiles[ti, 2] == 1 for ti in range(T))
        assert sum(tiles[:, 5] > 0) == 5                     # the other two: matrix-core CSR
    assert np.array_equal(h[h[12]:h[12] + 8 * len(segs)].reshape(-1, 8), segs)
    assert np.all(h[h[13]:h[13] + L * p.BH] == 0)                       # merge counters
    assert h[15] * 4 <= plan.numel() * 4
    # a problem that carries the plan validates it when asked to
    dp.prob.c.flags = sa.SA_FLAG_VALIDATE
    S, W, O = dp.pipeline()
    ref = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H)
    check(O, ref["O"], p.dtype, "context with plan")
    # a plan built for fewer heads is refused under validation
    small_prob = sa.Problem(1, 1, p.n, p.d, dp.prob.c.dtype, dp.row_ptr, dp.col_idx, p.nnz)
    nb = sa.sa_plan_bytes(small_prob)
    pl = torch.zeros((nb + 3) // 4, dtype=torch.int32, device=DEV)
    sa.sa_plan_build(small_prob, pl)
    if p.BH > 1:
        dp.prob.set_plan(pl)
        with pytest.raises(sa.SaError) as ei:
            dp.pipeline()
        assert ei.value.status == sa.SA_ERR_WORKSPACE


def test_plan_serves_smaller_shapes():
    """A plan built for B*H = 2 heads of d = 64 serves, stream-ordered, a problem on the same
    pattern with one head of d = 32 (its split rows use the plan's scratch at the plan's
    stride); pipeline and fused forward match the oracle."""
    big = small("longformer_long_rows")
    assert big.BH == 2 and big.d == 64
    owner = DevProblem(big, plan=True)
    p = gen.make("longformer_n4096", n=big.n, H=1, d=32, window=100)
    assert np.array_equal(p.row_ptr, big.row_ptr) and np.array_equal(p.col_idx, big.col_idx)
    dp = DevProblem(p)
    dp.prob.set_plan(owner.plan)
    dp.plan = owner.plan
    S, W, O = dp.pipeline()
    ref = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H)
    check(W, ref["W"], p.dtype, "weights")
    check(O, ref["O"], p.dtype, "context")
    Of, lse = dp.fused()
    refd = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, _pattern(p), want_weights=False)
    check(Of, refd["O"], p.dtype, "fused context")
    check(lse, refd["lse"], p.dtype, "fused lse")


def test_two_streams_one_pattern_own_plans():
    """Two streams run the pipeline and the fused forward concurrently on the same pattern,
    each with a plan of its own (a plan's long-row merge state serves one call at a time):
    every result equals the stream-ordered one bit for bit."""
    p = _elementwise(small("longformer_long_rows"))  # rows split into segments
    dps = [DevProblem(p, plan=True) for _ in range(2)]
    ref = [x.copy() for x in dps[0].pipeline()] + [dps[0].fused(want_lse=True)[0].copy()]
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = []
    for dp, st in zip(dps, streams):
        outs.append((torch.empty(p.BH * p.nnz, device=DEV), torch.empty(p.BH * p.nnz, device=DEV),
                     torch.empty(p.BH, p.n, p.d, device=DEV), torch.empty(p.BH, p.n, p.d, device=DEV),
                     torch.empty(p.BH, p.n, device=DEV)))
    torch.cuda.synchronize()
    for rep in range(4):
        for dp, st, (S, W, O, Of, lse) in zip(dps, streams, outs):
            with torch.cuda.stream(st):
                sa.sa_sddmm(dp.prob, dp.q, dp.k, S)
                sa.sa_sparse_softmax(dp.prob, S, W)
                sa.sa_spmm(dp.prob, W, dp.v, O)
                sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, Of, lse)
    torch.cuda.synchronize()
    for S, W, O, Of, _ in outs:
        got = [S.view(p.BH, p.nnz).cpu().numpy(), W.view(p.BH, p.nnz).cpu().numpy(), O.cpu().numpy(),
               Of.cpu().numpy()]
        for what, g_, r_ in zip(("scores", "weights", "context", "fused"), got, ref):
            assert np.array_equal(g_, r_), what


# ------------------------------------------------------------------------------ full size

FULL = ["longformer_n4096", "random_n8192", "bsr_n16384", "evoformer_l384"]


@functools.lru_cache(maxsize=2)
def full(name):
    return gen.make(name)


def _sample_rows(p, k=40, seed=0):
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (0, 1), (p.BH - 1, p.n - 1), (p.BH // 2, p.n // 2)}
    while len(pairs) < k:
        pairs.add((int(rng.integers(p.BH)), int(rng.integers(p.n))))
    return sorted(pairs)


@pytest.mark.parametrize("name", FULL[:3])
def test_full_size_pipeline_sampled(name):
    p = full(name)
    pe = _elementwise(p)
    say(f"full pipeline {name}: BH={p.BH} n={p.n} nnz/head={pe.nnz}")
    dp = DevProblem(pe, plan=True)
    S, W, O = dp.pipeline()
    pairs = _sample_rows(p)
    ref = oracle.attention_rows(p.q, p.k, p.v, p.scale, p.H, _pattern(p), pairs)
    got_o = np.stack([O[t, i] for t, i in pairs])
    check(got_o, ref["O"], p.dtype, "context (sampled rows)")
    got_w = np.concatenate([W[t, pe.row_ptr[i]:pe.row_ptr[i + 1]] for t, i in pairs])
    check(got_w, np.concatenate(ref["W"]), p.dtype, "weights (sampled rows)")
    # every row of every head: weights are nonnegative and sum to one
    assert np.all(W >= 0)
    sums = np.add.reduceat(W.astype(np.float64), pe.row_ptr[:-1], axis=1)
    assert np.abs(sums - 1.0).max() < 1e-5


@pytest.mark.parametrize("name", FULL)
def test_full_size_fused_sampled(name):
    p = full(name)
    say(f"full fused {name}: BH={p.BH} n={p.n} block={p.block}")
    dp = DevProblem(p)
    O, lse = dp.fused()
    pairs = _sample_rows(p)
    ref = oracle.attention_rows(p.q, p.k, p.v, p.scale, p.H, _pattern(p), pairs,
                                **dp.oracle_args())
    check(np.stack([O[t, i] for t, i in pairs]), ref["O"], p.dtype, "context (sampled rows)")
    check(np.array([lse[t, i] for t, i in pairs]), ref["lse"], p.dtype, "lse (sampled rows)")
    assert np.all(np.isfinite(O))


@pytest.mark.parametrize("name", ["longformer_long_rows", "random_bias_keymask"])
def test_graph_replay_matches_eager(name):
    """The pipeline and the fused forward captured as one HIP graph: every replay, with eager
    work and synchronisations in between, reproduces the eager results bit for bit (the long-row
    merge counters in the plan return to zero after each call)."""
    p = _elementwise(small(name))
    say(f"graph replay {name}: BH={p.BH} n={p.n} nnz={p.nnz}")
    dp = DevProblem(p, plan=True)
    ref = [x.copy() for x in dp.pipeline()] + [dp.fused(want_lse=True)[0].copy()]
    scores = torch.empty(p.BH * p.nnz, device=DEV)
    weights = torch.empty_like(scores)
    out = torch.empty(p.BH, p.n, p.d, device=DEV)
    fused = torch.empty_like(out)
    lse = torch.empty(p.BH, p.n, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.sa_sddmm(dp.prob, dp.q, dp.k, scores)
        sa.sa_sparse_softmax(dp.prob, scores, weights)
        sa.sa_spmm(dp.prob, weights, dp.v, out)
        sa.sa_fused_forward(dp.prob, dp.q, dp.k, dp.v, fused, lse)
    for rep in range(3):
        for x in (scores, weights, out, fused):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [scores.view(p.BH, p.nnz).cpu().numpy(), weights.view(p.BH, p.nnz).cpu().numpy(),
               out.cpu().numpy(), fused.cpu().numpy()]
        for what, g_, r_ in zip(("scores", "weights", "context", "fused"), got, ref):
            assert np.array_equal(g_, r_), f"replay {rep}: {what} differs from the eager result"
        dp.pipeline()  # eager work between replays
