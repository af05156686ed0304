"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a library routine for a special
case, a closed form, the pages' own worked mask example, an invariant of the
softmax, or brute force on tiny inputs. ``test_planted_mistakes_are_caught``
plants plausible mistakes in copies of the oracle and checks that a pin fails.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import csr as ocsr
from oracle import dense as odense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale, attn_mask=None):
    """torch's library SDPA in fp64 on the CPU (math path)."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    m = None if attn_mask is None else torch.from_numpy(np.ascontiguousarray(attn_mask))
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, scale=scale).numpy()


def _random_csr(n, rng, pmin=1, pmax=None, diag=True):
    pmax = n if pmax is None else pmax
    rows = []
    for i in range(n):
        k = int(rng.integers(pmin, pmax + 1))
        cols = rng.choice(n, size=min(k, n), replace=False)
        if diag:
            cols = np.union1d(cols, [i])
        rows.append(np.sort(cols))
    return gen.csr_from_rows(rows)


# --------------------------------------------------------------------------- library special cases

@pytest.mark.parametrize("n", [4, 64, 128, 256])
def test_all_ones_mask_equals_library_sdpa(n):
    """An all-ones mask without bias is plain softmax attention."""
    BH, d = 3, 16
    q, k, v = _rand((BH, n, d), 1), _rand((BH, n, d), 2), _rand((BH, n, d), 3)
    scale = 1.0 / math.sqrt(d)
    ref = _sdpa(q, k, v, scale)
    out = oracle.attention_dense(q, k, v, scale, BH, ("dense",), chunk=37)
    np.testing.assert_allclose(out["O"], ref, rtol=0, atol=1e-12)
    rp, ci = gen.expand_pattern(None, None, n, 1)
    out2 = oracle.attention_csr(q, k, v, rp, ci, scale, BH)
    np.testing.assert_allclose(out2["O"], ref, rtol=0, atol=1e-12)
    # weights equal torch's softmax of the score matrix
    Wref = torch.softmax(torch.from_numpy(scale * q @ k.transpose(0, 2, 1)), dim=-1).numpy()
    np.testing.assert_allclose(out2["W"].reshape(BH, n, n), Wref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.stack([out["W"][t] for t in range(BH)]).reshape(BH, n, n),
                               Wref, rtol=0, atol=1e-13)


def test_boolean_pattern_equals_library_sdpa():
    """A CSR pattern acts as SDPA's boolean attn_mask (True = attend); q != k, non-symmetric."""
    n, d, BH = 97, 8, 2
    rng = np.random.default_rng(7)
    rp, ci = _random_csr(n, rng, 1, 30)
    q, k, v = _rand((BH, n, d), 11), _rand((BH, n, d), 12), _rand((BH, n, d), 13)
    P = odense.pattern_rows(("csr", rp, ci), 0, n, n)
    assert not np.array_equal(P, P.T)
    ref = _sdpa(q, k, v, 0.3, attn_mask=np.broadcast_to(P, (BH, n, n)))
    out = oracle.attention_dense(q, k, v, 0.3, BH, ("csr", rp, ci), chunk=16)
    np.testing.assert_allclose(out["O"], ref, rtol=0, atol=1e-12)
    out2 = oracle.attention_csr(q, k, v, rp, ci, 0.3, BH)
    np.testing.assert_allclose(out2["O"], ref, rtol=0, atol=1e-12)


def test_bias_and_key_mask_equal_library_additive_mask():
    """Additive bias [1,H,n,n] and key mask [B,1,1,n] broadcast as the PR's shape lists say;
    SDPA's float attn_mask is added to scale*q.k^T."""
    B, H, n, d = 3, 2, 40, 8
    q, k, v = _rand((B * H, n, d), 21), _rand((B * H, n, d), 22), _rand((B * H, n, d), 23)
    bias = _rand((H, n, n), 24)
    km = np.zeros((B, 1, n))
    km[0, 0, 35:] = -np.inf
    km[1, 0, [3, 17, 30]] = -np.inf
    add = bias[None, :, :, :] + km[:, :, None, :]             # [B, H, n, n]
    ref = _sdpa(q.reshape(B, H, n, d), k.reshape(B, H, n, d), v.reshape(B, H, n, d), 0.25,
                attn_mask=add).reshape(B * H, n, d)
    out = oracle.attention_dense(q, k, v, 0.25, H, ("dense",), bias=bias, key_mask=km, chunk=9)
    np.testing.assert_allclose(out["O"], ref, rtol=0, atol=1e-12)
    rp, ci = gen.expand_pattern(None, None, n, 1)
    out2 = oracle.attention_csr(q, k, v, rp, ci, 0.25, H, bias=bias, key_mask=km)
    np.testing.assert_allclose(out2["O"], ref, rtol=0, atol=1e-12)
    # per-head key mask (head dim H): different keys masked per head
    kmh = np.zeros((B, H, n))
    kmh[:, 1, :5] = -np.inf
    add = bias[None] + kmh[:, :, None, :]
    ref = _sdpa(q.reshape(B, H, n, d), k.reshape(B, H, n, d), v.reshape(B, H, n, d), 0.25,
                attn_mask=add).reshape(B * H, n, d)
    out = oracle.attention_dense(q, k, v, 0.25, H, ("dense",), bias=bias, key_mask=kmh, km_heads=H)
    np.testing.assert_allclose(out["O"], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- closed forms

def test_hand_4x4_exact_rationals():
    """Tridiagonal mask, n=4, d=1, scale=1, q_i=1, k_j=ln(j+1), v_j=j+1: exp(s_ij) = j+1,
    so each row's weights are (j+1)/sum and the context is sum (j+1)^2 / sum (j+1)."""
    n = 4
    rows = [[0, 1], [0, 1, 2], [1, 2, 3], [2, 3]]
    rp, ci = gen.csr_from_rows(rows)
    q = np.ones((1, n, 1))
    k = np.log(np.arange(1, n + 1, dtype=np.float64)).reshape(1, n, 1)
    v = np.arange(1, n + 1, dtype=np.float64).reshape(1, n, 1)
    W_exp, O_exp = [], []
    for cols in rows:
        tot = sum(Fraction(j + 1) for j in cols)
        W_exp += [Fraction(j + 1) / tot for j in cols]
        O_exp.append(sum(Fraction((j + 1) ** 2) for j in cols) / tot)
    assert [float(x) for x in O_exp] == pytest.approx([5 / 3, 7 / 3, 29 / 9, 25 / 7], abs=1e-15)
    for out in (oracle.attention_csr(q, k, v, rp, ci, 1.0, 1),
                oracle.attention_dense(q, k, v, 1.0, 1, ("csr", rp, ci))):
        W = out["W"][0] if isinstance(out["W"], dict) else out["W"][0]
        np.testing.assert_allclose(W, [float(x) for x in W_exp], rtol=0, atol=1e-15)
        np.testing.assert_allclose(out["O"][0, :, 0], [float(x) for x in O_exp], rtol=0, atol=1e-14)
        # lse_i = log sum_j (j+1)
        np.testing.assert_allclose(out["lse"][0], [math.log(3), math.log(6), math.log(9), math.log(7)],
                                   rtol=0, atol=1e-14)


def test_hand_4x4_bf16_twin():
    """Same mask with k_j = j (exact in bf16), q_i = 1: W_ij = e^j / sum e^j'."""
    rows = [[0, 1], [0, 1, 2], [1, 2, 3], [2, 3]]
    rp, ci = gen.csr_from_rows(rows)
    q = np.ones((1, 4, 1)); k = np.arange(4.0).reshape(1, 4, 1); v = np.arange(1, 5.0).reshape(1, 4, 1)
    out = oracle.attention_csr(q, k, v, rp, ci, 1.0, 1)
    W = []
    for cols in rows:
        z = sum(math.exp(j) for j in cols)
        W += [math.exp(j) / z for j in cols]
    np.testing.assert_allclose(out["W"][0], W, rtol=0, atol=1e-15)


def _read_golden_masks():
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, "p4_msa_mask_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line[1:-1]
                blocks[cur] = []
                continue
            blocks[cur].append([float(x) for x in line.split()])
    return {k: np.array(v) for k, v in blocks.items()}


@pytest.mark.parametrize("name", ["mas_mask", "mas_mask_transposed"])
def test_pages_key_mask_example(name):
    """The PR's minimal MSA mask example used as key-padding masks [B,1,1,L] with Q = 0:
    every finite key gets weight 1/(number of finite keys), fully masked rows give 0."""
    M = _read_golden_masks()[name]                 # [B, L]
    B, L = M.shape
    d = 3
    q = np.zeros((B, L, d))
    k = _rand((B, L, d), 31)
    v = _rand((B, L, d), 32)
    km = M[:, None, :]
    out = oracle.attention_dense(q, k, v, 1.0, 1, ("dense",), key_mask=km)
    rp, ci = gen.expand_pattern(None, None, L, 1)
    out2 = oracle.attention_csr(q, k, v, rp, ci, 1.0, 1, key_mask=km)
    for b in range(B):
        fin = np.isfinite(M[b])
        cnt = fin.sum()
        for i in range(L):
            w = out["W"][b][i * L:(i + 1) * L]
            w2 = out2["W"][b, i * L:(i + 1) * L]
            exp_w = np.where(fin, 1.0 / cnt, 0.0) if cnt else np.zeros(L)
            np.testing.assert_allclose(w, exp_w, rtol=0, atol=1e-15)
            np.testing.assert_allclose(w2, exp_w, rtol=0, atol=1e-15)
            exp_o = v[b][fin].mean(axis=0) if cnt else np.zeros(d)
            np.testing.assert_allclose(out["O"][b, i], exp_o, rtol=0, atol=1e-14)
            np.testing.assert_allclose(out2["O"][b, i], exp_o, rtol=0, atol=1e-14)
            assert (out["lse"][b, i] == -np.inf) == (cnt == 0)
    if name == "mas_mask":
        # first sequence: the three finite keys share the weight equally
        np.testing.assert_allclose(out["W"][0][:6], [1 / 3, 1 / 3, 1 / 3, 0, 0, 0], atol=1e-15)


def test_scale_zero_gives_uniform_weights_and_mean_context():
    n, d, BH = 50, 5, 2
    rng = np.random.default_rng(41)
    rp, ci = _random_csr(n, rng, 1, 12)
    q, k, v = _rand((BH, n, d), 42), _rand((BH, n, d), 43), _rand((BH, n, d), 44)
    out = oracle.attention_csr(q, k, v, rp, ci, 0.0, BH)
    outd = oracle.attention_dense(q, k, v, 0.0, BH, ("csr", rp, ci))
    for i in range(n):
        a, e = rp[i], rp[i + 1]
        np.testing.assert_allclose(out["W"][:, a:e], 1.0 / (e - a), rtol=0, atol=1e-15)
        np.testing.assert_allclose(out["O"][:, i], v[:, ci[a:e]].mean(axis=1), rtol=0, atol=1e-14)
        np.testing.assert_allclose(outd["O"][:, i], v[:, ci[a:e]].mean(axis=1), rtol=0, atol=1e-14)
        np.testing.assert_allclose(out["lse"][:, i], math.log(e - a), rtol=0, atol=1e-14)


def test_diagonal_only_rows_copy_v():
    n, d, BH = 20, 4, 3
    rp, ci = gen.csr_from_rows([[i] for i in range(n)])
    q, k, v = _rand((BH, n, d), 51), _rand((BH, n, d), 52), _rand((BH, n, d), 53)
    for out in (oracle.attention_csr(q, k, v, rp, ci, 0.7, BH),
                oracle.attention_dense(q, k, v, 0.7, BH, ("csr", rp, ci))):
        W = out["W"] if not isinstance(out["W"], dict) else np.stack([out["W"][t] for t in range(BH)])
        assert np.array_equal(W, np.ones((BH, n)))
        assert np.array_equal(out["O"], v)


# --------------------------------------------------------------------------- invariants

def test_rows_sum_to_one_nonnegative_and_pattern_kept():
    p = gen.make("random_n8192", n=300, H=2, kmin=3, kmax=40)
    out = oracle.attention_csr(p.q, p.k, p.v, p.row_ptr, p.col_idx, p.scale, p.H)
    W = out["W"]
    assert W.shape == (p.BH, p.nnz)
    assert (W >= 0).all()
    for i in range(p.n):
        a, e = p.row_ptr[i], p.row_ptr[i + 1]
        np.testing.assert_allclose(W[:, a:e].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # the dense evaluation's weights, read at the CSR's stored positions, are the same values
    outd = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, ("csr", p.row_ptr, p.col_idx), chunk=64)
    for t in range(p.BH):
        np.testing.assert_allclose(outd["W"][t], W[t], rtol=0, atol=1e-13)
        # and are zero everywhere outside the pattern: total mass per row is 1 on the pattern
        assert outd["W"][t].shape == (p.nnz,)


def test_shift_invariance_through_bias():
    """Adding a per-row constant (here +1000, which would overflow exp without the max
    subtraction) through the bias leaves the weights unchanged."""
    n, d, H = 30, 4, 2
    q, k, v = _rand((H, n, d), 61), _rand((H, n, d), 62), _rand((H, n, d), 63)
    rng = np.random.default_rng(64)
    rp, ci = _random_csr(n, rng, 2, 9)
    bias = _rand((H, n, n), 65)
    shift = np.full((H, n, 1), 1000.0) + np.arange(n).reshape(1, n, 1)
    a = oracle.attention_csr(q, k, v, rp, ci, 0.5, H, bias=bias)
    b = oracle.attention_csr(q, k, v, rp, ci, 0.5, H, bias=bias + shift)
    np.testing.assert_allclose(b["W"], a["W"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["O"], a["O"], rtol=0, atol=1e-12)
    c = oracle.attention_dense(q, k, v, 0.5, H, ("csr", rp, ci), bias=bias + shift)
    np.testing.assert_allclose(c["O"], a["O"], rtol=0, atol=1e-12)


def test_empty_and_fully_masked_rows_convention():
    n, d = 6, 2
    rows = [[0, 1], [], [2], [0, 3, 5], [], [5]]
    rp, ci = gen.csr_from_rows(rows)
    q, k, v = _rand((1, n, d), 71), _rand((1, n, d), 72), _rand((1, n, d), 73)
    km = np.zeros((1, 1, n)); km[0, 0, 5] = -np.inf                  # row 5 fully masked
    for out in (oracle.attention_csr(q, k, v, rp, ci, 1.0, 1, key_mask=km),
                oracle.attention_dense(q, k, v, 1.0, 1, ("csr", rp, ci), key_mask=km)):
        W = out["W"] if not isinstance(out["W"], dict) else out["W"][0][None]
        for i in (1, 4, 5):
            assert np.array_equal(out["O"][0, i], np.zeros(d))
            assert out["lse"][0, i] == -np.inf
        assert W[0, rp[5]] == 0.0                                     # stored but masked entry
        assert W[0, rp[3] + 2] == 0.0                                 # key 5 inside row 3
        np.testing.assert_allclose(W[0, rp[3]:rp[3] + 2].sum(), 1.0, atol=1e-15)


# --------------------------------------------------------------------------- brute force

def _brute(q, k, v, scale, rows, bias=None, km=None, H=1):
    """Pure-Python loops with math.exp, straight from the definition."""
    BH, n, d = len(q), len(q[0]), len(q[0][0])
    O = [[[0.0] * d for _ in range(n)] for _ in range(BH)]
    W = [[] for _ in range(BH)]
    for t in range(BH):
        b, h = divmod(t, H)
        for i in range(n):
            s = []
            for j in rows[i]:
                x = scale * sum(q[t][i][c] * k[t][j][c] for c in range(d))
                if bias is not None:
                    x += bias[h][i][j]
                if km is not None:
                    x += km[b][0][j]
                s.append(x)
            fin = [x for x in s if x != -math.inf]
            if not fin:
                W[t] += [0.0] * len(s)
                continue
            m = max(fin)
            e = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
            z = sum(e)
            w = [x / z for x in e]
            W[t] += w
            for c in range(d):
                O[t][i][c] = sum(w[r] * v[t][j][c] for r, j in enumerate(rows[i]))
    return np.array(W), np.array(O)


def test_brute_force_tiny():
    B, H, n, d = 2, 2, 7, 3
    rng = np.random.default_rng(81)
    rows = [sorted(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False).tolist())
            for _ in range(n)]
    rows[3] = []
    rp, ci = gen.csr_from_rows(rows)
    q, k, v = _rand((B * H, n, d), 82), _rand((B * H, n, d), 83), _rand((B * H, n, d), 84)
    bias = _rand((H, n, n), 85)
    km = np.zeros((B, 1, n)); km[1, 0, [0, 4]] = -np.inf
    Wb, Ob = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, rows, bias.tolist(), km.tolist(), H)
    out = oracle.attention_csr(q, k, v, rp, ci, 0.6, H, bias=bias, key_mask=km)
    np.testing.assert_allclose(out["W"], Wb, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["O"], Ob, rtol=0, atol=1e-14)
    outd = oracle.attention_dense(q, k, v, 0.6, H, ("csr", rp, ci), bias=bias, key_mask=km, chunk=3)
    np.testing.assert_allclose(np.stack([outd["W"][t] for t in range(B * H)]), Wb, rtol=0, atol=1e-14)
    np.testing.assert_allclose(outd["O"], Ob, rtol=0, atol=1e-14)
    # sampled rows give the same rows
    pairs = [(0, 0), (3, 6), (2, 3), (1, 5)]
    r = oracle.attention_rows(q, k, v, 0.6, H, ("csr", rp, ci), pairs, bias=bias, key_mask=km)
    for x, (t, i) in enumerate(pairs):
        np.testing.assert_allclose(r["O"][x], Ob[t, i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["W"][x], Wb[t, rp[i]:rp[i + 1]], rtol=0, atol=1e-14)


def test_bsr_pattern_by_definition():
    """BSR: (i, j) is attended iff block (i // 64, j // 64) is stored; ragged last block."""
    rng = np.random.default_rng(91)
    n = 64 * 4 + 21
    brp, bci = gen.bsr_pattern(n, 2, rng)
    P = odense.pattern_rows(("bsr", brp, bci, 64), 0, n, n)
    stored = {(br, int(bc)) for br in range(len(brp) - 1) for bc in bci[brp[br]:brp[br + 1]]}
    for i in range(0, n, 5):
        for j in range(n):
            assert P[i, j] == ((i // 64, j // 64) in stored)
    q, k, v = _rand((2, n, 8), 92), _rand((2, n, 8), 93), _rand((2, n, 8), 94)
    rp, ci = gen.expand_pattern(brp, bci, n, 64)
    a = oracle.attention_dense(q, k, v, 0.3, 2, ("bsr", brp, bci, 64), chunk=50)
    b = oracle.attention_csr(q, k, v, rp, ci, 0.3, 2)
    np.testing.assert_allclose(a["O"], b["O"], rtol=0, atol=1e-13)
    for t in range(2):
        np.testing.assert_allclose(a["W"][t], b["W"][t], rtol=0, atol=1e-13)


def test_chunking_does_not_change_the_dense_oracle():
    p = gen.make("longformer_n4096", n=260, H=2, window=9)
    pat = ("csr", p.row_ptr, p.col_idx)
    a = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, pat, chunk=260)
    b = oracle.attention_dense(p.q, p.k, p.v, p.scale, p.H, pat, chunk=17)
    np.testing.assert_allclose(a["O"], b["O"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- planted mistakes

def _pins_pass(mod_patch, monkeypatch):
    """Run a subset of pins with a patched oracle; return True when all of them pass."""
    with monkeypatch.context() as m:
        mod_patch(m)
        try:
            test_all_ones_mask_equals_library_sdpa(64)
            test_boolean_pattern_equals_library_sdpa()
            test_bias_and_key_mask_equal_library_additive_mask()
            test_hand_4x4_exact_rationals()
            test_shift_invariance_through_bias()
            test_brute_force_tiny()
            test_empty_and_fully_masked_rows_convention()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return False
    return True


def _mut_sddmm_scale_on_bias(m):
    orig = ocsr.sddmm

    def bad(q, k, rp, ci, scale, H, bias=None, key_mask=None, km_heads=1):
        b2 = None if bias is None else bias * scale          # scale also applied to the bias
        return orig(q, k, rp, ci, scale, H, b2, key_mask, km_heads)
    m.setattr(ocsr, "sddmm", bad)
    m.setattr(oracle, "attention_csr", lambda *a, **kw: _compose(bad, *a, **kw))


def _mut_sddmm_swap_qk(m):
    orig = ocsr.sddmm

    def bad(q, k, rp, ci, scale, H, bias=None, key_mask=None, km_heads=1):
        return orig(k, q, rp, ci, scale, H, bias, key_mask, km_heads)   # k_i . q_j instead
    m.setattr(oracle, "attention_csr", lambda *a, **kw: _compose(bad, *a, **kw))


def _mut_softmax_no_max(m):
    def bad(S, rp, return_lse=False):
        S = np.asarray(S, dtype=np.float64)
        W = np.zeros_like(S); lse = np.full((S.shape[0], len(rp) - 1), -np.inf)
        with np.errstate(over="raise"):
            for i in range(len(rp) - 1):
                a, e = rp[i], rp[i + 1]
                if a == e:
                    continue
                x = np.exp(S[:, a:e]); W[:, a:e] = x / x.sum(axis=1, keepdims=True)
                lse[:, i] = np.log(x.sum(axis=1))
        return (W, lse) if return_lse else W
    m.setattr(ocsr, "sparse_softmax", bad)
    m.setattr(oracle, "attention_csr", lambda *a, **kw: _compose(ocsr.sddmm, *a, softmax=bad, **kw))


def _mut_spmm_transposed_index(m):
    def bad(W, rp, ci, v):
        BH, n, d = v.shape
        O = np.zeros((BH, n, d))
        for i in range(n):
            a, e = rp[i], rp[i + 1]
            O[:, i] = np.einsum("tj,td->td", W[:, a:e], v[:, i])      # uses v_i, not v_col
        return O
    m.setattr(oracle, "attention_csr", lambda *a, **kw: _compose(ocsr.sddmm, *a, spmm_fn=bad, **kw))


def _mut_dense_keymask_by_head(m):
    orig = odense._additive

    def bad(bias, key_mask, km_heads, H, t, i0, i1):
        b, h = divmod(t, H)
        return orig(bias, key_mask, km_heads, H, (t % H) * H + b, i0, i1) if key_mask is not None \
            else orig(bias, key_mask, km_heads, H, t, i0, i1)
    m.setattr(odense, "_additive", bad)


def _mut_empty_row_nan(m):
    def bad(S):
        m_ = S.max(axis=1, keepdims=True)
        with np.errstate(invalid="ignore"):
            E = np.exp(S - m_)
            l = E.sum(axis=1, keepdims=True)
            return E / l, (m_ + np.log(l))[:, 0]
    m.setattr(odense, "_softmax_rows", bad)


def _compose(sddmm_fn, q, k, v, rp, ci, scale, H, bias=None, key_mask=None, km_heads=1,
             softmax=None, spmm_fn=None):
    S = sddmm_fn(q, k, rp, ci, scale, H, bias, key_mask, km_heads)
    W, lse = (softmax or ocsr.sparse_softmax)(S, rp, return_lse=True)
    O = (spmm_fn or ocsr.spmm)(W, rp, ci, v)
    return {"S": S, "W": W, "O": O, "lse": lse}


@pytest.mark.parametrize("mutation", [_mut_sddmm_scale_on_bias, _mut_sddmm_swap_qk,
                                      _mut_softmax_no_max, _mut_spmm_transposed_index,
                                      _mut_dense_keymask_by_head, _mut_empty_row_nan])
def test_planted_mistakes_are_caught(mutation, monkeypatch):
    assert _pins_pass(lambda m: None, monkeypatch), "pins must pass on the unmodified oracle"
    assert not _pins_pass(mutation, monkeypatch), f"{mutation.__name__} went unnoticed"
