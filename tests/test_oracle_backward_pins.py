"""Pins of the fp64 backward oracle (gradients with respect to q, k, v).

What fixes the expected values: central finite differences of the forward definition
(oracle.dense, itself pinned in test_oracle_pins.py), torch's library SDPA with autograd
for the full mask, and invariants of the softmax gradient. The two evaluations in
oracle.backward (chain rule on the CSR, torch autograd of the dense definition) are
also checked against each other, and planted mistakes must make a pin fail.
"""
import numpy as np
import pytest
import torch

from oracle import backward as obw
from oracle import csr as ocsr
from oracle import dense as odense


def _csr_from_mask(P):
    row_ptr = np.zeros(P.shape[0] + 1, np.int32)
    cols = []
    for i in range(P.shape[0]):
        c = np.nonzero(P[i])[0]
        cols.append(c)
        row_ptr[i + 1] = row_ptr[i] + len(c)
    return row_ptr, (np.concatenate(cols) if cols else np.zeros(0)).astype(np.int32)


def _case(seed, B=1, H=2, n=6, d=4, density=0.5, bias=True, key_mask=True, empty_row=True):
    rng = np.random.default_rng(seed)
    BH = B * H
    q, k, v, dO = (rng.standard_normal((BH, n, d)) for _ in range(4))
    P = rng.random((n, n)) < density
    P[np.arange(n), np.arange(n)] = True
    if empty_row:
        P[n // 2] = False
    row_ptr, col_idx = _csr_from_mask(P)
    b = rng.standard_normal((H, n, n)) if bias else None
    km = None
    if key_mask:
        km = np.zeros((B, 1, n))
        km[:, :, -1] = -np.inf  # the last key masked for every batch
    return q, k, v, dO, row_ptr, col_idx, b, km


def _loss(q, k, v, dO, row_ptr, col_idx, scale, H, b, km):
    O = odense.attention_dense(q, k, v, scale, H, ("csr", row_ptr, col_idx), bias=b, key_mask=km,
                               want_weights=False)["O"]
    return float((O * dO).sum())


def _finite_difference(q, k, v, dO, row_ptr, col_idx, scale, H, b, km, h=1e-6):
    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        it = np.nditer(g, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = args[which][idx]
            args[which][idx] = orig + h
            fp = _loss(*args, dO, row_ptr, col_idx, scale, H, b, km)
            args[which][idx] = orig - h
            fm = _loss(*args, dO, row_ptr, col_idx, scale, H, b, km)
            args[which][idx] = orig
            g[idx] = (fp - fm) / (2 * h)
        out.append(g)
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_finite_differences(seed):
    q, k, v, dO, rp, ci, b, km = _case(seed)
    scale = 0.7
    fd = _finite_difference(q, k, v, dO, rp, ci, scale, 2, b, km)
    g = obw.grads_csr(q, k, v, rp, ci, scale, 2, dO, bias=b, key_mask=km)
    a = obw.grads_autograd(q, k, v, scale, 2, ("csr", rp, ci), dO, bias=b, key_mask=km)
    for name, ref in zip(("dQ", "dK", "dV"), fd):
        np.testing.assert_allclose(g[name], ref, atol=1e-7, rtol=1e-6, err_msg=name)
        np.testing.assert_allclose(a[name], ref, atol=1e-7, rtol=1e-6, err_msg=name)


@pytest.mark.parametrize("seed", [0, 1])
def test_bias_gradient_matches_finite_differences(seed):
    """dBias sums dS over the batches (the bias is shared by them); checked entry by entry
    against central differences of the forward, inside and outside the pattern."""
    q, k, v, dO, rp, ci, b, km = _case(seed, B=2, n=5, d=3)
    scale = 0.6
    g = obw.grads_csr(q, k, v, rp, ci, scale, 2, dO, bias=b, key_mask=km)
    a = obw.grads_autograd(q, k, v, scale, 2, ("csr", rp, ci), dO, bias=b, key_mask=km)
    h = 1e-6
    fd = np.zeros_like(b)
    for idx in np.ndindex(*b.shape):
        bp, bm = b.copy(), b.copy()
        bp[idx] += h
        bm[idx] -= h
        fd[idx] = (_loss(q, k, v, dO, rp, ci, scale, 2, bp, km) -
                   _loss(q, k, v, dO, rp, ci, scale, 2, bm, km)) / (2 * h)
    np.testing.assert_allclose(g["dBias"], fd, atol=1e-7, rtol=1e-6)
    np.testing.assert_allclose(a["dBias"], fd, atol=1e-7, rtol=1e-6)
    assert np.any(fd != 0)


def test_full_mask_equals_library_sdpa_gradients():
    rng = np.random.default_rng(7)
    BH, n, d = 3, 20, 8
    q, k, v, dO = (rng.standard_normal((BH, n, d)) for _ in range(4))
    scale = 1.0 / np.sqrt(d)
    rp, ci = _csr_from_mask(np.ones((n, n), bool))
    g = obw.grads_csr(q, k, v, rp, ci, scale, 1, dO)
    Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
    (O * torch.tensor(dO)).sum().backward()
    for name, t in (("dQ", Q), ("dK", K), ("dV", V)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), atol=1e-12, rtol=1e-10, err_msg=name)


def test_chain_rule_equals_autograd_on_a_larger_pattern():
    q, k, v, dO, rp, ci, b, km = _case(3, B=2, H=2, n=40, d=8, density=0.2)
    g = obw.grads_csr(q, k, v, rp, ci, 0.3, 2, dO, bias=b, key_mask=km)
    a = obw.grads_autograd(q, k, v, 0.3, 2, ("csr", rp, ci), dO, bias=b, key_mask=km)
    for name in ("dQ", "dK", "dV", "dBias"):
        np.testing.assert_allclose(g[name], a[name], atol=1e-12, rtol=1e-10, err_msg=name)
    np.testing.assert_allclose(g["O"], a["O"], atol=1e-12)


def test_softmax_gradient_rows_sum_to_zero_and_vanish_on_empty_rows():
    q, k, v, dO, rp, ci, b, km = _case(5, n=30, d=6, density=0.3)
    g = obw.grads_csr(q, k, v, rp, ci, 0.5, 2, dO, bias=b, key_mask=km)
    for i in range(30):
        a, e = rp[i], rp[i + 1]
        if a < e:
            np.testing.assert_allclose(g["dS"][:, a:e].sum(axis=1), 0.0, atol=1e-12)
    empty = 15
    assert rp[empty] == rp[empty + 1]
    np.testing.assert_array_equal(g["dQ"][:, empty], 0.0)


def test_zero_upstream_and_zero_scale():
    q, k, v, dO, rp, ci, b, km = _case(6, n=12)
    g = obw.grads_csr(q, k, v, rp, ci, 0.5, 2, np.zeros_like(dO), bias=b, key_mask=km)
    for name in ("dQ", "dK", "dV"):
        np.testing.assert_array_equal(g[name], 0.0)
    g = obw.grads_csr(q, k, v, rp, ci, 0.0, 2, dO, bias=b, key_mask=km)
    np.testing.assert_array_equal(g["dQ"], 0.0)
    np.testing.assert_array_equal(g["dK"], 0.0)


# ---- planted mistakes: each copy of a step has one plausible error, and a pin must fail

def _mut_no_row_term(W, dW, row_ptr):
    return np.asarray(W) * np.asarray(dW)


_REAL_BIAS_GRAD = obw.bias_grad


def _mut_bias_grad_first_batch_only(dS, row_ptr, col_idx, H, n):
    return _REAL_BIAS_GRAD(np.asarray(dS)[:H], row_ptr, col_idx, H, n)


def _mut_transpose_uses_column_as_row(X, row_ptr, col_idx, y, n):
    out = np.zeros((y.shape[0], n, y.shape[2]))
    for i in range(n):
        for p in range(row_ptr[i], row_ptr[i + 1]):
            out[:, i, :] += np.asarray(X)[:, p, None] * np.asarray(y)[:, int(col_idx[p]), :]
    return out


@pytest.mark.parametrize("target,mutation", [
    ("softmax_backward", _mut_no_row_term),
    ("spmm_transposed", _mut_transpose_uses_column_as_row),
])
def test_planted_mistakes_are_caught(target, mutation, monkeypatch):
    monkeypatch.setattr(obw, target, mutation)
    q, k, v, dO, rp, ci, b, km = _case(0)
    fd = _finite_difference(q, k, v, dO, rp, ci, 0.7, 2, b, km)
    g = obw.grads_csr(q, k, v, rp, ci, 0.7, 2, dO, bias=b, key_mask=km)
    assert any(not np.allclose(g[name], ref, atol=1e-6) for name, ref in zip(("dQ", "dK", "dV"), fd))


def test_planted_bias_gradient_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(obw, "bias_grad", _mut_bias_grad_first_batch_only)
    q, k, v, dO, rp, ci, b, km = _case(2, B=2, n=5, d=3)
    g = obw.grads_csr(q, k, v, rp, ci, 0.6, 2, dO, bias=b, key_mask=km)
    a = obw.grads_autograd(q, k, v, 0.6, 2, ("csr", rp, ci), dO, bias=b, key_mask=km)
    assert not np.allclose(g["dBias"], a["dBias"], atol=1e-6)


def test_planted_missing_scale_is_caught(monkeypatch):
    real = ocsr.spmm
    monkeypatch.setattr(ocsr, "spmm", lambda W, rp, ci, v: real(W, rp, ci, v) / 0.7 if W is not None else None)
    q, k, v, dO, rp, ci, b, km = _case(1)
    fd = _finite_difference(q, k, v, dO, rp, ci, 0.7, 2, b, km)
    g = obw.grads_csr(q, k, v, rp, ci, 0.7, 2, dO, bias=b, key_mask=km)
    assert not np.allclose(g["dQ"], fd[0], atol=1e-6)
