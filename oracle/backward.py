"""fp64 gradients of masked scaled dot-product attention (the backward pass).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the definition of :mod:`oracle.dense`. Given the gradient dO of a loss
with respect to the context O, the gradients with respect to q, k and v follow from
the chain rule through the three sparse steps of the gluon-nlp proposal ("Unified
Interface/Implementation for Sparse Attention", opening post), taken in reverse
order; the flash-attention PR "support attentions in AlphaFold2" raises training
through the fused kernel (its question on the bias gradient), which needs exactly
these quantities. For head t and a stored entry e = (i, j):

  dV[j]   = sum over stored (i, j) of W[i, j] dO[i]            (product with the
                                                               transposed pattern)
  dW[i,j] = dO[i] . v[j]                                       (scores-like step)
  D[i]    = sum over the row's entries of W[i, j] dW[i, j]
  dS[i,j] = W[i, j] (dW[i, j] - D[i])                          (softmax step)
  dQ[i]   = scale * sum over the row of dS[i, j] k[j]
  dK[j]   = scale * sum over stored (i, j) of dS[i, j] q[i]

dS is also the gradient with respect to the additive bias and key mask at the stored
entries (they enter S unscaled); the bias is shared by the batches, so its gradient sums
over them (the flash-attention PR's bias-gradient question):

  dBias[h, i, j] = sum over b of dS[b*H + h, (i, j)]   at stored (i, j); 0 elsewhere.

Rows without a finite score have W = 0, so all their terms vanish.

Two evaluations, pinned against each other and against finite differences in
``tests/test_oracle_backward_pins.py``:

* :func:`grads_autograd` -- torch autograd, in fp64 on the CPU, of the dense
  definition written with torch operations (the forward's formulas, nothing else);
* :func:`grads_csr` -- the formulas above, one sparse row at a time, in NumPy.
"""
from __future__ import annotations

import numpy as np

from . import csr as _csr
from .dense import pattern_rows


def softmax_backward(W, dW, row_ptr):
    """dS[t, e] = W[t, e] (dW[t, e] - sum_{e' in row} W[t, e'] dW[t, e'])."""
    W = np.asarray(W, dtype=np.float64)
    dW = np.asarray(dW, dtype=np.float64)
    dS = np.zeros_like(W)
    n = len(row_ptr) - 1
    for i in range(n):
        a, e = int(row_ptr[i]), int(row_ptr[i + 1])
        if a == e:
            continue
        D = (W[:, a:e] * dW[:, a:e]).sum(axis=1, keepdims=True)
        dS[:, a:e] = W[:, a:e] * (dW[:, a:e] - D)
    return dS


def spmm_transposed(X, row_ptr, col_idx, y, n):
    """out[t, j, :] = sum over stored entries e = (i, j) of X[t, e] * y[t, i, :]."""
    X = np.asarray(X, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    BH, _, d = y.shape
    out = np.zeros((BH, n, d))
    for i in range(n):
        a, e = int(row_ptr[i]), int(row_ptr[i + 1])
        for p in range(a, e):
            out[:, int(col_idx[p]), :] += X[:, p, None] * y[:, i, :]
    return out


def bias_grad(dS, row_ptr, col_idx, H, n):
    """dBias[h, i, j] = sum over batches b of dS[b*H + h, e] for the stored entry e = (i, j)."""
    dS = np.asarray(dS, dtype=np.float64)
    BH = dS.shape[0]
    out = np.zeros((H, n, n))
    for i in range(n):
        for e in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            for t in range(BH):
                out[t % H, i, int(col_idx[e])] += dS[t, e]
    return out


def grads_csr(q, k, v, row_ptr, col_idx, scale, H, dO, bias=None, key_mask=None, km_heads=1):
    """The formulas of the module docstring on the CSR pattern. Returns a dict with the
    forward's S, W, O and the gradients dW, dS, dQ, dK, dV and dBias (fp64)."""
    fwd = _csr.attention_csr(q, k, v, row_ptr, col_idx, scale, H, bias, key_mask, km_heads)
    n = q.shape[1]
    dO = np.asarray(dO, dtype=np.float64)
    dW = _csr.sddmm(dO, v, row_ptr, col_idx, 1.0, H)
    dS = softmax_backward(fwd["W"], dW, row_ptr)
    dQ = scale * _csr.spmm(dS, row_ptr, col_idx, k)
    dK = scale * spmm_transposed(dS, row_ptr, col_idx, q, n)
    dV = spmm_transposed(fwd["W"], row_ptr, col_idx, dO, n)
    dBias = bias_grad(dS, row_ptr, col_idx, H, n)
    return dict(fwd, dW=dW, dS=dS, dQ=dQ, dK=dK, dV=dV, dBias=dBias)


def grads_autograd(q, k, v, scale, H, pattern, dO, bias=None, key_mask=None, km_heads=1):
    """Gradients of sum(O * dO) with respect to q, k, v (and the bias, when given) by torch
    autograd (fp64, CPU) on the dense definition: S = scale q k^T + bias + key mask, -inf
    outside the pattern, a row softmax whose rows without a finite score are zero, O = W v."""
    import torch

    BH, n, d = q.shape
    t64 = lambda x: torch.tensor(np.asarray(x, dtype=np.float64))
    Q, K, V = (t64(x).requires_grad_(True) for x in (q, k, v))
    P = torch.tensor(pattern_rows(pattern, 0, n, n))
    S = scale * Q @ K.transpose(1, 2)
    heads = np.arange(BH)
    Bt = None
    if bias is not None:
        Bt = t64(bias).requires_grad_(True)
        S = S + Bt[heads % H]
    if key_mask is not None:
        km = np.asarray(key_mask, dtype=np.float64)
        S = S + t64(km[heads // H, (heads % H) if km_heads > 1 else 0])[:, None, :]
    S = S.masked_fill(~P, float("-inf"))
    m = S.max(dim=2, keepdim=True).values
    live = torch.isfinite(m)
    x = torch.exp(S - torch.where(live, m, torch.zeros_like(m)))
    x = torch.where(torch.isfinite(S), x, torch.zeros_like(x))
    l = x.sum(dim=2, keepdim=True)
    W = torch.where(live, x / torch.where(live, l, torch.ones_like(l)), torch.zeros_like(x))
    O = W @ V
    (O * t64(dO)).sum().backward()
    out = {"dQ": Q.grad.numpy(), "dK": K.grad.numpy(), "dV": V.grad.numpy(), "O": O.detach().numpy()}
    if Bt is not None:
        out["dBias"] = Bt.grad.numpy()
    return out
