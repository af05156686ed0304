"""CSR-only fp64 evaluation of the three sparse steps.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The steps follow the three bullet points of the gluon-nlp proposal "Unified
Interface/Implementation for Sparse Attention" (opening post):

1. ``sddmm``: a dot product between query i and key j for each nonzero (i, j)
   of the mask; the scores keep the mask's CSR pattern.
2. ``sparse_softmax``: a softmax over each sparse row; the weights keep the
   same pattern.
3. ``spmm``: the product of the CSR weights with the dense V gives the context.

Conventions are those of :mod:`oracle.dense` (additive bias/key mask, the
scale on q.k only, rows without a finite score give zero weights and output).
Each function loops over rows and vectorises over heads only, so that it can
be checked against the text by eye.
"""
from __future__ import annotations

import numpy as np


def sddmm(q, k, row_ptr, col_idx, scale, H, bias=None, key_mask=None, km_heads=1):
    """S[t, e] = scale * q[t, i] . k[t, col_idx[e]] (+ bias[h, i, j]) (+ key_mask[b, hm, j])
    for every stored entry e of row i. Returns fp64 [BH, nnz]."""
    BH, n, d = q.shape
    nnz = int(row_ptr[n])
    S = np.zeros((BH, nnz))
    heads = np.arange(BH)
    b_of, h_of = heads // H, heads % H
    kmt = None
    if key_mask is not None:                                        # [BH, n] per head
        kmt = np.asarray(key_mask, dtype=np.float64)[b_of, (h_of if km_heads > 1 else 0)]
    for i in range(n):
        a, e = int(row_ptr[i]), int(row_ptr[i + 1])
        if a == e:
            continue
        cols = np.asarray(col_idx[a:e], dtype=np.int64)
        qi = np.asarray(q[:, i, :], dtype=np.float64)               # [BH, d]
        kj = np.asarray(k[:, cols, :], dtype=np.float64)            # [BH, len, d]
        s = scale * np.einsum("td,tjd->tj", qi, kj)
        if bias is not None:
            s = s + np.asarray(bias[h_of, i], dtype=np.float64)[:, cols]
        if kmt is not None:
            s = s + kmt[:, cols]
        S[:, a:e] = s
    return S


def sparse_softmax(S, row_ptr, return_lse=False):
    """W[t, e] = exp(S[t,e] - m) / sum_{e' in row} exp(S[t,e'] - m), m the row max.
    Rows with no finite score give W = 0 (and lse = -inf)."""
    S = np.asarray(S, dtype=np.float64)
    BH = S.shape[0]
    n = len(row_ptr) - 1
    W = np.zeros_like(S)
    lse = np.full((BH, n), -np.inf)
    for i in range(n):
        a, e = int(row_ptr[i]), int(row_ptr[i + 1])
        if a == e:
            continue
        s = S[:, a:e]
        m = s.max(axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        x = np.exp(s - m)
        l = x.sum(axis=1, keepdims=True)
        W[ok, a:e] = x[ok] / l[ok]
        lse[ok, i] = m[ok, 0] + np.log(l[ok, 0])
    return (W, lse) if return_lse else W


def spmm(W, row_ptr, col_idx, v):
    """O[t, i, :] = sum_{e in row i} W[t, e] * v[t, col_idx[e], :]. Returns fp64 [BH, n, d]."""
    BH, n, d = v.shape
    O = np.zeros((BH, n, d))
    W = np.asarray(W, dtype=np.float64)
    for i in range(n):
        a, e = int(row_ptr[i]), int(row_ptr[i + 1])
        if a == e:
            continue
        cols = np.asarray(col_idx[a:e], dtype=np.int64)
        O[:, i, :] = np.einsum("tj,tjd->td", W[:, a:e], np.asarray(v[:, cols, :], dtype=np.float64))
    return O


def attention_csr(q, k, v, row_ptr, col_idx, scale, H, bias=None, key_mask=None, km_heads=1):
    """The three steps in sequence: returns dict(S, W, O, lse) in fp64."""
    S = sddmm(q, k, row_ptr, col_idx, scale, H, bias, key_mask, km_heads)
    W, lse = sparse_softmax(S, row_ptr, return_lse=True)
    O = spmm(W, row_ptr, col_idx, v)
    return {"S": S, "W": W, "O": O, "lse": lse}
