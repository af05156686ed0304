"""Dense fp64 definition of masked scaled dot-product attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For head t = b*H + h and query row i (the flattening of the q/k/v shape
``[total_size * head, seq, head_dim]`` in the flash-attention PR "support
attentions in AlphaFold2", first shape list):

  S[i, j] = scale * (q_i . k_j) + bias[h, i, j] + key_mask[b, hm, j]   if (i, j) in P
  S[i, j] = -inf                                                      otherwise

where P is the attention pattern: row i attends key j iff the mask holds a
nonzero at (i, j) (gluon-nlp issue "Unified Interface/Implementation for
Sparse Attention", opening post, the definition of atten_mask). The bias and
the key mask are additive (PR text: "(additive) attention_mask and (additive)
attention_bias"); the bias has shape [1, H, seq_q, seq_k] and the key mask
[total_size, 1 or H, 1, seq_k] (PR, the two shape lists). The scale multiplies
q.k only.

  m_i   = max_j S[i, j]
  W[i,j]= exp(S[i,j] - m_i) / sum_j' exp(S[i,j'] - m_i)      (row softmax)
  O_i   = sum_j W[i, j] v_j                                    (context)
  lse_i = m_i + log sum_j exp(S[i, j] - m_i)

A row with no finite score (empty row, or every key masked with -inf, e.g. the
fully masked rows of the transposed MSA mask in the PR's minimal example) gets
W = 0 at its stored entries, O_i = 0 and lse_i = -inf. The pages do not state
this case; it is the reading recorded in the design doc.

Patterns are passed as tuples:
  ("csr", row_ptr, col_idx)           element CSR, sorted unique columns per row
  ("bsr", row_ptr, col_idx, block)    CSR over block-rows of block x block tiles
  ("dense",)                          every (i, j)
"""
from __future__ import annotations

import numpy as np


def pattern_rows(pattern, i0: int, i1: int, n: int) -> np.ndarray:
    """Boolean rows [i1-i0, n] of the pattern: True where (i, j) is in P."""
    kind = pattern[0]
    P = np.zeros((i1 - i0, n), dtype=bool)
    if kind == "dense":
        P[:] = True
    elif kind == "csr":
        _, row_ptr, col_idx = pattern
        for i in range(i0, i1):
            P[i - i0, col_idx[row_ptr[i]:row_ptr[i + 1]]] = True
    elif kind == "bsr":
        _, row_ptr, col_idx, block = pattern
        for i in range(i0, i1):
            br = i // block
            for bc in col_idx[row_ptr[br]:row_ptr[br + 1]]:
                P[i - i0, bc * block:min((bc + 1) * block, n)] = True
    else:
        raise ValueError(kind)
    return P


def row_columns(pattern, i: int, n: int) -> np.ndarray:
    """Column indices of row i in the order the pattern stores them."""
    kind = pattern[0]
    if kind == "dense":
        return np.arange(n)
    if kind == "csr":
        _, row_ptr, col_idx = pattern
        return np.asarray(col_idx[row_ptr[i]:row_ptr[i + 1]], dtype=np.int64)
    _, row_ptr, col_idx, block = pattern
    br = i // block
    parts = [np.arange(bc * block, min((bc + 1) * block, n))
             for bc in col_idx[row_ptr[br]:row_ptr[br + 1]]]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _softmax_rows(S: np.ndarray):
    """Row softmax of an fp64 score block with -inf entries; returns (W, lse)."""
    m = S.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe)                     # exp(-inf) = 0 outside the pattern
    l = E.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        W = np.where(empty, 0.0, E / np.where(empty, 1.0, l))
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return W, lse[:, 0]


def _additive(bias, key_mask, km_heads, H, t, i0, i1):
    b, h = divmod(t, H)
    add = 0.0
    if bias is not None:
        add = add + np.asarray(bias[h, i0:i1, :], dtype=np.float64)
    if key_mask is not None:
        add = add + np.asarray(key_mask[b, h if km_heads > 1 else 0, :], dtype=np.float64)[None, :]
    return add


def attention_dense(q, k, v, scale, H, pattern, bias=None, key_mask=None, km_heads=1,
                    chunk=256, heads=None, want_weights=True):
    """Evaluate the definition for whole heads.

    q, k, v : [BH, n, d] (any float dtype; widened to fp64)
    returns dict(O=[BH,n,d] f64, lse=[BH,n] f64, W=list per head of the weights at
    the pattern's stored positions in storage order, or None)
    """
    BH, n, d = q.shape
    heads = range(BH) if heads is None else heads
    O = np.zeros((BH, n, d))
    lse = np.full((BH, n), -np.inf)
    Ws = {}
    for t in heads:
        qt = np.asarray(q[t], dtype=np.float64)
        kt = np.asarray(k[t], dtype=np.float64)
        vt = np.asarray(v[t], dtype=np.float64)
        wrow = [] if want_weights else None
        for i0 in range(0, n, chunk):
            i1 = min(n, i0 + chunk)
            S = scale * (qt[i0:i1] @ kt.T)
            S = S + _additive(bias, key_mask, km_heads, H, t, i0, i1)
            S = np.where(pattern_rows(pattern, i0, i1, n), S, -np.inf)
            W, lse[t, i0:i1] = _softmax_rows(S)
            O[t, i0:i1] = W @ vt
            if want_weights:
                for i in range(i0, i1):
                    wrow.append(W[i - i0, row_columns(pattern, i, n)])
        if want_weights:
            Ws[t] = np.concatenate(wrow) if wrow else np.zeros(0)
    return {"O": O, "lse": lse, "W": Ws if want_weights else None}


def attention_rows(q, k, v, scale, H, pattern, pairs, bias=None, key_mask=None, km_heads=1):
    """Evaluate the definition for selected (t, i) rows only, one row at a time.

    Used on workloads whose full dense evaluation is too large. Returns
    dict(O=[len(pairs), d], lse=[len(pairs)], W=list of the row's weights in storage order).
    """
    BH, n, d = q.shape
    O = np.zeros((len(pairs), d))
    lse = np.zeros(len(pairs))
    Ws = []
    for r, (t, i) in enumerate(pairs):
        kt = np.asarray(k[t], dtype=np.float64)
        s = scale * (kt @ np.asarray(q[t, i], dtype=np.float64))
        if bias is not None or key_mask is not None:
            s = s + np.atleast_2d(_additive(bias, key_mask, km_heads, H, t, i, i + 1))[0]
        s = np.where(pattern_rows(pattern, i, i + 1, n)[0], s, -np.inf)
        W, l = _softmax_rows(s[None, :])
        O[r] = W[0] @ np.asarray(v[t], dtype=np.float64)
        lse[r] = l[0]
        Ws.append(W[0, row_columns(pattern, i, n)])
    return {"O": O, "lse": lse, "W": Ws}
