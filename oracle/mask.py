"""Mask inputs in other forms than CSR, turned into the CSR pattern and key mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* :func:`coo_to_csr` -- the gluon-nlp proposal ("Unified Interface/Implementation for
  Sparse Attention", opening post) accepts the (n, n) mask in COO form as well as CSR. A
  COO list is a set of (row, column) pairs: the mask holds exactly the pairs inside
  [0, n) x [0, n), each once, whatever their order or repetition.
* :func:`key_mask_from_lengths` -- the flash-attention pull request "support attentions in
  AlphaFold2" (key-padding discussion) proposes one int per batch, the number of valid keys,
  for masks whose masked keys are a suffix: the additive key mask is 0 before that length
  and -inf from it on.
* :func:`varlen_csr` -- the same pull request packs variable-length sequences one after
  another with the prefix of their starts (cu_seqlens); attention stays inside each
  sequence, here optionally within a window |i - j| <= w.

* :func:`topk_rows` -- a mask generated from scores at run time: each query keeps the k
  keys of largest score, a constant number per query (the SPARSEK abstract); equal scores
  are taken lowest column first, NaN counts as -inf and -0 as +0.

Each is written from its definition with Python sets, sorts and loops, for small inputs.
"""
from __future__ import annotations

import numpy as np


def coo_to_csr(n, rows, cols):
    """Returns (row_ptr int32 [n+1], col_idx int32, counts = (stored, dropped, merged))."""
    kept = [(int(r), int(c)) for r, c in zip(rows, cols) if 0 <= r < n and 0 <= c < n]
    pairs = sorted(set(kept))
    row_ptr = np.zeros(n + 1, np.int64)
    for r, _ in pairs:
        row_ptr[r + 1] += 1
    row_ptr = np.cumsum(row_ptr)
    col_idx = np.array([c for _, c in pairs], np.int64)
    counts = (len(pairs), len(rows) - len(kept), len(kept) - len(pairs))
    return row_ptr.astype(np.int32), col_idx.astype(np.int32), counts


def key_mask_from_lengths(seqlen_k, n):
    """[B, n] fp64: 0 for keys j < seqlen_k[b] (taken within [0, n]), -inf for the others."""
    B = len(seqlen_k)
    km = np.full((B, n), -np.inf)
    for b in range(B):
        km[b, :min(max(int(seqlen_k[b]), 0), n)] = 0.0
    return km


def varlen_csr(cu_seqlens, total, window=-1):
    """CSR over the packed tokens 0 .. total-1: token i in sequence b (cu[b] <= i < cu[b+1])
    attends keys j of the same sequence, with |i - j| <= window when window >= 0."""
    seq_of = {}
    for b in range(len(cu_seqlens) - 1):
        for i in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
            seq_of[i] = b
    row_ptr, cols = [0], []
    for i in range(total):
        if i in seq_of:
            b = seq_of[i]
            for j in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
                if window < 0 or abs(i - j) <= window:
                    cols.append(j)
        row_ptr.append(len(cols))
    return np.array(row_ptr, np.int32), np.array(cols, np.int32)


def topk_rows(scores, k):
    """(row_ptr, col_idx) of the k largest scores of every row, columns ascending."""
    S = np.asarray(scores, dtype=np.float32)
    rows, n = S.shape
    kk = max(0, min(int(k), n))
    cols = []
    for i in range(rows):
        vals = [(-np.inf if np.isnan(x) else float(x) + 0.0, j) for j, x in enumerate(S[i])]
        best = sorted(vals, key=lambda vj: (-vj[0], vj[1]))[:kk]   # larger first, then lower j
        cols.extend(sorted(j for _, j in best))
    return np.arange(rows + 1, dtype=np.int64).astype(np.int32) * kk, np.array(cols, np.int32)
