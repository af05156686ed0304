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

Each is written from its definition with Python sets and loops, for small inputs.
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
