"""Block cover of an element CSR pattern.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The block-sparse replies of the gluon-nlp issue ("[Proposal] Unified Interface/Implementation
for Sparse Attention") compute whole 64x64 blocks; an element pattern is carried onto such
kernels by its cover, the set of 64x64 blocks of the (n, n) grid that hold at least one of
its entries, with one 64-bit word per row of each block marking the entries (and the same
per key of each block of the transposed cover). Written from that definition with Python
sets, sorts and loops, for small inputs.
"""
from __future__ import annotations

import numpy as np

B = 64


def block_cover(n, row_ptr, col_idx):
    """Returns dict(row_ptr, col_idx, t_row_ptr, t_col_idx, bits, bits_t): the cover as block
    CSR over ceil(n/64) block-rows (each block-row's block-columns ascending), its transpose
    (each block-column's block-rows ascending), and uint64 words [nnz, 64]: bits[j][r] has
    bit c set when (64R + r, 64C + c) is an entry of block j = (R, C); bits_t[j][c] has bit r
    set for the same entry, j indexing the transposed cover."""
    nb = (n + B - 1) // B
    entries = set()
    for r in range(n):
        for e in range(int(row_ptr[r]), int(row_ptr[r + 1])):
            c = int(col_idx[e])
            if 0 <= c < n:
                entries.add((r, c))
    blocks = sorted({(r // B, c // B) for r, c in entries})
    t_blocks = sorted((C, R) for R, C in blocks)
    pos = {blk: j for j, blk in enumerate(blocks)}
    t_pos = {blk: j for j, blk in enumerate(t_blocks)}
    words = np.zeros((len(blocks), B), dtype=np.uint64)
    t_words = np.zeros((len(blocks), B), dtype=np.uint64)
    for r, c in entries:
        R, C = r // B, c // B
        words[pos[(R, C)], r % B] |= np.uint64(1) << np.uint64(c % B)
        t_words[t_pos[(C, R)], c % B] |= np.uint64(1) << np.uint64(r % B)

    def csr(pairs):
        rp = np.zeros(nb + 1, np.int64)
        for a, _ in pairs:
            rp[a + 1] += 1
        return np.cumsum(rp).astype(np.int32), np.array([b for _, b in pairs], np.int32)

    rp, ci = csr(blocks)
    trp, tci = csr(t_blocks)
    return dict(row_ptr=rp, col_idx=ci, t_row_ptr=trp, t_col_idx=tci, bits=words, bits_t=t_words)


def pattern_of_cover(n, cover):
    """The set of (row, column) pairs the words of a cover mark (bits only)."""
    out = set()
    rp, ci, words = cover["row_ptr"], cover["col_idx"], cover["bits"]
    for R in range(len(rp) - 1):
        for j in range(int(rp[R]), int(rp[R + 1])):
            C = int(ci[j])
            for r in range(B):
                w = int(words[j, r])
                for c in range(B):
                    if (w >> c) & 1:
                        out.add((R * B + r, C * B + c))
    return out
