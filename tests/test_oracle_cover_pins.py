"""Pins of the block-cover oracle (oracle.cover) against facts fixed by its definition: the
dense pattern covers every block with every in-range bit set, a block-diagonal pattern
covers only the diagonal blocks, the words mark exactly the pattern (round trip, both
layouts), and hand-worked small cases give the block lists and words spelled out here."""
import numpy as np

import gen
from oracle import cover as ocv


def _csr(n, pairs):
    pairs = sorted(set(pairs))
    rp = np.zeros(n + 1, np.int64)
    for r, _ in pairs:
        rp[r + 1] += 1
    return np.cumsum(rp).astype(np.int32), np.array([c for _, c in pairs], np.int32)


def test_dense_pattern_covers_every_block():
    n = 150  # three block-rows, the last with 22 rows
    rp, ci = _csr(n, [(i, j) for i in range(n) for j in range(n)])
    cv = ocv.block_cover(n, rp, ci)
    assert list(cv["row_ptr"]) == [0, 3, 6, 9]
    assert list(cv["col_idx"]) == [0, 1, 2] * 3
    assert list(cv["t_row_ptr"]) == [0, 3, 6, 9] and list(cv["t_col_idx"]) == [0, 1, 2] * 3
    full, tail = (1 << 64) - 1, (1 << 22) - 1
    for j, (R, C) in enumerate((R, C) for R in range(3) for C in range(3)):
        rows = 64 if R < 2 else 22
        want = full if C < 2 else tail
        assert [int(w) for w in cv["bits"][j, :rows]] == [want] * rows
        assert not cv["bits"][j, rows:].any()


def test_block_diagonal_pattern_covers_the_diagonal():
    n = 256
    rp, ci = _csr(n, [(i, j) for i in range(n) for j in range(n) if i // 64 == j // 64])
    cv = ocv.block_cover(n, rp, ci)
    assert list(cv["row_ptr"]) == [0, 1, 2, 3, 4] and list(cv["col_idx"]) == [0, 1, 2, 3]
    assert np.array_equal(cv["bits"], cv["bits_t"])


def test_hand_worked_case():
    # entries (0, 70), (1, 0), (65, 1), (65, 127): blocks (0,0), (0,1), (1,0), (1,1)
    n = 128
    rp, ci = _csr(n, [(0, 70), (1, 0), (65, 1), (65, 127)])
    cv = ocv.block_cover(n, rp, ci)
    assert list(cv["row_ptr"]) == [0, 2, 4] and list(cv["col_idx"]) == [0, 1, 0, 1]
    w = cv["bits"]
    assert int(w[0, 1]) == 1 and int(w[0].sum()) == 1              # (1, 0)
    assert int(w[1, 0]) == 1 << 6 and int(w[1].sum()) == 1 << 6    # (0, 70)
    assert int(w[2, 1]) == 1 << 1 and int(w[2].sum()) == 2         # (65, 1)
    assert int(w[3, 1]) == 1 << 63                                  # (65, 127)
    # transposed cover: block-column 0 holds block-rows 0, 1; column 1 the same
    t = cv["bits_t"]
    assert list(cv["t_row_ptr"]) == [0, 2, 4] and list(cv["t_col_idx"]) == [0, 1, 0, 1]
    assert int(t[0, 0]) == 1 << 1      # key 0, query 1
    assert int(t[1, 1]) == 1 << 1      # key 1, query 65
    assert int(t[2, 6]) == 1           # key 70, query 0
    assert int(t[3, 63]) == 1 << 1     # key 127, query 65


def test_round_trip_both_layouts():
    p = gen.make("random_n8192", n=200, H=1, kmin=1, kmax=30)
    cv = ocv.block_cover(p.n, p.row_ptr, p.col_idx)
    want = {(r, int(c)) for r in range(p.n) for c in p.col_idx[p.row_ptr[r]:p.row_ptr[r + 1]]}
    assert ocv.pattern_of_cover(p.n, cv) == want
    swapped = dict(row_ptr=cv["t_row_ptr"], col_idx=cv["t_col_idx"], bits=cv["bits_t"])
    assert ocv.pattern_of_cover(p.n, swapped) == {(c, r) for r, c in want}
    assert cv["row_ptr"][-1] == cv["t_row_ptr"][-1] == len(cv["col_idx"])


def test_a_dropped_entry_is_seen():
    """Planted mistake: the oracle run on a pattern missing one entry differs in one word."""
    n = 100
    pairs = [(i, (7 * i) % n) for i in range(n)] + [(i, i) for i in range(n)]
    rp, ci = _csr(n, pairs)
    rp2, ci2 = _csr(n, [x for x in pairs if x != (3, 21)])
    a, b = ocv.block_cover(n, rp, ci), ocv.block_cover(n, rp2, ci2)
    assert (a["bits"] != b["bits"]).sum() == 1 and (a["bits_t"] != b["bits_t"]).sum() == 1
