"""Pins of oracle.mask (masks given as COO pairs, key lengths, packed sequences or generated
as the top-k scores of every row).

What fixes the expected values: small cases worked out by hand (written out below), a
pattern drawn by the generators and scattered back as shuffled, repeated COO pairs, the
dense boolean matrix of the pairs, and attention itself -- a key mask from lengths must
give the attention over the first keys only, and a packed batch must give each sequence's
own attention (torch's library SDPA on each sequence); top-k rows are checked against
numpy's stable argsort and the threshold property. Planted mistakes must fail a pin.
"""
import numpy as np
import pytest
import torch

import gen
from oracle import dense as odense
from oracle import mask as omask


# ---- pins, written as checks of a function under test so that mutants can be run too

def pin_coo_hand(f):
    # n = 4; (5, 0) and (-1, 1) lie outside, (2, 1) is given twice
    rows = [2, 0, 2, 5, 0, 1, -1, 2]
    cols = [1, 3, 1, 0, 0, 2, 1, 0]
    rp, ci, counts = f(4, rows, cols)
    return (list(rp) == [0, 2, 3, 5, 5] and list(ci) == [0, 3, 2, 0, 1]
            and tuple(counts) == (5, 2, 1))


def pin_coo_round_trip(f, seed=0):
    p = gen.make("window_n128")
    rows = np.repeat(np.arange(p.n), np.diff(p.row_ptr))
    cols = p.col_idx.astype(np.int64)
    rng = np.random.default_rng(seed)
    extra = rng.integers(0, len(rows), 300)                # repeats of stored pairs
    R = np.concatenate([rows, rows[extra], [p.n, 3, -2]])  # and three pairs outside
    C = np.concatenate([cols, cols[extra], [0, p.n + 7, 1]])
    order = rng.permutation(len(R))
    rp, ci, counts = f(p.n, R[order], C[order])
    return (np.array_equal(rp, p.row_ptr) and np.array_equal(ci, p.col_idx)
            and tuple(counts) == (len(rows), 3, 300))


def pin_coo_dense_matrix(f, seed=1):
    rng = np.random.default_rng(seed)
    n = 23
    R, C = rng.integers(-2, n + 2, 400), rng.integers(-2, n + 2, 400)
    P = np.zeros((n, n), bool)
    for r, c in zip(R, C):
        if 0 <= r < n and 0 <= c < n:
            P[r, c] = True
    rp, ci, _ = f(n, R, C)
    ok = rp[-1] == P.sum()
    for i in range(n):
        ok = ok and np.array_equal(ci[rp[i]:rp[i + 1]], np.nonzero(P[i])[0])
    return bool(ok)


def pin_key_mask_hand(f):
    km = f([2, 5, -1, 0], 4)
    want = np.array([[0, 0, -np.inf, -np.inf], [0, 0, 0, 0], [-np.inf] * 4, [-np.inf] * 4])
    return np.array_equal(km, want)


def pin_key_mask_truncation(f, seed=2):
    """With keys j >= L masked, attention equals attention over the first L keys only."""
    rng = np.random.default_rng(seed)
    B, H, n, d = 3, 2, 12, 8
    lens = [12, 7, 1]
    q, k, v = (rng.standard_normal((B * H, n, d)) for _ in range(3))
    km = f(lens, n)[:, None, :]                             # [B, 1, n]
    full = ("csr", np.arange(0, n * n + 1, n), np.tile(np.arange(n), n))
    O = odense.attention_dense(q, k, v, 0.5, H, full, key_mask=km, want_weights=False)["O"]
    ok = True
    for t in range(B * H):
        L = lens[t // H]
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[t]), torch.tensor(k[t, :L]), torch.tensor(v[t, :L]), scale=0.5)
        ok = ok and np.allclose(O[t], want.numpy(), atol=1e-12)
    return bool(ok)


def pin_varlen_hand(f):
    # sequences [0, 2) and [2, 5); token 5 belongs to none
    rp, ci = f([0, 2, 5], 6, -1)
    ok = list(rp) == [0, 2, 4, 7, 10, 13, 13] and list(ci) == [0, 1, 0, 1] + [2, 3, 4] * 3
    rp, ci = f([0, 2, 5], 6, 1)
    return ok and list(rp) == [0, 2, 4, 6, 9, 11, 11] and \
        list(ci) == [0, 1, 0, 1, 2, 3, 2, 3, 4, 3, 4]


def pin_varlen_per_sequence_attention(f, seed=3):
    """Packed attention over the varlen pattern = each sequence's own full attention."""
    rng = np.random.default_rng(seed)
    cu = [0, 5, 6, 14, 20]
    total, H, d = 20, 2, 8
    q, k, v = (rng.standard_normal((H, total, d)) for _ in range(3))
    rp, ci = f(cu, total, -1)
    O = odense.attention_dense(q, k, v, 0.3, H, ("csr", rp, ci), want_weights=False)["O"]
    ok = True
    for b in range(len(cu) - 1):
        s = slice(cu[b], cu[b + 1])
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[:, s]), torch.tensor(k[:, s]), torch.tensor(v[:, s]), scale=0.3)
        ok = ok and np.allclose(O[:, s], want.numpy(), atol=1e-12)
    return bool(ok)


def pin_topk_hand(f):
    nan, inf = np.nan, np.inf
    S = np.array([[1, 3, 3, 2],
                  [-0.0, 0.0, nan, -inf],
                  [5, -inf, nan, 5],
                  [0, 0, 0, 0]], np.float32)
    rp, ci = f(S, 2)
    ok = list(rp) == [0, 2, 4, 6, 8] and list(ci) == [1, 2, 0, 1, 0, 3, 0, 1]
    rp, ci = f(S, 3)
    ok = ok and list(ci) == [1, 2, 3, 0, 1, 2, 0, 1, 3, 0, 1, 2]
    rp, ci = f(S, 9)   # k past n keeps every column
    return ok and list(rp) == [0, 4, 8, 12, 16] and list(ci) == [0, 1, 2, 3] * 4


def pin_topk_stable_argsort(f, seed=4):
    """Against numpy's stable argsort of the negated scores (ties: lower column first)."""
    rng = np.random.default_rng(seed)
    S = rng.integers(-3, 4, (40, 57)).astype(np.float32)   # many ties
    S[rng.random(S.shape) < 0.05] = -np.inf
    rp, ci = f(S, 11)
    ok = list(rp) == list(range(0, 41 * 11, 11))
    for i in range(40):
        want = np.sort(np.argsort(-S[i], kind="stable")[:11])
        ok = ok and np.array_equal(ci[11 * i:11 * i + 11], want)
    return bool(ok)


def pin_topk_threshold(f, seed=5):
    """Every kept score is >= every dropped score of the row."""
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((30, 100)).astype(np.float32)
    rp, ci = f(S, 13)
    ok = True
    for i in range(30):
        kept = np.zeros(100, bool)
        kept[ci[13 * i:13 * i + 13]] = True
        ok = ok and kept.sum() == 13 and S[i][kept].min() >= S[i][~kept].max()
    return bool(ok)


COO_PINS = [pin_coo_hand, pin_coo_round_trip, pin_coo_dense_matrix]
TOPK_PINS = [pin_topk_hand, pin_topk_stable_argsort, pin_topk_threshold]
KM_PINS = [pin_key_mask_hand, pin_key_mask_truncation]
VARLEN_PINS = [pin_varlen_hand, pin_varlen_per_sequence_attention]


@pytest.mark.parametrize("pin", COO_PINS)
def test_coo_to_csr(pin):
    assert pin(omask.coo_to_csr)


@pytest.mark.parametrize("pin", TOPK_PINS)
def test_topk_rows(pin):
    assert pin(omask.topk_rows)


@pytest.mark.parametrize("pin", KM_PINS)
def test_key_mask_from_lengths(pin):
    assert pin(omask.key_mask_from_lengths)


@pytest.mark.parametrize("pin", VARLEN_PINS)
def test_varlen_csr(pin):
    assert pin(omask.varlen_csr)


# ---- planted mistakes

def _coo_keeps_repeats(n, rows, cols):
    pairs = sorted((int(r), int(c)) for r, c in zip(rows, cols) if 0 <= r < n and 0 <= c < n)
    rp = np.zeros(n + 1, np.int64)
    for r, _ in pairs:
        rp[r + 1] += 1
    return np.cumsum(rp), np.array([c for _, c in pairs]), (len(pairs), 0, 0)


def _coo_clamps_instead_of_dropping(n, rows, cols):
    return omask.coo_to_csr(n, np.clip(rows, 0, n - 1), np.clip(cols, 0, n - 1))


def _key_mask_off_by_one(seqlen_k, n):
    return omask.key_mask_from_lengths([s + 1 for s in seqlen_k], n)


def _varlen_end_inclusive(cu, total, window=-1):
    cu2 = list(cu[:-1]) + [cu[-1]]
    rp, cols = [0], []
    for i in range(total):
        for b in range(len(cu2) - 1):
            if cu2[b] <= i < cu2[b + 1]:
                cols += [j for j in range(cu2[b], min(cu2[b + 1] + 1, total))
                         if window < 0 or abs(i - j) <= window]
        rp.append(len(cols))
    return np.array(rp), np.array(cols)


def _topk_ties_high_first(scores, k):
    S = np.asarray(scores, np.float32)
    rows, n = S.shape
    kk = min(k, n)
    cols = []
    for i in range(rows):
        v = np.where(np.isnan(S[i]), -np.inf, S[i])
        order = sorted(range(n), key=lambda j: (-v[j], -j))[:kk]
        cols.extend(sorted(order))
    return np.arange(rows + 1) * kk, np.array(cols)


def _topk_nan_as_largest(scores, k):
    S = np.array(scores, np.float32)
    S[np.isnan(S)] = np.inf
    return omask.topk_rows(S, k)


@pytest.mark.parametrize("mutant,pins", [
    (_topk_ties_high_first, TOPK_PINS),
    (_topk_nan_as_largest, TOPK_PINS),
    (_coo_keeps_repeats, COO_PINS),
    (_coo_clamps_instead_of_dropping, COO_PINS),
    (_key_mask_off_by_one, KM_PINS),
    (_varlen_end_inclusive, VARLEN_PINS),
])
def test_planted_mistakes_fail_a_pin(mutant, pins):
    assert not all(pin(mutant) for pin in pins)
