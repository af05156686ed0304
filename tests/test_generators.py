"""Properties of the seeded input generators (CPU)."""
import numpy as np
import pytest
import torch

import gen


def _check_csr(rp, ci, n, diag=True):
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0)
    assert len(ci) == rp[-1]
    assert ci.dtype == np.int32 and rp.dtype == np.int32
    for i in range(n):
        row = ci[rp[i]:rp[i + 1]]
        assert np.all(np.diff(row) > 0), "sorted and unique"
        assert row.min() >= 0 and row.max() < n
        if diag:
            assert i in row


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e-39]   # ties and a subnormal
    ours = gen.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_window_n128():
    p = gen.make("window_n128")
    assert (p.BH, p.n, p.d, p.dtype) == (1, 128, 32, "f32")
    _check_csr(p.row_ptr, p.col_idx, p.n)
    lens = np.diff(p.row_ptr)
    assert lens.min() == 9 and lens.max() == 17 and p.nnz == 2104
    for i in range(p.n):
        assert np.array_equal(p.col_idx[p.row_ptr[i]:p.row_ptr[i + 1]],
                              np.arange(max(0, i - 8), min(127, i + 8) + 1))
    assert p.scale == pytest.approx(1 / np.sqrt(32))


def test_longformer_n4096():
    p = gen.make("longformer_n4096")
    assert (p.BH, p.n, p.d, p.dtype) == (12, 4096, 64, "bf16")
    _check_csr(p.row_ptr, p.col_idx, p.n)
    lens = np.diff(p.row_ptr)
    assert lens[0] == lens[1] == 4096
    assert p.nnz == 1052026
    assert np.all((lens[2:] >= 131) & (lens[2:] <= 259))
    assert np.sum(lens == 259) == 3838
    for i in (2, 500, 4095):
        row = set(p.col_idx[p.row_ptr[i]:p.row_ptr[i + 1]].tolist())
        assert {0, 1} <= row
        assert row - {0, 1} == set(range(max(0, i - 128), min(4095, i + 128) + 1)) - {0, 1}
    assert p.q_bits.dtype == np.uint16
    assert np.array_equal(gen.bf16_bits_to_f32(p.q_bits), p.q)


def test_random_rows():
    p = gen.make("random_n8192", n=2000, H=2)
    _check_csr(p.row_ptr, p.col_idx, p.n)
    lens = np.diff(p.row_ptr)
    assert lens.min() >= 32 and lens.max() <= 512
    assert abs(lens.mean() - 272) < 10
    q2 = gen.make("random_n8192", n=2000, H=2)
    assert np.array_equal(q2.col_idx, p.col_idx) and np.array_equal(q2.q, p.q)   # seeded


def test_bsr():
    p = gen.make("bsr_n16384", n=64 * 40, H=2)
    assert p.block == 64
    nb = 40
    _check_csr(p.row_ptr, p.col_idx, nb)
    assert np.all(np.diff(p.row_ptr) == 9)
    rp, ci = p.element_csr()
    assert rp[-1] == 64 * 40 * 9 * 64
    full = gen.make("bsr_n16384")
    assert full.nnz == 256 * 9 and full.n == 16384 and full.d == 128


def test_evoformer():
    p = gen.make("evoformer_l384")
    assert (p.B, p.H, p.n, p.d) == (32, 8, 384, 32)
    assert p.row_ptr is None
    assert p.bias.shape == (8, 384, 384) and p.bias.dtype == np.float32
    assert p.key_mask.shape == (32, 1, 384)
    for b in range(32):
        m = p.key_mask[b, 0]
        pb = int(np.sum(~np.isfinite(m)))
        assert 0 <= pb <= 64
        assert np.all(np.isfinite(m[:384 - pb])) and np.all(m[384 - pb:] == -np.inf)
        assert np.all(m[:384 - pb] == 0)
