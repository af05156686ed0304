"""Seeded synthetic inputs for masked scaled dot-product attention over a CSR mask.

This module only draws inputs: Q/K/V, the attention pattern (CSR, BSR or dense),
the additive pair bias and the additive key-padding mask. It computes no score,
softmax or product; both the HIP path and the fp64 oracle receive what it returns.

Workloads (sizes and structure follow the five workloads named for the method):

* ``window_n128``   -- one head, n=128, d=32, fp32, sliding window |i-j|<=8
  (local attention as mask generation: gluon-nlp issue "Unified
  Interface/Implementation for Sparse Attention", opening proposal; the
  "Sparse Attention" concept notes, section on how it works, local window).
* ``longformer_n4096`` -- 12 heads, n=4096, d=64, bf16, window |i-j|<=128 plus
  global tokens 0 and 1 that attend to and are attended by every position
  (the same notes: global tokens).
* ``random_n8192``  -- 16 heads, n=8192, d=64, bf16, row i keeps k_i ~ U{32..512}
  columns, drawn without replacement, diagonal forced in (variable per-token
  window, gluon-nlp issue, second reply by the proposer).
* ``bsr_n16384``    -- 16 heads, n=16384, d=128, bf16, 64x64 blocks; each
  block-row keeps its diagonal block plus 8 distinct random block-columns
  (block-sparse attention, gluon-nlp issue, replies).
* ``evoformer_l384`` -- 32 sequences x 8 heads, L=384, d=32, bf16, dense
  pattern with an fp32 pair bias [1,8,L,L] ~ N(0,1) and a key-padding mask
  [32,1,1,L] whose last p_b keys are -inf, p_b ~ U{0..64} (flash-attention
  PR "support attentions in AlphaFold2", the shape list of mask and bias).

Readings taken where the workload text is silent are listed in the design doc
(RNG, seeds, inclusive bounds, shared CSR across heads).

bf16 inputs are drawn as fp32 N(0,1) and rounded to bf16 with
round-to-nearest-even; ``q/k/v`` hold those values widened exactly to fp32,
``*_bits`` hold the raw bf16 bit patterns the GPU receives.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

BLOCK = 64  # block edge of the block-sparse workload


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    Inputs are finite (normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Problem:
    """One attention problem. Arrays are host NumPy arrays.

    q, k, v : float32 [B*H, n, d] (bf16-representable values when dtype == "bf16")
    row_ptr, col_idx : int32 CSR over rows (block=1) or block-rows (block=64);
                       None for the dense pattern.
    bias : float32 [H, n, n] or None ([1, H, n, n] with the leading 1 dropped)
    key_mask : float32 [B, key_mask_heads, n] or None (0 / -inf additive)
    """

    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    row_ptr: Optional[np.ndarray]
    col_idx: Optional[np.ndarray]
    block: int = 1
    scale: float = 1.0
    bias: Optional[np.ndarray] = None
    key_mask: Optional[np.ndarray] = None
    key_mask_heads: int = 1
    seed: int = 0
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def nnz(self) -> int:
        """Stored entries of row_ptr/col_idx (blocks when block == 64)."""
        return 0 if self.row_ptr is None else int(self.row_ptr[-1])

    def element_csr(self):
        """The pattern as element CSR (expands blocks, enumerates the dense case)."""
        return expand_pattern(self.row_ptr, self.col_idx, self.n, self.block)

    def attended_pairs(self) -> int:
        """Count of (t, i, j) with j in the pattern of row i and a finite key mask."""
        rp, ci = self.element_csr()
        if self.key_mask is None:
            return self.BH * int(rp[-1])
        total = 0
        for t in range(self.BH):
            b, h = divmod(t, self.H)
            km = self.key_mask[b, h if self.key_mask_heads > 1 else 0]
            total += int(np.isfinite(km[ci]).sum())
        return total


def expand_pattern(row_ptr, col_idx, n, block):
    """Element-level CSR of a pattern given as CSR (block=1), BSR or dense (None)."""
    if row_ptr is None:
        rp = np.arange(n + 1, dtype=np.int64) * n
        ci = np.tile(np.arange(n, dtype=np.int32), n)
        return rp, ci
    if block == 1:
        return row_ptr.astype(np.int64), col_idx.astype(np.int32)
    nbr = len(row_ptr) - 1
    rows_cols = []
    lens = np.zeros(n, dtype=np.int64)
    for br in range(nbr):
        bcs = col_idx[row_ptr[br]:row_ptr[br + 1]]
        cols = np.concatenate([np.arange(bc * block, min((bc + 1) * block, n)) for bc in bcs]) \
            if len(bcs) else np.zeros(0, dtype=np.int64)
        for i in range(br * block, min((br + 1) * block, n)):
            rows_cols.append(cols)
            lens[i] = len(cols)
    rp = np.zeros(n + 1, dtype=np.int64)
    rp[1:] = np.cumsum(lens)
    ci = np.concatenate(rows_cols).astype(np.int32) if rows_cols else np.zeros(0, np.int32)
    return rp, ci


# ----------------------------------------------------------------------------- patterns

def csr_from_rows(rows) -> tuple:
    lens = np.array([len(r) for r in rows], dtype=np.int64)
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col_idx = np.concatenate([np.asarray(r, dtype=np.int32) for r in rows]) if len(rows) \
        else np.zeros(0, np.int32)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def window_pattern(n: int, w: int, global_tokens=()) -> tuple:
    """Sliding window |i-j| <= w, optionally united with global tokens that
    attend to every key and are attended by every query."""
    g = np.asarray(sorted(set(global_tokens)), dtype=np.int64)
    gset = set(g.tolist())
    rows = []
    for i in range(n):
        if i in gset:
            rows.append(np.arange(n))
            continue
        lo, hi = max(0, i - w), min(n - 1, i + w)
        cols = np.arange(lo, hi + 1)
        if len(g):
            cols = np.union1d(cols, g[g < n])
        rows.append(cols)
    return csr_from_rows(rows)


def random_rows_pattern(n: int, kmin: int, kmax: int, rng: np.random.Generator) -> tuple:
    """Row i keeps k_i ~ U{kmin..kmax} (clipped to n) columns: the diagonal plus
    k_i - 1 distinct off-diagonal columns drawn uniformly without replacement."""
    ks = rng.integers(kmin, kmax + 1, size=n)
    rows = []
    for i in range(n):
        k = int(min(ks[i], n))
        off = rng.choice(n - 1, size=k - 1, replace=False)
        off = np.where(off >= i, off + 1, off)
        rows.append(np.sort(np.concatenate([off, [i]])))
    return csr_from_rows(rows)


def bsr_pattern(n: int, extra: int, rng: np.random.Generator, block: int = BLOCK) -> tuple:
    """Block-rows of a BSR with the diagonal block plus ``extra`` distinct random
    block-columns each (fewer when there are not enough block-columns)."""
    nb = (n + block - 1) // block
    rows = []
    for br in range(nb):
        k = min(extra, nb - 1)
        off = rng.choice(nb - 1, size=k, replace=False) if k > 0 else np.zeros(0, np.int64)
        off = np.where(off >= br, off + 1, off)
        rows.append(np.sort(np.concatenate([off, [br]])))
    return csr_from_rows(rows)


def key_padding_mask(B: int, n: int, pmax: int, rng: np.random.Generator) -> np.ndarray:
    """[B, 1, n] additive mask: 0, then -inf on the last p_b keys, p_b ~ U{0..pmax}."""
    p = rng.integers(0, pmax + 1, size=B)
    m = np.zeros((B, 1, n), dtype=np.float32)
    for b in range(B):
        if p[b] > 0:
            m[b, 0, n - p[b]:] = -np.inf
    return m


# ----------------------------------------------------------------------------- tensors

def _qkv(rng, BH, n, d, dtype):
    out = []
    for _ in range(3):
        x = rng.standard_normal((BH, n, d), dtype=np.float32)
        if dtype == BF16:
            bits = bf16_round_bits(x)
            out.append((bf16_bits_to_f32(bits).reshape(BH, n, d), bits.reshape(BH, n, d)))
        else:
            out.append((x, None))
    return out


WORKLOADS = ("window_n128", "longformer_n4096", "random_n8192", "bsr_n16384", "evoformer_l384")
BASE_SEED = {name: 1000 + i + 1 for i, name in enumerate(WORKLOADS)}


def make(name: str, seed: Optional[int] = None, **over) -> Problem:
    """Build a workload by name. Keyword overrides shrink it for fast tests:
    n, H, B, d, dtype, window, kmin, kmax, extra, pmax, scale, bias (bool),
    key_mask (bool), global_tokens."""
    seed = BASE_SEED[name] if seed is None else seed
    ss = np.random.SeedSequence(seed)
    s_qkv, s_mask, s_bias, s_kpm = ss.spawn(4)
    rng_qkv = np.random.default_rng(s_qkv)
    rng_mask = np.random.default_rng(s_mask)
    rng_bias = np.random.default_rng(s_bias)
    rng_kpm = np.random.default_rng(s_kpm)

    if name == "window_n128":
        B, H, n, d, dtype = 1, 1, 128, 32, F32
        n = over.get("n", n); H = over.get("H", H); d = over.get("d", d)
        dtype = over.get("dtype", dtype)
        row_ptr, col_idx = window_pattern(n, over.get("window", 8))
        block = 1
    elif name == "longformer_n4096":
        B, H, n, d, dtype = 1, 12, 4096, 64, BF16
        n = over.get("n", n); H = over.get("H", H); d = over.get("d", d)
        dtype = over.get("dtype", dtype)
        row_ptr, col_idx = window_pattern(n, over.get("window", 128),
                                          over.get("global_tokens", (0, 1)))
        block = 1
    elif name == "random_n8192":
        B, H, n, d, dtype = 1, 16, 8192, 64, BF16
        n = over.get("n", n); H = over.get("H", H); d = over.get("d", d)
        dtype = over.get("dtype", dtype)
        row_ptr, col_idx = random_rows_pattern(n, over.get("kmin", 32), over.get("kmax", 512),
                                               rng_mask)
        block = 1
    elif name == "bsr_n16384":
        B, H, n, d, dtype = 1, 16, 16384, 128, BF16
        n = over.get("n", n); H = over.get("H", H); d = over.get("d", d)
        dtype = over.get("dtype", dtype)
        row_ptr, col_idx = bsr_pattern(n, over.get("extra", 8), rng_mask)
        block = BLOCK
    elif name == "evoformer_l384":
        B, H, n, d, dtype = 32, 8, 384, 32, BF16
        B = over.get("B", B); n = over.get("n", n); H = over.get("H", H); d = over.get("d", d)
        dtype = over.get("dtype", dtype)
        row_ptr, col_idx = None, None
        block = 1
    else:
        raise KeyError(name)
    B = over.get("B", B)

    (q, qb), (k, kb), (v, vb) = _qkv(rng_qkv, B * H, n, d, dtype)
    bias = None
    key_mask = None
    if over.get("bias", name == "evoformer_l384"):
        bias = rng_bias.standard_normal((H, n, n), dtype=np.float32)
    if over.get("key_mask", name == "evoformer_l384"):
        key_mask = key_padding_mask(B, n, over.get("pmax", 64), rng_kpm)
    scale = over.get("scale", 1.0 / math.sqrt(d))
    return Problem(name=name, B=B, H=H, n=n, d=d, dtype=dtype, q=q, k=k, v=v,
                   row_ptr=row_ptr, col_idx=col_idx, block=block, scale=float(scale),
                   bias=bias, key_mask=key_mask, key_mask_heads=1, seed=seed,
                   q_bits=qb, k_bits=kb, v_bits=vb)


def random_scores(BH: int, nnz: int, seed: int, spread: float = 3.0) -> np.ndarray:
    """fp32 scores [BH, nnz] ~ spread * N(0,1): a seeded input for the softmax step alone."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    return (spread * rng.standard_normal((BH, nnz))).astype(np.float32)


def random_weights(BH: int, nnz: int, seed: int) -> np.ndarray:
    """fp32 nonnegative values [BH, nnz] ~ U[0,1): a seeded input for the SpMM step alone."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    return rng.random((BH, nnz), dtype=np.float32)
