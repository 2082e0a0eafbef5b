"""CPU oracle for the W4A16 GEMM -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. It shares no code with the HIP library
(no kernels, headers, helpers, tables or constants) and never imports it.

What it computes is the plain definition the method reaches faster:

    Y[m, n] = sum_k X[m, k] * Wd[n, k],    Wd[n, k] = S[n, k // 128] * (q[n, k] - 8)

in float64, with no rounding of the dequantised weights, of partial sums or of
the output. Sources (pages by title; sections in quotes):

* "Add Triton BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950", Summary and
  Implementation "Fused A-operand dot": the op is bf16 activations times a
  row-major packed int4 weight; the low nibble of a byte goes with the even-K
  activation and the high nibble with the odd-K activation.
* "[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for gfx1151", section 1
  "Magic-constant bf16 dequant": a nibble n decodes as scale * (n - 8); the
  benchmarks there are "symmetric" (no zero-point tensor).
* The 128-wide K group with one bf16 scale per output row per group, stored
  row-major ``[N, K/128]``, is the plainest reading of the scale tensor whose
  byte size (rows * groups * 2) the same page gives in section 3 "Exact
  buffer-descriptor sizing".
* Split-K and the reduce: "Add Triton BF16xINT4 ...", Implementation "Split-K
  without atomics" -- fp32 partial sums in a ``[SPLIT_K, M, N]`` workspace,
  summed by a separate reduce step and cast to bf16.
* Grouped: same page, Implementation "Native fused grouped kernel" -- group g
  owns rows ``[start_g, start_g + M_sizes[g])`` with
  ``start = cumsum(M_sizes) - M_sizes``.
* Batched: same page, Summary (the batched op beside the plain and grouped
  ones) -- B independent problems of one shape, ``Y[b] = X[b] . Wd_b^T``.

Readings where the pages are silent (each is listed with its reason in the
design notes): split-K slices are contiguous runs of whole 128-groups, each
``ceil(G_k / SK)`` groups long (trailing slices may be empty and then hold
zeros); the reduce sums slices in order s = 0..SK-1 in float32 and rounds to
bf16 to nearest-even; the grouped weights and scales are ``[G, N, K/2]`` and
``[G, N, K/128]``.

Every function below is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle.py`` against printed constants, closed forms, invariants
and brute force; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

GROUP = 128


# ---------------------------------------------------------------- bf16 bits

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64. A bf16 value is the upper half
    of the float32 with the same bits, so the conversion is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN
    (quiet), overflow goes to infinity. Written from the definition of RNE on
    the 16 discarded low bits: round up when they exceed half, or equal half
    and the kept LSB is odd."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    up = (low > half) | ((low == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    out = (keep + up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(a)
    out[nan] = ((u[nan] >> np.uint64(16)).astype(np.uint32) | np.uint32(0x0040))
    return out.astype(np.uint16)


# ---------------------------------------------------------------- int4 packing

def pack_int4(q: np.ndarray) -> np.ndarray:
    """q[..., K] (values 0..15, high bits ignored) -> P[..., K/2] with
    P[..., j] = q[..., 2j] | q[..., 2j+1] << 4 (low nibble = even k)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    lo = q[..., 0::2] & np.uint8(0x0F)
    hi = q[..., 1::2] & np.uint8(0x0F)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """P[..., K/2] -> q[..., K]: even k from the low nibble, odd k from the
    high nibble."""
    p = np.asarray(p, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = p & np.uint8(0x0F)
    q[..., 1::2] = p >> np.uint8(4)
    return q


# ---------------------------------------------------------------- dequant / GEMM

def dequant(p: np.ndarray, s_bits: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Wd[..., n, k] = S[..., n, k // group] * (q[..., n, k] - 8), float64,
    exact (a bf16 scale times an integer in [-8, 7] fits a double)."""
    q = unpack_int4(p).astype(np.float64)
    s = bf16_to_f64(s_bits)
    K = q.shape[-1]
    if K % group or s.shape[-1] != K // group:
        raise ValueError("scale shape does not match K / group")
    return np.repeat(s, group, axis=-1) * (q - 8.0)


def gemm(x_bits: np.ndarray, p: np.ndarray, s_bits: np.ndarray,
         group: int = GROUP) -> np.ndarray:
    """Y = X . Wd^T in float64. X [M, K] bf16 bits, P [N, K/2], S [N, K/g]."""
    x = bf16_to_f64(x_bits)
    wd = dequant(p, s_bits, group)
    if x.shape[1] != wd.shape[1]:
        raise ValueError("K mismatch")
    return x @ wd.T


def gemm_entries(x_bits: np.ndarray, p: np.ndarray, s_bits: np.ndarray,
                 rows: np.ndarray, cols: np.ndarray,
                 group: int = GROUP) -> np.ndarray:
    """Y[rows[i], cols[i]] one by one (for sampled checks at full size)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(rows.shape[0], dtype=np.float64)
    ucols, inv = np.unique(cols, return_inverse=True)
    wd = dequant(p[ucols], s_bits[ucols], group)
    for i in range(rows.shape[0]):
        out[i] = float(bf16_to_f64(x_bits[rows[i]]) @ wd[inv[i]])
    return out


# ---------------------------------------------------------------- split-K

def splitk_group_ranges(num_groups: int, split_k: int) -> List[Tuple[int, int]]:
    """Slice s covers K-groups [s*c, min((s+1)*c, num_groups)) with
    c = ceil(num_groups / split_k); trailing slices may be empty."""
    if split_k < 1:
        raise ValueError("split_k must be >= 1")
    c = -(-num_groups // split_k)
    return [(min(s * c, num_groups), min((s + 1) * c, num_groups))
            for s in range(split_k)]


def gemm_splitk_partials(x_bits: np.ndarray, p: np.ndarray, s_bits: np.ndarray,
                         split_k: int, group: int = GROUP) -> np.ndarray:
    """[SK, M, N] float64: slice s holds the sum restricted to its K range
    (zeros for an empty slice)."""
    x = bf16_to_f64(x_bits)
    wd = dequant(p, s_bits, group)
    G = x.shape[1] // group
    out = np.zeros((split_k, x.shape[0], wd.shape[0]), dtype=np.float64)
    for s, (g0, g1) in enumerate(splitk_group_ranges(G, split_k)):
        if g1 > g0:
            k0, k1 = g0 * group, g1 * group
            out[s] = x[:, k0:k1] @ wd[:, k0:k1].T
    return out


def splitk_reduce_bf16(ws: np.ndarray) -> np.ndarray:
    """Reduce of a float32 workspace [SK, M, N]: float32 sum in slice order
    s = 0..SK-1, then round to bf16 (nearest even). Returns bf16 bits."""
    ws = np.asarray(ws, dtype=np.float32)
    acc = ws[0].copy()
    for s in range(1, ws.shape[0]):
        acc = (acc + ws[s]).astype(np.float32)
    return f32_to_bf16_rne(acc)


# ---------------------------------------------------------------- grouped

def group_starts(m_sizes: Sequence[int]) -> np.ndarray:
    """Exclusive prefix sum: start_g = sum_{h<g} M_sizes[h]."""
    ms = np.asarray(m_sizes, dtype=np.int64)
    return np.cumsum(ms) - ms


def gemm_grouped(x_bits: np.ndarray, p: np.ndarray, s_bits: np.ndarray,
                 m_sizes: Sequence[int], group: int = GROUP) -> np.ndarray:
    """Rows [start_g, start_g + M_sizes[g]) of Y are those rows of X times
    Wd_g^T, with P [G, N, K/2] and S [G, N, K/g]. Empty groups add nothing."""
    ms = np.asarray(m_sizes, dtype=np.int64)
    starts = group_starts(ms)
    M_total = int(ms.sum())
    if x_bits.shape[0] != M_total:
        raise ValueError("X rows must equal sum(M_sizes)")
    N = p.shape[1]
    y = np.zeros((M_total, N), dtype=np.float64)
    for g in range(ms.shape[0]):
        r0, r1 = int(starts[g]), int(starts[g] + ms[g])
        if r1 > r0:
            y[r0:r1] = gemm(x_bits[r0:r1], p[g], s_bits[g], group)
    return y


def gemm_batched(x_bits: np.ndarray, p: np.ndarray, s_bits: np.ndarray,
                 group: int = GROUP) -> np.ndarray:
    """Y[b] = X[b] . Wd_b^T for X [B, M, K], P [B, N, K/2], S [B, N, K/g]:
    each problem is the plain definition on its own operands."""
    B = x_bits.shape[0]
    if p.shape[0] != B or s_bits.shape[0] != B:
        raise ValueError("X, P and S must hold the same number of problems")
    return np.stack([gemm(x_bits[b], p[b], s_bits[b], group) for b in range(B)])


# ---------------------------------------------------------------- the gate

def gate(y_bits: np.ndarray, y_ref: np.ndarray, rel: float = 4e-3,
         abs_: float = 1e-3, min_cos: float = 0.99999) -> dict:
    """The acceptance test for a bf16 result against the float64 reference:
    max|y - y_ref| <= rel * max|y_ref| + abs_ and cos(y, y_ref) >= min_cos,
    both over the flattened arrays in float64. A non-finite y fails."""
    y = bf16_to_f64(y_bits).ravel()
    r = np.asarray(y_ref, dtype=np.float64).ravel()
    if y.shape != r.shape:
        raise ValueError("shape mismatch")
    finite = bool(np.all(np.isfinite(y)))
    if y.size == 0:
        return dict(ok=True, max_err=0.0, tol=abs_, cos=1.0, finite=True)
    max_err = float(np.max(np.abs(y - r))) if finite else math.inf
    tol = rel * float(np.max(np.abs(r))) + abs_
    ny, nr = float(np.linalg.norm(y)), float(np.linalg.norm(r))
    if ny == 0.0 and nr == 0.0:
        cos = 1.0
    elif ny == 0.0 or nr == 0.0 or not finite:
        cos = 0.0
    else:
        cos = float(np.dot(y, r) / (ny * nr))
    return dict(ok=bool(finite and max_err <= tol and cos >= min_cos),
                max_err=max_err, tol=tol, cos=cos, finite=finite)
