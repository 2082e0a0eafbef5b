"""Seeded input generator for the W4A16 GEMM workloads.

Distributions follow the workloads the pages benchmark (the fused gate_up
prefill shape of "[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for
gfx1151", Benchmark results (per-GEMM); the decode projection dims of
"gfx1151: 61.7% of ... per-token byte budget runs KQuantGemmK with 8-12 of 32
lanes idle", The byte budget): no checkpoint is involved, so every tensor is
drawn here.

Recipe, per workload, with one fresh ``numpy.random.default_rng(seed)``
(PCG64) and this fixed draw order:

1. grouped only: ``M_sizes`` -- a multinomial split of ``M_total`` over the
   non-empty groups (equal probabilities), forced-empty groups get 0 (the
   batched workload: B groups of M rows, no draw);
2. ``X``: float32 standard normal ``[M, K]``, rounded to bf16;
3. ``q``: uniform integers 0..15 ``[N, K]`` (``[G, N, K]`` grouped), one
   unsigned nibble per byte, not packed;
4. ``S``: uniform on [0.005, 0.02) in float64, cast to float32, rounded to
   bf16, ``[N, K/g]`` (``[G, N, K/g]`` grouped) for the group size g (128,
   or 32 for the per-layer workloads at group 32).

The float32 -> bf16 rounding of the draws is done by PyTorch's CPU
conversion (round to nearest even), i.e. by a library routine, so this module
contains none of the method's own arithmetic. bf16 tensors are carried as
their raw uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

GROUP = 128

# The six workloads, by what they are.
CONFIGS = {
    "tiny": dict(M=1, N=256, K=512),
    "decode_gemv": dict(M=1, N=17408, K=5120),
    "decode_splitk": dict(M=16, N=8192, K=8192),
    "prefill": dict(M=1322, N=19456, K=2560),
    "grouped": dict(G=8, M_total=2048, N=2048, K=4096, empty=(2, 5)),
    # B independent problems of M rows (the grouped shape, split evenly)
    "batched": dict(B=8, M=256, N=2048, K=4096),
}


@dataclass
class Inputs:
    x: np.ndarray            # uint16 bf16 bits, [M, K]
    q: np.ndarray            # uint8 nibble values 0..15, [N, K] or [G, N, K]
    s: np.ndarray            # uint16 bf16 bits, [N, K/128] or [G, N, K/128]
    m_sizes: Optional[np.ndarray] = None   # int32 [G] (grouped only)
    group_size: int = GROUP

    @property
    def M(self) -> int:
        return int(self.x.shape[0])

    @property
    def K(self) -> int:
        return int(self.x.shape[1])

    @property
    def N(self) -> int:
        return int(self.q.shape[-2])

    @property
    def G(self) -> Optional[int]:
        return None if self.m_sizes is None else int(self.m_sizes.shape[0])


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(M: int, N: int, K: int, seed: int = 0, *,
                G: Optional[int] = None,
                m_sizes: Optional[Sequence[int]] = None,
                empty: Sequence[int] = (),
                x_scale: float = 1.0,
                s_range=(0.005, 0.02),
                group: int = GROUP) -> Inputs:
    """Draw one workload. For grouped inputs give ``G`` and either explicit
    ``m_sizes`` (then ``M`` must equal their sum) or ``M`` as ``M_total`` to
    split multinomially over the groups not listed in ``empty``."""
    if K % GROUP or GROUP % group:
        raise ValueError("K must be a multiple of 128 and the group size divide 128")
    rng = np.random.default_rng(seed)
    ms = None
    if G is not None:
        if m_sizes is not None:
            ms = np.asarray(m_sizes, dtype=np.int32)
            if ms.shape != (G,) or int(ms.sum()) != M:
                raise ValueError("m_sizes must have G entries summing to M")
        else:
            live = [g for g in range(G) if g not in set(empty)]
            ms = np.zeros(G, dtype=np.int32)
            if live:
                ms[live] = rng.multinomial(M, [1.0 / len(live)] * len(live))
    x = rng.standard_normal((M, K), dtype=np.float32)
    if x_scale != 1.0:
        x = (x * np.float32(x_scale)).astype(np.float32)
    wshape = (N, K) if G is None else (G, N, K)
    q = rng.integers(0, 16, wshape, dtype=np.uint8)
    s = rng.uniform(s_range[0], s_range[1], wshape[:-1] + (K // group,))
    return Inputs(x=_to_bf16_bits(x), q=q,
                  s=_to_bf16_bits(s.astype(np.float32)), m_sizes=ms, group_size=group)


def make_config(name: str, seed: int = 0) -> Inputs:
    c = CONFIGS[name]
    if "B" in c:   # batched: the grouped layout with B groups of M rows each
        return make_inputs(c["B"] * c["M"], c["N"], c["K"], seed, G=c["B"],
                           m_sizes=[c["M"]] * c["B"])
    if "G" in c:
        return make_inputs(c["M_total"], c["N"], c["K"], seed, G=c["G"],
                           empty=c["empty"])
    return make_inputs(c["M"], c["N"], c["K"], seed)


def make_workspace(SK: int, M: int, N: int, seed: int = 0,
                   tie_fraction: float = 0.25) -> np.ndarray:
    """A float32 ``[SK, M, N]`` split-K workspace for exercising the reduce
    step on its own. A ``tie_fraction`` of the (m, n) entries are built to sit
    exactly half-way between two neighbouring bf16 values in slice 0 with the
    other slices zero, so that round-to-nearest-even ties are reached."""
    rng = np.random.default_rng(seed)
    ws = (rng.standard_normal((SK, M, N), dtype=np.float32) * np.float32(8.0))
    ws = ws.astype(np.float32)
    flat = ws.reshape(SK, -1)
    n_tie = int(flat.shape[1] * tie_fraction)
    if n_tie:
        idx = rng.choice(flat.shape[1], n_tie, replace=False)
        hi = rng.integers(0x0080, 0x7F00, n_tie, dtype=np.uint32)
        sign = rng.integers(0, 2, n_tie, dtype=np.uint32) << 15
        bits = ((hi | sign) << 16) | np.uint32(0x8000)
        flat[0, idx] = bits.view(np.float32)
        flat[1:, idx] = 0.0
    return ws
