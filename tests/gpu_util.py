"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its binding, bring bf16 results back as bit patterns."""
from __future__ import annotations

import numpy as np
import torch

import bf16_activation_quantized_amd as w4
import oracle


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DevCase:
    """Device copies of one seeded case; the weights are packed by the
    library's own pack kernel (checked bit-exact against the oracle's
    packer by the caller when wanted)."""

    def __init__(self, c):
        self.c = c
        self.x = bf16_dev(c.x)
        self.q = u8_dev(c.q)
        self.s = bf16_dev(c.s)
        self.w = w4.w4a16_pack_int4(self.q)
        self.m_sizes = None if c.m_sizes is None else torch.from_numpy(c.m_sizes).to(dev())
        self.p_host = oracle.pack_int4(c.q)

    def packed_matches_oracle(self) -> bool:
        return np.array_equal(self.w.cpu().numpy(), self.p_host)


def check_gate(y_bits: np.ndarray, y_ref: np.ndarray, what: str):
    g = oracle.gate(y_bits, y_ref)
    assert g["ok"], f"{what}: {g}"
    return g


BF16_NAN = 0x7FC0


def nan_filled(shape) -> torch.Tensor:
    """A bf16 device tensor filled with NaN: outputs that a kernel never
    writes stay NaN, which the gate's finiteness check then catches."""
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=dev())


def check_full(y: torch.Tensor, y_ref: np.ndarray, what: str):
    """Every output element written (finite) and the whole output against the
    oracle's."""
    torch.cuda.synchronize()
    yb = bits_host(y).reshape(y_ref.shape)
    unwritten = int(np.count_nonzero((yb & 0x7FFF) > 0x7F80))
    assert unwritten == 0, f"{what}: {unwritten} outputs left NaN (never written)"
    return check_gate(yb, y_ref, what)
