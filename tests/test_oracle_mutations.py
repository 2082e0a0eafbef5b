"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies the oracle's source, applies one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, ...), loads the
copy as a separate module and checks that at least one pin fails on it. The
real oracle is never modified.
"""
import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "w4a16_ref.py")

MUTATIONS = {
    "nibble_order_swapped": (
        "q[..., 0::2] = p & np.uint8(0x0F)\n    q[..., 1::2] = p >> np.uint8(4)",
        "q[..., 1::2] = p & np.uint8(0x0F)\n    q[..., 0::2] = p >> np.uint8(4)"),
    "pack_order_swapped": (
        "return (lo | (hi << np.uint8(4))).astype(np.uint8)",
        "return (hi | (lo << np.uint8(4))).astype(np.uint8)"),
    "offset_dropped": ("* (q - 8.0)", "* (q - 0.0)"),
    "offset_sign": ("* (q - 8.0)", "* (q + 8.0)"),
    "offset_off_by_one": ("* (q - 8.0)", "* (q - 7.0)"),
    "scale_group_64": ("np.repeat(s, group, axis=-1)",
                       "np.tile(np.repeat(s, group // 2, axis=-1), 2)"),
    "scale_tiled_not_repeated": ("np.repeat(s, group, axis=-1)",
                                 "np.tile(s, group)"),
    "gemm_group_ignored": ("wd = dequant(p, s_bits, group)\n    if x.shape[1]",
                           "wd = dequant(p, np.repeat(s_bits[..., ::128 // group], 1, axis=-1), 128)\n    if x.shape[1]"),
    "entries_group_ignored": ("wd = dequant(p[ucols], s_bits[ucols], group)",
                              "wd = dequant(p[ucols], s_bits[ucols][..., ::128 // group], 128)"),
    "grouped_group_dropped": ("y[r0:r1] = gemm(x_bits[r0:r1], p[g], s_bits[g], group)",
                              "y[r0:r1] = gemm(x_bits[r0:r1], p[g], s_bits[g][..., ::128 // group])"),
    "batched_group_dropped": ("gemm(x_bits[b], p[b], s_bits[b], group) for b in range(B)",
                              "gemm(x_bits[b], p[b], s_bits[b][..., ::128 // group]) for b in range(B)"),
    "transposed_operand": ("return x @ wd.T", "return (wd @ x.T).T[:, ::-1]"),
    "bf16_low_half": ("astype(np.uint32) << np.uint32(16)",
                      "astype(np.uint32) << np.uint32(15)"),
    "rne_truncates": ("up = (low > half) | ((low == half) & ((keep & np.uint64(1)) == np.uint64(1)))",
                      "up = low > np.uint64(0xFFFF)"),
    "rne_ties_away": ("up = (low > half) | ((low == half) & ((keep & np.uint64(1)) == np.uint64(1)))",
                      "up = low >= half"),
    "splitk_floor": ("c = -(-num_groups // split_k)", "c = max(1, num_groups // split_k)"),
    "splitk_slice_k_unscaled": ("k0, k1 = g0 * group, g1 * group", "k0, k1 = g0, g1"),
    "reduce_skips_last": ("for s in range(1, ws.shape[0]):", "for s in range(1, ws.shape[0] - 1):"),
    "starts_inclusive": ("return np.cumsum(ms) - ms", "return np.cumsum(ms)"),
    "grouped_wrong_weights": ("y[r0:r1] = gemm(x_bits[r0:r1], p[g], s_bits[g], group)",
                              "y[r0:r1] = gemm(x_bits[r0:r1], p[0], s_bits[0], group)"),
    "batched_wrong_weights": ("gemm(x_bits[b], p[b], s_bits[b], group) for b in range(B)",
                              "gemm(x_bits[b], p[0], s_bits[b], group) for b in range(B)"),
    "batched_wrong_scales": ("gemm(x_bits[b], p[b], s_bits[b], group) for b in range(B)",
                             "gemm(x_bits[b], p[b], s_bits[B - 1 - b], group) for b in range(B)"),
    "gate_no_abs": ("max_err = float(np.max(np.abs(y - r)))", "max_err = float(np.max(y - r))"),
}


def _mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:   # AssertionError or a shape error both count
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
