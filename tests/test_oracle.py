"""The CPU oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins

pytestmark = []


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_no_pin_is_missing():
    # every public oracle function is exercised by at least one pin
    import inspect
    src = "".join(inspect.getsource(p) for p in oracle_pins.ALL_PINS)
    for name in oracle.__all__ if hasattr(oracle, "__all__") else [
            "bf16_to_f64", "f32_to_bf16_rne", "pack_int4", "unpack_int4",
            "dequant", "gemm", "gemm_entries", "splitk_group_ranges",
            "gemm_splitk_partials", "splitk_reduce_bf16", "group_starts",
            "gemm_grouped", "gemm_batched", "gate"]:
        assert f"o.{name}(" in src, name
