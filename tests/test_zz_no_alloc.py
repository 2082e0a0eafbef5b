"""GPU check of w4a16_gemm_noalloc (the entry point for callers that cannot
allocate): called through the C ABI, its output against w4a16_gemm's with a
workspace of w4a16_gemm_workspace_bytes (the same kernels: bit for bit) and
against the oracle's gate, on two calls in a row, the second on a smaller
input; sizes beyond the scratch are rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import bf16_activation_quantized_amd as w4
import oracle
from synth import make_inputs
from gpu_util import DevCase, bits_host, check_full, nan_filled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4._lib()


def _noalloc(d, M, N, K, sk, group):
    """The entry point through ctypes, on a NaN-filled y; returns y."""
    y = nan_filled((M, N))
    L = w4._lib()
    st = L.w4a16_gemm_noalloc(w4._ptr(d.x), w4._ptr(d.w), w4._ptr(d.s), w4._ptr(y), M, N, K, group, sk,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, w4.status_string(st)
    return y


def _reference(d, M, N, K, sk, group):
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, sk, group_size=group)
    assert need <= w4.NOALLOC_SCRATCH_BYTES
    ws = torch.full((max(need // 4, 1) + 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws, group_size=group)
    return y


# pairs of calls in a row, the second smaller: (first, second), each (M, N, K, split_k, group)
PAIRS = [
    ((16, 8192, 8192, 8, 128), (5, 1000, 1024, 2, 128)),      # small batch, split-K partials in the scratch
    ((1, 17408, 5120, 2, 128), (1, 300, 1280, 4, 128)),       # GEMV with split-K
    ((100, 8192, 640, 2, 128), (129, 8448, 384, 1, 128)),     # tile: partials + pre-pass row sums
    ((1322, 8192, 2560, 0, 128), (200, 8192, 1280, 0, 128)),  # tile, automatic split, pre-pass row sums
    ((130, 2048, 512, 2, 32), (40, 257, 384, 4, 32)),         # group 32
    ((64, 300, 640, 0, 128), (17, 100, 128, 1, 128)),         # no scratch needed at all
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemm_on_two_calls(first, second):
    for (M, N, K, sk, group), seed in ((first, 1), (second, 2)):
        c = make_inputs(M, N, K, seed=seed * 1000 + M + N + K, group=group)
        d = DevCase(c)
        y = _noalloc(d, M, N, K, sk, group)
        ref = _reference(d, M, N, K, sk, group)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), bits_host(ref)), (M, N, K, sk, group)
        check_full(y, oracle.gemm(c.x, d.p_host, c.s, group), f"noalloc M={M} N={N} K={K} sk={sk} g={group}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 16 x 65536 x 8 slices of fp32 partials = 32 MiB > the 16 MiB scratch:
    # rejected on the host, nothing enqueued (y keeps its NaNs)
    M, N, K = 16, 65536, 1024
    c = make_inputs(M, N, K, seed=9)
    d = DevCase(c)
    y = nan_filled((M, N))
    L = w4._lib()
    st = L.w4a16_gemm_noalloc(w4._ptr(d.x), w4._ptr(d.w), w4._ptr(d.s), w4._ptr(y), M, N, K, 128, 8, None)
    assert st == 5                                        # W4A16_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.all((bits_host(y) & 0x7FFF) > 0x7F80)
