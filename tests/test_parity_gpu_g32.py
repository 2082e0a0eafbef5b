"""GPU parity at group size 32 (one bf16 scale per output row per 32 k): the
tile kernel's 32-group mode, called through the C ABI, against the CPU
oracle with the same group size, on the same seeded inputs and with the same
gate as the 128-group tests (max|y - y_ref| <= 4e-3 * max|y_ref| + 1e-3,
cos >= 0.99999).

The quantisation follows the per-GEMM table of the gfx1151 skinny-GEMM page
("Benchmark results (per-GEMM)": the decoder GEMMs at M = 1322 with one
scale per 32 k).
"""
import numpy as np
import pytest
import torch

import bf16_activation_quantized_amd as w4
import oracle
from synth import make_inputs
from gpu_util import DevCase, bits_host, check_full, check_gate, nan_filled

pytestmark = pytest.mark.gpu

G32 = 32


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4._lib()   # raises if the HIP library is missing: no fallback


def _gemm(d, **kw):
    y = w4.w4a16_gemm(d.x, d.w, d.s, group_size=G32, **kw)
    torch.cuda.synchronize()
    return bits_host(y)


TILE_CASES = [
    # M, N, K, split_k, rows per tile (None = automatic)
    (1, 256, 128, 0, None),     # decode row count: the tile kernel at M = 1
    (16, 300, 512, 0, None),
    (17, 100, 128, 1, 128),       # one 128-k stage (4 scale groups), M and N tails
    (130, 256, 256, 1, 128),
    (300, 1000, 640, 1, 128),     # steady state, N tail of 232 columns
    (129, 513, 384, 2, 128),      # split-K slices of 2 and 1 stages, N * K/32 odd rows
    (257, 300, 256, 8, 128),      # more slices than stages: empty slices write zeros
    (1322, 512, 2560, 1, 128),    # the prefill row count and depth
    (97, 256, 256, 1, 96),       # one row past a 96-row tile
    (300, 1000, 640, 1, 96),
    (95, 129, 512, 0, 96),
    (113, 256, 256, 1, 112),      # one row past a 112-row tile
    (1322, 512, 2560, 1, 112),
    (224, 257, 384, 4, 112),
    (81, 256, 256, 1, 80),       # one row past an 80-row tile
    (300, 1000, 640, 2, 80),
    (1322, 512, 2560, 1, 80),
    (600, 700, 1280, 0, None),
    (64, 64, 1024, 4, None),
    (130, 300, 16384, 0, None),   # 512 scale groups per row, automatic split
    (40, 257, 16384, 16, 80),      # 16 slices of 8 stages, N * K/32 odd rows
]


@pytest.mark.parametrize("M,N,K,sk,cfg", TILE_CASES)
def test_g32_tile_parity(M, N, K, sk, cfg):
    c = make_inputs(M, N, K, seed=M + N * 3 + K + 32, group=G32)
    assert c.s.shape == (N, K // G32)
    d = DevCase(c)
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, group_size=G32, split_k=sk,
                  path=w4.PATH_TILE if cfg is not None else None, variant=cfg)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s, G32), f"g32 tile M={M} N={N} K={K} sk={sk} rows={cfg}")


@pytest.mark.parametrize("prepass", [True, False])
@pytest.mark.parametrize("M,N,K,sk,rows", [(130, 2048, 512, 1, 128), (97, 2049, 384, 2, 80), (1, 2304, 256, 1, 96)])
def test_g32_rowsum_paths(M, N, K, sk, rows, prepass):
    # from 8 column tiles the 32-group row sums come from the pre-pass when the
    # workspace has room for them, else the tile kernel forms them
    c = make_inputs(M, N, K, seed=M + N + K + 320, group=G32)
    d = DevCase(c)
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, sk, path=w4.PATH_TILE, variant=rows, group_size=G32)
    split = (sk * M * N * 4 + 255) // 256 * 256 if sk > 1 else 0
    assert need > split
    ws = torch.full(((need if prepass else max(split, 16)) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws, path=w4.PATH_TILE, variant=rows, group_size=G32)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s, G32), f"g32 M={M} N={N} K={K} sk={sk} pre-pass={prepass}")


def test_g32_scales_differ_within_a_stage():
    # 4 different scales per 128 k: a kernel that used one scale per 128 k
    # (or the scales of the wrong 32-group) fails this gate. Scale group j of
    # every row is 2^-(j mod 4 + 4), so mixing any two groups of a stage
    # changes the result by at least a factor 2 in some term.
    M, N, K = 130, 300, 512
    c = make_inputs(M, N, K, seed=3232, group=G32)
    ex = 0x3D80 - (np.arange(K // G32) % 4) * 0x80     # bf16 2^-4, 2^-5, 2^-6, 2^-7
    c.s[:] = ex.astype(np.uint16)[None, :]
    d = DevCase(c)
    for cfg in (128, 96, 112, 80):
        y = _gemm(d, split_k=1, path=w4.PATH_TILE, variant=cfg)
        ref = oracle.gemm(c.x, d.p_host, c.s, G32)
        check_gate(y, ref, f"g32 stepped scales cfg={cfg}")
        wrong = oracle.gemm(c.x, d.p_host, c.s[:, ::4], 128)   # one scale per 128 k
        assert not oracle.gate(y, wrong)["ok"]


@pytest.mark.parametrize("sk", [1, 2])
def test_g32_degenerate_zero_outputs(sk):
    M, N, K = 40, 256, 384
    c = make_inputs(M, N, K, seed=88, group=G32)
    # q == 8 everywhere: the oracle gives exactly 0; the tile kernel forms
    # -136 * sum(x) + sum(136 * x) per 32-group in two fp32 summation orders,
    # so only a rounding residue far below the gate's absolute term remains
    zero_q = DevCase(type(c)(x=c.x, q=np.full_like(c.q, 8), s=c.s, group_size=G32))
    y8 = oracle.bf16_to_f64(_gemm(zero_q, split_k=sk))
    assert np.all(np.isfinite(y8)) and float(np.max(np.abs(y8))) <= 1e-3
    zero_s = DevCase(type(c)(x=c.x, q=c.q, s=np.zeros_like(c.s), group_size=G32))
    assert np.all((_gemm(zero_s, split_k=sk) & 0x7FFF) == 0)        # s == 0 -> +-0
    zero_x = DevCase(type(c)(x=np.zeros_like(c.x), q=c.q, s=c.s, group_size=G32))
    assert np.all((_gemm(zero_x, split_k=sk) & 0x7FFF) == 0)


def test_g32_n1_k128_and_m0():
    for M in (1, 3, 20):
        c = make_inputs(M, 1, 128, seed=M + 32, group=G32)
        d = DevCase(c)
        check_gate(_gemm(d), oracle.gemm(c.x, d.p_host, c.s, G32), f"g32 N=1 K=128 M={M}")
    # M = 0: nothing is enqueued and no byte of the buffer behind y is written
    c = make_inputs(1, 64, 256, seed=5, group=G32)
    d = DevCase(c)
    buf = nan_filled((16, 64))
    before = bits_host(buf)
    w4.w4a16_gemm(d.x[:0], d.w, d.s, y=buf[:0], group_size=G32)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(buf), before)


GROUPED_CASES = [
    # m_sizes, N, K, rows per tile (None = automatic)
    ([37], 256, 384, None),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, None),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 128),
    ([96, 97, 95, 0, 1], 256, 640, 96),
    ([112, 113, 111, 0, 1], 256, 640, 112),
    ([80, 81, 79, 0, 1], 256, 640, 80),
    ([5, 70, 33], 257, 384, 128),     # N * K/32 odd per weight group
    ([0, 0, 0, 50], 128, 128, None),
]


@pytest.mark.parametrize("ms,N,K,cfg", GROUPED_CASES)
def test_g32_grouped_parity(ms, N, K, cfg):
    c = make_inputs(sum(ms), N, K, seed=len(ms) * 31 + N + K + 32, G=len(ms), m_sizes=ms, group=G32)
    d = DevCase(c)
    y = nan_filled((sum(ms), N))
    w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y, variant=cfg, group_size=G32)
    ref = oracle.gemm_grouped(c.x, d.p_host, c.s, c.m_sizes, G32)
    check_full(y, ref, f"g32 grouped {ms} N={N} K={K} rows={cfg}")


BATCHED_CASES = [
    # B, M, N, K, split_k, rows per tile (None = automatic)
    (3, 1, 256, 512, 0, None),
    (4, 16, 300, 640, 2, None),
    (2, 130, 513, 384, 0, None),
    (3, 97, 257, 256, 4, 96),
    (2, 113, 300, 256, 2, 112),
    (3, 100, 300, 384, 1, 80),
]


@pytest.mark.parametrize("B,M,N,K,sk,cfg", BATCHED_CASES)
def test_g32_batched_parity(B, M, N, K, sk, cfg):
    c = make_inputs(B * M, N, K, seed=B * 1000 + M + N + K + 32, G=B, m_sizes=[M] * B, group=G32)
    d = DevCase(c)
    y = nan_filled((B, M, N))
    w4.w4a16_gemm_batched(d.x.view(B, M, K), d.w, d.s, y=y, split_k=sk, variant=cfg, group_size=G32)
    ref = oracle.gemm_batched(c.x.reshape(B, M, K), d.p_host, c.s, G32)
    check_full(y, ref, f"g32 batched B={B} M={M} N={N} K={K} sk={sk}")
    yb = bits_host(y.view(B * M, N)).reshape(B, M, N)
    for b in range(B):
        check_gate(yb[b], ref[b], f"g32 batched B={B} M={M} N={N} K={K} sk={sk} problem {b}")


def test_g32_repeat_bitwise_and_graph_replay():
    M, N, K = 300, 1000, 1280
    c = make_inputs(M, N, K, seed=77, group=G32)
    d = DevCase(c)
    ws = torch.empty(w4.w4a16_gemm_workspace_bytes(M, N, K, 4, group_size=G32) // 4 + 1,
                     dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=4, workspace=ws, group_size=G32)
    torch.cuda.synchronize()
    y0 = bits_host(y)
    check_gate(y0, oracle.gemm(c.x, d.p_host, c.s, G32), "g32 split 4")
    for _ in range(2):
        w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=4, workspace=ws, group_size=G32)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), y0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=4, workspace=ws, group_size=G32)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        y.fill_(0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), y0), f"replay {i}"


# ------------------------------------------------------------------ the four decoder GEMMs, full size

LAYER_GEMMS = [
    # name, N, K (the per-GEMM table of the gfx1151 page, M = 1322)
    ("gate_up", 19456, 2560),
    ("qkv", 6144, 2560),
    ("o_proj", 4096, 2560),
    ("down", 2560, 9728),
]


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("name,N,K", LAYER_GEMMS)
def test_layer_gemm_full_size(name, N, K, group):
    # default path, tile choice and split (what the per-layer bench times),
    # the whole output against the oracle, every element written
    M = 1322
    c = make_inputs(M, N, K, seed=1322 + N + K, group=group)
    d = DevCase(c)
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, group_size=group)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s, group), f"g{group} {name} {M}x{N}x{K}")
