"""GPU parity: the HIP library (called through its C ABI) against the CPU
oracle, on the same seeded inputs.

Floating-point results must pass the gate max|y - y_ref| <= 4e-3 * max|y_ref|
+ 1e-3 and cos >= 0.99999 against the float64 oracle; integer work (packing)
and the reduce step (float32 sum in slice order, then round to nearest even,
decided in the same precision on both sides) must be bit-exact.
"""
import numpy as np
import pytest
import torch

import bf16_activation_quantized_amd as w4
import oracle
from synth import make_config, make_inputs, make_workspace
from gpu_util import DevCase, bf16_dev, bits_host, check_gate, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4._lib()   # raises if the HIP library is missing: no fallback


def _run(case, sk=0, path=None, variant=None, M=None):
    y = w4.w4a16_gemm(case.x, case.w, case.s, split_k=sk, path=path, variant=variant)
    torch.cuda.synchronize()
    return bits_host(y)


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("rows,K", [(3, 18), (7, 10), (256, 512), (1000, 1280), (5, 4098), (1, 2)])
def test_pack_bit_exact(rows, K):
    rng = np.random.default_rng(rows * 7 + K)
    q = rng.integers(0, 256, (rows, K), dtype=np.uint8)   # high bits must be ignored
    out = w4.w4a16_pack_int4(u8_dev(q))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.pack_int4(q & 0x0F))


# ------------------------------------------------------------------ decode GEMV (M = 1)

GEMV_CASES = [
    # N, K, split_k, variant (1000 * layout [0 flat, 1 half-wave, 2 MFMA] + layout digits;
    #   flat / half-wave: 100 * non-temporal + 10 * prefetch depth + row blocks (rows) per wave)
    # None = the default (MFMA 2110 where the slice length has an MFMA geometry,
    # otherwise half-wave 124)
    (256, 512, 0, None),      # the tiny workload (MFMA, 4-row blocks)
    (17408, 5120, 1, None),   # the decode workload (MFMA, 2-row blocks)
    (1001, 5120, 1, 131),     # odd N: last 2-row block half outside
    (999, 8192, 1, 22),       # flat, 1-row blocks, 4 runs of 1 KiB
    (777, 4096, 1, 113),      # flat, 1-row blocks, 2 runs
    (1003, 2560, 1, 24),      # flat, 4-row blocks, 5 runs
    (1002, 1024, 1, 21),      # flat, 2-row blocks, 1 run
    (1000, 1280, 1, 1011),    # half-wave layout (flat does not fit 40 chunks/row)
    (1000, 1280, 1, 1022),
    (1001, 1280, 1, 1134),
    (999, 640, 1, 1149),
    (1003, 5120, 1, 1037),    # half-wave layout forced
    (37, 128, 1, None),
    (513, 2560, 2, None),
    (300, 9216, 0, None),     # 72 groups: auto split so that a slice holds <= 64
    (300, 1024, 16, None),    # more slices than groups: empty slices write zeros
    (64, 384, 4, None),       # 3 groups over 4 slices
    (1, 8192, 1, None),       # single row, 64 groups in one slice
    (3, 5120, 1, None),       # fewer rows than one wave's blocks
    (40, 10240, 2, 24),       # flat with split-K: 40 groups per slice
    (41, 7680, 2, None),      # 30 groups per slice -> half-wave fallback
    # MFMA layout: 2000 + 100 * (4 * x-in-LDS + waves / 4 - 1) + 10 * depth
    #              + row blocks per wave (0: one workgroup per compute unit)
    (17408, 5120, 1, 2024),   # 2-row blocks, 5 instructions, x in registers
    (17408, 5120, 1, 2514),   # x in LDS, 8 waves
    (17408, 5120, 1, 2610),   # x in LDS, 12 waves, one workgroup per CU
    (17408, 5120, 1, 2620),
    (17408, 5120, 1, 2710),   # 16 waves
    (17408, 5120, 1, 2110),   # 8 waves, x in registers, one workgroup per CU
    (17408, 5120, 1, 2120),
    (1001, 5120, 1, 2115),
    (1003, 2560, 1, 2110),    # 4-row blocks, 5 instructions
    (1002, 1024, 1, 2210),    # 12 waves, x in registers (2-row blocks, 1 instruction)
    (1001, 5120, 1, 2413),
    (999, 8192, 1, 2022),     # 1-row blocks, 4 instructions
    (777, 4096, 1, 2431),     # 1-row blocks, 2 instructions, depth 3
    (1003, 2560, 1, 2424),    # 4-row blocks, 5 instructions
    (1002, 1024, 1, 2012),    # 2-row blocks, 1 instruction
    (1002, 1024, 1, 2610),
    (256, 512, 1, 2421),      # 4-row blocks, 1 instruction (the tiny shape)
    (256, 512, 1, 2610),      # fewer blocks than one workgroup per CU can take
    (40, 10240, 2, 2524),     # with split-K
    (40, 10240, 2, 2610),
    (5, 5120, 1, 2011),       # fewer rows than one block per wave
    (5, 5120, 1, 2710),
    (33, 8192, 4, 2620),      # split-K, 16 groups per slice, 1-row blocks
    (1001, 896, 2, 2410),     # N * G odd: the last scale is the low half of a word
    (1001, 896, 2, 2110),     #   that ends past the tensor (4 + 3 groups per slice)
    (1000, 640, 1, 2213),     # 5 groups per slice: no MFMA geometry -> half-wave 124
    (17408, 5120, 1, 122),    # flat layout at the decode shape
    (17408, 5120, 1, 1124),   # half-wave layout at the decode shape
]


@pytest.mark.parametrize("N,K,sk,variant", GEMV_CASES)
def test_gemv_parity(N, K, sk, variant):
    c = make_inputs(1, N, K, seed=N + K + sk)
    d = DevCase(c)
    assert d.packed_matches_oracle()
    y = _run(d, sk=sk, path=w4.PATH_GEMV, variant=variant)
    check_gate(y, oracle.gemm(c.x, d.p_host, c.s), f"gemv N={N} K={K} sk={sk} v={variant}")


# ------------------------------------------------------------------ skinny MFMA (M <= 16)

SKINNY_CASES = [
    # M, N, K, split_k, variant (10 * waves + column tiles per wave; or streaming)
    (1, 256, 512, 1, 44),
    (2, 1000, 1024, 1, 44),
    (3, 17, 384, 1, 41),
    (5, 64, 128, 1, 42),
    (15, 1000, 1024, 2, 84),
    (16, 513, 2048, 4, 81),
    (16, 256, 1024, 8, 82),
    (16, 100, 384, 16, 44),   # more slices than groups
    (7, 300, 640, 1, 82),
    (16, 8192, 1024, 0, None),
    # X row quads loaded per group follow M (1: M <= 4, 2: <= 8, 3: <= 12, 4)
    (4, 300, 640, 1, 82),
    (8, 300, 640, 2, 82),
    (9, 513, 1024, 1, 82),
    (12, 300, 640, 1, 41),
    (13, 257, 384, 1, 84),
    (4, 100, 40960, 1, 82),       # a slice too long to stage its scales in LDS (320 groups)
    # two row tiles of 16 (17 <= M <= 32; 6 or 8 row quads), 8 waves of 1 or 2 column tiles
    (17, 300, 640, 1, 82),
    (20, 257, 1024, 2, 81),
    (24, 513, 2048, 4, 82),
    (25, 100, 384, 16, 82),       # more slices than groups
    (31, 1000, 1024, 1, 81),
    (32, 8192, 1024, 0, 82),
    (32, 300, 40960, 1, 82),      # a slice too long to stage its scales in LDS
    # three row tiles (33 <= M <= 48; 10 or 12 row quads), 8 waves of 1 column tile
    (33, 300, 640, 1, 81),
    (40, 257, 1024, 2, 81),
    (41, 513, 2048, 4, 81),
    (48, 100, 384, 16, 81),       # more slices than groups
    (48, 1000, 1024, 0, None),    # forced path, default variant and split
    (47, 300, 40960, 1, 81),      # a slice too long to stage its scales in LDS
    # streaming layout: 1000 + 100 * row tiles + 10 * units in flight + waves / 4
    (1, 256, 512, 1, 1131),
    (3, 17, 384, 1, 1121),        # fewer rows than one 16-row block
    (5, 100, 640, 1, 3131),       # ragged unit (5 groups in a 16-group unit)
    (15, 1000, 1024, 2, 2121),
    (16, 513, 2048, 4, 2122),
    (16, 1000, 4096, 1, 3112),    # 32 groups in one slice (the LDS maximum)
    (16, 777, 1280, 4, 1222),     # uneven slices (3, 3, 3, 1 groups)
    (16, 100, 384, 16, 1131),     # more slices than groups (empty slices write zeros)
    (16, 512, 8192, 1, 1131),     # slice too long for LDS: group-striped fallback
    (16, 8192, 8192, 0, None),    # small-batch decode workload, default split
    (9, 2048, 8192, 2, 1122),
]


@pytest.mark.parametrize("M,N,K,sk,variant", SKINNY_CASES)
def test_skinny_parity(M, N, K, sk, variant):
    c = make_inputs(M, N, K, seed=M * 1000 + N + K)
    d = DevCase(c)
    y = _run(d, sk=sk, path=w4.PATH_SKINNY, variant=variant)
    check_gate(y, oracle.gemm(c.x, d.p_host, c.s), f"skinny M={M} N={N} K={K} sk={sk} v={variant}")


# ------------------------------------------------------------------ tile MFMA (prefill)

TILE_CASES = [
    # M, N, K, split_k, tile config
    (17, 100, 128, 1, 0),
    (130, 256, 256, 1, 0),
    (300, 1000, 640, 1, 1),
    (129, 513, 384, 2, 0),
    (64, 64, 1024, 4, 1),
    (257, 300, 256, 8, 1),    # more slices than groups
    (1, 256, 256, 1, 0),      # one row through the tile kernel (M tail)
    (255, 129, 512, 0, 0),
    (600, 700, 1280, 0, 1),
    # LDS-DMA kernel, 8 waves, 3 stages: 2 = 128 x 256 tiles, 3 = 96 x 256 tiles
    (17, 100, 128, 1, 2),     # one group: no second stage in flight; M and N tails
    (130, 256, 256, 1, 2),    # two groups
    (300, 1000, 640, 1, 2),   # steady state, N tail of 232 columns
    (129, 513, 384, 2, 2),    # split-K slices of 2 and 1 groups
    (257, 300, 256, 8, 2),    # more slices than groups: empty slices write zeros
    (1, 256, 256, 1, 2),
    (255, 129, 512, 0, 2),
    (1322, 512, 2560, 1, 2),  # the prefill row count and depth
    (64, 64, 1024, 4, 2),
    (600, 700, 1280, 0, 2),
    (77, 257, 640, 1, 2),
    (129, 511, 384, 1, 2),    # N * G odd, no split
    (17, 100, 128, 1, 3),
    (97, 256, 256, 1, 3),     # one row past a 96-row tile
    (300, 1000, 640, 1, 3),
    (129, 513, 384, 2, 3),
    (257, 300, 256, 8, 3),
    (1322, 512, 2560, 1, 3),
    (95, 129, 512, 0, 3),
    # 4 = 112 x 256 tiles (7 row tiles: the X stage is 28 DMA blocks over 8 waves)
    (17, 100, 128, 1, 4),
    (113, 256, 256, 1, 4),    # one row past a 112-row tile
    (300, 1000, 640, 1, 4),
    (129, 513, 384, 2, 4),
    (257, 300, 256, 8, 4),
    (1322, 512, 2560, 1, 4),
    (111, 129, 512, 0, 4),
    (224, 257, 384, 1, 4),    # exactly two tiles; N * G odd
    # 6 = 144 x 256 tiles (36 X DMA blocks over 8 waves, 3 x 52.6 KiB stages)
    (17, 100, 128, 1, 6),
    (145, 256, 256, 1, 6),    # one row past a 144-row tile
    (300, 1000, 640, 1, 6),
    (129, 513, 384, 2, 6),
    (257, 300, 256, 8, 6),
    (1322, 512, 2560, 1, 6),
    (143, 129, 512, 0, 6),
    # 7 = 64 x 256 and 8 = 48 x 256 tiles (16 and 12 X DMA blocks over 8 waves)
    (17, 100, 128, 1, 7),
    (65, 256, 256, 1, 7),     # one row past a 64-row tile
    (300, 1000, 640, 2, 7),
    (1322, 512, 2560, 1, 7),
    (17, 100, 128, 1, 8),
    (49, 256, 256, 1, 8),     # one row past a 48-row tile
    (300, 1000, 640, 8, 8),
    (47, 129, 512, 0, 8),
    # 5 = 80 x 256 tiles (20 X DMA blocks over 8 waves)
    (17, 100, 128, 1, 5),
    (81, 256, 256, 1, 5),
    (300, 1000, 640, 1, 5),
    (257, 300, 256, 8, 5),
    (1322, 512, 2560, 1, 5),
]


@pytest.mark.parametrize("M,N,K,sk,cfg", TILE_CASES)
def test_tile_parity(M, N, K, sk, cfg):
    c = make_inputs(M, N, K, seed=M + N * 3 + K)
    d = DevCase(c)
    y = _run(d, sk=sk, path=w4.PATH_TILE, variant=cfg)
    check_gate(y, oracle.gemm(c.x, d.p_host, c.s), f"tile M={M} N={N} K={K} sk={sk} cfg={cfg}")


# ------------------------------------------------------------------ grouped

GROUPED_CASES = [
    # m_sizes, N, K, tile config
    ([37], 256, 384, None),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 0),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 1),
    ([0, 0, 0, 50], 128, 128, None),
    ([128, 128, 128], 256, 512, 1),
    ([1, 1, 1, 1, 1], 64, 128, 0),
    ([37], 256, 384, 2),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 2),
    ([1, 1, 1, 1, 1], 64, 128, 2),
    ([128, 128, 128], 256, 512, 2),
    ([0, 0, 0, 50], 128, 128, 2),
    ([5, 70, 33], 257, 384, 2),   # N * G odd per weight group: unaligned group bases
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 3),   # 96-row tiles
    ([96, 97, 95, 0, 1], 256, 640, 3),
    ([37], 256, 384, 3),
    ([0, 0, 0, 50], 128, 128, 3),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 4),   # 112-row tiles
    ([112, 113, 111, 0, 1], 256, 640, 4),
    ([37], 256, 384, 4),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 5),   # 80-row tiles
    ([80, 81, 79, 0, 1], 256, 640, 5),
    ([0, 0, 0, 0, 0, 0, 0, 700], 512, 256, 5),      # all rows in the last group
    ([144, 145, 143, 0, 1], 256, 640, 6),           # 144-row tiles
    ([64, 65, 63, 0, 1], 256, 640, 7),              # 64-row tiles
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 8),   # 48-row tiles
]


@pytest.mark.parametrize("ms,N,K,cfg", GROUPED_CASES)
def test_grouped_parity(ms, N, K, cfg):
    c = make_inputs(sum(ms), N, K, seed=len(ms) * 31 + N + K, G=len(ms), m_sizes=ms)
    d = DevCase(c)
    assert d.packed_matches_oracle()
    y = w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, variant=cfg)
    torch.cuda.synchronize()
    check_gate(bits_host(y), oracle.gemm_grouped(c.x, d.p_host, c.s, c.m_sizes), f"grouped {ms} N={N} K={K}")


# ------------------------------------------------------------------ batched

BATCHED_CASES = [
    # B, M, N, K, split_k, tile configuration (None = automatic)
    (1, 17, 100, 128, 0, None),
    (3, 1, 256, 512, 0, None),      # one row per problem
    (4, 16, 300, 640, 2, None),     # N tail, split-K
    (2, 130, 513, 384, 0, None),    # M tail across tiles, N * G odd per problem
    (3, 97, 257, 256, 4, None),     # more slices than groups per slice of 1
    (5, 33, 129, 1280, 8, None),
    (2, 64, 256, 2560, 16, 2),      # 16 slices of 20 groups
    (2, 144, 256, 256, 1, 6),       # 144-row tiles: exactly one per problem
    (3, 100, 300, 384, 1, 5),       # 80-row tiles: a problem spans two tiles
    (2, 113, 300, 256, 2, 4),
    (3, 50, 200, 256, 2, 0),        # the LDS-dequant tile kernel
    (2, 70, 130, 384, 1, 1),
]


@pytest.mark.parametrize("B,M,N,K,sk,cfg", BATCHED_CASES)
def test_batched_parity(B, M, N, K, sk, cfg):
    c = make_inputs(B * M, N, K, seed=B * 1000 + M + N + K, G=B, m_sizes=[M] * B)
    d = DevCase(c)
    assert d.packed_matches_oracle()
    x = d.x.view(B, M, K)
    y = w4.w4a16_gemm_batched(x, d.w, d.s, split_k=sk, variant=cfg)
    torch.cuda.synchronize()
    ref = oracle.gemm_batched(c.x.reshape(B, M, K), d.p_host, c.s)
    check_gate(bits_host(y.view(B * M, N)), ref.reshape(B * M, N), f"batched B={B} M={M} N={N} K={K} sk={sk}")
    # every problem on its own gate too (a swapped problem would pass the joint gate only by luck)
    yb = bits_host(y.view(B * M, N)).reshape(B, M, N)
    for b in range(B):
        check_gate(yb[b], ref[b], f"batched problem {b}")


def test_batched_repeat_bitwise():
    B, M, N, K = 3, 40, 300, 640
    c = make_inputs(B * M, N, K, seed=7, G=B, m_sizes=[M] * B)
    d = DevCase(c)
    x = d.x.view(B, M, K)
    y0 = bits_host(w4.w4a16_gemm_batched(x, d.w, d.s, split_k=4).view(B * M, N))
    y1 = bits_host(w4.w4a16_gemm_batched(x, d.w, d.s, split_k=4).view(B * M, N))
    torch.cuda.synchronize()
    assert np.array_equal(y0, y1)


# ------------------------------------------------------------------ full sizes, sampled outputs

def _sample_entries(rng, M, N, n_random, row_edges=(), col_edges=()):
    """Random (row, col) pairs plus the corners of the given row and column
    boundaries (tile edges, last row and column)."""
    rows = list(rng.integers(0, M, n_random))
    cols = list(rng.integers(0, N, n_random))
    for r in list(row_edges) + [0, M - 1]:
        for c in list(col_edges) + [0, N - 1]:
            if 0 <= r < M and 0 <= c < N:
                rows.append(r)
                cols.append(c)
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


def _gate_sampled(y_bits, rows, cols, ref, what):
    got = y_bits[rows, cols]
    assert np.all(np.isfinite(oracle.bf16_to_f64(y_bits))), f"{what}: non-finite output"
    check_gate(got, ref, what)


def test_prefill_full_size_sampled():
    # the deep-prefill workload in the launch configuration bench.py times
    # (default path and tile configuration), checked on sampled entries
    c = make_config("prefill")
    d = DevCase(c)
    y = bits_host(w4.w4a16_gemm(d.x, d.w, d.s))
    torch.cuda.synchronize()
    M, N = c.M, c.N
    rng = np.random.default_rng(11)
    rows, cols = _sample_entries(rng, M, N, 3000, row_edges=(111, 112, 127, 128, 143, 144, 1231, 1232, 1279, 1280, 1295, 1296, 1321),
                                 col_edges=(255, 256, 19199, 19200, 19455))
    ref = oracle.gemm_entries(c.x, d.p_host, c.s, rows, cols)
    _gate_sampled(y, rows, cols, ref, "prefill 1322x19456x2560 sampled")


def test_grouped_full_size_sampled():
    c = make_config("grouped")
    d = DevCase(c)
    y = bits_host(w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes))
    torch.cuda.synchronize()
    ms = c.m_sizes.astype(np.int64)
    starts = oracle.group_starts(ms)
    rng = np.random.default_rng(12)
    all_rows, all_cols, all_ref = [], [], []
    for g in range(ms.shape[0]):
        if ms[g] == 0:
            continue
        r0 = int(starts[g])
        rows, cols = _sample_entries(rng, int(ms[g]), c.N, 300, row_edges=(127, 128), col_edges=(255, 256))
        ref = oracle.gemm_entries(c.x[r0:r0 + int(ms[g])], d.p_host[g], c.s[g], rows, cols)
        all_rows.append(rows + r0)
        all_cols.append(cols)
        all_ref.append(ref)
    _gate_sampled(y, np.concatenate(all_rows), np.concatenate(all_cols), np.concatenate(all_ref),
                  f"grouped G=8 {list(ms)} sampled")


def test_batched_full_size_sampled():
    # the batched workload in the launch configuration bench.py times
    # (automatic tile height and split), checked on sampled entries per problem
    c = make_config("batched")
    B, M, N, K = c.G, c.M // c.G, c.N, c.K
    d = DevCase(c)
    y = bits_host(w4.w4a16_gemm_batched(d.x.view(B, M, K), d.w, d.s).view(B * M, N))
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    all_rows, all_cols, all_ref = [], [], []
    for b in range(B):
        r0 = b * M
        rows, cols = _sample_entries(rng, M, N, 300, row_edges=(79, 80, 127, 128), col_edges=(255, 256))
        ref = oracle.gemm_entries(c.x[r0:r0 + M], d.p_host[b], c.s[b], rows, cols)
        all_rows.append(rows + r0)
        all_cols.append(cols)
        all_ref.append(ref)
    _gate_sampled(y, np.concatenate(all_rows), np.concatenate(all_cols), np.concatenate(all_ref),
                  f"batched B={B} {M}x{N}x{K} sampled")


def test_grouped_empty_total_is_noop():
    c = make_inputs(0, 64, 128, seed=5, G=3, m_sizes=[0, 0, 0])
    d = DevCase(c)
    y = torch.full((0, 64), 1.0, dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ split-K partials and reduce

@pytest.mark.parametrize("path,M,N,K,sk", [
    (w4.PATH_GEMV, 1, 300, 1280, 4),
    (w4.PATH_SKINNY, 16, 256, 1024, 8),
    (w4.PATH_SKINNY, 5, 100, 384, 4),
    (w4.PATH_TILE, 130, 256, 640, 2),
])
def test_splitk_workspace_slices(path, M, N, K, sk):
    c = make_inputs(M, N, K, seed=sk * 100 + M)
    d = DevCase(c)
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, sk, path=path)
    ws = torch.empty(need // 4 + 4, dtype=torch.float32, device="cuda")
    y = w4.w4a16_gemm(d.x, d.w, d.s, split_k=sk, workspace=ws, path=path)
    torch.cuda.synchronize()
    part = ws[: sk * M * N].view(sk, M, N).cpu().numpy().astype(np.float64)
    ref = oracle.gemm_splitk_partials(c.x, d.p_host, c.s, sk)
    # fp32 accumulation bound: the kernels accumulate x * (128 + q) against
    # -136 * sum(x), so the error scales with 143 * sum |x| * s per slice
    x = np.abs(oracle.bf16_to_f64(c.x))
    srep = np.repeat(oracle.bf16_to_f64(c.s), 128, axis=1) * 143.0
    for s, (g0, g1) in enumerate(oracle.splitk_group_ranges(K // 128, sk)):
        k0, k1 = g0 * 128, g1 * 128
        mag = x[:, k0:k1] @ srep[:, k0:k1].T if k1 > k0 else np.zeros((M, N))
        err = np.abs(part[s] - ref[s])
        assert np.all(err <= 4e-6 * mag + 1e-30), (s, float(err.max()), float(mag.max()))
    # and the final output is the reduce of exactly these partials
    assert np.array_equal(bits_host(y), oracle.splitk_reduce_bf16(ws[: sk * M * N].view(sk, M, N).cpu().numpy()))


@pytest.mark.parametrize("sk,M,N", [(1, 3, 37), (2, 16, 64), (3, 5, 7), (8, 16, 8192), (16, 1, 17408), (64, 2, 6)])
def test_splitk_reduce_bit_exact(sk, M, N):
    ws = make_workspace(sk, M, N, seed=sk + M + N)
    y = w4.w4a16_splitk_reduce(torch.from_numpy(ws).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(y), oracle.splitk_reduce_bf16(ws))


# ------------------------------------------------------------------ degenerate inputs

@pytest.mark.parametrize("path,M", [(w4.PATH_GEMV, 1), (w4.PATH_SKINNY, 4), (w4.PATH_TILE, 40)])
def test_degenerate_zero_outputs(path, M):
    N, K = 200, 384
    c = make_inputs(M, N, K, seed=9)
    # q == 8 everywhere: the oracle gives exactly 0; the MFMA paths form
    # -136 * sum(x) + sum(136 * x) in two fp32 summation orders, so only a
    # rounding residue (far below the gate's absolute term) may remain
    # (the gate's cosine is undefined for an all-zero reference, so only its
    # absolute term, 1e-3, is checked)
    zero_q = DevCase(type(c)(x=c.x, q=np.full_like(c.q, 8), s=c.s))
    y8 = oracle.bf16_to_f64(_run(zero_q, path=path))
    assert np.all(np.isfinite(y8)) and float(np.max(np.abs(y8))) <= 1e-3
    zero_s = DevCase(type(c)(x=c.x, q=c.q, s=np.zeros_like(c.s)))
    assert np.all((_run(zero_s, path=path) & 0x7FFF) == 0)       # s == 0 -> +-0
    zero_x = DevCase(type(c)(x=np.zeros_like(c.x), q=c.q, s=c.s))
    assert np.all((_run(zero_x, path=path) & 0x7FFF) == 0)


def test_n1_and_k128():
    for M in (1, 3, 20):
        c = make_inputs(M, 1, 128, seed=M)
        d = DevCase(c)
        check_gate(_run(d), oracle.gemm(c.x, d.p_host, c.s), f"N=1 M={M}")


def test_m0_leaves_output_untouched():
    c = make_inputs(1, 64, 256, seed=3)
    d = DevCase(c)
    x0 = d.x[:0]
    y = torch.full((0, 64), 2.0, dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(x0, d.w, d.s, y=y)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ determinism and graphs

@pytest.mark.parametrize("path,M,N,K,sk", [
    (w4.PATH_GEMV, 1, 1000, 2560, 1),
    (w4.PATH_SKINNY, 16, 1024, 2048, 4),
    (w4.PATH_TILE, 300, 512, 1024, 1),
])
def test_repeat_bitwise_and_graph_replay(path, M, N, K, sk):
    c = make_inputs(M, N, K, seed=77)
    d = DevCase(c)
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, sk, path=path)
    ws = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws, path=path)
    torch.cuda.synchronize()
    ref = bits_host(y)
    check_gate(ref, oracle.gemm(c.x, d.p_host, c.s), "eager")
    for _ in range(3):
        w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws, path=path)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws, path=path)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        y.fill_(0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), ref), f"replay {i}"


def test_grouped_graph_replay():
    ms = [3, 0, 129, 5, 0, 255, 1, 64]
    c = make_inputs(sum(ms), 300, 256, seed=12, G=len(ms), m_sizes=ms)
    d = DevCase(c)
    y = torch.empty((sum(ms), 300), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(w4.w4a16_gemm_grouped_workspace_bytes(len(ms), sum(ms), 300, 256) // 4,
                     dtype=torch.float32, device="cuda")
    w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y, workspace=ws)
    torch.cuda.synchronize()
    ref = bits_host(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), ref), f"replay {i}"
