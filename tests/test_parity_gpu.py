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
from gpu_util import DevCase, bf16_dev, bits_host, check_full, check_gate, nan_filled, u8_dev

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
    # N, K, split_k, variant (None = the MFMA layout where the slice length has
    # a tiling of 16 (row, group) pairs per instruction, else the half-wave
    # layout; 1 = the half-wave layout forced)
    (256, 512, 0, None),      # the tiny workload (MFMA, 4-row blocks)
    (17408, 5120, 1, None),   # the decode workload (MFMA, 2-row blocks)
    (1001, 5120, 1, None),    # odd N: last 2-row block half outside
    (1003, 2560, 1, None),    # 4-row blocks, 5 instructions
    (1002, 1024, 1, None),    # 2-row blocks, 1 instruction
    (999, 8192, 1, None),     # 1-row blocks, 4 instructions
    (777, 4096, 1, None),     # 1-row blocks, 2 instructions
    (1000, 1280, 1, None),    # 10 groups: 8-row blocks, no MFMA tiling -> half-wave
    (999, 640, 1, None),      # 5 groups: half-wave
    (37, 128, 1, None),
    (513, 2560, 2, None),
    (300, 9216, 0, None),     # 72 groups: auto split so that a slice holds <= 64
    (300, 1024, 16, None),    # more slices than groups: empty slices write zeros
    (64, 384, 4, None),       # 3 groups over 4 slices
    (1, 8192, 1, None),       # single row, 64 groups in one slice
    (3, 5120, 1, None),       # fewer rows than one wave's blocks
    (5, 5120, 1, None),
    (256, 512, 1, None),      # fewer blocks than one workgroup per compute unit can take
    (41, 7680, 2, None),      # 30 groups per slice -> half-wave fallback
    (33, 8192, 4, None),      # split-K, 16 groups per slice, 1-row blocks
    (1001, 896, 2, None),     # N * G odd: the last scale is the low half of a word
                              #   that ends past the tensor (4 + 3 groups per slice)
    (40, 10240, 2, None),     # with split-K: 40 groups per slice
    # blocks per workgroup not a multiple of the 8 waves: the leftover blocks'
    # instructions are dealt to all waves (rem = 7, 7 with q = 0, 1, 0 .. 7)
    (7680, 5120, 1, None),    # 15 two-row blocks per workgroup: 1 full step + 7 leftover blocks
    (7680, 5120, 2, None),    # 20 groups per slice: 4-row blocks, 7 per workgroup, all leftover
    (12310, 5120, 1, None),   # 24 or 25 blocks per workgroup (rem 0 or 1)
    (6000, 8192, 1, None),    # 1-row blocks of 64 groups (I = 4), rem varies
    (8192, 3584, 1, None),    # 28 groups: 4-row blocks of 7 instructions (one leftover per step)
    (8200, 3584, 1, None),
    # two or more blocks per wave on average: the two-deep ring of register
    # sets (one instance per block shape below 7 instructions)
    (8192, 5120, 1, None),    # 2-row blocks, exactly 16 per workgroup (2 per wave)
    (20000, 2560, 1, None),   # 4-row blocks of 5 instructions, 19 or 20 per workgroup
    (17000, 1536, 1, None),   # 4-row blocks of 3 instructions
    (16500, 512, 1, None),    # 4-row blocks of 1 instruction
    (9000, 3072, 1, None),    # 2-row blocks of 3 instructions
    (8400, 1024, 1, None),    # 2-row blocks of 1 instruction
    (4400, 6144, 1, None),    # 1-row blocks of 3 instructions
    (4500, 4096, 1, None),    # 1-row blocks of 2 instructions
    (4200, 2048, 1, None),    # 1-row blocks of 1 instruction
    # the half-wave layout forced
    (17408, 5120, 1, 1),
    (1000, 1280, 1, 1),
    (1001, 1280, 1, 1),
    (1003, 5120, 1, 1),
    (999, 640, 2, 1),
    (40, 10240, 2, 1),
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
    # M, N, K, split_k, column tiles of 16 per wave (None = 1 up to 8 rows and
    # past 32, 2 between)
    (1, 256, 512, 1, 1),
    (2, 1000, 1024, 1, 2),
    (3, 17, 384, 1, 1),
    (5, 64, 128, 1, 2),
    (15, 1000, 1024, 2, 2),
    (16, 513, 2048, 4, 1),
    (16, 256, 1024, 8, 2),
    (16, 100, 384, 16, 1),    # more slices than groups
    (7, 300, 640, 1, 2),
    (16, 8192, 1024, 0, None),
    # X row quads loaded per group follow M (1: M <= 4, 2: <= 8, 3: <= 12, 4)
    (4, 300, 640, 1, 2),
    (8, 300, 640, 2, 2),
    (9, 513, 1024, 1, 2),
    (12, 300, 640, 1, 1),
    (13, 257, 384, 1, 2),
    (4, 100, 40960, 1, 2),        # a slice too long to stage its scales in LDS (320 groups)
    # two row tiles of 16 (17 <= M <= 32; 6 or 8 row quads)
    (17, 300, 640, 1, 2),
    (20, 257, 1024, 2, 1),
    (24, 513, 2048, 4, 2),
    (25, 100, 384, 16, 2),        # more slices than groups
    (31, 1000, 1024, 1, 1),
    (32, 8192, 1024, 0, 2),
    (32, 300, 40960, 1, 2),       # a slice too long to stage its scales in LDS
    # three row tiles (33 <= M <= 48; 10 or 12 row quads), one column tile per wave
    (33, 300, 640, 1, 1),
    (40, 257, 1024, 2, 1),
    (41, 513, 2048, 4, 1),
    (48, 100, 384, 16, 1),        # more slices than groups
    (48, 1000, 1024, 0, None),    # forced path, default variant and split
    (47, 300, 40960, 1, 1),       # a slice too long to stage its scales in LDS
    (16, 8192, 8192, 0, None),    # small-batch decode workload, default split
    (9, 2048, 8192, 2, 2),
    # 3..6: X and the weights staged in LDS by DMA (3 stages of 8 groups; 6,
    # 5, 4 stages of 4 groups)
] + [case[:4] + (v,) for v in (3, 4, 5, 6) for case in (
    (16, 8192, 8192, 1),          # the small-batch decode workload
    (16, 8192, 8192, 4),
    (1, 256, 512, 1),             # one partial stage
    (3, 17, 384, 1),              # N tail inside the first column tile; 3 groups
    (5, 100, 1280, 2),            # slices of 5 groups
    (16, 513, 2048, 4),           # N tail of one column; empty groups in the last stage
    (16, 100, 384, 16),           # more slices than groups: empty slices write zeros
    (8, 1000, 5120, 1),           # 40 groups
    (12, 777, 3584, 1),           # 28 groups (odd scale words: N * G even, n * G odd rows)
    (16, 2049, 9728, 2),          # 76 groups over 2 slices
)]


@pytest.mark.parametrize("M,N,K,sk,variant", SKINNY_CASES)
def test_skinny_parity(M, N, K, sk, variant):
    c = make_inputs(M, N, K, seed=M * 1000 + N + K)
    d = DevCase(c)
    y = _run(d, sk=sk, path=w4.PATH_SKINNY, variant=variant)
    check_gate(y, oracle.gemm(c.x, d.p_host, c.s), f"skinny M={M} N={N} K={K} sk={sk} v={variant}")


# ------------------------------------------------------------------ tile MFMA (prefill)

TILE_CASES = [
    # M, N, K, split_k, rows per tile (LDS-DMA kernel, 8 waves, 3 stages)
    (17, 100, 128, 1, 128),   # one group: no second stage in flight; M and N tails
    (130, 256, 256, 1, 128),  # two groups
    (300, 1000, 640, 1, 128), # steady state, N tail of 232 columns
    (129, 513, 384, 2, 128),  # split-K slices of 2 and 1 groups
    (257, 300, 256, 8, 128),  # more slices than groups: empty slices write zeros
    (1, 256, 256, 1, 128),
    (255, 129, 512, 0, 128),
    (1322, 512, 2560, 1, 128),  # the prefill row count and depth
    (64, 64, 1024, 4, 128),
    (600, 700, 1280, 0, 128),
    (77, 257, 640, 1, 128),
    (129, 511, 384, 1, 128),  # N * G odd, no split
    (17, 100, 128, 1, 96),
    (97, 256, 256, 1, 96),    # one row past a 96-row tile
    (300, 1000, 640, 1, 96),
    (129, 513, 384, 2, 96),
    (257, 300, 256, 8, 96),
    (1322, 512, 2560, 1, 96),
    (95, 129, 512, 0, 96),
    # 112-row tiles (7 row tiles: the X stage is 28 DMA blocks over 8 waves)
    (17, 100, 128, 1, 112),
    (113, 256, 256, 1, 112),  # one row past a 112-row tile
    (300, 1000, 640, 1, 112),
    (129, 513, 384, 2, 112),
    (257, 300, 256, 8, 112),
    (1322, 512, 2560, 1, 112),
    (111, 129, 512, 0, 112),
    (224, 257, 384, 1, 112),  # exactly two tiles; N * G odd
    # 144-row tiles (36 X DMA blocks over 8 waves, 3 x 52.6 KiB stages; the
    # ninth row tile's sums are taken by a different wave each group)
    (17, 100, 128, 1, 144),
    (145, 256, 256, 1, 144),  # one row past a 144-row tile
    (300, 1000, 640, 1, 144),
    (129, 513, 384, 2, 144),
    (257, 300, 256, 8, 144),
    (1322, 512, 2560, 1, 144),
    (143, 129, 512, 0, 144),
    (150, 300, 2048, 1, 144), # 16 groups: every wave takes the ninth row tile twice
    # 64- and 48-row tiles (16 and 12 X DMA blocks over 8 waves; 4 and 3 of
    # the 8 waves form the row sums)
    (17, 100, 128, 1, 64),
    (65, 256, 256, 1, 64),    # one row past a 64-row tile
    (300, 1000, 640, 2, 64),
    (1322, 512, 2560, 1, 64),
    (17, 100, 128, 1, 48),
    (49, 256, 256, 1, 48),    # one row past a 48-row tile
    (300, 1000, 640, 8, 48),
    (47, 129, 512, 0, 48),
    # 80-row tiles (20 X DMA blocks over 8 waves)
    (17, 100, 128, 1, 80),
    (81, 256, 256, 1, 80),
    (300, 1000, 640, 1, 80),
    (257, 300, 256, 8, 80),
    (1322, 512, 2560, 1, 80),
    # automatic tile height and split
    (200, 700, 1280, 0, None),
    (1000, 300, 4096, 0, None),
]


@pytest.mark.parametrize("M,N,K,sk,cfg", TILE_CASES)
def test_tile_parity(M, N, K, sk, cfg):
    c = make_inputs(M, N, K, seed=M + N * 3 + K)
    d = DevCase(c)
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, path=w4.PATH_TILE, variant=cfg)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s), f"tile M={M} N={N} K={K} sk={sk} rows={cfg}")


# Row sums of X on the tile path: with a wide N (at least 32 column tiles) and
# a workspace of w4a16_gemm_workspace_bytes, a pre-pass forms them into the
# workspace; with no workspace (or too small a one) the tile kernel forms
# them itself. Both ways, at the same shapes.
ROWSUM_CASES = [
    # M, N, K, split_k, rows per tile
    (300, 8192, 640, 1, 128),
    (129, 8448, 384, 2, 144),     # M tail, split-K; N = 33 column tiles
    (97, 8193, 512, 1, 96),       # N tail in the 33rd column tile
    (1, 8192, 256, 1, 48),
    (200, 8192, 1280, 4, 80),
]


@pytest.mark.parametrize("prepass", [True, False])
@pytest.mark.parametrize("M,N,K,sk,rows", ROWSUM_CASES)
def test_tile_rowsum_paths(M, N, K, sk, rows, prepass):
    c = make_inputs(M, N, K, seed=M + N + K + 5)
    d = DevCase(c)
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, sk, path=w4.PATH_TILE, variant=rows)
    split = sk * M * N * 4 if sk > 1 else 0
    split = (split + 255) // 256 * 256
    assert need > split                                   # the pre-pass row sums are part of it
    nbytes = need if prepass else max(split, 16)          # room for the partials only: in-kernel sums
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws, path=w4.PATH_TILE, variant=rows)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s), f"tile M={M} N={N} K={K} sk={sk} rows={rows} pre-pass={prepass}")
    if prepass:
        # the row sums the pre-pass left in the workspace: -136 * sum of each 128-group, fp32
        sx = ws[split // 4: split // 4 + (K // 128) * ((M + 3) // 4 * 4)].view(K // 128, -1)[:, :M].cpu().numpy()
        ref = -136.0 * oracle.bf16_to_f64(c.x).reshape(M, K // 128, 128).sum(axis=2).T
        assert np.allclose(sx, ref, rtol=1e-5, atol=1e-3)


# ------------------------------------------------------------------ grouped

GROUPED_CASES = [
    # m_sizes, N, K, rows per tile (None = automatic)
    ([37], 256, 384, None),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, None),
    ([0, 0, 0, 50], 128, 128, None),
    ([128, 128, 128], 256, 512, None),
    ([1, 1, 1, 1, 1], 64, 128, None),
    ([37], 256, 384, 128),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 128),
    ([1, 1, 1, 1, 1], 64, 128, 128),
    ([128, 128, 128], 256, 512, 128),
    ([0, 0, 0, 50], 128, 128, 128),
    ([5, 70, 33], 257, 384, 128),   # N * G odd per weight group: unaligned group bases
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 96),
    ([96, 97, 95, 0, 1], 256, 640, 96),
    ([37], 256, 384, 96),
    ([0, 0, 0, 50], 128, 128, 96),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 112),
    ([112, 113, 111, 0, 1], 256, 640, 112),
    ([37], 256, 384, 112),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 80),
    ([80, 81, 79, 0, 1], 256, 640, 80),
    ([0, 0, 0, 0, 0, 0, 0, 700], 512, 256, 80),      # all rows in the last group
    ([144, 145, 143, 0, 1], 256, 640, 144),
    ([64, 65, 63, 0, 1], 256, 640, 64),
    ([3, 0, 129, 5, 0, 255, 1, 64], 300, 256, 48),
]


@pytest.mark.parametrize("ms,N,K,cfg", GROUPED_CASES)
def test_grouped_parity(ms, N, K, cfg):
    c = make_inputs(sum(ms), N, K, seed=len(ms) * 31 + N + K, G=len(ms), m_sizes=ms)
    d = DevCase(c)
    assert d.packed_matches_oracle()
    y = nan_filled((sum(ms), N))
    w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y, variant=cfg)
    check_full(y, oracle.gemm_grouped(c.x, d.p_host, c.s, c.m_sizes), f"grouped {ms} N={N} K={K} rows={cfg}")


# ------------------------------------------------------------------ batched

BATCHED_CASES = [
    # B, M, N, K, split_k, rows per tile (None = automatic)
    (1, 17, 100, 128, 0, None),
    (3, 1, 256, 512, 0, None),      # one row per problem
    (4, 16, 300, 640, 2, None),     # N tail, split-K
    (2, 130, 513, 384, 0, None),    # M tail across tiles, N * G odd per problem
    (3, 97, 257, 256, 4, None),     # more slices than groups per slice of 1
    (5, 33, 129, 1280, 8, None),
    (2, 64, 256, 2560, 16, 128),    # 16 slices of 20 groups
    (2, 144, 256, 256, 1, 144),     # exactly one tile per problem
    (3, 100, 300, 384, 1, 80),      # a problem spans two tiles
    (2, 113, 300, 256, 2, 112),
    (3, 50, 200, 256, 2, 48),
    (2, 70, 130, 384, 1, 64),
]


@pytest.mark.parametrize("B,M,N,K,sk,cfg", BATCHED_CASES)
def test_batched_parity(B, M, N, K, sk, cfg):
    c = make_inputs(B * M, N, K, seed=B * 1000 + M + N + K, G=B, m_sizes=[M] * B)
    d = DevCase(c)
    assert d.packed_matches_oracle()
    x = d.x.view(B, M, K)
    y = nan_filled((B, M, N))
    w4.w4a16_gemm_batched(x, d.w, d.s, y=y, split_k=sk, variant=cfg)
    ref = oracle.gemm_batched(c.x.reshape(B, M, K), d.p_host, c.s)
    check_full(y, ref, f"batched B={B} M={M} N={N} K={K} sk={sk}")
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


# ------------------------------------------------------------------ full sizes, whole outputs
#
# Each workload in the launch configuration bench.py times (same entry point,
# same automatic or explicit split), its output pre-filled with NaN so that a
# tile that is never written fails, and compared element by element with the
# float64 oracle (about a second of host BLAS per workload).

def test_decode_gemv_full_size():
    c = make_config("decode_gemv")
    d = DevCase(c)
    y = nan_filled((c.M, c.N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s), "decode 1x17408x5120")


@pytest.mark.parametrize("sk", [0, 1, 2, 4, 8])
def test_decode_splitk_full_size(sk):
    # the small-batch decode workload at every split bench.py times; the
    # final output is also the bit-exact reduce of the kernel's own partials
    c = make_config("decode_splitk")
    d = DevCase(c)
    y = nan_filled((c.M, c.N))
    need = w4.w4a16_gemm_workspace_bytes(c.M, c.N, c.K, sk)
    ws = torch.full((max(need // 4, 1) + 4,), float("nan"), dtype=torch.float32, device="cuda")
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, split_k=sk, workspace=ws)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s), f"small-batch 16x8192x8192 sk={sk}")
    eff = sk if sk else w4.w4a16_gemm_auto_split_k(c.M, c.N, c.K)
    if eff > 1:
        part = ws[: eff * c.M * c.N].view(eff, c.M, c.N).cpu().numpy()
        assert np.array_equal(bits_host(y), oracle.splitk_reduce_bf16(part))


@pytest.mark.parametrize("prepass", [True, False])
def test_prefill_full_size(prepass):
    # as benched: the default choice with its workspace (the row sums from the
    # pre-pass); and with no workspace (the tile kernel forms them)
    c = make_config("prefill")
    d = DevCase(c)
    y = nan_filled((c.M, c.N))
    ws = None if prepass else torch.empty(4, dtype=torch.float32, device="cuda")
    w4.w4a16_gemm(d.x, d.w, d.s, y=y, workspace=ws)
    check_full(y, oracle.gemm(c.x, d.p_host, c.s), f"prefill 1322x19456x2560 pre-pass={prepass}")


def test_grouped_full_size():
    c = make_config("grouped")
    d = DevCase(c)
    y = nan_filled((c.M, c.N))
    w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y)
    ms = [int(v) for v in c.m_sizes]
    ref = oracle.gemm_grouped(c.x, d.p_host, c.s, c.m_sizes)
    check_full(y, ref, f"grouped G=8 {ms}")
    # every non-empty group on its own gate too
    starts = oracle.group_starts(c.m_sizes)
    yb = bits_host(y)
    for g, m in enumerate(ms):
        if m:
            r0 = int(starts[g])
            check_gate(yb[r0:r0 + m], ref[r0:r0 + m], f"grouped group {g}")


def test_batched_full_size():
    c = make_config("batched")
    B, M, N, K = c.G, c.M // c.G, c.N, c.K
    d = DevCase(c)
    y = nan_filled((B, M, N))
    w4.w4a16_gemm_batched(d.x.view(B, M, K), d.w, d.s, y=y)
    ref = oracle.gemm_batched(c.x.reshape(B, M, K), d.p_host, c.s)
    check_full(y, ref, f"batched B={B} {M}x{N}x{K}")
    yb = bits_host(y)
    for b in range(B):
        check_gate(yb[b], ref[b], f"batched problem {b}")


# The automatic path, tile height and split choice at the shape sets of the
# MI350X Triton page's Performance tables ("Add Triton BF16xINT4 rowwise GEMM
# for ROCm gfx942/gfx950"): decode rows M = 1, 16, 64, 128 at N x K = 896 x
# 5120, 2048 x 5120, 8192 x 3584, 7168 x 8192; prefill M = 2048, 4096 at
# 8192 x 3584 and 7168 x 8192. Whole outputs against the oracle.
AUTO_SHAPES = [(M, N, K) for N, K in ((896, 5120), (2048, 5120), (8192, 3584), (7168, 8192))
               for M in (1, 16, 64, 128)] + \
              [(M, N, K) for N, K in ((8192, 3584), (7168, 8192)) for M in (2048, 4096)]


@pytest.mark.parametrize("M,N,K", AUTO_SHAPES)
def test_auto_choice_page_shapes(M, N, K):
    c = make_inputs(M, N, K, seed=M + N + K + 7)
    d = DevCase(c)
    y = nan_filled((M, N))
    w4.w4a16_gemm(d.x, d.w, d.s, y=y)     # split_k 0, automatic path, the workspace it asks for
    check_full(y, oracle.gemm(c.x, d.p_host, c.s), f"auto {M}x{N}x{K} (sk {w4.w4a16_gemm_auto_split_k(M, N, K)})")


def _guarded_empty_call(call, n_cols):
    """Runs `call(y)` with y a (0, n_cols) view at the start of a NaN-filled
    buffer and checks that nothing of the buffer was written."""
    buf = nan_filled((64, n_cols))
    before = bits_host(buf)
    call(buf[:0])
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(buf), before)


def test_m0_writes_nothing():
    c = make_inputs(1, 64, 256, seed=3)
    d = DevCase(c)
    _guarded_empty_call(lambda y: w4.w4a16_gemm(d.x[:0], d.w, d.s, y=y), 64)
    _guarded_empty_call(lambda y: w4.w4a16_gemm(d.x[:0], d.w, d.s, y=y, split_k=4), 64)
    _guarded_empty_call(lambda y: w4.w4a16_gemm(d.x[:0], d.w, d.s, y=y, group_size=128, path=w4.PATH_TILE,
                                                 variant=128), 64)


def test_grouped_empty_total_writes_nothing():
    c = make_inputs(0, 64, 128, seed=5, G=3, m_sizes=[0, 0, 0])
    d = DevCase(c)
    _guarded_empty_call(lambda y: w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y), 64)


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


@pytest.mark.parametrize("sk,M,N", [(1, 3, 37), (2, 16, 64), (3, 5, 7), (8, 16, 8192), (16, 1, 17408), (64, 2, 6),
                                    (3, 4, 1001), (9, 7, 1000)])
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
    w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y)
    torch.cuda.synchronize()
    ref = bits_host(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.w4a16_gemm_grouped(d.x, d.w, d.s, d.m_sizes, y=y)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(y), ref), f"replay {i}"
