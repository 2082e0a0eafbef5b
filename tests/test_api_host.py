"""Host-side checks of the C-ABI library (CPU only: no kernel is launched).

Every call here either only queries host logic (workspace sizes, split-K
choice, status strings) or carries an argument error that the library must
reject before anything is enqueued.
"""
import ctypes
import os

import pytest

import bf16_activation_quantized_amd as w4

LIB_MISSING = not os.path.exists(w4.LIB_PATH)
pytestmark = pytest.mark.skipif(LIB_MISSING, reason="libw4a16.so not built")


@pytest.fixture(scope="module", autouse=True)
def _host_only():
    # the calls below pass fake device pointers that validation must reject;
    # where a GPU is visible a validation bug could launch on them, so these
    # tests run only on hosts without one
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only checks: a GPU is visible")

OK, ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_SPLIT, ERR_WS, ERR_ALIGN = 0, 1, 2, 3, 4, 5, 6


def L():
    return w4._lib()


def test_exports_every_declared_symbol():
    names = w4.header_functions()
    # the boundary: pack, plain / grouped / batched GEMM, the split-K reduce
    for n in ("w4a16_pack_int4", "w4a16_gemm", "w4a16_gemm_grouped", "w4a16_gemm_batched",
              "w4a16_splitk_reduce", "w4a16_gemm_workspace_bytes", "w4a16_status_string"):
        assert n in names, n
    lib = ctypes.CDLL(w4.LIB_PATH)
    for n in names + w4.header_functions(w4.INTERNAL_HEADER):
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(8):
        txt = w4.status_string(s)
        assert txt.startswith("W4A16_")
    assert "unknown" in w4.status_string(99)


# fake but 16-byte aligned device pointers: never dereferenced, because every
# call below fails validation first
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
D = ctypes.c_void_p(0x40000)
MIS = ctypes.c_void_p(0x10004)


def gemm(x=A, w=B, s=C, y=D, M=1, N=64, K=128, g=128, sk=0, ws=None, wsb=0):
    return L().w4a16_gemm(x, w, s, y, M, N, K, g, sk, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), ERR_SHAPE), (dict(N=0), ERR_SHAPE), (dict(K=0), ERR_SHAPE),
    (dict(K=100), ERR_GROUP), (dict(K=192), ERR_GROUP), (dict(g=64), ERR_GROUP),
    (dict(g=32, K=96), ERR_GROUP), (dict(g=16, K=128), ERR_GROUP),
    (dict(g=32, K=128, sk=2), ERR_WS),                       # group 32, split-K: partials needed
    (dict(sk=3), ERR_SPLIT), (dict(sk=-1), ERR_SPLIT), (dict(sk=32), ERR_SPLIT),
    (dict(x=None), ERR_NULL), (dict(w=None), ERR_NULL), (dict(s=None), ERR_NULL), (dict(y=None), ERR_NULL),
    (dict(x=MIS), ERR_ALIGN), (dict(y=MIS), ERR_ALIGN), (dict(w=MIS), ERR_ALIGN), (dict(s=MIS), ERR_ALIGN),
    (dict(M=4, N=1 << 20, K=1 << 14), ERR_SHAPE),            # W larger than 4 GiB (one resource)
    (dict(M=1 << 22, N=64, K=1 << 10), ERR_SHAPE),           # X larger than 4 GiB
    (dict(M=1 << 31, N=64, K=128), ERR_SHAPE),               # dimension limit
    (dict(M=1, N=64, K=128, sk=2), ERR_WS),                  # split-K needs a workspace
    (dict(M=64, N=64, K=256, sk=2), ERR_WS),                 # tile path, split-K: partials needed
    (dict(M=64, N=64, K=256, sk=2, ws=A, wsb=16), ERR_WS),   # too small
    (dict(M=64, N=64, K=256, sk=2, ws=MIS, wsb=1 << 20), ERR_ALIGN),
    (dict(M=1 << 16, N=1 << 15, K=128, sk=2, ws=A, wsb=1 << 30), ERR_SHAPE),   # partials >= 4 GiB
    (dict(M=0), OK),                                         # empty: nothing enqueued
    (dict(M=0, x=None, y=None), OK),                         # empty: pointers unused
])
def test_gemm_argument_errors(kw, want):
    assert gemm(**kw) == want


def test_gemm_m0_ok_even_without_workspace():
    assert gemm(M=0, N=1000, K=1024, sk=8) == OK


def grouped(x=A, w=B, s=C, ms=A, y=D, G=2, Mt=10, N=64, K=128, g=128):
    return L().w4a16_gemm_grouped(x, w, s, ms, y, G, Mt, N, K, g, None)


@pytest.mark.parametrize("kw,want", [
    (dict(G=0), ERR_SHAPE), (dict(G=-3), ERR_SHAPE), (dict(Mt=-1), ERR_SHAPE),
    (dict(K=130), ERR_GROUP), (dict(g=256), ERR_GROUP), (dict(g=32, K=96), ERR_GROUP),
    (dict(G=1 << 10, N=1 << 16, K=1 << 12, g=32), ERR_SHAPE),   # scales of all groups >= 4 GiB
    (dict(ms=None), ERR_NULL), (dict(x=None), ERR_NULL), (dict(y=None), ERR_NULL),
    (dict(ms=ctypes.c_void_p(0x10002)), ERR_ALIGN), (dict(x=MIS), ERR_ALIGN),
    (dict(Mt=0), OK),
    (dict(Mt=0, x=None, ms=None), OK),                      # empty: pointers unused
])
def test_grouped_argument_errors(kw, want):
    assert grouped(**kw) == want


def batched(x=A, w=B, s=C, y=D, Bn=3, M=5, N=64, K=128, g=128, sk=0, ws=A, wsb=1 << 20):
    return L().w4a16_gemm_batched(x, w, s, y, Bn, M, N, K, g, sk, ws, wsb, None)


@pytest.mark.parametrize("kw,want", [
    (dict(Bn=0), ERR_SHAPE), (dict(Bn=-1), ERR_SHAPE), (dict(M=-1), ERR_SHAPE), (dict(N=0), ERR_SHAPE),
    (dict(K=130), ERR_GROUP), (dict(g=64), ERR_GROUP),
    (dict(sk=3), ERR_SPLIT), (dict(sk=32), ERR_SPLIT),
    (dict(x=None), ERR_NULL), (dict(w=None), ERR_NULL), (dict(s=None), ERR_NULL), (dict(y=None), ERR_NULL),
    (dict(x=MIS), ERR_ALIGN), (dict(s=MIS), ERR_ALIGN), (dict(ws=MIS, sk=2), ERR_ALIGN),
    (dict(g=32, sk=2, wsb=2 * 15 * 64 * 4 - 4), ERR_WS),      # partials [2, 15, 64] fp32
    (dict(sk=2, ws=None), ERR_WS), (dict(sk=2, wsb=8), ERR_WS),
    (dict(Bn=1 << 16, M=1 << 16), ERR_SHAPE),              # B * M >= 2^31
    (dict(Bn=1 << 12, N=1 << 16, K=1 << 12), ERR_SHAPE),   # scales of all problems >= 4 GiB
    (dict(M=0), OK),
    (dict(M=0, x=None, w=None, s=None, y=None, ws=None), OK),   # empty: pointers unused
])
def test_batched_argument_errors(kw, want):
    assert batched(**kw) == want


def test_pack_argument_errors():
    f = L().w4a16_pack_int4
    assert f(A, B, 4, 3, None) == ERR_SHAPE          # odd K
    assert f(A, B, -1, 4, None) == ERR_SHAPE
    assert f(A, B, 4, 0, None) == ERR_SHAPE
    assert f(None, B, 4, 4, None) == ERR_NULL
    assert f(A, MIS, 4, 4, None) == ERR_ALIGN
    assert f(A, B, 0, 4, None) == OK                 # nothing to do


def test_reduce_argument_errors():
    f = L().w4a16_splitk_reduce
    assert f(A, B, 0, 4, 4, None) == ERR_SHAPE
    assert f(A, B, 65, 4, 4, None) == ERR_SHAPE
    assert f(A, B, 2, -1, 4, None) == ERR_SHAPE
    assert f(None, B, 2, 4, 4, None) == ERR_NULL
    assert f(MIS, B, 2, 4, 4, None) == ERR_ALIGN
    assert f(A, B, 2, 0, 4, None) == OK


def ex(cfg, M=2, N=64, K=128, g=128, sk=0, ws=None, wsb=0):
    return L().w4a16_gemm_ex(A, B, C, D, M, N, K, g, sk, ws, wsb, None, ctypes.byref(cfg))


def test_explicit_path_errors():
    assert ex(w4._Config(1, -1), M=2) == ERR_SHAPE          # GEMV path forced at M=2
    assert ex(w4._Config(1, 2), M=1) == ERR_SHAPE           # GEMV: 0 (MFMA) or 1 (half-wave) only
    assert ex(w4._Config(2, -1), M=49) == ERR_SHAPE         # small batch: three row tiles of 16 at most
    for v in (3, 4, 8):                                     # small batch: 1 or 2 column tiles per wave
        assert ex(w4._Config(2, v), M=20, sk=1) == ERR_SHAPE, v
    assert ex(w4._Config(2, 2), M=40, sk=1) == ERR_SHAPE    # past 32 rows one column tile only
    assert ex(w4._Config(7, -1)) == ERR_SHAPE               # no such path
    for v in (16, 32, 50, 160, 256):                        # tile heights 48 .. 144 in steps of 16
        assert ex(w4._Config(3, v), M=20, sk=1) == ERR_SHAPE, v
    # group size 32: the tile kernel with 80 .. 128-row tiles only
    for path, variant in ((1, -1), (2, -1), (3, 144), (3, 64), (3, 48)):
        assert ex(w4._Config(path, variant), M=1, g=32, sk=2, ws=A, wsb=1 << 20) == ERR_GROUP, (path, variant)
    for v in (144, 64, 48):
        cfg = w4._Config(3, v)
        st = L().w4a16_gemm_grouped_ex(A, B, C, A, D, 2, 10, 64, 128, 32, None, ctypes.byref(cfg))
        assert st == ERR_GROUP, v
        st = L().w4a16_gemm_batched_ex(A, B, C, D, 3, 5, 64, 128, 32, 2, A, 1 << 20, None, ctypes.byref(cfg))
        assert st == ERR_GROUP, v
    cfg = w4._Config(2, -1)                                 # grouped and batched run the tile kernel only
    assert L().w4a16_gemm_grouped_ex(A, B, C, A, D, 2, 10, 64, 128, 128, None, ctypes.byref(cfg)) == ERR_SHAPE
    assert L().w4a16_gemm_batched_ex(A, B, C, D, 3, 5, 64, 128, 128, 2, A, 1 << 20, None,
                                     ctypes.byref(cfg)) == ERR_SHAPE


def test_auto_split_rule():
    # the tile kernel splits only where tiles x SK fit one round of one
    # workgroup per compute unit (256 on the host without a device), and only
    # when the shorter slices pay for the partials and the reduce
    assert w4.w4a16_gemm_auto_split_k(1322, 19456, 2560) == 1    # 760+ tiles: no room
    assert w4.w4a16_gemm_auto_split_k(1322, 19456, 2560, 32) == 1
    assert w4.w4a16_gemm_auto_split_k(1, 17408, 5120, 64) == 0   # no such group size
    assert w4.w4a16_gemm_auto_split_k(4096, 17408, 5120) == 1
    assert w4.w4a16_gemm_auto_split_k(128, 17408, 5120) == 2     # 68 tiles of 128 x 256
    assert w4.w4a16_gemm_auto_split_k(1322, 2560, 9728) == 2     # tall K: 120 tiles of 112 rows
    assert w4.w4a16_gemm_auto_split_k(4096, 64, 8192) > 1        # 32 tiles, 64 groups
    for M, N, K in ((100, 256, 8192), (1322, 2560, 9728), (4096, 64, 8192)):
        sk = w4.w4a16_gemm_auto_split_k(M, N, K)
        assert sk in (1, 2, 4, 8, 16)
    # the decode GEMV splits only for its register budget (<= 64 groups per slice)
    assert w4.w4a16_gemm_auto_split_k(1, 17408, 5120) == 1
    assert w4.w4a16_gemm_auto_split_k(1, 256, 512) == 1
    assert w4.w4a16_gemm_auto_split_k(1, 8192, 16384) == 2
    for M in (1, 2, 16, 100):
        sk = w4.w4a16_gemm_auto_split_k(M, 256, 8192)
        assert sk in (1, 2, 4, 8, 16)
    # the decode GEMV holds at most 64 groups of x per lane: K = 32768 forces SK >= 4
    assert w4.w4a16_gemm_auto_split_k(1, 65536, 32768) >= 4
    assert w4.w4a16_gemm_auto_split_k(0, 64, 128) == 0
    assert w4.w4a16_gemm_auto_split_k(1, 64, 100) == 0


def test_auto_config_rule():
    """The automatic path, variant and split at the documented regime
    boundaries (256 compute units assumed on the host without a device)."""
    ac = w4.w4a16_gemm_auto_config
    assert ac(1, 17408, 5120) == (1, 0, 1)           # decode GEMV, MFMA layout, one slice
    assert ac(16, 8192, 8192) == (2, 6, 1)           # 9-16 rows: LDS-staged small batch
    assert ac(9, 8192, 8192)[:2] == (2, 6)
    assert ac(8, 8192, 8192)[:2] == (2, 1)           # up to 8 rows: one column tile per wave
    assert ac(24, 8192, 8192)[:2] == (2, 2)          # 17-32 rows: two column tiles per wave
    assert ac(16, 896, 5120) == (2, 6, 8)            # 28 workgroups: split to fill the GPU
    path, rows, sk = ac(1322, 19456, 2560)
    assert (path, rows, sk) == (3, 144, 1)            # prefill: 144-row tiles, 3 rounds
    # tile path at small M (measured against every explicit choice): 48-row
    # tiles, SK 16 only while 16 slices' partials stay small
    assert ac(64, 896, 5120) == (3, 48, 16)
    assert ac(128, 896, 5120) == (3, 48, 8)
    assert ac(64, 2048, 5120) == (3, 48, 8)
    assert ac(1322, 19456, 2560, 32)[0] == 3
    assert ac(1, 256, 512, 32)[0] == 3               # group 32 always on the tile kernel
    assert ac(0, 64, 128) == (0, -1, 0)              # nothing would run
    with pytest.raises(RuntimeError):
        ac(1, 64, 100)                               # K not a multiple of 128
    for M in (1, 2, 16, 17, 48, 49, 100, 1322):
        path, var, sk = ac(M, 4096, 4096)
        assert path in (1, 2, 3) and sk in (1, 2, 4, 8, 16)
        assert sk == w4.w4a16_gemm_auto_split_k(M, 4096, 4096)


def test_workspace_sizes():
    # the split-K partials [SK, M, N] fp32 (rounded up to 256 bytes) when the
    # effective split is above 1; on the tile path with a wide N (at least 32
    # column tiles of 256 at group 128, 8 at group 32) also room for the
    # pre-pass row sums [K/g, round_up(M, 4)] fp32, which the call then uses
    # (with less room, or none, the tile kernel forms the row sums itself)
    assert w4.w4a16_gemm_workspace_bytes(16, 8192, 8192, 8) == 8 * 16 * 8192 * 4
    assert w4.w4a16_gemm_workspace_bytes(16, 8192, 8192, 1) == 0
    assert w4.w4a16_gemm_workspace_bytes(1, 17408, 5120, 1) == 0
    assert w4.w4a16_gemm_workspace_bytes(1322, 19456, 2560, 1) == 20 * 1324 * 4
    assert w4.w4a16_gemm_workspace_bytes(1322, 19456, 2560, 0) == 20 * 1324 * 4   # auto: SK 1
    assert w4.w4a16_gemm_workspace_bytes(1322, 7936, 2560, 1) == 0                 # 31 column tiles
    assert w4.w4a16_gemm_workspace_bytes(1322, 7937, 2560, 1) == 20 * 1324 * 4     # 32
    assert w4.w4a16_gemm_workspace_bytes(100, 64, 256, 2) == ((2 * 100 * 64 * 4 + 255) // 256) * 256
    assert w4.w4a16_gemm_workspace_bytes(100, 8192, 256, 2) == 2 * 100 * 8192 * 4 + 2 * 100 * 4
    assert w4.w4a16_gemm_workspace_bytes(16, 64, 100, 1) == 0     # invalid K
    for M in (1, 2, 16, 20, 40, 64, 1322):
        for sk in (1, 2, 4):
            want = 0 if sk == 1 else ((sk * M * 512 * 4 + 255) // 256) * 256
            assert w4.w4a16_gemm_workspace_bytes(M, 512, 1024, sk) == want, (M, sk)
            assert w4.w4a16_gemm_workspace_bytes(M, 512, 1024, sk, group_size=32) == want, (M, sk)
    # group 32: the tile path at every M; pre-pass from 8 column tiles
    assert w4.w4a16_gemm_workspace_bytes(1322, 19456, 2560, 1, group_size=32) == 80 * 1324 * 4
    assert w4.w4a16_gemm_workspace_bytes(1, 2048, 512, 1, group_size=32) == 16 * 4 * 4
    assert w4.w4a16_gemm_workspace_bytes(1, 1792, 512, 1, group_size=32) == 0
    # batched: [SK, B*M, N] partials when SK > 1, pre-pass row sums over all B*M rows
    assert w4.w4a16_gemm_batched_workspace_bytes(8, 256, 2048, 4096, 1) == 0
    assert w4.w4a16_gemm_batched_workspace_bytes(3, 5, 64, 256, 2) == ((2 * 15 * 64 * 4 + 255) // 256) * 256
    assert w4.w4a16_gemm_batched_workspace_bytes(0, 5, 64, 256, 1) == 0
    assert w4.w4a16_gemm_batched_workspace_bytes(2, 0, 64, 256, 2) == 0
    assert w4.w4a16_gemm_batched_workspace_bytes(8, 256, 2048, 4096, 2, group_size=32) == \
        2 * 2048 * 2048 * 4 + 128 * 2048 * 4
    assert w4.w4a16_gemm_batched_workspace_bytes(2, 50, 8192, 256, 1) == 2 * 100 * 4
    # forced kernels
    assert w4.w4a16_gemm_workspace_bytes(16, 64, 256, 1, group_size=64) == 0
    assert w4.w4a16_gemm_workspace_bytes(16, 64, 256, 2, w4.PATH_SKINNY, group_size=32) == 0   # not allowed
    assert w4.w4a16_gemm_workspace_bytes(16, 64, 256, 2, w4.PATH_TILE, 144, group_size=32) == 0
    assert w4.w4a16_gemm_workspace_bytes(16, 64, 256, 2, w4.PATH_TILE, 128, group_size=32) == 2 * 16 * 64 * 4
    assert w4.w4a16_gemm_workspace_bytes(16, 8192, 256, 1, w4.PATH_TILE, 48) == 2 * 16 * 4
    assert w4.w4a16_gemm_workspace_bytes(16, 8192, 256, 1, w4.PATH_SKINNY) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(w4, "_lib_handle", None)
    monkeypatch.setattr(w4, "LIB_PATH", "/nonexistent/libw4a16.so")
    with pytest.raises(RuntimeError, match="not built"):
        w4._lib()
