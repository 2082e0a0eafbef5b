"""Python binding of the W4A16 GEMM library (libw4a16.so, C ABI in include/w4a16.h;
the kernel-forcing entry points used by tests and benchmarks are declared in
csrc/w4a16_internal.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library. PyTorch provides device memory and the current
stream. There is no fallback: if the library is not built, every call raises.

bf16 tensors are passed as torch.bfloat16 (their raw bits are what the
library reads); packed weights and nibbles are torch.uint8; group sizes are
torch.int32.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "w4a16.h")
INTERNAL_HEADER = os.path.join(_HERE, "csrc", "w4a16_internal.h")

GROUP_SIZE = 128
PATH_AUTO, PATH_GEMV, PATH_SKINNY, PATH_TILE = 0, 1, 2, 3

_STATUS_NAMES = {0: "W4A16_OK", 1: "W4A16_ERR_NULL", 2: "W4A16_ERR_SHAPE", 3: "W4A16_ERR_GROUP_SIZE",
                 4: "W4A16_ERR_SPLIT_K", 5: "W4A16_ERR_WORKSPACE", 6: "W4A16_ERR_ALIGN",
                 7: "W4A16_ERR_LAUNCH"}


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class _Config(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("variant", ctypes.c_int32)]


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"W4A16 HIP library not built ({LIB_PATH} missing); run "
                           "python -m bf16_activation_quantized_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "w4a16_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "w4a16_pack_int4": (ctypes.c_int, [P, P, I64, I64, P]),
        "w4a16_gemm_auto_split_k": (I32, [I64, I64, I64, I32]),
        "w4a16_gemm_workspace_bytes": (SZ, [I64, I64, I64, I32]),
        "w4a16_gemm_workspace_bytes_gs": (SZ, [I64, I64, I64, I32, I32]),
        "w4a16_gemm": (ctypes.c_int, [P, P, P, P, I64, I64, I64, I32, I32, P, SZ, P]),
        "w4a16_gemm_grouped": (ctypes.c_int, [P, P, P, P, P, I32, I64, I64, I64, I32, P]),
        "w4a16_gemm_batched_workspace_bytes": (SZ, [I32, I64, I64, I64, I32, I32]),
        "w4a16_gemm_batched": (ctypes.c_int, [P, P, P, P, I32, I64, I64, I64, I32, I32, P, SZ, P]),
        "w4a16_splitk_reduce": (ctypes.c_int, [P, P, I32, I64, I64, P]),
        "w4a16_gemm_noalloc": (ctypes.c_int, [P, P, P, P, I64, I64, I64, I32, I32, P]),
        # internal entry points that force a kernel (tests, benchmarks)
        "w4a16_gemm_auto_config": (ctypes.c_int, [I64, I64, I64, I32, P, P]),
        "w4a16_gemm_workspace_bytes_ex": (SZ, [I64, I64, I64, I32, I32, P]),
        "w4a16_gemm_ex": (ctypes.c_int, [P, P, P, P, I64, I64, I64, I32, I32, P, SZ, P, P]),
        "w4a16_gemm_grouped_ex": (ctypes.c_int, [P, P, P, P, P, I32, I64, I64, I64, I32, P, P]),
        "w4a16_gemm_batched_workspace_bytes_ex": (SZ, [I32, I64, I64, I64, I32, I32, P]),
        "w4a16_gemm_batched_ex": (ctypes.c_int, [P, P, P, P, I32, I64, I64, I64, I32, I32, P, SZ, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib_handle = L
    return L


def header_functions(path: str = HEADER) -> list:
    """Names of the functions a header (default include/w4a16.h) declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    try:
        return _lib().w4a16_status_string(int(status)).decode()
    except RuntimeError:
        return _STATUS_NAMES.get(int(status), "unknown")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _cfg(path: Optional[int], variant: Optional[int]):
    if path is None and variant is None:
        return None
    return ctypes.byref(_Config(int(path or 0), int(-1 if variant is None else variant)))


def _raise(status: int, what: str):
    if status != 0:
        raise W4A16Error(status, what)


# ------------------------------------------------------------------ entry points

def w4a16_pack_int4(q: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [..., K] uint8 nibbles -> packed [..., K/2] (low nibble = even k)."""
    _check(q, "q", torch.uint8)
    K = q.shape[-1]
    rows = q.numel() // K if K else 0
    if out is None:
        out = torch.empty(q.shape[:-1] + (K // 2,), dtype=torch.uint8, device=q.device)
    _check(out, "out", torch.uint8, q.shape[:-1] + (K // 2,))
    _raise(_lib().w4a16_pack_int4(_ptr(q), _ptr(out), rows, K, _stream(stream)), "w4a16_pack_int4")
    return out


def w4a16_gemm_auto_split_k(M: int, N: int, K: int, group_size: int = GROUP_SIZE) -> int:
    return int(_lib().w4a16_gemm_auto_split_k(M, N, K, group_size))


def w4a16_gemm_auto_config(M: int, N: int, K: int, group_size: int = GROUP_SIZE) -> tuple:
    """The automatic choice of w4a16_gemm at these sizes (internal entry
    point): (path, variant, split_k); path 0 when nothing would run (M = 0)."""
    cfg, sk = _Config(), ctypes.c_int32(0)
    _raise(_lib().w4a16_gemm_auto_config(M, N, K, group_size, ctypes.byref(cfg), ctypes.byref(sk)),
           "w4a16_gemm_auto_config")
    return int(cfg.path), int(cfg.variant), int(sk.value)


def w4a16_gemm_workspace_bytes(M: int, N: int, K: int, split_k: int = 0,
                               path: Optional[int] = None, variant: Optional[int] = None,
                               group_size: int = GROUP_SIZE) -> int:
    """Workspace bytes of w4a16_gemm (0 when the effective split is 1)."""
    cfg = _cfg(path, variant)
    if cfg is not None:
        return int(_lib().w4a16_gemm_workspace_bytes_ex(M, N, K, group_size, split_k, cfg))
    if group_size != GROUP_SIZE:
        return int(_lib().w4a16_gemm_workspace_bytes_gs(M, N, K, group_size, split_k))
    return int(_lib().w4a16_gemm_workspace_bytes(M, N, K, split_k))


def _workspace(need: int, workspace: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4 + 1, dtype=torch.float32, device=device)
    if workspace is not None:
        _check(workspace, "workspace", torch.float32)
    return workspace


def w4a16_gemm(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor,
               y: Optional[torch.Tensor] = None, split_k: int = 0,
               workspace: Optional[torch.Tensor] = None, path: Optional[int] = None,
               variant: Optional[int] = None, stream=None, group_size: int = GROUP_SIZE) -> torch.Tensor:
    """Y[M, N] = X[M, K] . dequant(W)[N, K]^T (bf16 out, fp32 accumulation).
    `path` / `variant` force a kernel (internal entry point w4a16_gemm_ex)."""
    _check(x, "x", torch.bfloat16)
    M, K = x.shape
    N = w_packed.shape[0]
    _check(w_packed, "w_packed", torch.uint8, (N, K // 2))
    _check(scales, "scales", torch.bfloat16, (N, K // group_size))
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, (M, N))
    workspace = _workspace(w4a16_gemm_workspace_bytes(M, N, K, split_k, path, variant, group_size), workspace,
                           x.device)
    wbytes = 0 if workspace is None else workspace.numel() * 4
    cfg = _cfg(path, variant)
    L = _lib()
    if cfg is None:
        st = L.w4a16_gemm(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(y), M, N, K, group_size, split_k,
                          _ptr(workspace), wbytes, _stream(stream))
    else:
        st = L.w4a16_gemm_ex(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(y), M, N, K, group_size, split_k,
                             _ptr(workspace), wbytes, _stream(stream), cfg)
    _raise(st, "w4a16_gemm")
    return y


NOALLOC_SCRATCH_BYTES = 16 << 20


def w4a16_gemm_noalloc(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor, y: torch.Tensor,
                       split_k: int = 0, stream=None, group_size: int = GROUP_SIZE) -> torch.Tensor:
    """w4a16_gemm with the library's own device scratch in place of a
    workspace (the C entry point allocates nothing; y must be given)."""
    _check(x, "x", torch.bfloat16)
    M, K = x.shape
    N = w_packed.shape[0]
    _check(w_packed, "w_packed", torch.uint8, (N, K // 2))
    _check(scales, "scales", torch.bfloat16, (N, K // group_size))
    _check(y, "y", torch.bfloat16, (M, N))
    _raise(_lib().w4a16_gemm_noalloc(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(y), M, N, K, group_size, split_k,
                                     _stream(stream)), "w4a16_gemm_noalloc")
    return y


def w4a16_gemm_grouped(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor,
                       m_sizes: torch.Tensor, y: Optional[torch.Tensor] = None,
                       variant: Optional[int] = None, stream=None, group_size: int = GROUP_SIZE) -> torch.Tensor:
    """Grouped GEMM in one launch; m_sizes stays on the device. `variant`
    forces the tile height in rows (internal entry point)."""
    _check(x, "x", torch.bfloat16)
    M_total, K = x.shape
    G, N = w_packed.shape[0], w_packed.shape[1]
    _check(w_packed, "w_packed", torch.uint8, (G, N, K // 2))
    _check(scales, "scales", torch.bfloat16, (G, N, K // group_size))
    _check(m_sizes, "m_sizes", torch.int32, (G,))
    if y is None:
        y = torch.empty((M_total, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, (M_total, N))
    L = _lib()
    if variant is None:
        st = L.w4a16_gemm_grouped(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(m_sizes), _ptr(y), G, M_total, N, K,
                                  group_size, _stream(stream))
    else:
        st = L.w4a16_gemm_grouped_ex(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(m_sizes), _ptr(y), G, M_total, N,
                                     K, group_size, _stream(stream), _cfg(PATH_TILE, variant))
    _raise(st, "w4a16_gemm_grouped")
    return y


def w4a16_gemm_batched_workspace_bytes(B: int, M: int, N: int, K: int, split_k: int = 0,
                                       variant: Optional[int] = None, group_size: int = GROUP_SIZE) -> int:
    L = _lib()
    if variant is None:
        return int(L.w4a16_gemm_batched_workspace_bytes(B, M, N, K, group_size, split_k))
    return int(L.w4a16_gemm_batched_workspace_bytes_ex(B, M, N, K, group_size, split_k, _cfg(PATH_TILE, variant)))


def w4a16_gemm_batched(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor,
                       y: Optional[torch.Tensor] = None, split_k: int = 0,
                       workspace: Optional[torch.Tensor] = None, variant: Optional[int] = None,
                       stream=None, group_size: int = GROUP_SIZE) -> torch.Tensor:
    """Y[b] = X[b] . dequant(W[b])^T for B independent problems, one launch."""
    _check(x, "x", torch.bfloat16)
    B, M, K = x.shape
    N = w_packed.shape[1]
    _check(w_packed, "w_packed", torch.uint8, (B, N, K // 2))
    _check(scales, "scales", torch.bfloat16, (B, N, K // group_size))
    if y is None:
        y = torch.empty((B, M, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, (B, M, N))
    workspace = _workspace(w4a16_gemm_batched_workspace_bytes(B, M, N, K, split_k, variant, group_size), workspace,
                           x.device)
    wbytes = 0 if workspace is None else workspace.numel() * 4
    L = _lib()
    if variant is None:
        st = L.w4a16_gemm_batched(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(y), B, M, N, K, group_size, split_k,
                                  _ptr(workspace), wbytes, _stream(stream))
    else:
        st = L.w4a16_gemm_batched_ex(_ptr(x), _ptr(w_packed), _ptr(scales), _ptr(y), B, M, N, K, group_size,
                                     split_k, _ptr(workspace), wbytes, _stream(stream), _cfg(PATH_TILE, variant))
    _raise(st, "w4a16_gemm_batched")
    return y


def w4a16_splitk_reduce(workspace: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = bf16_rne(sum over slices of workspace[SK, M, N]) in slice order."""
    _check(workspace, "workspace", torch.float32)
    SK, M, N = workspace.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=workspace.device)
    _check(y, "y", torch.bfloat16, (M, N))
    _raise(_lib().w4a16_splitk_reduce(_ptr(workspace), _ptr(y), SK, M, N, _stream(stream)), "w4a16_splitk_reduce")
    return y
