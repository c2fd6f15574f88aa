"""Torch-tensor entry points over the C ABI (argument marshalling only).

Each function checks what only the binding can check (tensor device, dtype,
contiguity), passes raw device pointers, sizes and the current HIP stream to
the library, and raises TernError on a non-OK status.  The library itself
validates shapes, group, alignment and dtypes before launching anything.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import (DTYPE_CODE, PATH_AUTO, PATH_GEMV, PATH_GEMV_B16, PATH_GEMV_FP4, PATH_GEMV_MFMA, PATH_MFMA,
                   TernError, lib)

_TORCH_CODE = {torch.float16: DTYPE_CODE["f16"], torch.bfloat16: DTYPE_CODE["bf16"],
               torch.float32: DTYPE_CODE["f32"]}
_PATHS = {"auto": PATH_AUTO, "gemv": PATH_GEMV, "mfma": PATH_MFMA, "gemv_mfma": PATH_GEMV_MFMA,
          "gemv_fp4": PATH_GEMV_FP4, "gemv_b16": PATH_GEMV_B16}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int = 2) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (reshape to 2-D and call .contiguous())")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise TernError(status, where)


def pack(T: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 [N,K] (values -1/0/+1) -> uint8 [N,K/4], 2 bits per weight."""
    _need(T, "T", torch.int8)
    N, K = T.shape
    if out is None:
        out = torch.empty((N, K // 4), dtype=torch.uint8, device=T.device)
    _need(out, "out", torch.uint8)
    if tuple(out.shape) != (N, K // 4):
        raise ValueError("out must be [N, K/4]")
    _check(lib.tern_pack(T.data_ptr(), out.data_ptr(), N, K, _stream(T)), "tern_pack")
    return out


def unpack(packed: torch.Tensor, K: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """uint8 [N,K/4] -> int8 [N,K] in {-1,0,+1}."""
    _need(packed, "packed", torch.uint8)
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed has {packed.shape[1]} bytes per row, K={K} needs {K // 4}")
    if out is None:
        out = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _need(out, "out", torch.int8)
    _check(lib.tern_unpack(packed.data_ptr(), out.data_ptr(), N, K, _stream(packed)), "tern_unpack")
    return out


def matmul_into(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, out: torch.Tensor,
                group: int = 128, path: str = "auto") -> torch.Tensor:
    """out[M,N] = x[M,K] . (T*S)^T; x fp16/bf16, scales fp16 [N,K/group]."""
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    _need(x, "x", x.dtype)
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.float16)
    if out.dtype not in _TORCH_CODE:
        raise TypeError("out must be float32, bfloat16 or float16")
    _need(out, "out", out.dtype)
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or tuple(scales.shape) != (N, K // group if group > 0 else 0) \
            or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, packed {tuple(packed.shape)}, "
                         f"scales {tuple(scales.shape)}, out {tuple(out.shape)}")
    st = lib.tern_matmul_path(x.data_ptr(), _TORCH_CODE[x.dtype], packed.data_ptr(), scales.data_ptr(),
                              out.data_ptr(), _TORCH_CODE[out.dtype], M, N, K, group, _PATHS[path],
                              _stream(x))
    _check(st, "tern_matmul")
    return out


def matmul(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
           out_dtype: torch.dtype = torch.bfloat16, group: int = 128, path: str = "auto") -> torch.Tensor:
    """Y[M,N] = x[M,K] . (T*S)^T with fp32 accumulation; returns a new tensor."""
    out = torch.empty((x.shape[0], packed.shape[0]), dtype=out_dtype, device=x.device)
    return matmul_into(x, packed, scales, out, group, path)


def dequant(packed: torch.Tensor, scales: torch.Tensor, out_dtype: torch.dtype = torch.float16,
            group: int = 128, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense W[N,K] = t * s (the pages' dequantise-then-GEMM comparison route)."""
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.float16)
    N = packed.shape[0]
    K = packed.shape[1] * 4
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=packed.device)
    if out.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("out must be float16 or bfloat16")
    _need(out, "out", out.dtype)
    if tuple(out.shape) != (N, K) or (group > 0 and tuple(scales.shape) != (N, K // group)):
        raise ValueError("shape mismatch")
    _check(lib.tern_dequant(packed.data_ptr(), scales.data_ptr(), out.data_ptr(), _TORCH_CODE[out.dtype],
                            N, K, group, _stream(packed)), "tern_dequant")
    return out


# --- zero-block skipping -----------------------------------------------------

def block_map(packed: torch.Tensor, group: int = 128) -> torch.Tensor:
    """packed [N,K/4] -> int32 [N, ceil(K/group/32)], the bits of tern_block_map (stored as int32)."""
    _need(packed, "packed", torch.uint8)
    N = packed.shape[0]
    K = packed.shape[1] * 4
    words = (K // group + 31) // 32
    out = torch.empty((N, words), dtype=torch.int32, device=packed.device)
    _check(lib.tern_block_map(packed.data_ptr(), out.data_ptr(), N, K, group, _stream(packed)),
           "tern_block_map")
    return out


def matmul_blockmap_into(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, bmap: torch.Tensor,
                         out: torch.Tensor, group: int = 128) -> torch.Tensor:
    """matmul_into that skips the blocks `bmap` (from block_map) leaves unmarked."""
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    _need(x, "x", x.dtype)
    _need(packed, "packed", torch.uint8)
    _need(scales, "scales", torch.float16)
    _need(bmap, "bmap", torch.int32)
    if out.dtype not in _TORCH_CODE:
        raise TypeError("out must be float32, bfloat16 or float16")
    _need(out, "out", out.dtype)
    M, K = x.shape
    N = packed.shape[0]
    words = (K // group + 31) // 32 if group > 0 else 0
    if packed.shape[1] * 4 != K or tuple(scales.shape) != (N, K // group if group > 0 else 0) \
            or tuple(bmap.shape) != (N, words) or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, packed {tuple(packed.shape)}, "
                         f"scales {tuple(scales.shape)}, bmap {tuple(bmap.shape)}, out {tuple(out.shape)}")
    st = lib.tern_matmul_blockmap(x.data_ptr(), _TORCH_CODE[x.dtype], packed.data_ptr(), scales.data_ptr(),
                                  bmap.data_ptr(), out.data_ptr(), _TORCH_CODE[out.dtype], M, N, K, group,
                                  _stream(x))
    _check(st, "tern_matmul_blockmap")
    return out


def matmul_blockmap(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, bmap: torch.Tensor,
                    out_dtype: torch.dtype = torch.bfloat16, group: int = 128) -> torch.Tensor:
    out = torch.empty((x.shape[0], packed.shape[0]), dtype=out_dtype, device=x.device)
    return matmul_blockmap_into(x, packed, scales, bmap, out, group)


# --- int8 block scales -------------------------------------------------------

def quantize_scales(scales: torch.Tensor, group: int = 128):
    """fp16 scales [N,G] -> (int8 codes [N,G], fp32 row factors [N]); scale = q * r."""
    _need(scales, "scales", torch.float16)
    N, G = scales.shape
    q = torch.empty((N, G), dtype=torch.int8, device=scales.device)
    r = torch.empty((N,), dtype=torch.float32, device=scales.device)
    _check(lib.tern_quantize_scales(scales.data_ptr(), q.data_ptr(), r.data_ptr(), N, G * group, group,
                                    _stream(scales)), "tern_quantize_scales")
    return q, r


def matmul_s8_into(x: torch.Tensor, packed: torch.Tensor, scales_q: torch.Tensor, row_factor: torch.Tensor,
                   out: torch.Tensor, group: int = 128, path: str = "auto") -> torch.Tensor:
    """out[M,N] = x . (T * (q * r))^T with int8 block codes q [N,K/group] and row factors r [N]."""
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    _need(x, "x", x.dtype)
    _need(packed, "packed", torch.uint8)
    _need(scales_q, "scales_q", torch.int8)
    _need(row_factor, "row_factor", torch.float32, ndim=1)
    if out.dtype not in _TORCH_CODE:
        raise TypeError("out must be float32, bfloat16 or float16")
    _need(out, "out", out.dtype)
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or tuple(scales_q.shape) != (N, K // group if group > 0 else 0) \
            or tuple(row_factor.shape) != (N,) or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, packed {tuple(packed.shape)}, "
                         f"scales_q {tuple(scales_q.shape)}, row_factor {tuple(row_factor.shape)}, "
                         f"out {tuple(out.shape)}")
    st = lib.tern_matmul_s8(x.data_ptr(), _TORCH_CODE[x.dtype], packed.data_ptr(), scales_q.data_ptr(),
                            row_factor.data_ptr(), out.data_ptr(), _TORCH_CODE[out.dtype], M, N, K, group,
                            _PATHS[path], _stream(x))
    _check(st, "tern_matmul_s8")
    return out


def matmul_s8(x: torch.Tensor, packed: torch.Tensor, scales_q: torch.Tensor, row_factor: torch.Tensor,
              out_dtype: torch.dtype = torch.bfloat16, group: int = 128, path: str = "auto") -> torch.Tensor:
    out = torch.empty((x.shape[0], packed.shape[0]), dtype=out_dtype, device=x.device)
    return matmul_s8_into(x, packed, scales_q, row_factor, out, group, path)


# --- one GPU's share of a sharded layer (no communication here) -------------

def shard_columns(packed: torch.Tensor, scales: torch.Tensor, rank: int, world: int):
    """Column-parallel shard: whole rows n of W (output columns of Y).

    Rows [rank*N/world, (rank+1)*N/world) of the packed matrix and of the
    scales (2kiu.com/news/5082861 §5.1: a column split cuts the packed weight
    and its scale by output rows).  Row slices of row-major tensors are
    contiguous views: nothing is copied.
    """
    N = packed.shape[0]
    a, b = N * rank // world, N * (rank + 1) // world
    return packed[a:b], scales[a:b]


def shard_k(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, rank: int, world: int,
            group: int = 128):
    """Row-parallel shard: a K range cut on 128-weight block boundaries.

    The block boundaries keep every scale with its weights (§3.2, third check,
    and §5.1 of the same page: a K split must align with the blocks).  Returns
    contiguous copies of x[:, k0:k1], packed[:, k0/4:k1/4], scales[:, g0:g1];
    the partial products of all ranks sum to the full result.
    """
    K = x.shape[1]
    groups = K // group
    g0, g1 = groups * rank // world, groups * (rank + 1) // world
    k0, k1 = g0 * group, g1 * group
    return (x[:, k0:k1].contiguous(), packed[:, k0 // 4:k1 // 4].contiguous(),
            scales[:, g0:g1].contiguous())


def stream_copy(src: torch.Tensor, dst: Optional[torch.Tensor] = None, nbytes: Optional[int] = None) -> None:
    """Calibration only: stream ``nbytes`` bytes of ``src`` (all of it by default) and copy
    them into ``dst`` when given; with no ``dst`` the bytes are only read.  Device tensors,
    contiguous, 16-byte aligned; nbytes a multiple of 16."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds src")
    dptr = 0
    if dst is not None:
        if not dst.is_cuda or not dst.is_contiguous() or dst.numel() * dst.element_size() < n:
            raise ValueError("dst must be a contiguous device tensor of at least nbytes")
        dptr = dst.data_ptr()
    _check(lib.tern_stream_copy(src.data_ptr(), dptr, n, _stream(src)), "tern_stream_copy")
