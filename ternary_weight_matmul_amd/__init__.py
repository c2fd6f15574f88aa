"""Ternary-weight matmul for AMD MI355X (gfx950): thin Python binding of libtern.so.

Every step of the computation runs in the HIP kernels behind the C ABI of
``include/tern.h``; this module only marshals arguments (device pointers,
sizes, dtype codes and the current HIP stream).  PyTorch supplies device
memory and streams.  If ``libtern.so`` has not been built, importing the
library raises: there is no fallback implementation.

    import ternary_weight_matmul_amd as tern
    packed = tern.pack(T)                     # int8 [N,K] in {-1,0,1} -> uint8 [N,K/4]
    T2 = tern.unpack(packed, K)               # uint8 [N,K/4] -> int8 [N,K]
    y = tern.matmul(x, packed, scales, out_dtype=torch.bfloat16)
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    DTYPE_CODE,
    PATH_AUTO,
    PATH_GEMV,
    PATH_MFMA,
    STATUS,
    TernError,
    lib,
    library_path,
)
from .ops import (block_map, dequant, matmul, matmul_blockmap, matmul_blockmap_into, matmul_into,  # noqa: F401
                  matmul_s8, matmul_s8_into, pack, quantize_scales, shard_columns, shard_k, stream_copy, unpack)

GROUP = 128
GEMV_MAX_M = 4
