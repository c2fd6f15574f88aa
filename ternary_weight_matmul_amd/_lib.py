"""ctypes loader for libtern.so (built in-tree by ``build.py``)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libtern.so"

STATUS = {
    0: "TERN_OK",
    1: "TERN_ERR_NULL",
    2: "TERN_ERR_SHAPE",
    3: "TERN_ERR_GROUP",
    4: "TERN_ERR_DTYPE",
    5: "TERN_ERR_ALIGN",
    6: "TERN_ERR_UNSUPPORTED",
    7: "TERN_ERR_HIP",
}
DTYPE_CODE = {"f16": 0, "bf16": 1, "f32": 2}
PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_GEMV_MFMA, PATH_GEMV_FP4, PATH_GEMV_B16 = 0, 1, 2, 3, 4, 5


class TernError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.tern_status_string(status).decode() if lib is not None else STATUS.get(status, "?")
        super().__init__(f"{where}: {msg}")


def library_path() -> str:
    return os.environ.get("TERN_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def _load() -> ctypes.CDLL:
    # One HIP runtime per process: torch ships its own libamdhip64 (soname
    # libamdhip64.so.7, loaded through an unversioned NEEDED entry).  Importing
    # torch first makes libtern.so's NEEDED libamdhip64.so.7 resolve to that
    # same, already-loaded runtime; loading libtern.so first would bring in a
    # second runtime, and torch's stream and memory handles would be foreign
    # to it.
    import torch  # noqa: F401

    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python ternary_weight_matmul_amd/build.py` "
            "(hipcc --offload-arch=gfx950). There is no non-HIP fallback.")
    L = ctypes.CDLL(path)
    i64, vp, i32, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    L.tern_status_string.argtypes = [c_int]
    L.tern_status_string.restype = ctypes.c_char_p
    L.tern_version.argtypes = []
    L.tern_version.restype = c_int
    L.tern_pack.argtypes = [vp, vp, i64, i64, vp]
    L.tern_pack.restype = c_int
    L.tern_unpack.argtypes = [vp, vp, i64, i64, vp]
    L.tern_unpack.restype = c_int
    L.tern_matmul.argtypes = [vp, c_int, vp, vp, vp, c_int, i64, i64, i64, i32, vp]
    L.tern_matmul.restype = c_int
    L.tern_matmul_path.argtypes = [vp, c_int, vp, vp, vp, c_int, i64, i64, i64, i32, c_int, vp]
    L.tern_matmul_path.restype = c_int
    L.tern_dequant.argtypes = [vp, vp, vp, c_int, i64, i64, i32, vp]
    L.tern_dequant.restype = c_int
    L.tern_block_map.argtypes = [vp, vp, i64, i64, i32, vp]
    L.tern_block_map.restype = c_int
    L.tern_matmul_blockmap.argtypes = [vp, c_int, vp, vp, vp, vp, c_int, i64, i64, i64, i32, vp]
    L.tern_matmul_blockmap.restype = c_int
    L.tern_quantize_scales.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    L.tern_quantize_scales.restype = c_int
    L.tern_matmul_s8.argtypes = [vp, c_int, vp, vp, vp, vp, c_int, i64, i64, i64, i32, c_int, vp]
    L.tern_matmul_s8.restype = c_int
    L.tern_stream_copy.argtypes = [vp, vp, ctypes.c_uint64, vp]
    L.tern_stream_copy.restype = c_int
    return L


lib = None
lib = _load()
