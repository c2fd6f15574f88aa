"""The C ABI on the CPU: the library loads, exports what include/tern.h
declares, and rejects bad arguments before touching a GPU.

No call here reaches a kernel launch: every call either fails validation or
has an empty size (which returns TERN_OK without launching).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tern.h")

tern = pytest.importorskip("ternary_weight_matmul_amd", reason="libtern.so not built")
L = tern.lib

OK, NULL, SHAPE, GROUP, DTYPE, ALIGN, UNSUP = 0, 1, 2, 3, 4, 5, 6
F16, BF16, F32 = 0, 1, 2
P = 4096  # a fake, 16-byte aligned, non-NULL device address; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tern_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("tern_pack", "tern_unpack", "tern_matmul", "tern_matmul_path",
                 "tern_status_string", "tern_version"):
        assert want in names


def test_every_declared_symbol_is_exported():
    so = ctypes.CDLL(tern.library_path())
    for name in declared_functions():
        assert hasattr(so, name), name


def test_status_strings():
    for code, name in tern.STATUS.items():
        s = L.tern_status_string(code).decode()
        assert s.startswith(name), (code, s)
    assert L.tern_status_string(99).decode().startswith("TERN_ERR_UNKNOWN")
    assert L.tern_version() >= 100


def mm(X=P, xd=F16, W=P, S=P, Y=P, yd=F32, M=1, N=16, K=128, G=128, path=0):
    return L.tern_matmul_path(X, xd, W, S, Y, yd, M, N, K, G, path, None)


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), SHAPE), (dict(N=-1), SHAPE), (dict(K=-4), SHAPE), (dict(K=130), SHAPE),
    (dict(K=1 << 31), SHAPE), (dict(M=1 << 31), SHAPE),
    (dict(K=192), GROUP), (dict(G=0), GROUP), (dict(G=-128), GROUP),
    (dict(K=256, G=64), UNSUP), (dict(K=256, G=256), UNSUP),
    (dict(xd=F32), DTYPE), (dict(xd=7), DTYPE), (dict(yd=9), DTYPE),
    (dict(X=0), NULL), (dict(W=0), NULL), (dict(S=0), NULL), (dict(Y=0), NULL),
    (dict(X=P + 8), ALIGN), (dict(W=P + 4), ALIGN), (dict(S=P + 1), ALIGN), (dict(Y=P + 2), ALIGN),
    (dict(Y=P + 1, yd=F16), ALIGN),
    (dict(M=5, path=1), UNSUP), (dict(path=6), UNSUP),
    (dict(M=1, K=128 * 1024, path=1), UNSUP),
    # the 16-row decode kernel: M <= 16, K <= 2^20
    (dict(M=17, path=5), UNSUP), (dict(M=4, K=(1 << 20) + 128, path=5), UNSUP),
    # the fp4 matrix-core decode kernel: bf16 activations only, M <= 4
    (dict(path=4), UNSUP), (dict(xd=BF16, M=5, path=4), UNSUP), (dict(xd=BF16, M=1, K=33280, path=4), UNSUP),
    # the matrix-core decode kernel: M <= 4, activations staged whole in LDS
    (dict(M=5, path=3), UNSUP), (dict(M=4, K=20480, path=3), UNSUP), (dict(M=1, K=128 * 1024, path=3), UNSUP),
])
def test_matmul_rejects(kw, want):
    assert mm(**kw) == want


@pytest.mark.parametrize("kw", [dict(M=0), dict(N=0), dict(M=0, N=0, K=0)])
def test_matmul_empty_is_ok_without_pointers(kw):
    assert mm(X=0, W=0, S=0, Y=0, **kw) == OK


def test_matmul_k0_needs_only_y():
    # K = 0 and M, N > 0: Y is written (zeros), X/W/S are never read
    assert mm(X=0, W=0, S=0, Y=0, K=0) == NULL


@pytest.mark.parametrize("fn", ["tern_pack", "tern_unpack"])
def test_pack_unpack_reject(fn):
    f = getattr(L, fn)
    assert f(P, P, 4, 6, None) == SHAPE
    assert f(P, P, -1, 8, None) == SHAPE
    assert f(0, P, 4, 8, None) == NULL
    assert f(P, 0, 4, 8, None) == NULL
    assert f(P + 4, P, 4, 8, None) == ALIGN
    assert f(P, P + 8, 4, 8, None) == ALIGN
    assert f(0, 0, 0, 8, None) == OK
    assert f(0, 0, 5, 0, None) == OK


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        tern.pack(torch.zeros((2, 8), dtype=torch.int8))


def test_single_hip_runtime_in_process():
    """The binding shares torch's HIP runtime instead of loading a second one."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


def mm8(X=P, xd=BF16, W=P, Q=P, R=P, Y=P, yd=F32, M=1, N=16, K=128, G=128, path=0):
    return L.tern_matmul_s8(X, xd, W, Q, R, Y, yd, M, N, K, G, path, None)


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), SHAPE), (dict(K=130), SHAPE), (dict(K=192), GROUP), (dict(K=256, G=64), UNSUP),
    (dict(xd=F32), DTYPE), (dict(yd=9), DTYPE),
    (dict(X=0), NULL), (dict(W=0), NULL), (dict(Q=0), NULL), (dict(R=0), NULL), (dict(Y=0), NULL),
    (dict(X=P + 8), ALIGN), (dict(W=P + 4), ALIGN), (dict(R=P + 2), ALIGN), (dict(Y=P + 2), ALIGN),
    (dict(M=5, path=1), UNSUP), (dict(path=6), UNSUP), (dict(M=5, path=3), UNSUP), (dict(xd=F16, path=4), UNSUP),
    (dict(M=17, path=5), UNSUP),
])
def test_matmul_s8_rejects(kw, want):
    assert mm8(**kw) == want


def test_matmul_s8_codes_need_no_alignment_and_empty_is_ok():
    # int8 codes may start at any byte: an odd code pointer passes the
    # alignment check, so the NULL row factor checked after it is reported
    assert mm8(Q=P + 1, R=0) == NULL
    assert mm8(X=0, W=0, Q=0, R=0, Y=0, M=0) == OK


def test_quantize_scales_rejects():
    f = L.tern_quantize_scales
    assert f(P, P, P, -1, 128, 128, None) == SHAPE
    assert f(P, P, P, 4, 192, 128, None) == GROUP
    assert f(P, P, P, 4, 256, 64, None) == UNSUP
    assert f(0, P, P, 4, 128, 128, None) == NULL
    assert f(P, 0, P, 4, 128, 128, None) == NULL
    assert f(P, P, 0, 4, 128, 128, None) == NULL
    assert f(P + 1, P, P, 4, 128, 128, None) == ALIGN
    assert f(P, P, P + 2, 4, 128, 128, None) == ALIGN
    assert f(0, 0, 0, 0, 128, 128, None) == OK


def test_block_map_rejects():
    f = L.tern_block_map
    assert f(P, P, -1, 128, 128, None) == SHAPE
    assert f(P, P, 4, 130, 128, None) == SHAPE
    assert f(P, P, 4, 192, 128, None) == GROUP
    assert f(P, P, 4, 256, 64, None) == UNSUP
    assert f(0, P, 4, 128, 128, None) == NULL
    assert f(P, 0, 4, 128, 128, None) == NULL
    assert f(P + 8, P, 4, 128, 128, None) == ALIGN
    assert f(P, P + 2, 4, 128, 128, None) == ALIGN
    assert f(0, 0, 0, 128, 128, None) == OK
    assert f(0, 0, 4, 0, 128, None) == OK


def mmb(X=P, xd=BF16, W=P, S=P, MAP=P, Y=P, yd=F32, M=1, N=16, K=128, G=128):
    return L.tern_matmul_blockmap(X, xd, W, S, MAP, Y, yd, M, N, K, G, None)


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), SHAPE), (dict(K=130), SHAPE), (dict(K=192), GROUP), (dict(K=256, G=64), UNSUP),
    (dict(xd=F32), DTYPE), (dict(X=0), NULL), (dict(S=0), NULL), (dict(MAP=0), NULL), (dict(Y=0), NULL),
    (dict(S=P + 1), ALIGN), (dict(MAP=P + 2), ALIGN), (dict(X=P + 8), ALIGN),
])
def test_matmul_blockmap_rejects(kw, want):
    assert mmb(**kw) == want
    assert mmb(X=0, W=0, S=0, MAP=0, Y=0, M=0) == OK


def test_stream_copy_rejects():
    """The calibration read/copy validates before launching; zero bytes launch nothing."""
    f = L.tern_stream_copy
    assert f(0, 0, 0, None) == OK
    assert f(P, P, 0, None) == OK
    assert f(0, 0, 16, None) == NULL
    assert f(P, 0, 17, None) == SHAPE
    assert f(P, 0, (1 << 40) + 16, None) == SHAPE
    assert f(P + 8, 0, 16, None) == ALIGN
    assert f(P, P + 4, 16, None) == ALIGN
