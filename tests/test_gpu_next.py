"""GPU tests of the comparison route (dequantise) and of one GPU's shard of a
sharded layer, against the CPU oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import TORCH_DT, check, device, out_bits, problem_to_device  # noqa: E402

tern = pytest.importorskip("ternary_weight_matmul_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


O = oracle.default


@pytest.mark.parametrize("N,K", [(1, 128), (7, 640), (64, 5120), (3, 17408)])
@pytest.mark.parametrize("wd", ["f16", "bf16"])
def test_dequant_bit_exact(N, K, wd):
    p = workloads.make_custom(N + K, 1, K, N, reserved_rate=0.05, scale_lo=1e-4, scale_hi=8.0)
    _, w, s = problem_to_device(p)
    W = tern.dequant(w, s, out_dtype=TORCH_DT[wd])
    torch.cuda.synchronize()
    got = O().decode(out_bits(W, wd), wd)
    want = O().round(O().dequant(p.packed, p.scales, N, K), wd)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_dequant_route_matches_fused_kernel():
    # dequantise + a library GEMM (hipBLASLt through torch) vs tern_matmul, both vs the oracle
    p = workloads.make_custom(41, 64, 1024, 256, x_dtype="f16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    W = tern.dequant(w, s, out_dtype=torch.float16)
    y_route = (x.float() @ W.float().t()).contiguous()
    torch.cuda.synchronize()
    Y, B = O().matmul(p.x, "f16", p.packed, p.scales, 64, 256, 1024, threads=4)
    check(out_bits(y_route, "f32"), "f32", Y, B, "dequant route")
    check(out_bits(tern.matmul(x, w, s, out_dtype=torch.float32), "f32"), "f32", Y, B, "fused")


@pytest.mark.parametrize("M,K,N,world", [(1, 5120, 640, 4), (3, 2048, 333, 3), (40, 1024, 520, 2)])
def test_column_shards_concatenate_to_the_full_result(M, K, N, world):
    p = workloads.make_custom(60 + M, M, K, N, x_dtype="bf16", y_dtype="bf16")
    x, w, s = problem_to_device(p)
    full = tern.matmul(x, w, s, out_dtype=torch.bfloat16)
    parts = []
    for r in range(world):
        wr, sr = tern.shard_columns(w, s, r, world)
        assert wr.is_contiguous() and sr.is_contiguous()
        parts.append(tern.matmul(x, wr, sr, out_dtype=torch.bfloat16))
    cat = torch.cat(parts, dim=1)
    torch.cuda.synchronize()
    assert torch.equal(cat.view(torch.int16), full.view(torch.int16))   # each column is computed alike


@pytest.mark.parametrize("M,K,N,world", [(1, 5120, 300, 4), (2, 17408, 64, 8), (24, 2048, 200, 2)])
def test_k_shards_sum_to_the_full_result(M, K, N, world):
    p = workloads.make_custom(80 + M, M, K, N, x_dtype="bf16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    total = torch.zeros((M, N), dtype=torch.float32, device=device())
    for r in range(world):
        xr, wr, sr = tern.shard_k(x, w, s, r, world)
        assert xr.shape[1] % 128 == 0
        # the shard's bytes are the corresponding slice of the full packed matrix
        k0 = xr.shape[1] * r if K // 128 % world == 0 else None
        if k0 is not None:
            assert torch.equal(wr, w[:, k0 // 4:(k0 + xr.shape[1]) // 4])
        total += tern.matmul(xr, wr, sr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Y, B = O().matmul(p.x, "bf16", p.packed, p.scales, M, N, K, threads=4)
    # one extra fp32 rounding per added shard partial
    check(out_bits(total, "f32"), "f32", Y, B, "K shards")
